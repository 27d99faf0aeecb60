"""Pins of the oracle's sampling at temperature > 0.

Philox4x32-10 against the known-answer vectors published with the algorithm
(Salmon et al., SC 2011, Random123 distribution); Gumbel-max draws against
softmax(l / T) by a chi-square test; speculative rejection sampling against
the guarantees on the walkthrough's page ("贪心模式与随机模式要分别说明",
"分布重叠怎样影响平均推进量"): the committed token is distributed as the
target's p, the acceptance rate is sum_v min(p, q) = 1 - TV(p, q), and
min(p, q) + [p - q]_+ = p; at a vanishing temperature everything reduces to
the greedy rule.
"""
import numpy as np
import pytest
from scipy import stats

import oracle


@pytest.mark.parametrize("ctr,key,want", [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(ctr, key, want):
    assert tuple(int(x) for x in oracle.philox4x32_10(ctr, key)) == want


def test_uniforms_are_open_interval_and_uniform():
    u = oracle.uniform01(7, 3, np.arange(200000), 5)
    assert (u > 0).all() and (u < 1).all()
    counts = np.histogram(u, bins=20, range=(0, 1))[0]
    assert stats.chisquare(counts).pvalue > 1e-4


def test_uniforms_of_one_generator_call_are_distinct_and_uncorrelated():
    """Four consecutive indices share a counter and take its four words: they
    must differ and show no correlation at lags 1..4 (a word reused for
    several indices, or a counter reused across groups, would); rows and
    streams give unrelated values."""
    u = oracle.uniform01(11, 0, np.arange(400000), 3)
    g = u.reshape(-1, 4)
    assert all(len(set(row)) == 4 for row in g[:20000])          # a call's words differ
    dup = len(u) - len(np.unique(u))                             # 32-bit birthday collisions only
    assert dup <= 3 * len(u) ** 2 / 2.0 ** 33 + 10, dup
    z = u - 0.5
    for lag in (1, 2, 3, 4):
        r = float(np.mean(z[:-lag] * z[lag:]) / np.mean(z * z))
        assert abs(r) < 0.01, (lag, r)
    w = oracle.uniform01(11, 0, np.arange(400000), 4)
    y = oracle.uniform01(11, 1, np.arange(400000), 3)
    for other in (w, y):
        assert abs(float(np.corrcoef(u, other)[0, 1])) < 0.01
    # the four words of one call are the generator's own outputs
    x = oracle.philox4x32_10((np.uint32(5), np.uint32(3), np.uint32(0), np.uint32(0)), (np.uint32(11), np.uint32(0)))
    np.testing.assert_array_equal(u[20:24], (np.array([int(v) for v in x], dtype=np.float64) + 0.5) / 2.0 ** 32)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_gumbel_draws_follow_softmax(T):
    V, N = 6, 60000
    logits = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4])
    tok, _ = oracle.sample_tokens(np.tile(logits, (N, 1)), T, seed=11, stream=0)
    counts = np.bincount(tok, minlength=V)
    want = oracle.softmax_t(logits, T) * N
    assert stats.chisquare(counts, want).pvalue > 1e-4


def _round(p_logits, q_logits, n, T, seed):
    """n one-position rounds: d ~ q drawn per request, then verification."""
    V = len(p_logits)
    d, _ = oracle.sample_tokens(np.tile(q_logits, (n, 1)), T, seed, stream=0)
    draft = np.tile(q_logits, (n, 1, 1))
    target = np.tile(np.stack([p_logits, p_logits]), (n, 1, 1))
    out = oracle.accept_sampled(d[:, None], draft, target, T, seed)
    first = np.where(out["A"] == 1, d, out["next"])      # the committed token at the position
    return d, out, first


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_committed_token_is_distributed_as_the_target(T):
    p_logits = np.array([1.0, 0.2, -0.5, 2.2, 0.0])
    q_logits = np.array([0.1, 1.5, -0.2, 1.0, 0.6])
    n = 20000
    _, out, first = _round(p_logits, q_logits, n, T, seed=23)
    counts = np.bincount(first, minlength=5)
    assert stats.chisquare(counts, oracle.softmax_t(p_logits, T) * n).pvalue > 1e-4
    # acceptance rate = sum_v min(p, q) = 1 - TV within 5 sigma
    p, q = oracle.softmax_t(p_logits, T), oracle.softmax_t(q_logits, T)
    beta = np.minimum(p, q).sum()
    assert abs(beta - (1 - 0.5 * np.abs(p - q).sum())) < 1e-15
    assert abs(out["A"].mean() - beta) < 5 * np.sqrt(beta * (1 - beta) / n)
    np.testing.assert_allclose(np.minimum(p, q) + np.maximum(p - q, 0), p, rtol=0, atol=1e-16)


def test_rejected_token_follows_the_residual():
    T = 1.0
    p_logits = np.array([0.0, 1.0, 2.0, -1.0, 0.5])
    q_logits = np.array([2.0, 0.2, 0.0, -1.0, 0.0])
    n = 20000
    _, out, _ = _round(p_logits, q_logits, n, T, seed=5)
    rej = out["A"] == 0
    p, q = oracle.softmax_t(p_logits, T), oracle.softmax_t(q_logits, T)
    res = np.maximum(p - q, 0)
    assert (res > 0).sum() >= 2
    counts = np.bincount(out["next"][rej], minlength=5)
    assert counts[res == 0].sum() == 0
    keep = res > 0
    assert stats.chisquare(counts[keep], res[keep] / res.sum() * rej.sum()).pvalue > 1e-4


def test_all_accepted_draws_the_extra_token_from_the_last_target_row():
    T, V, n = 1.0, 4, 8000
    same = np.array([0.5, -0.5, 1.0, 0.0])
    last = np.array([3.0, 0.0, 0.0, -3.0])
    d, _ = oracle.sample_tokens(np.tile(same, (n, 1)), T, 9, stream=0)
    out = oracle.accept_sampled(d[:, None], np.tile(same, (n, 1, 1)),
                                np.tile(np.stack([same, last]), (n, 1, 1)), T, 9)
    assert (out["A"] == 1).all()                               # p == q: always accepted
    counts = np.bincount(out["next"], minlength=V)
    assert stats.chisquare(counts, oracle.softmax_t(last, T) * n).pvalue > 1e-4


def test_vanishing_temperature_is_the_greedy_rule():
    rng = np.random.default_rng(3)
    B, K, V, T = 40, 5, 50, 1e-4
    draft = rng.normal(size=(B, K, V))
    target = rng.normal(size=(B, K + 1, V))
    for b in range(0, B, 2):                                   # half the rows agree at some positions
        target[b, :3] = draft[b, :3]
    cand, _ = oracle.sample_tokens(draft.reshape(B * K, V), T, 1, 0)
    cand = cand.reshape(B, K)
    np.testing.assert_array_equal(cand, draft.argmax(-1))
    out = oracle.accept_sampled(cand, draft, target, T, 1)
    A, nxt = oracle.accept_prefix(cand, target.argmax(-1))
    np.testing.assert_array_equal(out["A"], A)
    np.testing.assert_array_equal(out["next"], nxt)


def test_match_mode_passes_with_the_target_probability():
    """Match mode: greedy candidates against target tokens sampled at T; a
    position passes with the probability the target gives the candidate."""
    T, n = 1.0, 30000
    p_logits = np.array([1.0, 0.0, 2.0])
    cand = np.full((n, 1), 2)
    t, _ = oracle.sample_tokens(np.tile(p_logits, (n, 1)), T, 4, stream=3)
    tgt = np.stack([t, np.zeros(n, dtype=np.int64)], axis=1)
    A, _ = oracle.accept_prefix(cand, tgt)
    p2 = oracle.softmax_t(p_logits, T)[2]
    assert abs(A.mean() - p2) < 5 * np.sqrt(p2 * (1 - p2) / n)


@pytest.mark.parametrize("bad", [-1, 5])
def test_out_of_range_candidate_is_rejected(bad):
    """A candidate that is no vocabulary index (the draft reports -1 for an
    invalid request; V is one past the last index) is rejected at its
    position.  With p = q every in-range candidate is kept (u q < p for every
    u < 1), so A is exactly the out-of-range position, and the residual
    [p - q]_+ vanishes, so the next token follows p at that row."""
    V, K, n, T = 5, 4, 20000, 1.0
    rng = np.random.default_rng(8)
    rows = rng.normal(size=(K + 1, V))
    draft = np.tile(rows[:K], (n, 1, 1))
    target = np.tile(rows, (n, 1, 1))
    cand = np.tile(np.array([1, 3, bad, 0]), (n, 1))
    out = oracle.accept_sampled(cand, draft, target, T, seed=21)
    assert (out["A"] == 2).all()
    counts = np.bincount(out["next"], minlength=V)
    assert stats.chisquare(counts, oracle.softmax_t(rows[2], T) * n).pvalue > 1e-4
