"""Pins of the oracle's greedy prefix accept against what the pages fix.

The accept rule is pinned by the worked example and the verify-index rule
printed on the DLite walkthrough (golden fixtures), by exhaustive brute force
over every match pattern, by the closed forms P(A >= k) = prod c_i and
E[A + 1] = 1 + sum_k P(A >= k), and by a speculative-decoding loop with a
deterministic fake target, which must reproduce the target's greedy sequence.
"""
import itertools

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_target_tokens, match_probs
from tests._util import golden


def _pattern_to_tokens(pattern):
    """Candidates/targets whose position-wise equality is the given pattern."""
    K = len(pattern)
    cand = np.arange(10, 10 + K)[None, :]
    tgt = np.empty((1, K + 1), dtype=np.int64)
    for i, p in enumerate(pattern):
        tgt[0, i] = cand[0, i] if p else cand[0, i] + 1000
    tgt[0, K] = 7777
    return cand, tgt


def test_worked_example_from_page():
    rows = dict(r.split(":", 1) for r in golden("accept_worked_example.txt"))
    pattern = [int(t) for t in rows["pattern"].split()]
    cand, tgt = _pattern_to_tokens(pattern)
    A, nxt = oracle.accept_prefix(cand, tgt)
    assert int(A[0]) == int(rows["A"])
    # the correction token is the target's token at the first failure
    assert int(nxt[0]) == int(tgt[0, int(rows["A"])])


def test_verify_index_semantics():
    rows = dict(r.split(":", 1) for r in golden("verify_index.txt"))
    K = 4
    names = ["a"] + [f"d_{i}" for i in range(1, K + 1)]
    for a_str, name in rows.items():
        A_want = int(a_str)
        pattern = [1] * A_want + [0] * (K - A_want)
        cand, tgt = _pattern_to_tokens(pattern)
        A, nxt = oracle.accept_prefix(cand, tgt)
        assert int(A[0]) == A_want
        # the target token at verify index A is the output at input names[A]
        assert names[int(A[0])] == name.strip()
        assert int(nxt[0]) == int(tgt[0, A_want])


def _coded_verify_hidden(m, B, T, D):
    """[m, B, T, D] whose every element names its (layer, request, position)."""
    l, b, i = np.meshgrid(np.arange(m), np.arange(B), np.arange(T), indexing="ij")
    code = (1_000_000 * l + 100 * b + i).astype(np.float64)
    return np.repeat(code[..., None], D, axis=3)


def test_boundary_features_take_verify_index_a():
    """Next-round features come from verify index A (A = 0: a, A = 2: d_2)."""
    rows = dict(r.split(":", 1) for r in golden("verify_index.txt"))
    K, m, D = 4, 3, 5
    names = ["a"] + [f"d_{i}" for i in range(1, K + 1)]
    for a_str, name in rows.items():
        pattern = [1] * int(a_str) + [0] * (K - int(a_str))
        cand, tgt = _pattern_to_tokens(pattern)
        A, _ = oracle.accept_prefix(cand, tgt)
        vh = _coded_verify_hidden(m, 1, K + 1, D)
        H = oracle.boundary_features(vh, A)
        assert H.shape == (1, m, D)
        pos = H[0, :, 0] % 100
        assert (pos == names.index(name.strip())).all()
        assert (H[0, :, 0] // 1_000_000 == np.arange(m)).all()     # layer order kept


def test_boundary_features_never_use_rejected_positions():
    rng = np.random.default_rng(5)
    B, K, m, D = 64, 7, 2, 3
    cand = rng.integers(0, 3, size=(B, K))
    tgt = rng.integers(0, 3, size=(B, K + 1))
    A, _ = oracle.accept_prefix(cand, tgt)
    H = oracle.boundary_features(_coded_verify_hidden(m, B, K + 1, D), A)
    for b in range(B):
        p = int(H[b, 0, 0] % 100)
        assert int(H[b, 0, 0] // 100) % 10_000 == b
        assert (cand[b, :p] == tgt[b, :p]).all()            # every earlier draft passed
        assert p == K or cand[b, p] != tgt[b, p]            # d_{p+1} (if any) was rejected


def test_boundary_features_reject_out_of_range():
    vh = np.zeros((1, 2, 3, 4))
    with pytest.raises(ValueError):
        oracle.boundary_features(vh, np.array([0, 3]))
    with pytest.raises(ValueError):
        oracle.boundary_features(vh, np.array([-1, 0]))


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_verify_window_drops_the_tail(W):
    """A window of W inputs verifies the first W - 1 of the K drafted
    candidates (block 8 = anchor + 7 candidates: W = 8 is the full block)."""
    rng = np.random.default_rng(W)
    B, K = 500, 7
    cand = rng.integers(0, 3, size=(B, K))
    full_t = rng.integers(0, 3, size=(B, K + 1))
    A, nxt = oracle.accept_window(cand, full_t[:, :W], W)
    for b in range(B):   # first failure among the first W - 1, by scanning
        a = next((i for i in range(W - 1) if cand[b, i] != full_t[b, i]), W - 1)
        assert A[b] == a and nxt[b] == full_t[b, a]
    # the dropped tail never matters
    other = cand.copy()
    other[:, W - 1:] = 99
    A2, n2 = oracle.accept_window(other, full_t[:, :W], W)
    np.testing.assert_array_equal(A2, A)
    np.testing.assert_array_equal(n2, nxt)
    if W == K + 1:
        A3, n3 = oracle.accept_prefix(cand, full_t)
        np.testing.assert_array_equal(A3, A)
        np.testing.assert_array_equal(n3, nxt)


def test_round_accounting():
    for row in golden("round_accounting.txt"):
        lhs, rhs = row.split(":")
        K, A = (int(t) for t in lhs.split())
        commit, kv_verify, kv_crop = (int(t) for t in rhs.split())
        n = 100
        pattern = [1] * A + [0] * (K - A)
        cand, tgt = _pattern_to_tokens(pattern)
        got_A, _ = oracle.accept_prefix(cand, tgt)
        assert int(got_A[0]) + 1 == commit
        assert n + K + 1 == kv_verify and n + int(got_A[0]) + 1 == kv_crop


@pytest.mark.parametrize("K", range(1, 9))
def test_brute_force_all_patterns(K):
    """A equals the position of the first failure (or K), for all 2^K patterns."""
    pats = np.array(list(itertools.product([0, 1], repeat=K)))
    cand = np.tile(np.arange(K), (len(pats), 1))
    tgt = np.concatenate([np.where(pats == 1, cand, cand + 1),
                          np.full((len(pats), 1), -5)], axis=1)
    A, nxt = oracle.accept_prefix(cand, tgt)
    for row, p in enumerate(pats):
        s = "".join(map(str, p))
        want = s.find("0") if "0" in s else K
        assert A[row] == want
        assert nxt[row] == tgt[row, want]


@pytest.mark.parametrize("K", [1, 3, 7, 8])
def test_exact_enumeration_matches_closed_forms(K):
    """Sum over all 2^K patterns weighted by independent Bernoulli(c_i)."""
    rng = np.random.default_rng(K)
    c = rng.uniform(0.3, 0.97, size=K)
    pats = np.array(list(itertools.product([0, 1], repeat=K)))
    prob = np.prod(np.where(pats == 1, c, 1 - c), axis=1)
    cand = np.tile(np.arange(K), (len(pats), 1))
    tgt = np.concatenate([np.where(pats == 1, cand, cand + 1),
                          np.zeros((len(pats), 1), dtype=np.int64)], axis=1)
    A, _ = oracle.accept_prefix(cand, tgt)
    surv = oracle.prefix_survival(c)
    for k in range(1, K + 1):
        # P(A >= k) by enumeration vs the product of the pass probabilities
        assert abs(prob[A >= k].sum() - np.prod(c[:k])) < 1e-12
        assert abs(surv[k - 1] - np.prod(c[:k])) < 1e-12
    # P(A = j) = (prod_{i<=j} c_i)(1 - c_{j+1}), with c_{K+1} = 0
    for j in range(K + 1):
        cj = np.prod(c[:j]) * (1 - (c[j] if j < K else 0.0))
        assert abs(prob[A == j].sum() - cj) < 1e-12
    tau = (prob * (A + 1)).sum()
    assert abs(tau - oracle.expected_commit(c)) < 1e-12


def test_tau_geometric_closed_form():
    """Constant c: tau = (1 - c^(K+1)) / (1 - c); e.g. c=0.8, K=7 -> 4.1611392."""
    c = np.full(7, 0.8)
    assert abs(oracle.expected_commit(c) - 4.1611392) < 1e-9
    for cc in (0.5, 0.9, 0.99):
        for K in (1, 4, 7, 12):
            want = (1 - cc ** (K + 1)) / (1 - cc)
            assert abs(oracle.expected_commit(np.full(K, cc)) - want) < 1e-12


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_monte_carlo_accept_within_5_sigma(name):
    """Seeded rounds with the workloads' match model agree with the closed form.

    Candidates are arbitrary token ids; targets come from the workload
    generator, which passes position i with probability c_i exactly.
    """
    w = WORKLOADS[name]
    rounds = 200_000
    rng = np.random.default_rng(5)
    cand = rng.integers(0, w.vocab, size=(rounds, w.K))
    c = np.repeat(match_probs(w)[:1], rounds, axis=0)
    if w.match.startswith("uniform"):
        c = np.repeat(rng.uniform(0.5, 0.95, size=(rounds, 1)), w.K, axis=1)
    tgt = make_target_tokens(w, cand, c)
    A, nxt = oracle.accept_prefix(cand, tgt)
    surv = oracle.prefix_survival(c).mean(axis=0)
    for k in range(1, w.K + 1):
        p = surv[k - 1]
        sd = np.sqrt(p * (1 - p) / rounds)
        assert abs((A >= k).mean() - p) <= 5 * sd + 1e-12
    tau = oracle.expected_commit(c).mean()
    sd = (A + 1).std() / np.sqrt(rounds)
    assert abs((A + 1).mean() - tau) <= 5 * sd


class _FakeTarget:
    """Deterministic next-token function of the whole prefix (greedy target)."""

    def __init__(self, V):
        self.V = V

    def next(self, seq):
        h = 1469598103934665603
        for t in seq[-4:]:
            h = ((h ^ int(t)) * 1099511628211) % (1 << 61)
        return int((h + 7 * len(seq)) % self.V)

    def hidden(self, layer, seq):
        """A stand-in hidden state of `layer` after processing `seq` (exact in fp64)."""
        return float(sum((j + 1) * int(t) for j, t in enumerate(seq)) % 65521 + 100000 * layer)


@pytest.mark.parametrize("p_right", [0.0, 0.6, 0.95, 1.0])
def test_loop_reproduces_target_greedy_path(p_right):
    """Greedy drafting + prefix accept generates exactly the target's greedy path.

    DLite walkthrough, "贪心模式与随机模式要分别说明": with the same target forward
    and rule, greedy verification follows the target's greedy path; each round
    advances A + 1 tokens ("先拆开一次投机轮次的时间").
    """
    V, K, n_new = 97, 7, 300
    tgt_model = _FakeTarget(V)
    rng = np.random.default_rng(11)
    prompt = list(rng.integers(0, V, size=5))
    ref = list(prompt)
    while len(ref) < len(prompt) + n_new + K + 2:
        ref.append(tgt_model.next(ref))

    seq = list(prompt)                       # tokens already processed by the target
    anchor = tgt_model.next(seq)             # chosen, not yet processed
    rounds = 0
    while len(seq) < len(prompt) + n_new:
        # a noisy drafter: right with probability p_right
        ctx = seq + [anchor]
        cands = []
        for _ in range(K):
            good = tgt_model.next(ctx + cands)
            cands.append(good if rng.random() < p_right else (good + 1) % V)
        verify_in = [anchor] + cands
        t = [tgt_model.next(seq + verify_in[: i + 1]) for i in range(K + 1)]
        A, nxt = oracle.accept_prefix(np.array([cands]), np.array([t]))
        # hidden states of two layers at every verify input (causal: input i
        # sees the processed prefix and verify inputs 0..i)
        vh = np.array([[[[tgt_model.hidden(l, seq + verify_in[: i + 1])]
                         for i in range(K + 1)]] for l in range(2)], dtype=np.float64)
        H = oracle.boundary_features(vh, A)
        A = int(A[0])
        before = len(seq)
        seq = seq + [anchor] + cands[:A]
        assert len(seq) - before == A + 1
        # the next round is conditioned on the state after exactly the
        # committed tokens (the cache cropped to n + A + 1)
        assert [H[0, l, 0] for l in range(2)] == [tgt_model.hidden(l, seq) for l in range(2)]
        anchor = int(nxt[0])
        rounds += 1
    assert seq == ref[: len(seq)]
    assert anchor == ref[len(seq)]
    if p_right == 1.0:
        assert rounds == -(-n_new // (K + 1))
