"""Sampling at temperature on the GPU against the oracle, through the C ABI.

Both sides get the same synthetic fp32 logits and the same (seed, stream):
Philox counters make the draws identical, so tokens, accept lengths and
next tokens must be equal, except where the oracle's decision lies within
rounding of a threshold (top-two perturbed scores within 1e-9, or an
acceptance / inverse-CDF comparison within 1e-9 relative): those cases are
counted, printed and must stay under 1% of the rows.
"""
import numpy as np
import pytest
import torch

import oracle
from history_free_drafter_amd import binding as B
from synth import make_sampling_case

pytestmark = pytest.mark.gpu


def _ws(rows):
    return torch.empty(B.dlite_sampling_workspace_bytes(rows), dtype=torch.uint8, device="cuda")


def _sample_gpu(logits, T, seed, stream):
    N, V = logits.shape
    x = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    tok = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    B.dlite_sample_tokens(x, N, V, T, seed, stream, tok, _ws(N))
    torch.cuda.synchronize()
    return tok.cpu().numpy()


@pytest.mark.parametrize("N,V,T,seed", [(40, 5000, 0.5, 1), (40, 5000, 1.0, 2), (64, 777, 1.5, 3),
                                        (7, 151936, 1.0, 4), (3, 1, 1.0, 5)])
def test_sample_tokens_match_oracle(N, V, T, seed):
    print(f"\n[case] sample N={N} V={V} T={T}", flush=True)
    logits = (2.0 * np.random.default_rng(seed).standard_normal((N, V))).astype(np.float32)
    gpu = _sample_gpu(logits, T, seed, 0)
    ref, gap = oracle.sample_tokens(logits, T, seed, 0)
    clear = gap > 1e-9
    np.testing.assert_array_equal(gpu[clear], ref[clear])
    print(f"exempt rows {int((~clear).sum())} of {N}", flush=True)
    assert (~clear).sum() <= 0.01 * N
    assert ((gpu >= 0) & (gpu < V)).all()


def _accept_gpu(cand, draft, target, T, seed):
    Bn, K, V = draft.shape
    c = torch.from_numpy(np.ascontiguousarray(cand, dtype=np.int32)).cuda()
    d = torch.from_numpy(np.ascontiguousarray(draft)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(target)).cuda()
    A = torch.full((Bn,), -7, dtype=torch.int32, device="cuda")
    nx = torch.full((Bn,), -7, dtype=torch.int32, device="cuda")
    B.dlite_accept_sampled(c, d, t, Bn, K, V, T, seed, A, nx, _ws(Bn * (2 * K + 1)))
    torch.cuda.synchronize()
    return A.cpu().numpy(), nx.cpu().numpy()


@pytest.mark.parametrize("Bn,K,V,T,seed", [(64, 7, 3000, 1.0, 11), (64, 7, 3000, 0.75, 12),
                                           (200, 1, 64, 1.0, 13), (2, 7, 151936, 1.0, 14),
                                           (16, 16, 1000, 1.5, 15), (3, 64, 500, 2.0, 16),
                                           (8, 5, 2999, 1.0, 17)])
def test_accept_sampled_matches_oracle(Bn, K, V, T, seed):
    print(f"\n[case] accept B={Bn} K={K} V={V} T={T}", flush=True)
    draft, target = make_sampling_case(seed, Bn, K, V)
    cand = _sample_gpu(draft.reshape(Bn * K, V), T, seed, 0).reshape(Bn, K)
    ref_c, gap = oracle.sample_tokens(draft.reshape(Bn * K, V), T, seed, 0)
    clear_c = (gap > 1e-9).reshape(Bn, K).all(axis=1)
    np.testing.assert_array_equal(cand[clear_c], ref_c.reshape(Bn, K)[clear_c])
    print(f"exempt draft rows {int((~clear_c).sum())} of {Bn}", flush=True)
    assert (~clear_c).sum() <= 0.01 * Bn
    A, nx = _accept_gpu(cand, draft, target, T, seed)
    ref = oracle.accept_sampled(cand, draft, target, T, seed)     # same candidates on both sides
    clear = ref["margin"] > 1e-9
    np.testing.assert_array_equal(A[clear], ref["A"][clear])
    np.testing.assert_array_equal(nx[clear], ref["next"][clear])
    print(f"exempt requests {int((~clear).sum())} of {Bn}", flush=True)
    assert (~clear).sum() <= 0.01 * Bn
    print("accepted", A.mean(), "rejections", (A < K).mean(), flush=True)


def test_committed_tokens_follow_the_target_on_gpu():
    """4000 one-position rounds on the GPU: the committed token ~ p (chi-square)."""
    from scipy import stats
    n, V, T = 4000, 5, 1.0
    p_logits = np.array([1.0, 0.2, -0.5, 2.2, 0.0], dtype=np.float32)
    q_logits = np.array([0.1, 1.5, -0.2, 1.0, 0.6], dtype=np.float32)
    draft = np.tile(q_logits, (n, 1, 1))
    target = np.tile(np.stack([p_logits, p_logits]), (n, 1, 1))
    cand = _sample_gpu(draft.reshape(n, V), T, 77, 0).reshape(n, 1)
    A, nx = _accept_gpu(cand, draft, target, T, 77)
    first = np.where(A == 1, cand[:, 0], nx)
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, oracle.softmax_t(p_logits, T) * n).pvalue > 1e-4


def test_match_mode_on_gpu():
    """Match mode: greedy candidates, target tokens sampled at T, greedy prefix rule."""
    Bn, K, V, T, seed = 64, 7, 2000, 1.0, 21
    draft, target = make_sampling_case(seed, Bn, K, V, mix=0.95)
    cand = draft.argmax(-1).astype(np.int32)
    tt = _sample_gpu(target.reshape(Bn * (K + 1), V), T, seed, 3).reshape(Bn, K + 1)
    ref_t, gap = oracle.sample_tokens(target.reshape(Bn * (K + 1), V), T, seed, 3)
    clear = (gap > 1e-9).reshape(Bn, K + 1).all(axis=1)
    np.testing.assert_array_equal(tt[clear], ref_t.reshape(Bn, K + 1)[clear])
    c = torch.from_numpy(cand).cuda()
    t = torch.from_numpy(tt.astype(np.int32)).cuda()
    A = torch.empty(Bn, dtype=torch.int32, device="cuda")
    nx = torch.empty(Bn, dtype=torch.int32, device="cuda")
    B.dlite_accept_prefix(c, t, Bn, K, A, nx)
    torch.cuda.synchronize()
    A_ref, nx_ref = oracle.accept_prefix(cand, tt)
    np.testing.assert_array_equal(A.cpu().numpy(), A_ref)
    np.testing.assert_array_equal(nx.cpu().numpy(), nx_ref)


@pytest.mark.parametrize("bad", [-1, 5])
def test_out_of_range_candidate_is_rejected_on_gpu(bad):
    """Candidates -1 (the draft's mark of an invalid request) and V are
    rejected at their position on both sides: with p = q every in-range
    candidate is kept, so A is that position, and the next token equals the
    oracle's draw from p at that row."""
    V, K, n, T = 5, 4, 256, 1.0
    rng = np.random.default_rng(8)
    rows = rng.normal(size=(K + 1, V)).astype(np.float32)
    draft = np.ascontiguousarray(np.tile(rows[:K], (n, 1, 1)))
    target = np.ascontiguousarray(np.tile(rows, (n, 1, 1)))
    cand = np.tile(np.array([1, 3, bad, 0], dtype=np.int32), (n, 1))
    A, nx = _accept_gpu(cand, draft, target, T, 21)
    ref = oracle.accept_sampled(cand, draft, target, T, 21)
    assert (ref["A"] == 2).all()
    np.testing.assert_array_equal(A, ref["A"])
    clear = ref["margin"] > 1e-9
    np.testing.assert_array_equal(nx[clear], ref["next"][clear])
    assert (~clear).sum() <= 0.01 * n
