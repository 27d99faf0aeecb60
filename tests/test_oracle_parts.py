"""Pins of the oracle's drafter pieces.

Each piece is checked against something other than itself: a library routine
(torch CPU fp64 rms_norm / scaled_dot_product_attention / silu), an explicit
rotation matrix, closed-form special cases of the sequential head, planted
argmax ties, and invariants of the whole step (the depth-slot layout is
permutation invariant, requests are independent, nothing persists between
calls).  Gains are drawn U(0.5, 1.5) so a dropped or misplaced gain shows.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import custom, make_weights, make_features, make_anchors, tok_emb_rows
from tests._util import f64_weights, golden


def _rng(s=0):
    return np.random.default_rng(s)


# ------------------------------------------------------------------ norm ---

def test_rms_norm_matches_torch():
    r = _rng(1)
    x = r.normal(size=(5, 3, 64)) * 3.0
    g = r.uniform(0.5, 1.5, size=64)
    want = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-6), want, rtol=1e-13, atol=1e-13)


def test_feature_slots_add_depth_before_norm():
    r = _rng(2)
    H = r.normal(size=(2, 4, 32))
    e = r.normal(size=(4, 32))
    g = r.uniform(0.5, 1.5, size=32)
    z = oracle.feature_slots(H, e, g, 1e-6)
    for b in range(2):
        for l in range(4):
            want = F.rms_norm(torch.from_numpy(H[b, l] + e[l]), (32,),
                              torch.from_numpy(g), eps=1e-6).numpy()
            np.testing.assert_allclose(z[b, l], want, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ rope ---

def test_positions_match_figure3():
    rows = dict(r.split(":", 1) for r in golden("fig3_positions.txt"))
    ph = [int(t) for t in rows["placeholders"].split()]
    m = 5
    pos = oracle.local_positions(m, len(ph))
    assert list(pos[:m]) == [int(rows["feature"])] * m
    assert pos[m] == int(rows["anchor"])
    assert list(pos[m + 1:]) == ph


def test_rope_explicit_rotation_and_identity():
    r = _rng(3)
    d, theta = 16, 1e6
    x = r.normal(size=(4, 2, d))
    pos = np.array([0, 1, 5, 11])
    y = oracle.rope(x, pos, theta)
    np.testing.assert_allclose(y[0], x[0], rtol=0, atol=0)          # R(0) = I
    for si, p in enumerate(pos):
        for i in range(d // 2):
            a = p * theta ** (-2.0 * i / d)
            R = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
            for h in range(2):
                v = R @ np.array([x[si, h, i], x[si, h, i + d // 2]])
                assert abs(y[si, h, i] - v[0]) < 1e-13
                assert abs(y[si, h, i + d // 2] - v[1]) < 1e-13


def test_rope_scores_depend_on_relative_position_only():
    r = _rng(4)
    d = 32
    q = r.normal(size=(1, 1, d))
    k = r.normal(size=(1, 1, d))
    base = None
    for shift in range(0, 9, 2):
        qq = oracle.rope(q, np.array([3 + shift]), 1e6)
        kk = oracle.rope(k, np.array([1 + shift]), 1e6)
        s = float((qq * kk).sum())
        base = s if base is None else base
        assert abs(s - base) < 1e-12


# ------------------------------------------------------------- attention ---

@pytest.mark.parametrize("nq,nkv", [(4, 2), (8, 8), (6, 1)])
def test_block_attention_matches_torch_sdpa(nq, nkv):
    r = _rng(5)
    Lq, S, d = 5, 9, 16
    q = r.normal(size=(Lq, nq, d))
    k = r.normal(size=(S, nkv, d))
    v = r.normal(size=(S, nkv, d))
    G = nq // nkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    want = F.scaled_dot_product_attention(tq, tk, tv, is_causal=False).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.block_attention(q, k, v), want, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- swiglu ---

def test_swiglu_matches_torch():
    r = _rng(6)
    n = r.normal(size=(3, 24))
    wgu = r.normal(size=(2 * 40, 24)) * 0.2
    wd = r.normal(size=(24, 40)) * 0.2
    tn = torch.from_numpy(n)
    g = F.linear(tn, torch.from_numpy(wgu[:40]))
    u = F.linear(tn, torch.from_numpy(wgu[40:]))
    want = F.linear(F.silu(g) * u, torch.from_numpy(wd)).numpy()
    np.testing.assert_allclose(oracle.swiglu_ffn(n, wgu, wd), want, rtol=1e-12, atol=1e-12)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 301)
    np.testing.assert_allclose(oracle.silu(x), F.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-14, atol=1e-14)


# -------------------------------------------------------- sequential head ---

def test_scan_without_state_feedback_is_prefix_sum():
    """W_down[:, D:] = 0  ->  s_k = sum_{j<=k} W_up silu(W_down[:, :D] h_j)."""
    r = _rng(7)
    K, D, R = 6, 20, 8
    h = r.normal(size=(K, D))
    wd = r.normal(size=(R, D + R)) * 0.3
    wd[:, D:] = 0.0
    wu = r.normal(size=(R, R)) * 0.3
    s = oracle.sequential_head(h, wd, wu)
    inc = F.silu(torch.from_numpy(h @ wd[:, :D].T)).numpy() @ wu.T
    np.testing.assert_allclose(s, np.cumsum(inc, axis=0), rtol=1e-12, atol=1e-12)


def test_scan_first_state_uses_zero_initial_state():
    r = _rng(8)
    K, D, R = 3, 10, 4
    h = r.normal(size=(K, D))
    wd = r.normal(size=(R, D + R))
    wu = r.normal(size=(R, R))
    s = oracle.sequential_head(h, wd, wu)
    np.testing.assert_allclose(s[0], wu @ oracle.silu(wd[:, :D] @ h[0]), rtol=1e-13)
    # the second step feeds s_1 back through the state columns of W_down
    t2 = wd[:, :D] @ h[1] + wd[:, D:] @ s[0]
    np.testing.assert_allclose(s[1], s[0] + wu @ oracle.silu(t2), rtol=1e-12)


def test_scan_zero_up_projection_gives_zero_state_and_token_zero():
    r = _rng(9)
    K, D, R, V = 4, 12, 6, 50
    s = oracle.sequential_head(r.normal(size=(K, D)), r.normal(size=(R, D + R)),
                               np.zeros((R, R)))
    assert np.all(s == 0)
    logits, tok, margin = oracle.lm_head_argmax(s, r.normal(size=(V, R)))
    assert np.all(logits == 0) and np.all(tok == 0) and np.all(margin == 0)


# ---------------------------------------------------------------- argmax ---

def test_argmax_lowest_index_on_planted_ties():
    s = np.eye(3)
    lm = np.zeros((10, 3))
    lm[[2, 7], 0] = 5.0          # tie between 2 and 7 for row 0
    lm[[4, 9, 1], 1] = 3.0       # tie among 1, 4, 9 for row 1
    lm[8, 2] = 1.0
    lm[3, 2] = 0.5
    logits, tok, margin = oracle.lm_head_argmax(s, lm)
    assert list(tok) == [2, 1, 8]
    assert margin[0] == 0 and margin[1] == 0 and margin[2] == 0.5


def test_argmax_matches_numpy_on_random_logits():
    r = _rng(10)
    s = r.normal(size=(2, 5, 8))
    lm = r.normal(size=(300, 8))
    logits, tok, _ = oracle.lm_head_argmax(s, lm)
    np.testing.assert_array_equal(tok, np.argmax(np.einsum("bkr,vr->bkv", s, lm), axis=-1))


def test_projection_width_ratio():
    rows = dict(r.split(":", 1) for r in golden("projection_ratio.txt"))
    D, R, V, K = int(rows["D"]), int(rows["R"]), 151936, 7
    assert (K * D * V) / (K * R * V) == int(rows["ratio"])


# ----------------------------------------------------- whole-step checks ---

def _tiny(**kw):
    base = dict(B=3, m=3, D=32, n_layers=2, n_q=4, n_kv=2, d_h=8, ffn=48, K=4,
                rank=6, vocab=64, seed=3)
    base.update(kw)
    return custom(**base)


def _run(w, weights, H, anchors):
    Wf = f64_weights(w, weights)
    rows = np.stack([np.asarray(weights["tok_emb"][a], dtype=np.float64) for a in anchors])
    return oracle.draft_block(w, Wf, np.asarray(H, dtype=np.float64), rows)


def _unit_gains(weights, rng):
    """Replace the ~1 gains with U(0.5, 1.5) so gain mistakes are visible."""
    for k in ("feat_norm", "final_norm"):
        weights[k] = rng.uniform(0.5, 1.5, size=weights[k].shape).astype(np.float32)
    for lw in weights["layers"]:
        for k in ("attn_norm", "ffn_norm"):
            lw[k] = rng.uniform(0.5, 1.5, size=lw[k].shape).astype(np.float32)
    return weights


def _scale(weights, f):
    """Scale all matrices so activations are O(1) at tiny widths."""
    for k in ("seq_w_down", "seq_w_up", "lm_head", "ph_emb", "depth_emb", "tok_emb"):
        weights[k] = (weights[k] * f).astype(np.float32)
    for lw in weights["layers"]:
        for k in ("wqkv", "wo", "w_gate_up", "w_down"):
            lw[k] = (lw[k] * f).astype(np.float32)
    return weights


def test_depth_slot_layout_is_permutation_invariant():
    """All context slots share position 0 and attention is unmasked, so
    permuting the pairs (h^(l), e_depth^(l)) together changes nothing."""
    w = _tiny()
    weights = _scale(_unit_gains(make_weights(w), _rng(11)), 10.0)
    H, a = make_features(w), make_anchors(w)
    out = _run(w, weights, H, a)
    perm = np.array([2, 0, 1])
    wp = dict(weights)
    wp["depth_emb"] = weights["depth_emb"][perm]
    outp = _run(w, wp, H[:, perm], a)
    np.testing.assert_allclose(outp["s"], out["s"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(outp["cand"], out["cand"])
    # but the depth embedding is tied to its layer: permuting H alone changes s
    outq = _run(w, weights, H[:, perm], a)
    assert np.max(np.abs(outq["s"] - out["s"])) > 1e-6


def test_requests_are_independent_and_calls_stateless():
    w = _tiny()
    weights = _scale(_unit_gains(make_weights(w), _rng(12)), 10.0)
    H, a = make_features(w), make_anchors(w)
    full = _run(w, weights, H, a)
    again = _run(w, weights, H, a)
    for k in ("z", "h", "s", "logits"):
        np.testing.assert_array_equal(full[k], again[k])
    w1 = custom(**{**w.__dict__, "B": 1, "name": "one"})
    for b in range(w.B):
        one = _run(w1, weights, H[b:b + 1], a[b:b + 1])
        np.testing.assert_allclose(one["s"][0], full["s"][b], rtol=1e-13, atol=1e-13)


def test_zero_query_projection_gives_uniform_attention_over_all_slots():
    """W_q = 0 makes every score 0: each query averages V over all S slots
    (non-causal, features included)."""
    w = _tiny(n_layers=1, B=1)
    weights = _scale(_unit_gains(make_weights(w), _rng(13)), 10.0)
    lw = weights["layers"][0]
    lw["wqkv"][: w.n_q * w.d_h] = 0.0
    H, a = make_features(w), make_anchors(w)
    Wf = f64_weights(w, weights)
    z = oracle.feature_slots(np.asarray(H, np.float64), Wf["depth_emb"], Wf["feat_norm"], w.rms_eps)
    x = np.empty((1 + w.K, w.D))
    x[0] = weights["tok_emb"][a[0]]
    x[1:] = Wf["ph_emb"]
    slots = np.concatenate([z[0], x])
    n = oracle.rms_norm(slots, Wf["layers"][0]["attn_norm"], w.rms_eps)
    wv = Wf["layers"][0]["wqkv"][(w.n_q + w.n_kv) * w.d_h:]
    vmean = (n @ wv.T).mean(axis=0).reshape(w.n_kv, w.d_h)
    o = np.repeat(vmean, w.n_q // w.n_kv, axis=0).reshape(-1)
    x1 = x + o @ Wf["layers"][0]["wo"].T
    n2 = oracle.rms_norm(x1, Wf["layers"][0]["ffn_norm"], w.rms_eps)
    x1 = x1 + oracle.swiglu_ffn(n2, Wf["layers"][0]["w_gate_up"], Wf["layers"][0]["w_down"])
    got = oracle.draft_block(w, Wf, np.asarray(H, np.float64),
                             np.asarray(weights["tok_emb"][a], np.float64))
    np.testing.assert_allclose(got["x_layers"][0][0], x1, rtol=1e-12, atol=1e-12)


def test_identity_layer_leaves_stream_unchanged():
    """W_o = 0 and W_down = 0 make a layer the identity on the local stream, so a
    2-layer drafter equals the 1-layer drafter built from the other layer."""
    w2 = _tiny(n_layers=2)
    weights = _scale(_unit_gains(make_weights(w2), _rng(14)), 10.0)
    weights["layers"][0]["wo"][:] = 0
    weights["layers"][0]["w_down"][:] = 0
    H, a = make_features(w2), make_anchors(w2)
    out2 = _run(w2, weights, H, a)
    w1 = custom(**{**w2.__dict__, "n_layers": 1, "name": "one"})
    wts1 = dict(weights)
    wts1["layers"] = [weights["layers"][1]]
    out1 = _run(w1, wts1, H, a)
    np.testing.assert_allclose(out2["s"], out1["s"], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- generator ---

def test_bf16_rounding_matches_torch():
    from synth import f32_to_bf16_bits
    r = _rng(15)
    x = np.concatenate([r.normal(size=10000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), want)


def test_token_rows_regenerate_table():
    w = _tiny(vocab=3000)
    table = make_weights(w)["tok_emb"]
    rows = np.array([0, 1023, 1024, 2999, 5])
    np.testing.assert_array_equal(tok_emb_rows(w, rows), table[rows])
