"""Pins of the oracle's local token group and the gated head's warm-up token.

Local token group (DLite walkthrough, "锚点是已经确定、尚待目标前向处理的输入": the
draft input holds the anchor or a fixed-length local token group;
"局部位置编码切断草稿端的全局位置增长": the position builder takes the start of the
valid group as the origin).  Pinned by: the one-token group is the plain
anchor layout exactly; padding is invisible (a group padded at the front gives
the same result as the unpadded shorter group, whatever the padding rows
hold); a constructed layer whose scores depend only on position differences
checks the group's coordinates in closed form; and the scalar-loop second
oracle agrees to 1e-12.

Warm-up ("官方顺序头具体算了什么": one token before the anchor may warm the
state up).  Pinned by: warming up with w and then drafting from the anchor a
is a plain run from anchor w whose first chosen token is replaced by a; the
half-open gate's geometric state gains one step; an absent warm-up token
leaves the state at 0.
"""
import math

import numpy as np
import pytest

import oracle
from synth import custom
from tests.naive_drafter import naive_draft
from tests.test_oracle_positions import _naive_case, _slot_row


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a, float), np.asarray(b, float)
    assert a.shape == b.shape
    scale = max(1.0, float(np.max(np.abs(b))))
    assert float(np.max(np.abs(a - b))) <= tol * scale, float(np.max(np.abs(a - b)))


def _group_case(seed, G, B=3):
    w, weights, H, anchors = _naive_case(seed, 10.0, 2, 2, B=B)
    r = np.random.default_rng(seed + 100)
    rows = r.normal(size=(B, G, w.D))
    rows[:, -1] = anchors                      # the anchor closes the group
    return w, weights, H, anchors, rows


def test_group_of_one_is_the_anchor_layout():
    w, weights, H, anchors, rows = _group_case(1, 1)
    plain = oracle.draft_block(w, weights, H, anchors)
    grp = oracle.draft_block(w, weights, H, None, group_rows=rows,
                             group_valid=np.ones(w.B, dtype=int))
    for k in ("z", "h", "s", "logits", "cand"):
        np.testing.assert_array_equal(grp[k], plain[k])


@pytest.mark.parametrize("G,valid", [(4, [2, 4, 1]), (3, [3, 1, 2])])
def test_padding_is_invisible(G, valid):
    """A group of G slots with n real tokens equals the unpadded group of the
    last n tokens, and the padding rows' contents do not matter."""
    w, weights, H, anchors, rows = _group_case(2, G)
    valid = np.array(valid)
    out = oracle.draft_block(w, weights, H, None, group_rows=rows, group_valid=valid)
    junk = rows.copy()
    for b in range(w.B):
        junk[b, :G - valid[b]] = 1e3 * np.random.default_rng(b).normal(size=(G - valid[b], w.D))
    out2 = oracle.draft_block(w, weights, H, None, group_rows=junk, group_valid=valid)
    np.testing.assert_array_equal(out2["s"], out["s"])
    w1 = custom(**{**w.__dict__, "B": 1, "name": "one"})
    for b in range(w.B):
        n = int(valid[b])
        short = oracle.draft_block(w1, weights, H[b:b + 1], None, group_rows=rows[b:b + 1, G - n:],
                                   group_valid=np.array([n]))
        _close(short["h"][0], out["h"][b])
        _close(short["s"][0], out["s"][b])
        _close(short["x_layers"][-1][0], out["x_layers"][-1][b][G - n:])


def test_group_scores_follow_the_group_coordinates():
    """The constructed layer of the Figure 3 test with a group of G = 4 slots,
    3 of them real: scores a b n0^2 (cos(dp) + cos(f1 dp)) / sqrt(d_h) of the
    position difference dp, with group token j at j - 1 (origin at the first
    real token), the features at the anchor's position 2 and placeholder k at
    2 + k; the padding slot is no key."""
    m, K, D, dh, G, nv, theta = 2, 3, 8, 4, 4, 3, 50.0
    # eps 1e-30: the (zeroed) padding row normalises to 0 instead of NaN,
    # every other row is exactly unit-RMS as with eps = 0
    w = custom(B=1, m=m, D=D, n_layers=1, n_q=1, n_kv=1, d_h=dh, ffn=4, K=K,
               rank=4, vocab=16, rms_eps=1e-30, rope_theta=theta)
    S = m + G + K
    phis = [0.3 + 0.7 * s for s in range(S)]
    a, b = 1.1, 1.9
    H = np.stack([_slot_row(phis[l], D) for l in range(m)])[None]
    rows = np.stack([_slot_row(phis[m + j], D) for j in range(G)])[None]
    ph = _slot_row(phis[m + G], D)
    wqkv = np.zeros(((1 + 2) * dh, D))
    wqkv[0, 0] = wqkv[1, 0] = a
    wqkv[dh, 0] = wqkv[dh + 1, 0] = b
    wqkv[2 * dh, 2] = wqkv[2 * dh + 1, 3] = 1.0
    wo = np.zeros((D, dh))
    wo[4, 0] = wo[5, 1] = 1.0
    layer = dict(attn_norm=np.ones(D), wqkv=wqkv, wo=wo, ffn_norm=np.ones(D),
                 w_gate_up=np.random.default_rng(0).normal(size=(8, D)), w_down=np.zeros((D, 4)))
    weights = dict(depth_emb=np.zeros((m, D)), feat_norm=np.ones(D), ph_emb=ph,
                   layers=[layer], final_norm=np.ones(D))
    out = oracle.draft_block(w, weights, H, None, with_head=False, group_rows=rows,
                             group_valid=np.array([nv]))
    x1 = out["x_layers"][0][0]
    pad = G - nv
    key_pos = [nv - 1] * m + [j - pad for j in range(G)] + [nv - 1 + k for k in range(1, K + 1)]
    is_key = [True] * m + [j >= pad for j in range(G)] + [True] * K
    val_phi = phis[:m + G] + [phis[m + G]] * K
    n0 = 1.0 / math.sqrt(3.0 / D)
    f1 = theta ** (-2.0 / dh)
    for j in range(pad, G + K):                 # every real local row
        pq = key_pos[m + j]
        e = [math.exp(a * b * n0 * n0 * (math.cos(pq - pk) + math.cos(f1 * (pq - pk))) / math.sqrt(dh))
             if ok else 0.0 for pk, ok in zip(key_pos, is_key)]
        Z = sum(e)
        want4 = sum(e[s] / Z * n0 * math.cos(val_phi[s]) for s in range(S))
        want5 = sum(e[s] / Z * n0 * math.sin(val_phi[s]) for s in range(S))
        assert abs(x1[j, 4] - want4) < 1e-12, (j, x1[j, 4], want4)
        assert abs(x1[j, 5] - want5) < 1e-12, (j, x1[j, 5], want5)


@pytest.mark.parametrize("seed,G,valid", [(3, 3, [3, 1, 2]), (4, 2, [2, 2, 1])])
def test_naive_oracle_agrees_with_groups(seed, G, valid):
    w, weights, H, anchors, rows = _group_case(seed, G)
    valid = np.array(valid)
    got = oracle.draft_block(w, weights, H, None, group_rows=rows, group_valid=valid)
    ref = naive_draft(w, weights, H, None, group_rows=rows, group_valid=valid)
    _close(got["z"], ref["z"])
    for li in range(w.n_layers):
        g_, r_ = np.asarray(got["x_layers"][li]), np.asarray(ref["x_layers"][li])
        for b in range(w.B):     # padding rows are never read
            _close(g_[b, G - valid[b]:], r_[b, G - valid[b]:])
    _close(got["h"], ref["h"])
    _close(got["s"], ref["s"])
    _close(got["logits"], ref["logits"])
    np.testing.assert_array_equal(got["cand"], np.asarray(ref["cand"]))


def test_group_positions_span():
    """The span depends on the group and block lengths only."""
    for m in (1, 5):
        pos, valid = oracle.group_positions(m, 4, 4, 7)
        assert pos.min() == 0 and pos.max() == 4 - 1 + 7 and valid.all()
        pos, valid = oracle.group_positions(m, 4, 1, 7)     # only the anchor is real
        assert list(pos[:m]) == [0] * m and list(pos[m + 4:]) == list(range(1, 8))
        assert list(valid[m:m + 4]) == [False, False, False, True]


# ------------------------------------------------------------- warm-up ---

def _head(V, R, D, seed):
    r = np.random.default_rng(seed)
    return dict(emb=r.normal(size=(V, R)), w_s=r.normal(size=(2 * R, 2 * R)) * 0.4,
                b_s=r.normal(size=2 * R) * 0.3, w_h=r.normal(size=(R, R + D)) * 0.4,
                b_h=r.normal(size=R) * 0.3, w_o=r.normal(size=(V, R)))


@pytest.mark.parametrize("anchor,wtok", [(3, 7), (0, 0), (11, 5)])
def test_warmup_is_a_step_from_the_previous_token(anchor, wtok):
    V, R, D, K = 13, 6, 5, 5
    hd = _head(V, R, D, anchor + 17 * wtok)
    h = np.random.default_rng(1).normal(size=(K, D))
    warm = oracle.gated_head(h, anchor, hd, warmup=wtok)
    h2 = np.concatenate([np.zeros((1, D)), h])
    forced = np.concatenate([[anchor], warm["cand"]])
    plain = oracle.gated_head(h2, wtok, hd, forced=forced)
    _close(plain["s"][1:], warm["s"], 1e-14)
    _close(plain["logits"][1:], warm["logits"], 1e-14)
    np.testing.assert_array_equal(plain["cand"][1:], warm["cand"])
    # and it matters: without the warm-up the first state differs
    cold = oracle.gated_head(h, anchor, hd)
    assert np.max(np.abs(cold["s"][0] - warm["s"][0])) > 1e-6


def test_warmup_extends_the_half_open_geometric_state():
    R, D, V, K = 6, 5, 11, 6
    rng = np.random.default_rng(2)
    hd = _head(V, R, D, 9)
    c0 = rng.normal(size=R)
    hd["w_s"][:] = 0.0
    hd["b_s"] = np.concatenate([np.zeros(R), c0])             # f = 1/2, c = c0 every step
    out = oracle.gated_head(rng.normal(size=(K, D)), 3, hd, warmup=4)
    k = np.arange(1, K + 1)[:, None]
    np.testing.assert_allclose(out["s"], np.tanh(c0)[None, :] * (1.0 - 0.5 ** (k + 1)), rtol=1e-13)


@pytest.mark.parametrize("bad", [-1, 11])
def test_absent_warmup_token_leaves_the_state_at_zero(bad):
    R, D, V, K = 6, 5, 11, 4
    hd = _head(V, R, D, 10)
    h = np.random.default_rng(3).normal(size=(K, D))
    a = oracle.gated_head(h, 2, hd, warmup=bad)
    b = oracle.gated_head(h, 2, hd)
    for k in ("s", "logits", "cand"):
        np.testing.assert_array_equal(a[k], b[k])
