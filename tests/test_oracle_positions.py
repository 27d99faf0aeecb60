"""Pins of how the oracle's backbone uses the local positions.

The pieces (the position list, the rotary embedding, attention) are pinned on
their own elsewhere; these tests pin their composition inside the layer:

* a constructed layer whose attention scores depend only on the difference of
  the query's and the key's local positions, with values that name their slot,
  so the layer output is a closed form in Figure 3's coordinates (DLite
  walkthrough, "局部位置编码切断草稿端的全局位置增长": every feature slot and the
  anchor at 0, placeholder k at k) — a query rotated at the wrong position, an
  unrotated query, or feature keys at another position change it;
* a second, naive oracle in scalar loops (tests/naive_drafter.py), written
  separately, must agree with the numpy oracle to 1e-12 on tiny shapes.
"""
import math

import numpy as np
import pytest

import oracle
from synth import custom
from tests._util import golden
from tests.naive_drafter import naive_draft


def _fig3():
    rows = dict(r.split(":", 1) for r in golden("fig3_positions.txt"))
    return int(rows["feature"]), int(rows["anchor"]), int(rows["placeholders"].split()[0])


def _slot_row(phi, D):
    """(1, 1, cos phi, sin phi, 0, ...): every such row has mean square 3 / D."""
    y = np.zeros(D)
    y[0] = y[1] = 1.0
    y[2], y[3] = math.cos(phi), math.sin(phi)
    return y


@pytest.mark.parametrize("theta", [100.0, 7.0])
def test_attention_scores_follow_figure3_positions(theta):
    """q = a n0 (1, 1, 0, 0) and k = b n0 (1, 1, 0, 0) in every slot, so after
    the rotary embedding the score of a query at local position p and a key at
    p' is a b n0^2 (cos(p - p') + cos(f1 (p - p'))) / sqrt(d_h) with
    f1 = theta^(-1/2) (pairs (0, 2) and (1, 3) of a 4-wide head).  Values carry
    the slot's angle phi_s; W_o writes the attention output into coordinates 4
    and 5, the FFN adds nothing, so x_out[j, 4:6] is the softmax-weighted
    (cos phi, sin phi) n0 over all slots, evaluated here with Figure 3's
    positions written out."""
    m, K, D, dh = 3, 4, 8, 4
    w = custom(B=1, m=m, D=D, n_layers=1, n_q=1, n_kv=1, d_h=dh, ffn=4, K=K,
               rank=4, vocab=16, rms_eps=0.0, rope_theta=theta)
    S = m + 1 + K
    phis = [0.4 + 0.9 * s for s in range(S)]       # slot s: its own angle
    a, b = 1.3, 1.7
    H = np.stack([_slot_row(phis[l], D) for l in range(m)])[None]
    anchor = _slot_row(phis[m], D)[None]
    ph = _slot_row(phis[m + 1], D)                 # one shared placeholder row
    wqkv = np.zeros(((1 + 2) * dh, D))
    wqkv[0, 0] = wqkv[1, 0] = a                    # q = a n0 (1, 1, 0, 0)
    wqkv[dh, 0] = wqkv[dh + 1, 0] = b              # k = b n0 (1, 1, 0, 0)
    wqkv[2 * dh, 2] = wqkv[2 * dh + 1, 3] = 1.0    # v = (n2, n3, 0, 0)
    wo = np.zeros((D, dh))
    wo[4, 0] = wo[5, 1] = 1.0
    rng = np.random.default_rng(0)
    layer = dict(attn_norm=np.ones(D), wqkv=wqkv, wo=wo, ffn_norm=np.ones(D),
                 w_gate_up=rng.normal(size=(8, D)), w_down=np.zeros((D, 4)))
    weights = dict(depth_emb=np.zeros((m, D)), feat_norm=np.ones(D), ph_emb=ph,
                   layers=[layer], final_norm=np.ones(D))
    out = oracle.draft_block(w, weights, H, anchor, with_head=False)
    x1 = out["x_layers"][0][0]                     # [1 + K, D]

    feat_pos, anchor_pos, first_ph = _fig3()
    key_pos = [feat_pos] * m + [anchor_pos] + [first_ph + k for k in range(K)]
    val_phi = phis[:m] + [phis[m]] + [phis[m + 1]] * K
    n0 = 1.0 / math.sqrt(3.0 / D)
    f1 = theta ** (-2.0 / dh)
    for j in range(1 + K):
        pq = key_pos[m + j]
        sc = [a * b * n0 * n0 * (math.cos(pq - pk) + math.cos(f1 * (pq - pk))) / math.sqrt(dh)
              for pk in key_pos]
        mx = max(sc)
        e = [math.exp(v - mx) for v in sc]
        Z = sum(e)
        want4 = sum(e[s] / Z * n0 * math.cos(val_phi[s]) for s in range(S))
        want5 = sum(e[s] / Z * n0 * math.sin(val_phi[s]) for s in range(S))
        assert abs(x1[j, 4] - want4) < 1e-12, (j, x1[j, 4], want4)
        assert abs(x1[j, 5] - want5) < 1e-12, (j, x1[j, 5], want5)
    # the attention output really depends on the positions here: the same
    # layer with every slot at position 0 gives a different output
    flat = [math.exp(2 * a * b * n0 * n0 / math.sqrt(dh))] * S
    flat4 = sum(flat[s] / sum(flat) * n0 * math.cos(val_phi[s]) for s in range(S))
    assert abs(x1[K, 4] - flat4) > 1e-3


def _naive_case(seed, theta, G, layers, B=2):
    n_kv = 1
    w = custom(B=B, m=2, D=8, n_layers=layers, n_q=G * n_kv, n_kv=n_kv, d_h=4, ffn=12,
               K=3, rank=4, vocab=16, rms_eps=1e-6, rope_theta=theta)
    r = np.random.default_rng(seed)
    D, F, dh = w.D, w.ffn, w.d_h
    lay = []
    for _ in range(layers):
        lay.append(dict(attn_norm=r.uniform(0.5, 1.5, D),
                        wqkv=r.normal(size=((w.n_q + 2 * w.n_kv) * dh, D)) * 0.6,
                        wo=r.normal(size=(D, w.n_q * dh)) * 0.5,
                        ffn_norm=r.uniform(0.5, 1.5, D),
                        w_gate_up=r.normal(size=(2 * F, D)) * 0.5,
                        w_down=r.normal(size=(D, F)) * 0.5))
    weights = dict(depth_emb=r.normal(size=(w.m, D)), feat_norm=r.uniform(0.5, 1.5, D),
                   ph_emb=r.normal(size=D), layers=lay, final_norm=r.uniform(0.5, 1.5, D),
                   seq_w_down=r.normal(size=(w.rank, D + w.rank)) * 0.5,
                   seq_w_up=r.normal(size=(w.rank, w.rank)) * 0.5,
                   lm_head=r.normal(size=(w.vocab, w.rank)))
    H = r.normal(size=(B, w.m, D)) * 2.0
    anchors = r.normal(size=(B, D))
    return w, weights, H, anchors


@pytest.mark.parametrize("seed,theta,G,layers", [
    (1, 10.0, 1, 1), (2, 1e6, 2, 2), (3, 3.0, 4, 2), (4, 50.0, 2, 3)])
def test_naive_scalar_oracle_agrees(seed, theta, G, layers):
    w, weights, H, anchors = _naive_case(seed, theta, G, layers)
    got = oracle.draft_block(w, weights, H, anchors)
    ref = naive_draft(w, weights, H, anchors)

    def close(a, b):
        a, b = np.asarray(a, float), np.asarray(b, float)
        assert a.shape == b.shape
        scale = max(1.0, float(np.max(np.abs(b))))
        assert float(np.max(np.abs(a - b))) <= 1e-12 * scale, float(np.max(np.abs(a - b)))

    close(got["z"], ref["z"])
    for li in range(layers):
        close(got["x_layers"][li], ref["x_layers"][li])
    close(got["h"], ref["h"])
    close(got["s"], ref["s"])
    close(got["logits"], ref["logits"])
    np.testing.assert_array_equal(got["cand"], np.asarray(ref["cand"]))


def test_naive_oracle_sees_the_placeholder_positions():
    """The naive oracle's own check that positions matter at this shape: the
    placeholders' residual rows differ from each other only through their
    positions (they share one input row), so they must not be equal."""
    w, weights, H, anchors = _naive_case(5, 10.0, 2, 1)
    ref = naive_draft(w, weights, H, anchors)
    x = np.asarray(ref["x_layers"][0])
    assert np.max(np.abs(x[:, 1] - x[:, 2])) > 1e-3
    assert np.max(np.abs(x[:, 2] - x[:, 3])) > 1e-3
