"""Pins of the oracle's gated sequential head (the walkthrough's own head).

Special cases with closed forms: a counter chain in which the head must
emit a+1, a+2, ... (exercises the token feedback d_0 = a, the gate
orientation and both concatenation orders), the half-open gate with its
geometric state, the closed gate that reduces every position to one plain
projection, and all-zero logits (ties to index 0).
"""
import numpy as np
import pytest

import oracle


def _head(V, R, D, rng=None, zero=False):
    rng = rng or np.random.default_rng(0)
    f = (lambda *s: np.zeros(s)) if zero else (lambda *s: rng.normal(size=s) * 0.3)
    return dict(emb=f(V, R), w_s=f(2 * R, 2 * R), b_s=f(2 * R), w_h=f(R, R + D),
                b_h=f(R), w_o=f(V, R))


@pytest.mark.parametrize("anchor", [0, 5, 7])
def test_counter_chain_emits_successors_of_the_anchor(anchor):
    V = R = 8
    D, K, alpha = 4, 6, 3.0
    hd = _head(V, R, D, zero=True)
    hd["emb"] = np.eye(V)                                     # v = one-hot of d_{i-1}
    hd["b_s"][:R] = -40.0                                     # f = sigmoid(-40) ~ 0
    hd["w_s"][R:, R:] = alpha * np.eye(R)                     # c = alpha v
    shift = np.roll(np.eye(R), 1, axis=0)                     # e_d -> e_{d+1}
    hd["w_h"][:, :R] = shift                                  # r = shift s
    hd["w_o"] = np.eye(V)
    h = np.random.default_rng(1).normal(size=(K, D))          # u enters with weight 0
    out = oracle.gated_head(h, anchor, hd)
    want = [(anchor + i) % V for i in range(1, K + 1)]
    assert out["cand"].tolist() == want
    for i, d in enumerate([anchor] + want[:-1]):
        np.testing.assert_allclose(out["s"][i], np.tanh(alpha) * np.eye(R)[d], atol=1e-15)


def test_half_open_gate_has_geometric_state():
    R, D, V, K = 6, 5, 11, 7
    rng = np.random.default_rng(2)
    hd = _head(V, R, D, rng)
    c0 = rng.normal(size=R)
    hd["w_s"][:] = 0.0
    hd["b_s"] = np.concatenate([np.zeros(R), c0])             # f = 1/2, c = c0
    out = oracle.gated_head(rng.normal(size=(K, D)), 3, hd)
    k = np.arange(1, K + 1)[:, None]
    np.testing.assert_allclose(out["s"], np.tanh(c0)[None, :] * (1.0 - 0.5 ** k), rtol=1e-13)


def test_closed_gate_reduces_to_one_projection():
    R, D, V, K = 5, 9, 13, 4
    rng = np.random.default_rng(3)
    hd = _head(V, R, D, rng)
    hd["b_s"][:R] = 40.0                                      # f = 1: s stays 0
    hd["w_s"][:R] = 0.0
    u = rng.normal(size=(K, D))
    out = oracle.gated_head(u, 2, hd)
    assert np.abs(out["s"]).max() < 1e-15
    r = u @ hd["w_h"][:, R:].T + hd["b_h"][None, :]           # the u-columns come second
    np.testing.assert_allclose(out["r"], r, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["logits"], r @ hd["w_o"].T, rtol=1e-12, atol=1e-14)


def test_zero_logits_choose_index_zero_and_feed_it_back():
    R, D, V, K = 4, 3, 9, 5
    rng = np.random.default_rng(4)
    hd = _head(V, R, D, rng)
    hd["w_o"][:] = 0.0
    out = oracle.gated_head(rng.normal(size=(K, D)), 6, hd)
    assert (out["cand"] == 0).all()
    # the second step reads E_R[0]: the same run with anchor 0 agrees from step 2 on
    out0 = oracle.gated_head(rng.normal(size=(K, D)) * 0 + 0, 0, hd)
    assert out0["cand"].tolist() == [0] * K


def test_out_of_range_anchor_reads_a_zero_row_and_forcing_follows_given_tokens():
    R, D, V, K = 4, 3, 9, 5
    rng = np.random.default_rng(5)
    hd = _head(V, R, D, rng)
    h = rng.normal(size=(K, D))
    bad = oracle.gated_head(h, V + 3, hd)
    hz = dict(hd, emb=np.vstack([hd["emb"], np.zeros((1, R))]))
    ref = oracle.gated_head(h, V, hz)                          # row V of hz is zero
    np.testing.assert_array_equal(bad["s"][0], ref["s"][0])
    free = oracle.gated_head(h, 1, hd)
    forced = oracle.gated_head(h, 1, hd, forced=free["cand"])
    np.testing.assert_array_equal(free["logits"], forced["logits"])
    other = oracle.gated_head(h, 1, hd, forced=(free["cand"] + 1) % V)
    np.testing.assert_array_equal(other["logits"][0], free["logits"][0])
    assert not np.array_equal(other["logits"][1], free["logits"][1])
