"""Parity of dlite_draft_block_ex (local token group, gated-head warm-up) with
the fp64 oracle.

Local token group (DLite walkthrough, "锚点是已经确定、尚待目标前向处理的输入"
and "局部位置编码切断草稿端的全局位置增长"): the G - 1 tokens before each anchor
join it as local rows; leading negative ids are padding.  The oracle gets the
same group as rows of the token embedding (zero rows for ids outside [0, V)
after the first real one) and the count of real tokens.  Warm-up ("官方顺序头
具体算了什么"): one state update from the token before the anchor.

Tolerances and the clear-margin rule are those of the plain step's parity
tests: tensor-wise (row-wise for hidden rows and logits) relative error
<= 2e-2 (bf16 storage) / 2e-5 (fp32), tokens equal wherever the oracle's
top-2 margin is >= 1e-2 / 1e-6.
"""
import numpy as np
import pytest
import torch

import oracle
from history_free_drafter_amd import binding as B
from history_free_drafter_amd.runtime import DraftModel, to_device
from synth import WORKLOADS, as_f64, make_anchors, make_features, make_gated_head, make_weights
from tests._util import f64_weights
from tests.test_gpu_parity import MARGIN, TOL, SMALL, _announce, _dims_dict, _rel

pytestmark = pytest.mark.gpu


def _group_ids(w, G, seed):
    """[B, G-1] ids: a spread of padding lengths (none, some, all) and one
    out-of-range id after a real token."""
    r = np.random.default_rng(seed)
    ids = r.integers(0, w.vocab, size=(w.B, G - 1)).astype(np.int32)
    for b in range(w.B):
        pad = [0, G - 1, (G - 1) // 2, 1][b % 4] if G > 1 else 0
        ids[b, :pad] = -1 - r.integers(0, 5, size=pad)
    if w.B > 2 and G > 2:
        ids[2, -1] = w.vocab + 3            # after real tokens: a zero row, still a key
    return ids


def _oracle_group(w, weights, ids, anchors):
    """group_rows [B, G, D] and group_valid [B] of the oracle for these ids."""
    G = ids.shape[1] + 1
    E = as_f64(weights["tok_emb"])
    rows = np.zeros((w.B, G, w.D))
    valid = np.empty(w.B, dtype=int)
    for b in range(w.B):
        pad = 0
        while pad < G - 1 and ids[b, pad] < 0:
            pad += 1
        valid[b] = G - pad
        full = list(ids[b]) + [anchors[b]]
        for j in range(pad, G):
            if 0 <= full[j] < w.vocab:
                rows[b, j] = E[full[j]]
    return rows, valid


def _run_ex(w, weights, H, anchors, ids=None, warm=None, head=None, model=None, taps=True):
    dev = "cuda"
    model = model or DraftModel(_dims_dict(w), weights, dev)
    if head is not None:
        model.set_gated_head(head)
    G = 1 if ids is None else ids.shape[1] + 1
    tb = {}
    if taps:
        f = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device=dev)
        tb = dict(state=f(w.B, w.K, w.rank), logits=f(w.B, w.K, w.vocab))
        if head is None:
            tb.update(z=f(w.B, w.m, w.D), x=f(w.n_layers, w.B, G + w.K, w.D), hidden=f(w.B, w.K, w.D))
    idd = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids)).to(dev)
    wd = None if warm is None else torch.from_numpy(np.ascontiguousarray(warm, dtype=np.int32)).to(dev)
    model.draft_ex(to_device(H, dev), torch.from_numpy(anchors).to(dev), group_ids=idd,
                   warmup_ids=wd, gated=head is not None, taps=B.make_taps(**tb) if taps else None)
    torch.cuda.synchronize()
    assert model.status() == 0, "a bounded wait timed out"
    out = {k: v.cpu().numpy() for k, v in tb.items()}
    out["cand"] = model.candidates.cpu().numpy()
    out["max_logit"] = model.max_logit.cpu().numpy()
    return out, model


def _check_fixed(w, gpu, ref, valid, rows=None):
    rows = np.arange(w.B) if rows is None else np.asarray(rows)
    tol = TOL[w.dtype]
    G = gpu["x"].shape[2] - w.K
    rep = dict(z=_rel(gpu["z"][rows], ref["z"][rows]))
    for l in range(w.n_layers):
        last = l == w.n_layers - 1
        worst = 0.0
        for b in rows:      # padding rows hold no defined value; the last layer's group rows are skipped
            lo = G if last else G - int(valid[b])
            worst = max(worst, _rel(gpu["x"][l][b, lo:], ref["x_layers"][l][b, lo:], axis=-1))
        rep[f"x{l}"] = worst
    rep["h"] = _rel(gpu["hidden"][rows], ref["h"][rows], axis=-1)
    rep["s"] = _rel(gpu["state"][rows], ref["s"][rows])
    rep["logits"] = _rel(gpu["logits"][rows], ref["logits"][rows], axis=-1)
    bad = {k: v for k, v in rep.items() if not v <= tol}
    assert not bad, f"relative errors above {tol}: {bad} (all: {rep})"
    clear = ref["margin"][rows] >= MARGIN[w.dtype]
    mism = (gpu["cand"][rows] != ref["cand"][rows]) & clear
    assert not mism.any(), f"{int(mism.sum())} token mismatches at clear margins"
    Bi, Ki = np.meshgrid(np.arange(len(rows)), np.arange(w.K), indexing="ij")
    np.testing.assert_array_equal(gpu["max_logit"][rows], gpu["logits"][rows][Bi, Ki, gpu["cand"][rows]])
    return rep, float(1.0 - clear.mean())


def _case(key):
    w = WORKLOADS.get(key) or next(s for s in SMALL if s.name == key)
    weights = make_weights(w)
    return w, weights, make_features(w), make_anchors(w)


@pytest.mark.parametrize("key,G", [("small_bf16", 4), ("small_f32", 3), ("batch40_bf16", 5),
                                   ("k16_m64_bf16", 16), ("tiled_bf16", 2), ("batch5_f32", 6),
                                   ("fused_two_teams_bf16", 3)])
def test_token_group_matches_oracle(key, G):
    _announce(f"group {key} G={G}")
    w, weights, H, a = _case(key)
    ids = _group_ids(w, G, seed=G)
    rows, valid = _oracle_group(w, weights, ids, a)
    ref = oracle.draft_block(w, f64_weights(w, weights), as_f64(H), None, group_rows=rows,
                             group_valid=valid)
    gpu, _ = _run_ex(w, weights, H, a, ids)
    rep, exempt = _check_fixed(w, gpu, ref, valid)
    print(key, G, "valid", valid[:8].tolist(), rep, f"exempt={exempt:.3f}", flush=True)
    assert exempt < 0.5


def test_token_group_full_size():
    """The 8B-shaped drafter with a group of four tokens (one request)."""
    _announce("group qwen3_8b_b1 G=4")
    w, weights, H, a = _case("qwen3_8b_b1")
    ids = np.array([[-1, 12345, 99]], dtype=np.int32)     # one padding slot, three real tokens
    rows, valid = _oracle_group(w, weights, ids, a)
    ref = oracle.draft_block(w, f64_weights(w, weights), as_f64(H), None, group_rows=rows,
                             group_valid=valid)
    gpu, _ = _run_ex(w, weights, H, a, ids)
    rep, exempt = _check_fixed(w, gpu, ref, valid)
    print("qwen3_8b_b1 G=4", rep, f"exempt={exempt:.3f}", flush=True)


def test_all_padding_group_is_the_plain_step():
    """A group of padding only is the anchor layout: the same result as
    dlite_draft_block (to rounding: the slot count changes the summation
    grouping), and the same tokens at clear margins."""
    _announce("group all padding small_bf16")
    w, weights, H, a = _case("small_bf16")
    ids = np.full((w.B, 3), -1, dtype=np.int32)
    g, model = _run_ex(w, weights, H, a, ids)
    p, _ = _run_ex(w, weights, H, a, None, model=model)
    assert _rel(g["state"], p["state"]) <= TOL[w.dtype]
    assert _rel(g["logits"], p["logits"], axis=-1) <= TOL[w.dtype]
    ref = oracle.draft_block(w, f64_weights(w, weights), as_f64(H), as_f64(weights["tok_emb"][a]))
    clear = ref["margin"] >= MARGIN[w.dtype]
    np.testing.assert_array_equal(g["cand"][clear], p["cand"][clear])


def test_group_out_of_range_anchor_gives_minus_one():
    _announce("group bad anchor small_bf16")
    w, weights, H, a = _case("small_bf16")
    ids = _group_ids(w, 4, seed=1)
    good, model = _run_ex(w, weights, H, a, ids, taps=False)
    bad = a.copy()
    bad[1] = -3
    out, _ = _run_ex(w, weights, H, bad, ids, model=model, taps=False)
    assert (out["cand"][1] == -1).all() and (out["max_logit"][1] == 0).all()
    np.testing.assert_array_equal(out["cand"][0], good["cand"][0])


# ------------------------------------------------------ gated warm-up ---

def _check_gated(w, gpu, h, anchors, head, warm):
    hf = {k: as_f64(v) for k, v in head.items()}
    ref = oracle.gated_heads(h, anchors, hf, forced=gpu["cand"], warmups=warm)
    tol = TOL[w.dtype]
    rep = dict(state=_rel(gpu["state"], ref["s"]), logits=_rel(gpu["logits"], ref["logits"], axis=-1))
    assert all(v <= tol for v in rep.values()), rep
    clear = ref["margin"] >= MARGIN[w.dtype]
    mism = (gpu["cand"] != ref["cand"]) & clear
    assert not mism.any(), f"{int(mism.sum())} token mismatches at clear margins"
    return rep, float(1.0 - clear.mean())


@pytest.mark.parametrize("key,G", [("small_bf16", 1), ("small_f32", 3), ("batch40_bf16", 1),
                                   ("fused_gated_b6_bf16", 1), ("fused_gated_b6_bf16", 4)])
def test_gated_warmup_matches_oracle(key, G):
    """Per-step launches (small, batch40) and the fused persistent kernel
    (fused_gated_b6: B = 6, R = 512); warm-up ids include absent ones (-1
    and V + 1: the state starts at 0)."""
    _announce(f"gated warm-up {key} G={G}")
    w, weights, H, a = _case(key)
    head = make_gated_head(w)
    warm = np.random.default_rng(5).integers(0, w.vocab, size=w.B).astype(np.int32)
    warm[0] = -1
    if w.B > 1:
        warm[1] = w.vocab + 1
    ids = _group_ids(w, G, seed=3) if G > 1 else None
    if ids is None:
        base = oracle.draft_block(w, f64_weights(w, weights), as_f64(H), as_f64(weights["tok_emb"][a]),
                                  with_head=False)
    else:
        rows, valid = _oracle_group(w, weights, ids, a)
        base = oracle.draft_block(w, f64_weights(w, weights), as_f64(H), None, with_head=False,
                                  group_rows=rows, group_valid=valid)
    gpu, model = _run_ex(w, weights, H, a, ids, warm=warm, head=head)
    rep, exempt = _check_gated(w, gpu, base["h"], a, head, warm)
    print(key, G, rep, f"exempt={exempt:.3f}", flush=True)
    assert exempt < 0.5
    # an absent warm-up token is the plain gated step, bit for bit
    none = np.full(w.B, -1, dtype=np.int32)
    g0, _ = _run_ex(w, weights, H, a, ids, warm=none, head=head, model=model, taps=False)
    g1, _ = _run_ex(w, weights, H, a, ids, warm=None, head=head, model=model, taps=False)
    np.testing.assert_array_equal(g0["cand"], g1["cand"])
    np.testing.assert_array_equal(g0["max_logit"], g1["max_logit"])


def test_gated_warmup_full_size():
    _announce("gated warm-up qwen3_8b_b1")
    w, weights, H, a = _case("qwen3_8b_b1")
    head = make_gated_head(w)
    warm = np.array([4321], dtype=np.int32)
    base = oracle.draft_block(w, f64_weights(w, weights), as_f64(H), as_f64(weights["tok_emb"][a]),
                              with_head=False)
    gpu, _ = _run_ex(w, weights, H, a, None, warm=warm, head=head)
    rep, exempt = _check_gated(w, gpu, base["h"], a, head, warm)
    print("qwen3_8b_b1 warm-up", rep, f"exempt={exempt:.3f}", flush=True)
