"""dlite_draft_block_noalloc against dlite_draft_block, through the C ABI.

The allocation-free variant runs the same kernels on the library's own
scratch array, so its candidates, winning logits and taps must equal the
workspace entry point's bitwise.  Two calls in a row, the second with fewer
requests, check that the array's left-over contents from the first call do
not leak into the second; dimensions past the array's size are rejected
before anything is enqueued.
"""
import numpy as np
import pytest
import torch

from history_free_drafter_amd import binding as B
from history_free_drafter_amd.runtime import DraftModel, to_device
from synth import WORKLOADS, custom, make_anchors, make_features, make_weights

pytestmark = pytest.mark.gpu


def _dims(w):
    return dict(B=w.B, m=w.m, D=w.D, n_layers=w.n_layers, n_q=w.n_q, n_kv=w.n_kv, d_h=w.d_h,
                ffn=w.ffn, K=w.K, rank=w.rank, vocab=w.vocab, dtype=w.dtype,
                rms_eps=w.rms_eps, rope_theta=w.rope_theta)


def _both(w, weights, H, a):
    model = DraftModel(_dims(w), weights, "cuda")
    Hd, ad = to_device(H), torch.from_numpy(a).cuda()
    st = lambda: torch.full((w.B, w.K, w.rank), float("nan"), device="cuda")
    s1, s2 = st(), st()
    model.draft(Hd, ad, taps=B.make_taps(state=s1))
    torch.cuda.synchronize()
    assert model.status() == 0
    ref = (model.candidates.cpu().numpy().copy(), model.max_logit.cpu().numpy().copy(), s1.cpu().numpy())
    cand = torch.full((w.B, w.K), -9, dtype=torch.int32, device="cuda")
    maxl = torch.full((w.B, w.K), float("nan"), device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    B.dlite_draft_block_noalloc(model.dims, model.wstruct, Hd, ad, cand, maxl,
                                taps=B.make_taps(state=s2), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = (cand.cpu().numpy(), maxl.cpu().numpy(), s2.cpu().numpy())
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)
    return got


@pytest.mark.parametrize("big,small", [("qwen3_8b_b1x3", "qwen3_8b_b1"),
                                       ("batch24_bf16", "batch5_bf16")])
def test_noalloc_matches_workspace_entry_point(big, small):
    print(f"\n[case] noalloc {big} then {small}", flush=True)
    shapes = {
        "qwen3_8b_b1": WORKLOADS["qwen3_8b_b1"],
        "qwen3_8b_b1x3": custom(**{**WORKLOADS["qwen3_8b_b1"].__dict__, "B": 3, "name": "b3"}),
        "batch24_bf16": custom(name="b24", B=24, m=3, D=256, n_layers=2, n_q=4, n_kv=2, d_h=64,
                               ffn=320, K=5, rank=64, vocab=1500, dtype="bf16",
                               weight_std=1.0 / 16),
        "batch5_bf16": custom(name="b5", B=5, m=3, D=256, n_layers=2, n_q=4, n_kv=2, d_h=64,
                              ffn=320, K=5, rank=64, vocab=1500, dtype="bf16",
                              weight_std=1.0 / 16),
    }
    wb, ws = shapes[big], shapes[small]
    weights = make_weights(wb)              # the smaller shape differs only in B
    Hb, ab = make_features(wb), make_anchors(wb)
    _both(wb, weights, Hb, ab)
    _both(ws, weights, Hb[:ws.B], ab[:ws.B])


def test_noalloc_rejects_dimensions_past_its_scratch():
    w = custom(**{**WORKLOADS["qwen3_8b_b64_m36"].__dict__, "name": "big"})
    d = B.make_dims(w.B, w.m, w.D, w.n_layers, w.n_q, w.n_kv, w.d_h, w.ffn, w.K, w.rank, w.vocab,
                    B.DLITE_BF16)
    assert B.dlite_workspace_bytes(d) > 64 << 20
    f = torch.empty(16, dtype=torch.int32, device="cuda")
    wt = B.DliteWeights(*([f.data_ptr()] * 4), None, *([f.data_ptr()] * 4))
    rc = B.load_library().dlite_draft_block_noalloc(d, wt, f.data_ptr(), f.data_ptr(),
                                                     f.data_ptr(), None, None, None, None)
    assert rc == -4
    assert "64" in B.load_library().dlite_last_error().decode() or "scratch" in \
        B.load_library().dlite_last_error().decode()
