"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before enqueuing anything.

No compute call is made here; every call below returns from argument
validation, which runs before any HIP call.
"""
import ctypes
import os
import re

import pytest

from history_free_drafter_amd import binding as B
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "dlite.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dlite_\w+)\s*\(", txt)))


def test_library_exports_every_header_function():
    lib = B.load_library()
    names = _header_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in B.dlite_version()


def _dims(w, **over):
    d = dict(B=w.B, m=w.m, D=w.D, n_layers=w.n_layers, n_q=w.n_q, n_kv=w.n_kv, d_h=w.d_h,
             ffn=w.ffn, K=w.K, rank=w.rank, vocab=w.vocab,
             dtype=B.DLITE_BF16 if w.dtype == "bf16" else B.DLITE_F32)
    d.update(over)
    return B.make_dims(**d)


def test_workspace_size_does_not_depend_on_history():
    # the ABI has no history-length argument at all; sizes scale with B, m, K only
    w = WORKLOADS["qwen3_8b_b1"]
    n1 = B.dlite_workspace_bytes(_dims(w))
    n2 = B.dlite_workspace_bytes(_dims(w, B=2))
    assert 0 < n1 < n2 <= 2 * n1 + 4096
    assert n1 % 256 == 0


@pytest.mark.parametrize("field,value", [
    ("B", 0), ("m", 0), ("m", 65), ("D", 100), ("D", 32), ("n_q", 6), ("d_h", 96),
    ("ffn", 48), ("K", 0), ("K", 17), ("rank", 48), ("rank", 1024), ("vocab", 0),
])
def test_invalid_dims_rejected(field, value):
    w = WORKLOADS["qwen3_8b_b1"]
    d = _dims(w, **{field: value})
    with pytest.raises(B.DliteError) as e:
        B.dlite_workspace_bytes(d)
    assert e.value.code == -2
    assert field.split("_")[0] in B.load_library().dlite_last_error().decode() or True


def test_invalid_dtype_rejected():
    lib = B.load_library()
    d = _dims(WORKLOADS["tiny_f32"], dtype=7)
    assert lib.dlite_workspace_bytes(ctypes.byref(d)) == 0
    assert b"dtype" in lib.dlite_last_error()


def _fake_weights(n_layers, addr=0x100000):
    layers = (B.DliteLayerWeights * n_layers)(
        *[B.DliteLayerWeights(*([addr] * 6)) for _ in range(n_layers)])
    w = B.DliteWeights(addr, addr, addr, addr, ctypes.cast(layers, ctypes.POINTER(B.DliteLayerWeights)),
                       addr, addr, addr, addr)
    return w, layers


def test_draft_block_validation_codes():
    lib = B.load_library()
    wl = WORKLOADS["tiny_f32"]
    d = _dims(wl)
    need = B.dlite_workspace_bytes(d)
    w, keep = _fake_weights(wl.n_layers)
    fake = 0x200000
    call = lambda dims, weights, feats, anchors, cand, ws, nbytes: lib.dlite_draft_block(
        dims, weights, feats, anchors, cand, None, None, ws, nbytes, None)
    assert call(None, ctypes.byref(w), fake, fake, fake, fake, need) == -1
    assert call(ctypes.byref(d), None, fake, fake, fake, fake, need) == -1
    assert call(ctypes.byref(d), ctypes.byref(w), None, fake, fake, fake, need) == -1
    assert call(ctypes.byref(d), ctypes.byref(w), fake, None, fake, fake, need) == -1
    assert call(ctypes.byref(d), ctypes.byref(w), fake, fake, None, fake, need) == -1
    assert call(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, None, need) == -1
    assert call(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, fake, need - 1) == -4
    assert b"needed" in lib.dlite_last_error()
    assert call(ctypes.byref(d), ctypes.byref(w), fake + 8, fake, fake, fake, need) == -5
    assert call(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, fake + 64, need) == -5
    layers_null = B.DliteWeights(*[fake] * 4, None, *[fake] * 4)
    assert call(ctypes.byref(d), ctypes.byref(layers_null), fake, fake, fake, fake, need) == -1
    bad = _dims(wl, K=0)
    assert call(ctypes.byref(bad), ctypes.byref(w), fake, fake, fake, fake, need) == -2


def test_draft_block_at_validation_codes():
    lib = B.load_library()
    wl = WORKLOADS["tiny_f32"]
    d = _dims(wl)
    need = B.dlite_workspace_bytes(d)
    w, keep = _fake_weights(wl.n_layers)
    fake = 0x200000
    call = lambda dims, vh, T, A, ws, nbytes: lib.dlite_draft_block_at(
        dims, ctypes.byref(w), vh, T, A, fake, fake, None, None, ws, nbytes, None)
    assert call(None, fake, 8, fake, fake, need) == -1
    assert call(ctypes.byref(d), None, 8, fake, fake, need) == -1
    assert call(ctypes.byref(d), fake, 8, None, fake, need) == -1
    assert call(ctypes.byref(d), fake, 0, fake, fake, need) == -2
    assert call(ctypes.byref(d), fake, 66, fake, fake, need) == -2
    assert call(ctypes.byref(d), fake + 8, 8, fake, fake, need) == -5
    assert call(ctypes.byref(d), fake, 8, fake, fake, need - 1) == -4
    assert call(ctypes.byref(_dims(wl, K=0)), fake, 8, fake, fake, need) == -2
    assert lib.dlite_draft_block_at(ctypes.byref(d), ctypes.byref(w), fake, 8, fake, None, fake,
                                    None, None, fake, need, None) == -1


def test_draft_block_gated_validation_codes():
    lib = B.load_library()
    wl = WORKLOADS["tiny_f32"]
    d = _dims(wl)
    need = B.dlite_workspace_bytes(d)
    w, keep = _fake_weights(wl.n_layers)
    fake = 0x200000
    head = B.DliteGatedHead(*[fake] * 6)
    call = lambda dims, hd, nbytes: lib.dlite_draft_block_gated(
        dims, ctypes.byref(w), hd, fake, fake, fake, None, None, fake, nbytes, None)
    assert call(ctypes.byref(d), None, need) == -1
    assert call(ctypes.byref(d), ctypes.byref(B.DliteGatedHead(*[fake] * 5, None)), need) == -1
    assert call(ctypes.byref(d), ctypes.byref(B.DliteGatedHead(fake + 4, *[fake] * 5)), need) == -5
    assert call(ctypes.byref(d), ctypes.byref(head), need - 1) == -4
    # the fixed head's weights are not needed by the gated head
    nohead = B.DliteWeights(*[fake] * 4, w.layers, fake, None, None, None)
    assert lib.dlite_draft_block_gated(ctypes.byref(d), ctypes.byref(nohead), ctypes.byref(head),
                                       fake, fake, fake, None, None, fake, need - 1, None) == -4


def test_sampling_validation_codes():
    lib = B.load_library()
    f, ws = 0x300000, 0x400000
    need = B.dlite_sampling_workspace_bytes(7)
    assert lib.dlite_sample_tokens(None, 7, 10, 1.0, 1, 0, f, ws, need, None) == -1
    assert lib.dlite_sample_tokens(f, 7, 10, 1.0, 1, 0, None, ws, need, None) == -1
    assert lib.dlite_sample_tokens(f, 0, 10, 1.0, 1, 0, f, ws, need, None) == -2
    assert lib.dlite_sample_tokens(f, 7, 10, 0.0, 1, 0, f, ws, need, None) == -2
    assert lib.dlite_sample_tokens(f, 7, 10, float("nan"), 1, 0, f, ws, need, None) == -2
    assert lib.dlite_sample_tokens(f, 7, 10, 1.0, 1, 0, f, ws + 8, need, None) == -5
    assert lib.dlite_sample_tokens(f, 7, 10, 1.0, 1, 0, f, ws, need - 1, None) == -4
    need2 = B.dlite_sampling_workspace_bytes(4 * 15)
    assert lib.dlite_accept_sampled(f, f, f, 4, 7, 10, 1.0, 1, f, None, ws, need2, None) == -1
    assert lib.dlite_accept_sampled(f, f, f, 4, 65, 10, 1.0, 1, f, f, ws, need2, None) == -2
    assert lib.dlite_accept_sampled(f, f, f, 4, 7, 10, -1.0, 1, f, f, ws, need2, None) == -2
    assert lib.dlite_accept_sampled(f, f, f, 4, 7, 10, 1.0, 1, f, f, ws, need2 - 1, None) == -4
    assert B.load_library().dlite_sampling_workspace_bytes(0) == 0


def test_accept_window_validation_codes():
    lib = B.load_library()
    f = 0x300000
    assert lib.dlite_accept_window(None, 7, f, 4, 8, f, None, None) == -1
    assert lib.dlite_accept_window(f, 7, f, 4, 9, f, None, None) == -2
    assert lib.dlite_accept_window(f, 7, f, 4, 0, f, None, None) == -2
    assert lib.dlite_accept_window(f, 0, f, 4, 1, f, None, None) == -2
    assert lib.dlite_accept_window(f, 7, f, 0, 8, f, None, None) == -2


def test_accept_validation_codes():
    lib = B.load_library()
    f = 0x300000
    assert lib.dlite_accept_prefix(None, f, 4, 7, f, None, None) == -1
    assert lib.dlite_accept_prefix(f, None, 4, 7, f, None, None) == -1
    assert lib.dlite_accept_prefix(f, f, 4, 7, None, None, None) == -1
    assert lib.dlite_accept_prefix(f, f, 0, 7, f, None, None) == -2
    assert lib.dlite_accept_prefix(f, f, 4, 0, f, None, None) == -2
    assert lib.dlite_accept_prefix(f, f, 4, 65, f, None, None) == -2


def test_draft_status_validation_codes():
    lib = B.load_library()
    f = 0x300000
    n = B.dlite_workspace_bytes(_dims(WORKLOADS["tiny_f32"]))
    assert lib.dlite_draft_status(None, n, f, None) == -1
    assert lib.dlite_draft_status(f, n, None, None) == -1
    assert lib.dlite_draft_status(f + 16, n, f, None) == -5
    assert lib.dlite_draft_status(f, 64, f, None) == -4


def test_block_options_workspace_and_validation_codes():
    lib = B.load_library()
    wl = WORKLOADS["tiny_f32"]
    d = _dims(wl)
    plain = B.dlite_workspace_bytes(d)
    assert B.dlite_workspace_bytes_ex(d, None) == plain
    assert B.dlite_workspace_bytes_ex(d, B.make_block_options(0)) == plain
    assert B.dlite_workspace_bytes_ex(d, B.make_block_options(1)) == plain
    need4 = B.dlite_workspace_bytes_ex(d, B.make_block_options(4, 0x500000))
    assert need4 > plain and need4 % 256 == 0
    for G in (-1, 17):
        with pytest.raises(B.DliteError) as e:
            B.dlite_workspace_bytes_ex(d, B.make_block_options(G, 0x500000))
        assert e.value.code == -2 and b"group" in lib.dlite_last_error()
    w, keep = _fake_weights(wl.n_layers)
    fake = 0x200000
    head = B.DliteGatedHead(*[fake] * 6)
    call = lambda hd, opts, nbytes: lib.dlite_draft_block_ex(
        ctypes.byref(d), ctypes.byref(w), hd, opts, fake, fake, fake, None, None, fake, nbytes, None)
    # a group without its ids, a warm-up token without the gated head
    assert call(None, ctypes.byref(B.make_block_options(4)), need4) == -1
    assert call(None, ctypes.byref(B.make_block_options(1, None, fake)), plain) == -5
    assert b"gated" in lib.dlite_last_error()
    # a group needs the larger workspace
    assert call(None, ctypes.byref(B.make_block_options(4, fake)), plain) == -4
    assert call(ctypes.byref(head), ctypes.byref(B.make_block_options(4, fake, fake)), need4 - 1) == -4
    assert call(None, ctypes.byref(B.make_block_options(17, fake)), need4) == -2
    # the largest block: m = 64 features, a group of 16 and 16 placeholders
    big = _dims(WORKLOADS["tiny_f32"], m=64, K=16)
    assert B.dlite_workspace_bytes_ex(big, B.make_block_options(16, fake)) > 0


def test_gumbel_bucket_bounds_hold():
    """The draw kernel's per-bucket bounds of -log(-log u) (generated header)
    enclose the fp64 value at every bucket's first and last word and at
    random words, and are tight enough to prune (hi - lo small except near
    u = 1)."""
    import numpy as np
    txt = open(os.path.join(ROOT, "history_free_drafter_amd", "csrc", "gumbel_bounds.hpp")).read()
    body = txt[txt.index("{", txt.index("kGumbelBounds[2 *")) + 1:txt.index("};")]
    vals = np.array([float.fromhex(t.strip().rstrip("f")) for t in body.split(",") if t.strip()])
    lo, hi = vals[0::2], vals[1::2]
    nb = len(lo)
    shift = 32 - int(np.log2(nb))
    g = lambda x: -np.log(-np.log((x.astype(np.float64) + 0.5) / 2.0 ** 32))
    b = np.arange(nb, dtype=np.uint64)
    first, last = b << np.uint64(shift), ((b + np.uint64(1)) << np.uint64(shift)) - np.uint64(1)
    assert (lo <= g(first)).all() and (g(last) <= hi).all()
    x = np.random.default_rng(0).integers(0, 2 ** 32, 200000, dtype=np.uint64)
    k = (x >> np.uint64(shift)).astype(int)
    gx = g(x)
    assert (lo[k] <= gx).all() and (gx <= hi[k]).all()
    assert np.median(hi - lo) < 0.01
