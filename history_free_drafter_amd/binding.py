"""ctypes binding of libdlite.so: the C ABI declared in include/dlite.h.

Argument marshalling only.  Every step of the draft and accept computations
runs in the library's HIP kernels; torch is used for device memory and for the
current stream.  If the library is missing the import fails loudly: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdlite.so")

DLITE_F32, DLITE_BF16 = 0, 1
ERRORS = {-1: "DLITE_ERR_NULL", -2: "DLITE_ERR_SHAPE", -3: "DLITE_ERR_DTYPE",
          -4: "DLITE_ERR_WORKSPACE", -5: "DLITE_ERR_UNSUPPORTED", -6: "DLITE_ERR_HIP"}
EXPORTS = ["dlite_workspace_bytes", "dlite_draft_block", "dlite_draft_block_noalloc",
           "dlite_draft_block_at", "dlite_workspace_bytes_ex", "dlite_draft_block_ex",
           "dlite_draft_block_gated", "dlite_sampling_workspace_bytes", "dlite_sample_tokens",
           "dlite_accept_sampled", "dlite_accept_window",
           "dlite_accept_prefix", "dlite_draft_status", "dlite_set_stage_events",
           "dlite_last_error", "dlite_version"]
STAGES = ["features", "qkv", "attention", "oproj", "gate_up", "down", "final_norm",
          "seq_proj", "scan", "lm_head"]


class DliteDims(Structure):
    _fields_ = [(n, c_int32) for n in
                ("B", "m", "D", "n_layers", "n_q", "n_kv", "d_h", "ffn", "K", "rank",
                 "vocab", "dtype")] + [("rms_eps", c_float), ("rope_theta", c_float)]


class DliteLayerWeights(Structure):
    _fields_ = [(n, c_void_p) for n in
                ("attn_norm", "wqkv", "wo", "ffn_norm", "w_gate_up", "w_down")]


class DliteWeights(Structure):
    _fields_ = [("depth_emb", c_void_p), ("feat_norm", c_void_p), ("tok_emb", c_void_p),
                ("ph_emb", c_void_p), ("layers", POINTER(DliteLayerWeights)),
                ("final_norm", c_void_p), ("seq_w_down", c_void_p), ("seq_w_up", c_void_p),
                ("lm_head", c_void_p)]


class DliteGatedHead(Structure):
    _fields_ = [(n, c_void_p) for n in ("emb", "w_s", "b_s", "w_h", "b_h", "w_o")]


class DliteBlockOptions(Structure):
    _fields_ = [("group", c_int32), ("group_ids", c_void_p), ("warmup_ids", c_void_p)]


class DliteTaps(Structure):
    _fields_ = [(n, c_void_p) for n in ("z", "x", "hidden", "state", "logits")]


class DliteError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdlite.so once and declare the prototypes of its exports."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -m history_free_drafter_amd.build)")
    lib = ctypes.CDLL(path)
    lib.dlite_workspace_bytes.argtypes = [POINTER(DliteDims)]
    lib.dlite_workspace_bytes.restype = c_size_t
    lib.dlite_draft_block.argtypes = [POINTER(DliteDims), POINTER(DliteWeights), c_void_p,
                                      c_void_p, c_void_p, c_void_p, POINTER(DliteTaps),
                                      c_void_p, c_size_t, c_void_p]
    lib.dlite_draft_block.restype = c_int
    lib.dlite_draft_block_noalloc.argtypes = [POINTER(DliteDims), POINTER(DliteWeights), c_void_p,
                                              c_void_p, c_void_p, c_void_p, POINTER(DliteTaps),
                                              c_void_p, c_void_p]
    lib.dlite_draft_block_noalloc.restype = c_int
    lib.dlite_draft_block_gated.argtypes = [POINTER(DliteDims), POINTER(DliteWeights),
                                            POINTER(DliteGatedHead), c_void_p, c_void_p,
                                            c_void_p, c_void_p, POINTER(DliteTaps), c_void_p,
                                            c_size_t, c_void_p]
    lib.dlite_draft_block_gated.restype = c_int
    lib.dlite_draft_block_at.argtypes = [POINTER(DliteDims), POINTER(DliteWeights), c_void_p,
                                         c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                         POINTER(DliteTaps), c_void_p, c_size_t, c_void_p]
    lib.dlite_draft_block_at.restype = c_int
    lib.dlite_workspace_bytes_ex.argtypes = [POINTER(DliteDims), POINTER(DliteBlockOptions)]
    lib.dlite_workspace_bytes_ex.restype = c_size_t
    lib.dlite_draft_block_ex.argtypes = [POINTER(DliteDims), POINTER(DliteWeights),
                                         POINTER(DliteGatedHead), POINTER(DliteBlockOptions),
                                         c_void_p, c_void_p, c_void_p, c_void_p,
                                         POINTER(DliteTaps), c_void_p, c_size_t, c_void_p]
    lib.dlite_draft_block_ex.restype = c_int
    lib.dlite_accept_window.argtypes = [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p,
                                        c_void_p, c_void_p]
    lib.dlite_accept_window.restype = c_int
    lib.dlite_sampling_workspace_bytes.argtypes = [c_int32]
    lib.dlite_sampling_workspace_bytes.restype = c_size_t
    lib.dlite_sample_tokens.argtypes = [c_void_p, c_int32, c_int32, ctypes.c_float, ctypes.c_uint64,
                                        ctypes.c_uint32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dlite_sample_tokens.restype = c_int
    lib.dlite_accept_sampled.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                         ctypes.c_float, ctypes.c_uint64, c_void_p, c_void_p, c_void_p,
                                         c_size_t, c_void_p]
    lib.dlite_accept_sampled.restype = c_int
    lib.dlite_accept_prefix.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                        c_void_p, c_void_p]
    lib.dlite_accept_prefix.restype = c_int
    lib.dlite_draft_status.argtypes = [c_void_p, c_size_t, c_void_p, c_void_p]
    lib.dlite_draft_status.restype = c_int
    lib.dlite_set_stage_events.argtypes = [c_int, c_void_p, c_void_p]
    lib.dlite_set_stage_events.restype = c_int
    lib.dlite_last_error.argtypes = []
    lib.dlite_last_error.restype = c_char_p
    lib.dlite_version.argtypes = []
    lib.dlite_version.restype = c_char_p
    _lib = lib
    return lib


def _ptr(t):
    """Device address of a torch tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc):
    if rc != 0:
        raise DliteError(rc, load_library().dlite_last_error().decode())


def make_dims(B, m, D, n_layers, n_q, n_kv, d_h, ffn, K, rank, vocab, dtype,
              rms_eps=1e-6, rope_theta=1e6) -> DliteDims:
    return DliteDims(B, m, D, n_layers, n_q, n_kv, d_h, ffn, K, rank, vocab, dtype,
                     rms_eps, rope_theta)


def make_weights(w: dict):
    """dlite_weights from a dict of device tensors (keys as in include/dlite.h).

    Returns (struct, keepalive): keep `keepalive` referenced while the struct
    is in use (it owns the host array of layer structs).
    """
    layers = (DliteLayerWeights * len(w["layers"]))(
        *[DliteLayerWeights(*[_ptr(lw[k]) for k in
                              ("attn_norm", "wqkv", "wo", "ffn_norm", "w_gate_up", "w_down")])
          for lw in w["layers"]])
    s = DliteWeights(_ptr(w["depth_emb"]), _ptr(w["feat_norm"]), _ptr(w["tok_emb"]),
                     _ptr(w["ph_emb"]), ctypes.cast(layers, POINTER(DliteLayerWeights)),
                     _ptr(w["final_norm"]), _ptr(w["seq_w_down"]), _ptr(w["seq_w_up"]),
                     _ptr(w["lm_head"]))
    return s, layers


def make_taps(z=None, x=None, hidden=None, state=None, logits=None) -> DliteTaps:
    return DliteTaps(_ptr(z), _ptr(x), _ptr(hidden), _ptr(state), _ptr(logits))


def dlite_workspace_bytes(dims: DliteDims) -> int:
    n = load_library().dlite_workspace_bytes(ctypes.byref(dims))
    if n == 0:
        raise DliteError(-2, load_library().dlite_last_error().decode())
    return n


def dlite_draft_block(dims, weights, features, anchor_ids, candidates, max_logit=None,
                      taps=None, workspace=None, workspace_bytes=None, stream=None):
    """Enqueue one draft step; see include/dlite.h for the contract."""
    ws_bytes = workspace_bytes
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load_library().dlite_draft_block(
        ctypes.byref(dims), ctypes.byref(weights), _ptr(features), _ptr(anchor_ids),
        _ptr(candidates), _ptr(max_logit), ctypes.byref(taps) if taps is not None else None,
        _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc)


def dlite_draft_block_noalloc(dims, weights, features, anchor_ids, candidates, max_logit=None,
                              taps=None, status=None, stream=None):
    """Enqueue one draft step with the library's own scratch (no workspace, no allocation)."""
    rc = load_library().dlite_draft_block_noalloc(
        ctypes.byref(dims), ctypes.byref(weights), _ptr(features), _ptr(anchor_ids),
        _ptr(candidates), _ptr(max_logit), ctypes.byref(taps) if taps is not None else None,
        _ptr(status), _stream(stream))
    _check(rc)


def make_gated_head(h: dict):
    """dlite_gated_head from a dict of device tensors (keys as in include/dlite.h)."""
    return DliteGatedHead(*[_ptr(h[k]) for k in ("emb", "w_s", "b_s", "w_h", "b_h", "w_o")])


def dlite_draft_block_gated(dims, weights, head, features, anchor_ids, candidates,
                            max_logit=None, taps=None, workspace=None, workspace_bytes=None,
                            stream=None):
    """Enqueue a draft step with the gated sequential head; see include/dlite.h."""
    ws_bytes = workspace_bytes
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load_library().dlite_draft_block_gated(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(head) if head is not None else None,
        _ptr(features), _ptr(anchor_ids), _ptr(candidates), _ptr(max_logit),
        ctypes.byref(taps) if taps is not None else None, _ptr(workspace), ws_bytes,
        _stream(stream))
    _check(rc)


def dlite_draft_block_at(dims, weights, verify_hidden, T, accept_len, anchor_ids, candidates,
                         max_logit=None, taps=None, workspace=None, workspace_bytes=None,
                         stream=None):
    """Enqueue a draft step fed from the verify pass at index A; see include/dlite.h."""
    ws_bytes = workspace_bytes
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load_library().dlite_draft_block_at(
        ctypes.byref(dims), ctypes.byref(weights), _ptr(verify_hidden), T, _ptr(accept_len),
        _ptr(anchor_ids), _ptr(candidates), _ptr(max_logit),
        ctypes.byref(taps) if taps is not None else None, _ptr(workspace), ws_bytes,
        _stream(stream))
    _check(rc)


def make_block_options(group=1, group_ids=None, warmup_ids=None) -> DliteBlockOptions:
    """dlite_block_options: group length, [B, G-1] group ids, [B] warm-up ids (device)."""
    return DliteBlockOptions(group, _ptr(group_ids), _ptr(warmup_ids))


def dlite_workspace_bytes_ex(dims: DliteDims, opts=None) -> int:
    n = load_library().dlite_workspace_bytes_ex(ctypes.byref(dims),
                                                ctypes.byref(opts) if opts is not None else None)
    if n == 0:
        raise DliteError(-2, load_library().dlite_last_error().decode())
    return n


def dlite_draft_block_ex(dims, weights, head, opts, features, anchor_ids, candidates,
                         max_logit=None, taps=None, workspace=None, workspace_bytes=None,
                         stream=None):
    """Enqueue a draft step with a local token group and/or the gated head's
    warm-up token (head None: the fixed head); see include/dlite.h."""
    ws_bytes = workspace_bytes
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load_library().dlite_draft_block_ex(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(head) if head is not None else None,
        ctypes.byref(opts) if opts is not None else None, _ptr(features), _ptr(anchor_ids),
        _ptr(candidates), _ptr(max_logit), ctypes.byref(taps) if taps is not None else None,
        _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc)


def dlite_accept_window(candidates, K, target_tokens, B, W, accept_len, next_anchor=None,
                        stream=None):
    """Enqueue greedy verification of a W-input window; see include/dlite.h."""
    _check(load_library().dlite_accept_window(_ptr(candidates), K, _ptr(target_tokens), B, W,
                                              _ptr(accept_len), _ptr(next_anchor), _stream(stream)))


def dlite_sampling_workspace_bytes(rows: int) -> int:
    n = load_library().dlite_sampling_workspace_bytes(rows)
    if n == 0:
        raise DliteError(-2, load_library().dlite_last_error().decode())
    return n


def dlite_sample_tokens(logits, N, V, temperature, seed, stream_id, tokens, workspace, stream=None):
    """Enqueue temperature sampling of N rows; see include/dlite.h."""
    rc = load_library().dlite_sample_tokens(
        _ptr(logits), N, V, temperature, seed, stream_id, _ptr(tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)


def dlite_accept_sampled(candidates, draft_logits, target_logits, B, K, V, temperature, seed,
                         accept_len, next_token, workspace, stream=None):
    """Enqueue speculative rejection sampling of one round; see include/dlite.h."""
    rc = load_library().dlite_accept_sampled(
        _ptr(candidates), _ptr(draft_logits), _ptr(target_logits), B, K, V, temperature, seed,
        _ptr(accept_len), _ptr(next_token), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)


def dlite_accept_prefix(candidates, target_tokens, B, K, accept_len, next_anchor=None,
                        stream=None):
    """Enqueue greedy prefix acceptance; see include/dlite.h."""
    rc = load_library().dlite_accept_prefix(_ptr(candidates), _ptr(target_tokens), B, K,
                                            _ptr(accept_len), _ptr(next_anchor),
                                            _stream(stream))
    _check(rc)


def dlite_draft_status(workspace, status, workspace_bytes=None, stream=None):
    """Enqueue a copy of the last draft step's status word into status[0] (device uint32/int32)."""
    ws_bytes = workspace_bytes
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().dlite_draft_status(_ptr(workspace), ws_bytes, _ptr(status),
                                             _stream(stream)))


def dlite_set_stage_events(stage, before, after):
    """Record HIP events around one stage of later draft calls (None, None: off)."""
    if isinstance(stage, str):
        stage = STAGES.index(stage)
    _check(load_library().dlite_set_stage_events(stage, before, after))


def dlite_version() -> str:
    return load_library().dlite_version().decode()
