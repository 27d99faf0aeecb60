"""Device buffers for the draft step: weights, workspace and outputs.

torch is used only to allocate device memory and to name the stream; every
computation is a call into libdlite.so through `binding`.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as _b


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a stored array: uint16 bf16 bit patterns -> bfloat16, else as is."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


class DraftModel:
    """Weights resident on the GPU plus a workspace sized for the dimensions."""

    def __init__(self, dims: dict, weights: dict, device="cuda"):
        dt = _b.DLITE_BF16 if dims["dtype"] == "bf16" else _b.DLITE_F32
        self.shape = dict(dims)
        self.dims = _b.make_dims(dims["B"], dims["m"], dims["D"], dims["n_layers"],
                                 dims["n_q"], dims["n_kv"], dims["d_h"], dims["ffn"],
                                 dims["K"], dims["rank"], dims["vocab"], dt,
                                 dims.get("rms_eps", 1e-6), dims.get("rope_theta", 1e6))
        self.device = device
        self.w = {k: (to_device(v, device) if v is not None and k != "layers" else None)
                  for k, v in weights.items() if k != "layers"}
        self.w["layers"] = [{k: to_device(v, device) for k, v in lw.items()}
                            for lw in weights["layers"]]
        self.wstruct, self._keep = _b.make_weights(self.w)
        self.ws_bytes = _b.dlite_workspace_bytes(self.dims)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        B, K = dims["B"], dims["K"]
        self.candidates = torch.empty((B, K), dtype=torch.int32, device=device)
        self.max_logit = torch.empty((B, K), dtype=torch.float32, device=device)
        self.accept_len = torch.empty((B,), dtype=torch.int32, device=device)
        self.next_anchor = torch.empty((B,), dtype=torch.int32, device=device)
        self.status_word = torch.zeros((1,), dtype=torch.int32, device=device)

    def draft(self, features: torch.Tensor, anchors: torch.Tensor, taps=None, stream=None,
              weights=None):
        _b.dlite_draft_block(self.dims, weights if weights is not None else self.wstruct,
                             features, anchors, self.candidates, self.max_logit, taps,
                             self.workspace, self.ws_bytes, stream)
        return self.candidates

    def status(self, stream=None) -> int:
        """Status word of the last draft call (0 = every bounded wait ended
        normally); synchronises the stream to read it."""
        _b.dlite_draft_status(self.workspace, self.status_word, self.ws_bytes, stream)
        if stream is None:
            torch.cuda.current_stream().synchronize()
        else:
            stream.synchronize()
        return int(self.status_word.item())

    def set_gated_head(self, head: dict):
        """Upload the gated head's weights (storage-form arrays keyed as dlite_gated_head)."""
        self.gh = {k: to_device(v, self.device) for k, v in head.items()}
        self.ghstruct = _b.make_gated_head(self.gh)

    def draft_gated(self, features: torch.Tensor, anchors: torch.Tensor, taps=None, stream=None,
                    weights=None, head=None):
        _b.dlite_draft_block_gated(self.dims, weights if weights is not None else self.wstruct,
                                   head if head is not None else self.ghstruct, features, anchors,
                                   self.candidates, self.max_logit, taps, self.workspace,
                                   self.ws_bytes, stream)
        return self.candidates

    def draft_at(self, verify_hidden: torch.Tensor, accept_len: torch.Tensor,
                 anchors: torch.Tensor, taps=None, stream=None):
        """Draft from the previous verify pass: verify_hidden [m, B, T, D] at index accept_len."""
        _b.dlite_draft_block_at(self.dims, self.wstruct, verify_hidden, int(verify_hidden.shape[2]),
                                accept_len, anchors, self.candidates, self.max_logit, taps,
                                self.workspace, self.ws_bytes, stream)
        return self.candidates

    def draft_ex(self, features: torch.Tensor, anchors: torch.Tensor, group_ids=None,
                 warmup_ids=None, gated=False, taps=None, stream=None):
        """Draft with a local token group (group_ids [B, G-1] int32: the tokens
        before each anchor, leading negatives = padding) and/or the gated head's
        warm-up token (warmup_ids [B] int32).  The workspace grows on demand."""
        G = 1 if group_ids is None else int(group_ids.shape[1]) + 1
        opts = _b.make_block_options(G, group_ids, warmup_ids)
        need = _b.dlite_workspace_bytes_ex(self.dims, opts)
        if need > self.ws_bytes:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
            self.ws_bytes = need
        _b.dlite_draft_block_ex(self.dims, self.wstruct, self.ghstruct if gated else None, opts,
                                features, anchors, self.candidates, self.max_logit, taps,
                                self.workspace, self.ws_bytes, stream)
        return self.candidates

    def accept(self, target_tokens: torch.Tensor, stream=None):
        B, K = self.shape["B"], self.shape["K"]
        _b.dlite_accept_prefix(self.candidates, target_tokens, B, K, self.accept_len,
                               self.next_anchor, stream)
        return self.accept_len, self.next_anchor
