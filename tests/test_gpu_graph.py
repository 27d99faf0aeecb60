"""The draft step and accept captured in a HIP graph and replayed.

The library allocates nothing and keeps no state between calls, and it clears
its own counters with a kernel (no memset nodes), so one draft + accept pair
can be captured once and replayed.  Each replay must give bitwise the eager
result, also with other eager calls (which overwrite the same output buffers)
and synchronisations between the replays, and the step's status word must
stay 0.  Inputs are seeded device draws of the workload shapes (no oracle is
involved: the graph is compared with the same library run eagerly).
"""
import numpy as np
import pytest
import torch

from history_free_drafter_amd import binding as B
from synth import WORKLOADS

pytestmark = pytest.mark.gpu


def _device_model(w, seed, gated=False):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch.bfloat16

    def mat(*shape, std=0.02):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(dt)

    def gain(n):
        return (1.0 + torch.randn(n, generator=g, device="cuda") * 0.02).to(dt)

    D, F, r, V = w.D, w.ffn, w.rank, w.vocab
    qkv = (w.n_q + 2 * w.n_kv) * w.d_h
    wt = dict(depth_emb=mat(w.m, D), feat_norm=gain(D), tok_emb=mat(V, D), ph_emb=mat(D),
              final_norm=gain(D), seq_w_down=mat(r, D + r), seq_w_up=mat(r, r), lm_head=mat(V, r))
    wt["layers"] = [dict(attn_norm=gain(D), wqkv=mat(qkv, D), wo=mat(D, w.n_q * w.d_h),
                         ffn_norm=gain(D), w_gate_up=mat(2 * F, D), w_down=mat(D, F))
                    for _ in range(w.n_layers)]
    head = None
    if gated:
        head = dict(emb=mat(V, r, std=1.0), w_s=mat(2 * r, 2 * r), b_s=mat(2 * r),
                    w_h=mat(r, r + D), b_h=mat(r), w_o=mat(V, r))
    dims = B.make_dims(w.B, w.m, D, w.n_layers, w.n_q, w.n_kv, w.d_h, F, w.K, r, V, B.DLITE_BF16)
    H = torch.randn(w.B, w.m, D, generator=g, device="cuda").to(dt)
    anchors = torch.randint(0, V, (w.B,), generator=g, device="cuda", dtype=torch.int32)
    tgt = torch.randint(0, V, (w.B, w.K + 1), generator=g, device="cuda", dtype=torch.int32)
    return dims, wt, head, H, anchors, tgt


class _Step:
    def __init__(self, w, seed, gated=False):
        self.w = w
        self.dims, self.wt, self.head, self.H, self.anchors, self.tgt = _device_model(w, seed, gated)
        self.ws_struct, self._keep = B.make_weights(self.wt)
        self.head_struct = B.make_gated_head(self.head) if gated else None
        self.ws_bytes = B.dlite_workspace_bytes(self.dims)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.cand = torch.empty((w.B, w.K), dtype=torch.int32, device="cuda")
        self.maxl = torch.empty((w.B, w.K), dtype=torch.float32, device="cuda")
        self.A = torch.empty((w.B,), dtype=torch.int32, device="cuda")
        self.nxt = torch.empty((w.B,), dtype=torch.int32, device="cuda")
        self.status = torch.zeros((1,), dtype=torch.int32, device="cuda")

    def run(self, anchors=None):
        a = self.anchors if anchors is None else anchors
        if self.head_struct is not None:
            B.dlite_draft_block_gated(self.dims, self.ws_struct, self.head_struct, self.H, a,
                                      self.cand, self.maxl, None, self.ws, self.ws_bytes)
        else:
            B.dlite_draft_block(self.dims, self.ws_struct, self.H, a, self.cand, self.maxl, None,
                                self.ws, self.ws_bytes)
        B.dlite_accept_prefix(self.cand, self.tgt, self.w.B, self.w.K, self.A, self.nxt)

    def outputs(self):
        torch.cuda.synchronize()
        B.dlite_draft_status(self.ws, self.status, self.ws_bytes)
        torch.cuda.synchronize()
        assert int(self.status.item()) == 0, "a bounded wait timed out"
        return [t.cpu().numpy().copy() for t in (self.cand, self.maxl, self.A, self.nxt)]

    def scribble(self):
        for t in (self.cand, self.A, self.nxt):
            t.fill_(-5)
        self.maxl.fill_(float("nan"))


def _replays(step, n=10):
    step.run()
    eager = step.outputs()
    other = torch.randint(0, step.w.vocab, (step.w.B,), device="cuda", dtype=torch.int32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm the capture stream once
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="thread_local"):
        step.run()
    torch.cuda.synchronize()
    for i in range(n):
        step.scribble()
        if i % 2:                            # eager work on the same buffers in between
            step.run(anchors=other)
            step.outputs()
        graph.replay()
        got = step.outputs()
        for g_, e_ in zip(got, eager):
            np.testing.assert_array_equal(g_, e_)
    return eager


@pytest.mark.parametrize("key", ["qwen3_8b_b1", "qwen3_8b_b64_m36"])
def test_draft_and_accept_replay_from_a_graph(key):
    print(f"\n[case] graph {key}", flush=True)
    step = _Step(WORKLOADS[key], 101)
    eager = _replays(step)
    print(key, "candidates", eager[0][0].tolist(), "A", eager[2][:4].tolist(), flush=True)


def test_gated_head_replays_from_a_graph():
    """The gated head's single cooperative launch (a few requests at rank 512)
    captured with the rest of the step."""
    print("\n[case] graph gated qwen3_8b_b1", flush=True)
    step = _Step(WORKLOADS["qwen3_8b_b1"], 102, gated=True)
    _replays(step)
