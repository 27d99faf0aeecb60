"""Seeded synthetic workloads for the DLite draft step.

This module only draws numbers: shapes, seeds, Gaussian weights, features,
anchor ids, per-position match probabilities and target tokens built from a
given candidate array.  It performs none of the drafter's arithmetic, so the
fp64 oracle and the HIP path can both consume its output without sharing any
of the method's code.

Storage convention: every floating tensor is returned as a numpy array in its
*storage* form.  For bf16 workloads that is ``uint16`` bf16 bit patterns
(rounded to nearest-even from an fp32 draw); for fp32 workloads it is
``float32``.  :func:`as_f64` widens either form exactly.

Workload shapes follow the drafter described in the DLite walkthrough
(pinghaoyang.com.cn, "DLite 完全拆解"): m boundary features of width D, one
anchor, K placeholders, a rank-r sequential head and a vocabulary of V.  The
paper's block of 8 counts the anchor plus 7 predictions, so K=7 (section
"草稿块长与验证块长不是一个参数").
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Rows of the token-embedding table are drawn in blocks with their own seed,
# so that any subset of rows can be regenerated without drawing the whole table.
TOK_BLOCK = 1024


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    m: int
    D: int
    n_layers: int
    n_q: int
    n_kv: int
    d_h: int
    ffn: int
    K: int
    rank: int
    vocab: int
    dtype: str
    seed: int
    match: str                 # "const:<c>", "pow:<c>" (c_i=c^i), "uniform:<lo>:<hi>" (per request)
    feat_scale_step: float = 0.0   # slot l multiplied by (1 + step*l)
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    weight_std: float = 0.02
    gain_std: float = 0.02     # norm gains are 1 + N(0, gain_std)

    @property
    def S(self) -> int:
        """Slots per request: m context features, the anchor, K placeholders."""
        return self.m + 1 + self.K

    @property
    def qkv_rows(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.d_h

    def weight_bytes(self) -> int:
        """Bytes of weights the step reads once (token table: only B rows)."""
        e = 2 if self.dtype == BF16 else 4
        D, F, r, V = self.D, self.ffn, self.rank, self.vocab
        per_layer = (self.qkv_rows * D + D * self.n_q * self.d_h
                     + 2 * F * D + D * F + 2 * D)
        n = (self.m * D + D + self.B * D + D + self.n_layers * per_layer + D
             + r * (D + r) + r * r + V * r)
        return n * e


def _w(name, B, m, D, L, nq, nkv, dh, F, K, r, V, dt, i, match, step=0.0):
    return Workload(name, B, m, D, L, nq, nkv, dh, F, K, r, V, dt,
                    20261016 + i, match, step)


# The workloads: a tiny fp32 block, Qwen3-4B and Qwen3-8B shaped single
# requests, a 32-request two-layer batch, a 64-request all-layer batch, and
# the 8B single request with the five-layer backbone the paper trains.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    _w("tiny_f32", 1, 4, 256, 1, 4, 2, 64, 512, 7, 32, 4096, F32, 1,
       "const:0.8", 0.25),
    _w("qwen3_4b_b1", 1, 12, 2560, 1, 32, 8, 128, 9728, 7, 320, 151936, BF16,
       2, "pow:0.85"),
    _w("qwen3_8b_b1", 1, 14, 4096, 1, 32, 8, 128, 12288, 7, 512, 151936, BF16,
       3, "pow:0.85"),
    _w("qwen3_8b_b32_l2", 32, 14, 4096, 2, 32, 8, 128, 12288, 7, 512, 151936,
       BF16, 4, "uniform:0.5:0.95"),
    _w("qwen3_8b_b64_m36", 64, 36, 4096, 1, 32, 8, 128, 12288, 7, 512, 151936,
       BF16, 5, "pow:0.9"),
    _w("qwen3_8b_b1_l5", 1, 14, 4096, 5, 32, 8, 128, 12288, 7, 512, 151936,
       BF16, 6, "pow:0.85"),
]}


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit fields (small test shapes)."""
    base = dict(B=1, m=2, D=64, n_layers=1, n_q=2, n_kv=1, d_h=64, ffn=128,
                K=3, rank=16, vocab=256, dtype=F32, seed=7, match="const:0.8")
    base.update(kw)
    return Workload(name=name, **base)


# ---------------------------------------------------------------- storage ---

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of a stored tensor (bf16 bits or fp32) to float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == BF16 else a32.astype(np.float32)


# ------------------------------------------------------------------ draws ---

def _streams(w: Workload) -> Dict[str, np.random.SeedSequence]:
    names = ["weights", "features", "anchors", "match", "tokens", "tok_emb", "verify", "gated"]
    kids = np.random.SeedSequence(w.seed).spawn(len(names))
    return dict(zip(names, kids))


def _normal(rng, shape, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _gain(rng, n, std):
    return (np.float32(1.0) + _normal(rng, (n,), std)).astype(np.float32)


def tok_emb_rows(w: Workload, rows) -> np.ndarray:
    """Regenerate selected rows of the token-embedding table (storage form)."""
    rows = np.asarray(rows, dtype=np.int64)
    seq = _streams(w)["tok_emb"]
    out = np.empty((len(rows), w.D), dtype=np.uint16 if w.dtype == BF16 else np.float32)
    cache = {}
    for i, v in enumerate(rows):
        blk = int(v) // TOK_BLOCK
        if blk not in cache:
            cache[blk] = _tok_block(w, seq, blk)
        out[i] = cache[blk][int(v) - blk * TOK_BLOCK]
    return out


def _tok_block(w: Workload, seq, blk: int) -> np.ndarray:
    n = min(TOK_BLOCK, w.vocab - blk * TOK_BLOCK)
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seq.entropy, spawn_key=seq.spawn_key + (blk,))))
    return _store(_normal(rng, (n, w.D), w.weight_std), w.dtype)


def tok_emb_table(w: Workload, threads: int = 8) -> np.ndarray:
    """The whole [V, D] token-embedding table (storage form), drawn per block."""
    seq = _streams(w)["tok_emb"]
    nblk = (w.vocab + TOK_BLOCK - 1) // TOK_BLOCK
    out = np.empty((w.vocab, w.D), dtype=np.uint16 if w.dtype == BF16 else np.float32)

    def fill(b):
        out[b * TOK_BLOCK:(b + 1) * TOK_BLOCK] = _tok_block(w, seq, b)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def make_weights(w: Workload, with_tok_table: bool = True) -> dict:
    """Drafter weights, all ~N(0, 0.02) except norm gains (1 + N(0, 0.02)).

    Matrix layouts (row-major, out_features x in_features):
      layers[i]: attn_norm [D], wqkv [(n_q+2 n_kv) d_h, D] (q heads, k heads,
      v heads), wo [D, n_q d_h], ffn_norm [D], w_gate_up [2F, D] (gate rows
      then up rows), w_down [D, F]; depth_emb [m, D]; feat_norm [D];
      tok_emb [V, D]; ph_emb [D]; final_norm [D]; seq_w_down [r, D + r]
      (columns: hidden part then state part); seq_w_up [r, r]; lm_head [V, r].
    """
    rng = np.random.Generator(np.random.PCG64(_streams(w)["weights"]))
    s, g = w.weight_std, w.gain_std
    D, F, r, V = w.D, w.ffn, w.rank, w.vocab
    st = lambda a: _store(a, w.dtype)
    out = {
        "depth_emb": st(_normal(rng, (w.m, D), s)),
        "feat_norm": st(_gain(rng, D, g)),
        "ph_emb": st(_normal(rng, (D,), s)),
        "final_norm": None, "layers": [],
    }
    for _ in range(w.n_layers):
        out["layers"].append({
            "attn_norm": st(_gain(rng, D, g)),
            "wqkv": st(_normal(rng, (w.qkv_rows, D), s)),
            "wo": st(_normal(rng, (D, w.n_q * w.d_h), s)),
            "ffn_norm": st(_gain(rng, D, g)),
            "w_gate_up": st(_normal(rng, (2 * F, D), s)),
            "w_down": st(_normal(rng, (D, F), s)),
        })
    out["final_norm"] = st(_gain(rng, D, g))
    out["seq_w_down"] = st(_normal(rng, (r, D + r), s))
    out["seq_w_up"] = st(_normal(rng, (r, r), s))
    out["lm_head"] = st(_normal(rng, (V, r), s))
    if with_tok_table:
        out["tok_emb"] = tok_emb_table(w)
    return out


def make_gated_head(w: Workload) -> dict:
    """Weights of the gated sequential head (R = rank), storage form.

    emb [V, R] ~ N(0, 1) (the previous token's R-wide embedding);
    w_s [2R, 2R] (rows: g then c; columns: state then embedding), b_s [2R],
    w_h [R, R + D] (columns: state then backbone row), b_h [R], w_o [V, R]:
    ~ N(0, weight_std).
    """
    rng = np.random.Generator(np.random.PCG64(_streams(w)["gated"]))
    s, R, D, V = w.weight_std, w.rank, w.D, w.vocab
    st = lambda a: _store(a, w.dtype)
    return {
        "emb": st(_normal(rng, (V, R), 1.0)),
        "w_s": st(_normal(rng, (2 * R, 2 * R), s)),
        "b_s": st(_normal(rng, (2 * R,), s)),
        "w_h": st(_normal(rng, (R, R + D), s)),
        "b_h": st(_normal(rng, (R,), s)),
        "w_o": st(_normal(rng, (V, R), s)),
    }


def make_features(w: Workload) -> np.ndarray:
    """Boundary features H [B, m, D] ~ N(0,1); slot l scaled by (1 + step*l)."""
    rng = np.random.Generator(np.random.PCG64(_streams(w)["features"]))
    h = rng.standard_normal((w.B, w.m, w.D), dtype=np.float32)
    if w.feat_scale_step:
        h *= (1.0 + w.feat_scale_step * np.arange(w.m, dtype=np.float32))[None, :, None]
    return _store(h, w.dtype)


def make_verify_hidden(w: Workload, T: int):
    """Hidden states of the m selected target layers at T verify inputs.

    Returns (verify_hidden [m, B, T, D] stored like the features, A [B]):
    N(0,1) rows with the features' per-slot scaling, and accept lengths that
    take 0 and T - 1 at the first two requests and are uniform on [0, T)
    elsewhere.
    """
    rng = np.random.Generator(np.random.PCG64(_streams(w)["verify"]))
    h = rng.standard_normal((w.m, w.B, T, w.D), dtype=np.float32)
    if w.feat_scale_step:
        h *= (1.0 + w.feat_scale_step * np.arange(w.m, dtype=np.float32))[:, None, None, None]
    A = rng.integers(0, T, size=w.B).astype(np.int32)
    A[0] = 0
    if w.B > 1:
        A[1] = T - 1
    return _store(h, w.dtype), A


def make_anchors(w: Workload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(_streams(w)["anchors"]))
    return rng.integers(0, w.vocab, size=w.B, dtype=np.int64).astype(np.int32)


def match_probs(w: Workload) -> np.ndarray:
    """Per-request, per-position pass probabilities c[b, i], i = 1..K."""
    kind, *args = w.match.split(":")
    i = np.arange(1, w.K + 1, dtype=np.float64)
    if kind == "const":
        return np.full((w.B, w.K), float(args[0]))
    if kind == "pow":
        return np.tile(float(args[0]) ** i, (w.B, 1))
    if kind == "uniform":
        rng = np.random.Generator(np.random.PCG64(_streams(w)["match"]))
        c = rng.uniform(float(args[0]), float(args[1]), size=w.B)
        return np.repeat(c[:, None], w.K, axis=1)
    raise ValueError(w.match)


def make_target_tokens(w: Workload, cand: np.ndarray, c: Optional[np.ndarray] = None,
                       seed_offset: int = 0) -> np.ndarray:
    """Target greedy tokens t[b, 0..K] for the verify input [a, d_1..d_K].

    Position i < K agrees with the candidate d_{i+1} with probability c[b, i];
    otherwise it is drawn uniformly from the vocabulary minus d_{i+1}, so the
    pass probability is exactly c.  The last position (the bonus token after
    the whole block) is uniform over the vocabulary.
    """
    cand = np.asarray(cand, dtype=np.int64)
    B, K = cand.shape
    c = match_probs(w) if c is None else c
    seq = _streams(w)["tokens"]
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seq.entropy, spawn_key=seq.spawn_key + (seed_offset,))))
    hit = rng.random((B, K)) < c
    other = rng.integers(0, w.vocab - 1, size=(B, K))
    other = other + (other >= cand)          # skip the candidate itself
    t = np.empty((B, K + 1), dtype=np.int64)
    t[:, :K] = np.where(hit, cand, other)
    t[:, K] = rng.integers(0, w.vocab, size=B)
    return t.astype(np.int32)


def make_sampling_case(seed: int, B: int, K: int, V: int, scale: float = 2.0, mix: float = 0.7):
    """Logits for sampling tests: draft [B, K, V] and target [B, K + 1, V] fp32.

    Draft rows ~ scale * N(0, 1); target rows at the candidate positions are
    mix * draft + sqrt(1 - mix^2) * scale * N(0, 1) (overlapping but different
    distributions, so both acceptances and rejections occur); the target's
    last row is independent.
    """
    rng = np.random.default_rng(seed)
    draft = (scale * rng.standard_normal((B, K, V))).astype(np.float32)
    target = np.empty((B, K + 1, V), dtype=np.float32)
    noise = scale * rng.standard_normal((B, K + 1, V))
    target[:, :K] = mix * draft + np.sqrt(1.0 - mix * mix) * noise[:, :K]
    target[:, K] = noise[:, K]
    return draft, target
