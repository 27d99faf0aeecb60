"""Plain fp64 CPU oracle for the DLite draft step and greedy prefix accept.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product library never
does.  It is deliberately slow and direct: numpy float64 throughout, one
library matmul per linear map, no fusion and no reordering beyond what the
definitions below state.  It shares no code with the HIP implementation.

Sources.  Citations name the page and its section:
  [W]  "DLite 完全拆解" walkthrough, pinghaoyang.com.cn (the primary source);
  [S]  DLite paper summary, yomxxx.com;
  [F]  DFlash article, charlestar.github.io (shared verification math).

Where the pages leave a step open the plainest reading is taken; each such
reading is marked READING below.

Pinned by the tests under tests/ (closed forms, worked examples printed on the
pages, library cross-checks, invariants and special cases).  Parity status of
the composed drafter: the pages print no value for any draft tensor, so the
composition is pinned through its pinned parts plus invariants only.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- pieces ---


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMS normalisation over the last axis with a learned gain.

    [W] section "历史并没有消失，而是由目标模型编码": the official code normalises
    the depth-embedded feature.  READING: RMSNorm with gain, eps = 1e-6.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def feature_slots(H: np.ndarray, depth_emb: np.ndarray, gain: np.ndarray,
                  eps: float) -> np.ndarray:
    """z[b, l] = Norm(h^(l) + e_depth^(l)) for each of the m selected layers.

    [W] "历史并没有消失，而是由目标模型编码", equation for z_t^(l): a learned
    depth vector of width D is added to each layer's hidden state.  [W]
    "沿序列维拼接，保留各层的独立身份": the m features stay m separate sequence
    slots of width D (not one concatenated m*D vector).
    H: [B, m, D]; depth_emb: [m, D]  ->  [B, m, D].
    """
    return rms_norm(H + depth_emb[None, :, :], gain, eps)


def local_positions(m: int, K: int) -> np.ndarray:
    """Local RoPE positions of the S = m + 1 + K slots of one request.

    [W] "局部位置编码切断草稿端的全局位置增长" (Figure 3 layout): the target
    features and the anchor sit at local position 0, the placeholders follow
    at 1, 2, 3, ...  Slot order: [features 0..m-1, anchor, placeholders 1..K].
    """
    return np.concatenate([np.zeros(m + 1, dtype=np.int64),
                           np.arange(1, K + 1, dtype=np.int64)])


def group_positions(m: int, G: int, n_valid: int, K: int):
    """Local positions and key validity of the m + G + K slots of one request
    whose local input is a token group of G slots, n_valid of them real.

    [W] "局部位置编码切断草稿端的全局位置增长": the official position builder
    allows a fixed-length local token group and takes the start of the valid
    group as the coordinate origin, so the span depends only on the group and
    block lengths.  READING: the group holds the last G tokens up to and
    including the anchor, padded at the front when fewer exist; valid group
    token j sits at j - (G - n_valid) (the anchor at n_valid - 1), the feature
    slots share the anchor's position (Figure 3: "the same boundary"), and
    placeholder k sits at n_valid - 1 + k.  Padding slots are no keys (their
    position is irrelevant and set to 0).  G = 1 is Figure 3's layout.
    Slot order: [features 0..m-1, group 0..G-1, placeholders 1..K].
    Returns (pos [S] int64, key_valid [S] bool).
    """
    if not 1 <= n_valid <= G:
        raise ValueError("the group must hold the anchor (1 <= n_valid <= G)")
    pad = G - n_valid
    pos = np.concatenate([np.full(m, n_valid - 1, dtype=np.int64),
                          np.maximum(np.arange(G, dtype=np.int64) - pad, 0),
                          n_valid - 1 + np.arange(1, K + 1, dtype=np.int64)])
    valid = np.ones(m + G + K, dtype=bool)
    valid[m:m + pad] = False
    return pos, valid


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing (i, i + d/2).

    READING: frequency of pair i is theta^(-2i/d), theta = 1e6, as in the
    Qwen3 targets the pages use.  x: [..., S, heads, d]; pos: [S].
    """
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]          # [S, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def block_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    key_valid: np.ndarray = None) -> np.ndarray:
    """Non-causal attention of the local queries over every slot of the block.

    [W] "锚点是已经确定、尚待目标前向处理的输入": inside the short block the
    drafter attends non-causally, so all placeholders are computed at once.
    [W] "本轮临时 K/V 仍然需要计算": Q for the anchor and placeholders, K and V
    for the context features and the local inputs; nothing persists.
    Grouped heads: query head h reads key/value head floor(h / G).
    q: [Lq, n_q, d]; k, v: [S, n_kv, d]  ->  [Lq, n_q, d].  key_valid [S]
    (optional): slots that are keys (padding of a local token group is not).
    """
    n_q, d = q.shape[1], q.shape[2]
    G = n_q // k.shape[1]
    out = np.empty_like(q)
    if key_valid is not None:        # only the slots that are keys take part
        k, v = k[key_valid], v[key_valid]
    for h in range(n_q):
        kh, vh = k[:, h // G, :], v[:, h // G, :]
        sc = (q[:, h, :] @ kh.T) / np.sqrt(d)                      # [Lq, S]
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu_ffn(n: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """W_down (silu(W_gate n) * W_up n); w_gate_up holds gate rows then up rows.

    READING: the backbone layer form is not printed; a pre-norm Qwen3-style
    block (grouped attention + SwiGLU, no biases) is taken.
    """
    F = w_gate_up.shape[0] // 2
    g = n @ w_gate_up[:F].T
    u = n @ w_gate_up[F:].T
    return (silu(g) * u) @ w_down.T


# --------------------------------------------------------------- backbone ---


def backbone_layer(ctx: np.ndarray, x: np.ndarray, pos: np.ndarray, lw: dict,
                   dims, key_valid: np.ndarray = None) -> np.ndarray:
    """One history-free backbone layer for one request.

    ctx: [m, D] context slots (fixed across layers, READING of [W] "本轮临时
    K/V 仍然需要计算": context features only supply K and V);
    x: [L, D] residual stream of the local rows: the anchor (or the local
    token group) and the placeholders; pos [m + L] their local positions;
    key_valid [m + L] (optional) which slots are keys.
    Returns the updated local residual stream.
    """
    n_q, n_kv, d_h, eps = dims.n_q, dims.n_kv, dims.d_h, dims.rms_eps
    m = ctx.shape[0]
    slots = np.concatenate([ctx, x], axis=0)                         # [S, D]
    n_slots = rms_norm(slots, lw["attn_norm"], eps)
    wq = lw["wqkv"][: n_q * d_h]
    wk = lw["wqkv"][n_q * d_h: (n_q + n_kv) * d_h]
    wv = lw["wqkv"][(n_q + n_kv) * d_h:]
    q = (n_slots[m:] @ wq.T).reshape(-1, n_q, d_h)
    k = (n_slots @ wk.T).reshape(-1, n_kv, d_h)
    v = (n_slots @ wv.T).reshape(-1, n_kv, d_h)
    q = rope(q, pos[m:], dims.rope_theta)
    k = rope(k, pos, dims.rope_theta)
    o = block_attention(q, k, v, key_valid).reshape(x.shape[0], n_q * d_h)
    x = x + o @ lw["wo"].T
    n2 = rms_norm(x, lw["ffn_norm"], eps)
    return x + swiglu_ffn(n2, lw["w_gate_up"], lw["w_down"])


# ---------------------------------------------------------- sequential head ---


def sequential_head(h: np.ndarray, w_down: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """Low-rank recurrent state over the K block positions.

    [W] "把条件分布拆成历史与本块前缀": a narrow state s_i in R^R, R << D, restores
    the in-block dependency; it is reset at block start ("官方顺序头具体算了什么").
    READING (the recurrence is fixed by the build's statement, because the
    pages print only a different, token-fed gated head):
        s_0 = 0,  s_k = s_{k-1} + W_up silu(W_down [h_k ; s_{k-1}]).
    h: [K, D]; w_down: [r, D + r]; w_up: [r, r]  ->  s: [K, r] (s_1..s_K).
    """
    K = h.shape[0]
    r = w_up.shape[0]
    s = np.zeros(r)
    out = np.empty((K, r))
    for k in range(K):
        t = w_down @ np.concatenate([h[k], s])
        s = s + w_up @ silu(t)
        out[k] = s
    return out


def lm_head_argmax(s: np.ndarray, lm_head: np.ndarray):
    """Vocabulary projection applied once, after the head, then greedy choice.

    [W] "避免的是昂贵的中间词表投影" and [S] "设计": the R -> V projection is done
    once after the in-block dependencies are integrated.  [W] "贪心模式与随机模式
    要分别说明": at temperature 0 the token with the largest logit is chosen.
    READING: ties go to the lowest vocabulary index.
    s: [..., r]; lm_head: [V, r]  ->  logits [..., V], tokens [...], margin [...]
    (margin = largest minus second-largest logit).
    """
    logits = s @ lm_head.T
    tok = np.argmax(logits, axis=-1)          # first index of the maximum
    top2 = np.partition(logits, -2, axis=-1)[..., -2:]
    margin = top2[..., 1] - top2[..., 0]
    return logits, tok.astype(np.int64), margin


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def gated_state_step(s: np.ndarray, v: np.ndarray, head: dict) -> np.ndarray:
    """One gated state update ([W] "官方顺序头具体算了什么"):
    [g; c] = W_s [s; v] + b_s, s' = sigmoid(g) * s + (1 - sigmoid(g)) * tanh(c)."""
    R = s.shape[0]
    gc = head["w_s"] @ np.concatenate([s, v]) + head["b_s"]
    f = sigmoid(gc[:R])
    return f * s + (1.0 - f) * np.tanh(gc[R:])


def gated_head(h: np.ndarray, anchor: int, head: dict, forced=None, warmup=None) -> dict:
    """The walkthrough's own sequential head for one request, greedy.

    [W] "官方顺序头具体算了什么": the previous token enters through an R-wide
    embedding, d_0 = a, v_i = E_R(d_{i-1}); then
        [g_i ; c_i] = W_s [s_{i-1} ; v_i] + b_s,   f_i = sigmoid(g_i),
        s_i = f_i * s_{i-1} + (1 - f_i) * tanh(c_i),
        r_i = W_h [s_i ; u_i] + b_h,               logits_i = W_o r_i,
    and d_i is chosen from logits_i before position i + 1 ([W] "贪心模式与随机
    模式要分别说明": the largest logit at temperature 0; ties to the lowest
    index, as everywhere here).
    READING: s_0 = 0 (the state starts at the block start, no warm-up token);
    u_i = h_i, the final-normed backbone row of placeholder i; an anchor id
    outside [0, V) reads a zero embedding row (its candidates are reported
    as -1 by the caller).
    Warm-up ([W], same section: when the configuration allows, one token
    before the anchor warms the state up over a fixed length).  READING: with
    warmup = w in [0, V), one state update with v = E_R(w) from s = 0 and no
    output precedes position 1 (so s_0 is that state); warmup None or outside
    [0, V) (no token before the anchor) leaves s_0 = 0.
    h: [K, D]; head: emb [V, R], w_s [2R, 2R], b_s [2R], w_h [R, R + D],
    b_h [R], w_o [V, R].  forced: optional [K] tokens fed back in place of
    the chosen ones (to follow a run that chose differently at a near tie).
    Returns s [K, R], r [K, R], logits [K, V], cand [K], margin [K].
    """
    K = h.shape[0]
    emb = head["emb"]
    w_h, b_h, w_o = head["w_h"], head["b_h"], head["w_o"]
    R = emb.shape[1]
    V = w_o.shape[0]
    s = np.zeros(R)
    if warmup is not None and 0 <= int(warmup) < emb.shape[0]:
        s = gated_state_step(s, emb[int(warmup)], head)
    out = dict(s=np.empty((K, R)), r=np.empty((K, R)), logits=np.empty((K, V)),
               cand=np.empty(K, dtype=np.int64), margin=np.empty(K))
    d_prev = int(anchor)
    for i in range(K):
        v = emb[d_prev] if 0 <= d_prev < emb.shape[0] else np.zeros(R)
        s = gated_state_step(s, v, head)
        r = w_h @ np.concatenate([s, h[i]]) + b_h
        logits, tok, margin = lm_head_argmax(r, w_o)
        out["s"][i], out["r"][i], out["logits"][i] = s, r, logits
        out["cand"][i], out["margin"][i] = tok, margin
        d_prev = int(tok) if forced is None else int(forced[i])
    return out


def gated_heads(h: np.ndarray, anchors: np.ndarray, head: dict, forced=None,
                warmups=None) -> dict:
    """gated_head for every request: h [B, K, D], anchors [B] ids, forced
    [B, K] or None, warmups [B] ids (the token before each anchor) or None."""
    runs = [gated_head(h[b], int(anchors[b]), head, None if forced is None else forced[b],
                       None if warmups is None else int(warmups[b]))
            for b in range(h.shape[0])]
    return {k: np.stack([o[k] for o in runs]) for k in runs[0]}


# ------------------------------------------------------------------- step ---


def draft_block(dims, weights: dict, H: np.ndarray, anchor_rows: np.ndarray,
                with_head: bool = True, group_rows: np.ndarray = None,
                group_valid: np.ndarray = None) -> dict:
    """The whole draft step for a batch: K greedy candidates per request.

    dims: object with B, m, D, n_layers, n_q, n_kv, d_h, K, rms_eps, rope_theta.
    weights: fp64 arrays keyed as in the library's weight layout (layers list).
    H: [B, m, D] boundary features; anchor_rows: [B, D] = tok_emb[anchor].
    Local token group (optional, [W] "锚点是已经确定、尚待目标前向处理的输入":
    the draft input holds the anchor or a fixed-length local token group):
    group_rows [B, G, D] = tok_emb of the last G tokens ending at the anchor
    (rows of padding slots are ignored), group_valid [B] = real tokens per
    request (a suffix of the group); anchor_rows is then not read.  The group
    rows are local rows like the anchor (they query and are updated in every
    layer); positions follow group_positions.
    Returns dict with z [B,m,D], x_layers (list of [B,L,D], L = 1 + K or
    G + K), h [B,K,D], s [B,K,r], logits [B,K,V], cand [B,K], margin [B,K].

    [W] "从目标隐藏状态到并行草稿表示" (Figure 3) and the generation loop in
    "一轮执行后，缓存、锚点与隐藏状态怎样对齐": features + anchor + placeholders
    -> parallel backbone -> sequential head -> proposals.
    """
    B, m, K = dims.B, dims.m, dims.K
    z = feature_slots(H, weights["depth_emb"], weights["feat_norm"], dims.rms_eps)
    if group_rows is None:
        G = 1
        pos = [local_positions(m, K)] * B
        valid = [None] * B
        lead = np.asarray(anchor_rows)[:, None, :]
    else:
        G = group_rows.shape[1]
        pv = [group_positions(m, G, int(group_valid[b]), K) for b in range(B)]
        pos = [p for p, _ in pv]
        valid = [v for _, v in pv]
        lead = np.where(np.stack([v[m:m + G] for v in valid])[:, :, None], group_rows, 0.0)
    # [W] "锚点是已经确定…": the anchor (or the token group) enters through
    # its embedding; READING: one shared learned placeholder vector for all K
    # slots.
    x = np.empty((B, G + K, dims.D))
    x[:, :G] = lead
    x[:, G:] = weights["ph_emb"][None, None, :]
    x_layers = []
    for lw in weights["layers"]:
        x = np.stack([backbone_layer(z[b], x[b], pos[b], lw, dims, valid[b]) for b in range(B)])
        x_layers.append(x.copy())
    # READING: a final RMSNorm before the head; only placeholder rows are drafted.
    h = rms_norm(x[:, G:], weights["final_norm"], dims.rms_eps)
    if not with_head:   # the backbone only (for another sequential head)
        return dict(z=z, x_layers=x_layers, h=h)
    s = np.stack([sequential_head(h[b], weights["seq_w_down"], weights["seq_w_up"])
                  for b in range(B)])
    logits, cand, margin = lm_head_argmax(s, weights["lm_head"])
    return dict(z=z, x_layers=x_layers, h=h, s=s, logits=logits, cand=cand,
                margin=margin)


# ----------------------------------------------------------------- accept ---


def accept_prefix(cand: np.ndarray, target: np.ndarray):
    """Greedy verification: longest accepted prefix and the next anchor.

    [W] "一次因果前向评估整条候选": only the leading run of passes is committed;
    the official code takes a cumulative product of the boolean matches.
    [W] "先拆开一次投机轮次的时间": 0 <= A <= K and a round commits A + 1 tokens.
    [W] "一轮执行后…": the next anchor is the target token at verify index A
    (index 0 is the anchor's own output when nothing passed).
    cand: [B, K] draft tokens d_1..d_K; target: [B, K + 1] target tokens at
    the verify inputs [a, d_1..d_K].  Returns A [B], next_anchor [B].
    """
    cand = np.asarray(cand)
    target = np.asarray(target)
    K = cand.shape[1]
    passed = (cand == target[:, :K]).astype(np.int64)
    A = np.cumprod(passed, axis=1).sum(axis=1)
    nxt = target[np.arange(target.shape[0]), A]
    return A.astype(np.int64), nxt.astype(np.int64)


def accept_window(cand: np.ndarray, target: np.ndarray, W: int):
    """Greedy verification of a window of W inputs (anchor included).

    [W] "草稿块长与验证块长不是一个参数": a verify window shorter than the
    block still lets the drafter predict all K candidates; only the first
    W - 1 are sent to the target and the tail is dropped.  cand [B, K];
    target [B, W] (the target's tokens at the W window inputs).  Returns A
    [B] in 0 .. W - 1 and the next anchor target[b, A].
    """
    cand = np.asarray(cand)
    target = np.asarray(target)
    return accept_prefix(cand[:, :W - 1], target[:, :W])


def boundary_features(verify_hidden: np.ndarray, A: np.ndarray) -> np.ndarray:
    """The next round's boundary features, taken from the verify pass at index A.

    [W] "一轮执行后，缓存、锚点与隐藏状态怎样对齐", step 5 and the state-relation
    pseudo-code after it: the m selected target layers' hidden states are read
    at verify index A_b of the input [a, d_1..d_K], the last input that stays
    (index 0 is the anchor a when nothing passed, index 2 is d_2 when two
    passed); positions of rejected candidates are never used.
    verify_hidden: [m, B, T, D], one [B, T, D] block per selected layer (T
    verify inputs per request); A: [B] with 0 <= A_b < T.  Returns [B, m, D].
    """
    verify_hidden = np.asarray(verify_hidden)
    A = np.asarray(A)
    m, B, T, D = verify_hidden.shape
    if A.shape != (B,) or (A < 0).any() or (A >= T).any():
        raise ValueError("accept lengths must lie in [0, T)")
    H = np.empty((B, m, D), dtype=verify_hidden.dtype)
    for b in range(B):
        H[b] = verify_hidden[:, b, int(A[b]), :]
    return H


def prefix_survival(c: np.ndarray) -> np.ndarray:
    """P(A >= k) = prod_{i<=k} c_i for k = 1..K ([F] "为什么验证仍然只接受最长前缀")."""
    return np.cumprod(np.asarray(c, dtype=np.float64), axis=-1)


def expected_commit(c: np.ndarray) -> np.ndarray:
    """tau = E[A + 1] = 1 + sum_j P(A >= j) ([W] "分布重叠怎样影响平均推进量")."""
    return 1.0 + prefix_survival(c).sum(axis=-1)


# ------------------------------------------------- sampling at temperature ---
# Random numbers: Philox4x32-10 (J. Salmon, M. Moraes, R. Dror, D. Shaw,
# "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written from its
# published definition: ten rounds, each two 32 x 32 -> 64-bit products of
# counter words 0 and 2 with the round multipliers, the high halves xor-ed
# with the other counter words and the key, the key bumped by the Weyl
# constants.  A uniform in (0, 1) is (x0 + 1/2) / 2^32 (exact in fp64).

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counter words ctr[0..3] and key words key[0..1]
    (scalars or equal-shape uint arrays); returns the four output words."""
    m = 0xFFFFFFFF
    c = [np.asarray(x, dtype=np.uint64) & m for x in ctr]
    k = [np.asarray(x, dtype=np.uint64) & m for x in key]
    for _ in range(10):
        p0 = c[0] * _PHILOX_M[0]
        p1 = c[2] * _PHILOX_M[1]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & m, (p0 >> 32) ^ c[3] ^ k[1], p0 & m]
        k = [(k[0] + _PHILOX_W[0]) & m, (k[1] + _PHILOX_W[1]) & m]
    return [x.astype(np.uint32) for x in c]


def uniform01(seed: int, stream: int, a, b) -> np.ndarray:
    """Uniform in (0, 1) with index a of row b in the given stream.

    READING (the pages name no generator): word a mod 4 of Philox4x32-10 at
    counter (a div 4, b, stream, 0) under key (seed low, seed high), as
    u = (word + 1/2) / 2^32; one generator call yields four uniforms.
    """
    a = np.asarray(a)
    b = np.broadcast_to(np.asarray(b), a.shape)
    x = philox4x32_10((a >> 2, b, np.full(a.shape, stream), np.zeros(a.shape)),
                      (np.full(a.shape, seed & 0xFFFFFFFF), np.full(a.shape, (seed >> 32) & 0xFFFFFFFF)))
    word = np.choose(a & 3, x)
    return (word.astype(np.float64) + 0.5) / 4294967296.0


def softmax_t(logits: np.ndarray, T: float) -> np.ndarray:
    """softmax(logits / T) in fp64 along the last axis."""
    z = np.asarray(logits, dtype=np.float64) / T
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def sample_tokens(logits: np.ndarray, T: float, seed: int, stream: int):
    """One token per row of logits [N, V] drawn from softmax(logits / T).

    [W] "贪心模式与随机模式要分别说明": at a positive temperature the draft
    samples its candidates (and, in match mode, the target its tokens).
    READING: drawn by the Gumbel-max rule, argmax_v (l_v / T - log(-log u_v))
    with u_v = uniform01(seed, stream, v, row), which is distributed exactly as
    softmax(l / T) (ties to the lowest index).  Returns tokens [N] and the gap
    between the two best perturbed scores (for comparisons at near ties).
    """
    x = np.asarray(logits, dtype=np.float64)
    N, V = x.shape
    v, n = np.meshgrid(np.arange(V), np.arange(N))
    u = uniform01(seed, stream, v, n)
    score = x / T - np.log(-np.log(u))
    tok = np.argmax(score, axis=1)
    if V == 1:   # a single token: no runner-up
        return tok.astype(np.int64), np.full(N, np.inf)
    top2 = np.partition(score, -2, axis=1)[:, -2:]
    return tok.astype(np.int64), top2[:, 1] - top2[:, 0]


def inverse_cdf(w: np.ndarray, u: float):
    """The first index whose running sum of the weights w exceeds u * sum(w)
    (the last positive weight if rounding leaves none); also the distance of
    u * sum(w) to the nearest running sum (for comparisons near a boundary)."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    t = u * c[-1]
    idx = int(np.searchsorted(c, t, side="right"))
    if idx >= len(c):
        idx = int(np.nonzero(np.asarray(w) > 0)[0][-1])
    return idx, float(np.min(np.abs(c - t)))


def accept_sampled(cand: np.ndarray, draft_logits: np.ndarray, target_logits: np.ndarray,
                   T: float, seed: int) -> dict:
    """Speculative rejection sampling of one round per request.

    [W] "贪心模式与随机模式要分别说明": with p the target's and q the draft's
    conditional distribution at a candidate position and d ~ q the candidate,
    d is accepted with probability min(1, p(d) / q(d)); at the first rejection
    the token is drawn from the normalised positive residual [p - q]_+, so the
    committed token is distributed as p; the leading run of accepted
    candidates is committed (the first-failure rule of the greedy case).
    READING: when all K pass, the extra token is drawn from the target's
    distribution after the last candidate; p = softmax(target / T),
    q = softmax(draft / T) in fp64; the acceptance test is u q(d) < p(d) with
    u = uniform01(seed, 1, i, b); the residual (or extra) draw is
    inverse_cdf(weights, uniform01(seed, 2, i, b)) at the deciding position i.
    A candidate outside [0, V) is rejected at its position (READING).
    cand [B, K]; draft_logits [B, K, V]; target_logits [B, K + 1, V].
    Returns A [B], next token [B], and per request the margin of its last
    decision (for comparisons near a threshold).
    """
    B, K = cand.shape
    A = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    margin = np.full(B, np.inf)
    for b in range(B):
        for i in range(K + 1):
            p = softmax_t(target_logits[b, i], T)
            if i == K:
                w = p
            else:
                q = softmax_t(draft_logits[b, i], T)
                d = int(cand[b, i])
                # READING: a candidate that is no vocabulary index (the draft
                # reports -1 for an invalid request) has no probability under
                # q or p and is rejected at its position.
                if 0 <= d < len(p):
                    u = float(uniform01(seed, 1, i, b))
                    margin[b] = min(margin[b], abs(u * q[d] - p[d]) / max(p[d], q[d], 1e-300))
                    if u * q[d] < p[d]:
                        A[b] += 1
                        continue
                w = np.maximum(p - q, 0.0)
                if not (w > 0).any():
                    w = p
            tok, gap = inverse_cdf(w, float(uniform01(seed, 2, i, b)))
            nxt[b] = tok
            margin[b] = min(margin[b], gap / max(w.sum(), 1e-300))
            break
    return dict(A=A, next=nxt, margin=margin)
