/*
 * dlite.h — C ABI of the DLite draft step on AMD Instinct MI355X (gfx950).
 *
 * The operations, following the statement of the problem on the DLite pages:
 *
 *   dlite_draft_block   boundary features [B, m, D] + anchor ids [B] + drafter
 *                       weights  ->  K greedy candidates per request [B, K].
 *   dlite_accept_prefix candidates [B, K] + target greedy tokens [B, K + 1]
 *                       ->  accepted prefix length A [B] and next anchor [B].
 *   dlite_draft_block_at the next round's draft step with its features read
 *                       from the verify pass's hidden states at index A.
 *   dlite_draft_block_gated the draft step with the pages' gated sequential
 *                       head (token-fed state, one vocabulary pass per step).
 *
 * Sources (page title and section; no code is printed on them):
 *   [W] "DLite 完全拆解" walkthrough (pinghaoyang.com.cn);
 *   [S] DLite paper summary (yomxxx.com);
 *   [F] DFlash article (charlestar.github.io), shared verification math.
 *
 * Conventions for every entry point.
 *   Ownership   All tensor pointers are DEVICE pointers owned by the caller,
 *               except the dlite_dims / dlite_weights / dlite_taps structs and
 *               the dlite_weights.layers array, which are host memory and are
 *               read only during the call.  The library allocates no device
 *               memory and keeps no state between calls; all scratch lives in
 *               the caller's workspace.
 *   Layout      Row-major, densest axis last.  Matrices are
 *               [out_features, in_features].
 *   Streams     Work is enqueued on `stream` and the call returns without
 *               synchronising; outputs are valid once the stream has
 *               completed.  Buffers must stay alive until then.  Two calls
 *               that share a workspace must be ordered on one stream.
 *   Errors      0 on success, else a negative DLITE_ERR_* code; arguments are
 *               validated before anything is enqueued, so a failed call
 *               launches nothing.  dlite_last_error() returns a message for
 *               the calling thread's last failure.  No exception crosses the
 *               ABI.
 *   Determinism Outputs are bitwise reproducible for identical inputs: no
 *               floating-point atomics, fixed reduction orders.
 */
#ifndef DLITE_H
#define DLITE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of weights, features and norm gains. */
enum { DLITE_F32 = 0, DLITE_BF16 = 1 };

enum {
  DLITE_OK = 0,
  DLITE_ERR_NULL = -1,        /* a required pointer is NULL                    */
  DLITE_ERR_SHAPE = -2,       /* a dimension is out of range or inconsistent   */
  DLITE_ERR_DTYPE = -3,       /* unknown storage type                          */
  DLITE_ERR_WORKSPACE = -4,   /* workspace smaller than dlite_workspace_bytes  */
  DLITE_ERR_UNSUPPORTED = -5, /* valid but unsupported configuration           */
  DLITE_ERR_HIP = -6          /* the HIP runtime reported a launch error       */
};

/*
 * Problem dimensions.
 *   B        requests in the batch (1 .. 4096)
 *   m        selected target layers = context slots per request ([W] section
 *            "历史并没有消失，而是由目标模型编码"; 1 .. 64)
 *   D        target hidden width = drafter width (multiple of 64, <= 16384)
 *   n_layers drafter backbone layers (1 .. 16)
 *   n_q,n_kv query / key-value heads, n_q % n_kv == 0, n_q / n_kv <= 16
 *   d_h      head width, 64 or 128
 *   ffn      SwiGLU inner width F (multiple of 32)
 *   K        placeholders = drafted tokens per request (1 .. 16); the paper's
 *            block of 8 is the anchor plus K = 7 ([W] "草稿块长与验证块长不是一个参数")
 *   rank     sequential-head state width r (multiple of 32; <= 512 for bf16,
 *            <= 256 for fp32)
 *   vocab    vocabulary size V (1 .. 2^30)
 *   dtype    DLITE_BF16 or DLITE_F32 for all weights and the features
 *   rms_eps  RMSNorm epsilon (e.g. 1e-6)
 *   rope_theta RoPE base (e.g. 1e6)
 */
typedef struct dlite_dims {
  int32_t B, m, D, n_layers, n_q, n_kv, d_h, ffn, K, rank, vocab;
  int32_t dtype;
  float rms_eps, rope_theta;
} dlite_dims;

/* One backbone layer (pre-norm grouped attention + SwiGLU, no biases). */
typedef struct dlite_layer_weights {
  const void *attn_norm;  /* [D] RMSNorm gain before attention                 */
  const void *wqkv;       /* [(n_q + 2 n_kv) d_h, D]: q heads, k heads, v heads */
  const void *wo;         /* [D, n_q d_h]                                       */
  const void *ffn_norm;   /* [D] RMSNorm gain before the FFN                    */
  const void *w_gate_up;  /* [2F, D]: F gate rows, then F up rows               */
  const void *w_down;     /* [D, F]                                             */
} dlite_layer_weights;

typedef struct dlite_weights {
  const void *depth_emb;  /* [m, D] depth embedding e_depth ([W] eq. for z_t^(l)) */
  const void *feat_norm;  /* [D] gain of the feature RMSNorm                       */
  const void *tok_emb;    /* [V, D] anchor token embedding (only B rows are read)  */
  const void *ph_emb;     /* [D] shared placeholder input                          */
  const dlite_layer_weights *layers; /* HOST array of n_layers entries             */
  const void *final_norm; /* [D] gain of the RMSNorm before the sequential head    */
  const void *seq_w_down; /* [r, D + r]: columns 0..D-1 act on h_k, D.. on s_{k-1} */
  const void *seq_w_up;   /* [r, r]                                                */
  const void *lm_head;    /* [V, r] vocabulary projection of the state             */
} dlite_weights;

/*
 * Weights of the gated sequential head printed in [W] "官方顺序头具体算了什么"
 * (R = dims.rank, storage type dims.dtype).  Used by dlite_draft_block_gated
 * in place of seq_w_down / seq_w_up / lm_head.
 */
typedef struct dlite_gated_head {
  const void *emb;  /* [V, R] embedding E_R of the previous token (d_0 = anchor)  */
  const void *w_s;  /* [2R, 2R] W_s: rows g then c; columns s_{i-1} then v_i     */
  const void *b_s;  /* [2R] b_s                                                 */
  const void *w_h;  /* [R, R + D] W_h: columns s_i then u_i (the backbone row)   */
  const void *b_h;  /* [R] b_h                                                  */
  const void *w_o;  /* [V, R] W_o: vocabulary projection of r_i                  */
} dlite_gated_head;

/*
 * Optional fp32 copies of intermediate tensors, for checking.  Any member may
 * be NULL.  z, x, state and logits are predicated stores of the kernels that
 * run either way; hidden (which the fast path never forms in fp32: the final
 * RMSNorm is folded into the GEMMs around it) adds one small kernel.
 *   z       [B, m, D]               normalised, depth-embedded feature slots
 *   x       [n_layers, B, G + K, D] group (G = 1: the anchor) + placeholder
 *                                   residual stream after each layer (the
 *                                   group rows of the last layer are not
 *                                   computed and are left as is; padding rows
 *                                   of a token group hold no defined value)
 *   hidden  [B, K, D]               h_k after the final RMSNorm
 *   state   [B, K, r]               sequential-head states s_1..s_K
 *   logits  [B, K, V]               vocabulary logits
 */
typedef struct dlite_taps {
  float *z, *x, *hidden, *state, *logits;
} dlite_taps;

/*
 * Workspace bytes dlite_draft_block needs for these dimensions; 0 if the
 * dimensions are invalid (see dlite_last_error).  It depends on B, m, K and the
 * model widths only: there is no history-length argument, because the drafter
 * keeps no history KV ([W] "本轮临时 K/V 仍然需要计算").
 */
size_t dlite_workspace_bytes(const dlite_dims *dims);

/*
 * dlite_draft_block — one DLite draft step for a batch of requests.
 *
 * Computes, per request b ([W] Figure 3 data flow, sections
 * "从目标隐藏状态到并行草稿表示" and "轻量顺序头：只补块内依赖"; [S] "设计"):
 *   z_l   = RMSNorm(H[b,l] + depth_emb[l]; feat_norm), l < m: m sequence slots
 *   x_0   = tok_emb[anchor_ids[b]],  x_k = ph_emb (k = 1..K); local positions
 *           0 for every z_l and the anchor, k for placeholder k
 *   n_layers pre-norm layers: non-causal grouped attention of the 1 + K local
 *           rows over all m + 1 + K slots with RoPE (rotate-half), then SwiGLU;
 *           context slots only provide keys and values
 *   h_k   = RMSNorm(x_k; final_norm)
 *   s_0 = 0, s_k = s_{k-1} + seq_w_up silu(seq_w_down [h_k; s_{k-1}])
 *   candidates[b, k-1] = argmax_v (lm_head s_k)_v, lowest index on ties
 *
 * features    [B, m, D] (dtype)       target hidden states at the pivot position
 * anchor_ids  [B] int32                ids in [0, V); an out-of-range id gives a
 *                                      zero anchor embedding and candidates -1
 * candidates  [B, K] int32 (out)
 * max_logit   [B, K] fp32 (out, may be NULL): the winning logit
 * taps        may be NULL
 * workspace   device buffer of at least dlite_workspace_bytes(dims) bytes,
 *             256-byte aligned; contents on entry are ignored
 * stream      HIP stream (0 = default stream)
 */
int dlite_draft_block(const dlite_dims *dims, const dlite_weights *weights,
                      const void *features, const int32_t *anchor_ids,
                      int32_t *candidates, float *max_logit,
                      const dlite_taps *taps, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * dlite_draft_block_noalloc — dlite_draft_block for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same computation, kernels and results as dlite_draft_block; the scratch is
 * a fixed 64 MiB array inside the library (one per GPU, on the current
 * device, created with the code object and held until the process ends)
 * instead of the caller's workspace.  The call allocates nothing.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, or two host threads) race and give undefined results; order them
 * on one stream.  The array keeps the last call's contents; the step clears
 * what must start at zero itself.
 *
 * Dimensions whose dlite_workspace_bytes exceeds 64 MiB (at the 8B-shaped
 * drafter: more than about 20 requests) are rejected with DLITE_ERR_WORKSPACE
 * before anything is enqueued.
 * status  [1] uint32 (device, out, may be NULL): the call's status word, as
 *         dlite_draft_status reports it for a workspace (0 = every bounded
 *         wait ended normally), written on the stream after the step.
 * All other arguments and errors are as dlite_draft_block.
 */
int dlite_draft_block_noalloc(const dlite_dims *dims, const dlite_weights *weights,
                              const void *features, const int32_t *anchor_ids,
                              int32_t *candidates, float *max_logit, const dlite_taps *taps,
                              uint32_t *status, hipStream_t stream);

/*
 * dlite_draft_block_gated — the draft step with the walkthrough's own gated
 * sequential head in place of the fixed recurrence.
 *
 * [W] "官方顺序头具体算了什么": with d_0 = anchor and s_0 = 0, for i = 1..K
 *   v_i = E_R(d_{i-1}),  [g_i ; c_i] = W_s [s_{i-1} ; v_i] + b_s,
 *   s_i = sigmoid(g_i) * s_{i-1} + (1 - sigmoid(g_i)) * tanh(c_i),
 *   r_i = W_h [s_i ; u_i] + b_h,  logits_i = W_o r_i,
 *   d_i = candidates[b, i-1] = argmax logits_i (lowest index on ties),
 * where u_i is the final-normed backbone row of placeholder i (the same h_k
 * the fixed head reads).  The backbone is the one of dlite_draft_block.  The
 * K vocabulary passes are dependent (each choice feeds the next step).
 *
 * head        weights of the head (host struct, device tensors); weights'
 *             seq_w_down / seq_w_up / lm_head are not read and may be NULL
 * rank        a multiple of 8, at most 512 (else DLITE_ERR_UNSUPPORTED)
 * taps        state: s_i; logits: logits_i; others as dlite_draft_block
 * An out-of-range anchor id reads a zero row of E_R and of the token
 * embedding; that request's candidates are -1.  All other arguments, the
 * workspace (dlite_workspace_bytes covers both heads) and the errors are as
 * dlite_draft_block.
 */
int dlite_draft_block_gated(const dlite_dims *dims, const dlite_weights *weights,
                            const dlite_gated_head *head, const void *features,
                            const int32_t *anchor_ids, int32_t *candidates, float *max_logit,
                            const dlite_taps *taps, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Options of dlite_draft_block_ex.  A zeroed struct (or NULL) is the plain
 * step of dlite_draft_block / dlite_draft_block_gated.
 *
 * group       G in [0, 16] (0 and 1: the anchor alone).  The local input is a
 *             token group: the G - 1 tokens before the anchor and the anchor
 *             ([W] "锚点是已经确定、尚待目标前向处理的输入": the draft input
 *             holds the anchor or a fixed-length local token group;
 *             "局部位置编码切断草稿端的全局位置增长": the origin of the local
 *             positions is the start of the group's valid part).
 * group_ids   [B, G - 1] int32, device (read when G > 1): the tokens before
 *             each anchor, oldest first.  Leading ids < 0 are padding (the
 *             sequence holds fewer tokens): padding slots are neither keys nor
 *             read.  Any other id outside [0, V) gives a zero input row.
 *             With n = G - padding real tokens: group token j sits at local
 *             position j - padding (the anchor at n - 1), every feature slot at
 *             n - 1, placeholder k at n - 1 + k.  All G group rows query and
 *             are updated in every layer like the anchor row (rows of the
 *             group are local rows); only placeholders are drafted.
 * warmup_ids  [B] int32, device, or NULL; gated head only (else
 *             DLITE_ERR_UNSUPPORTED).  [W] "官方顺序头具体算了什么": one token
 *             before the anchor may warm the state up.  An id w in [0, V)
 *             runs one state update from s = 0 with v = E_R(w) and no output
 *             before position 1; an id outside [0, V) leaves s_0 = 0.
 */
typedef struct dlite_block_options {
  int32_t group;
  const int32_t *group_ids;
  const int32_t *warmup_ids;
} dlite_block_options;

/* Workspace bytes of dlite_draft_block_ex for these dimensions and options
 * (the group length changes the slot count); 0 if invalid. */
size_t dlite_workspace_bytes_ex(const dlite_dims *dims, const dlite_block_options *opts);

/*
 * dlite_draft_block_ex — the draft step with a local token group and/or the
 * gated head's warm-up token (dlite_block_options).
 *
 * head     NULL: the fixed recurrence of dlite_draft_block; else the gated
 *          head of dlite_draft_block_gated (same weights and rules)
 * opts     may be NULL (the plain step)
 * taps     x is [n_layers, B, G + K, D]; the others as dlite_draft_block
 * workspace  at least dlite_workspace_bytes_ex(dims, opts) bytes
 * A request whose anchor id is outside [0, V) gets candidates -1, as in
 * dlite_draft_block.  All other arguments and errors are as
 * dlite_draft_block; G > 1 with group_ids NULL is DLITE_ERR_NULL, G outside
 * [0, 16] or an attention block too large for LDS (m + G + K slots) is
 * DLITE_ERR_SHAPE / DLITE_ERR_UNSUPPORTED.
 */
int dlite_draft_block_ex(const dlite_dims *dims, const dlite_weights *weights,
                         const dlite_gated_head *head, const dlite_block_options *opts,
                         const void *features, const int32_t *anchor_ids, int32_t *candidates,
                         float *max_logit, const dlite_taps *taps, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * dlite_draft_block_at — the draft step of the next round, fed straight from
 * the previous round's verify pass (no host round trip between rounds).
 *
 * [W] "一轮执行后，缓存、锚点与隐藏状态怎样对齐", step 5 and the state-relation
 * pseudo-code: the next round's boundary features are the m selected target
 * layers' hidden states at verify index A_b of the input [a, d_1..d_K] (the
 * last input that stays: index 0 is the anchor when nothing passed), and the
 * next anchor is the target token there.  Identical to dlite_draft_block with
 *   features[b, l, :] = verify_hidden[l, b, accept_len[b], :]
 * (the same kernels; the feature build reads the rows in place).
 *
 * verify_hidden [m, B, T, D] (dtype)  per selected layer, that layer's hidden
 *                                    states at the T verify inputs of every
 *                                    request (one [B, T, D] block per layer)
 * T             verify inputs per request (the previous round's K + 1), 1..65
 * accept_len    [B] int32, device: A of the previous round (dlite_accept_prefix
 *               output).  A value outside [0, T) cannot be checked before the
 *               launch; the kernels then read position 0 (in bounds) and the
 *               request's candidates are -1 and max_logit 0.
 * anchor_ids    [B] int32: the next anchors (dlite_accept_prefix's next_anchor)
 * All other arguments, the workspace and the errors are as dlite_draft_block.
 */
int dlite_draft_block_at(const dlite_dims *dims, const dlite_weights *weights,
                         const void *verify_hidden, int32_t T, const int32_t *accept_len,
                         const int32_t *anchor_ids, int32_t *candidates, float *max_logit,
                         const dlite_taps *taps, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * dlite_draft_status — the health word of the last draft step that used
 * `workspace` (dlite_draft_block, _at or _gated), copied on `stream` into
 * status[0] (a DEVICE uint32 owned by the caller), so it can be read without
 * stalling the stream or be captured with the step.
 *
 * Several kernels of the step exchange data between workgroups that wait on
 * each other (the sequential-head scan team, the fused scan + vocabulary and
 * gated-head kernels).  Every such wait is bounded: rather than hang, a wait
 * that runs out of its spin budget sets DLITE_STATUS_WAIT_TIMEOUT here and
 * the kernel finishes.  A nonzero word therefore means that call's candidates
 * are NOT reliable; the caller must treat it as an error.  The word is zeroed
 * by the first kernel of every draft step, so it describes exactly one call.
 *
 * workspace, workspace_bytes  the buffer passed to that draft call
 * status                      [1] uint32 (device, out): 0 = every wait ended
 *                             normally, else a mask of DLITE_STATUS_* bits
 * Errors as elsewhere (NULL pointers, a workspace that is not 256-byte
 * aligned or smaller than any draft step's).
 */
enum { DLITE_STATUS_WAIT_TIMEOUT = 1 };
int dlite_draft_status(const void *workspace, size_t workspace_bytes, uint32_t *status,
                       hipStream_t stream);

/*
 * dlite_accept_prefix — greedy verification of one round.
 *
 * [W] "一次因果前向评估整条候选": only the leading run of matches is committed.
 * [W] "一轮执行后，缓存、锚点与隐藏状态怎样对齐": the next anchor (the
 * correction, or the bonus token when all K pass) is the target token at verify
 * index A.  A round commits A + 1 tokens ([W] "先拆开一次投机轮次的时间").
 *
 * candidates    [B, K] int32    draft tokens d_1..d_K
 * target_tokens [B, K + 1] int32 target greedy token at each verify input
 *                               [a, d_1, .., d_K]
 * accept_len    [B] int32 (out)  A = number of leading i with
 *                               candidates[b, i] == target_tokens[b, i], 0..K
 * next_anchor   [B] int32 (out, may be NULL)  target_tokens[b, A]
 * Integer only; bit-exact.  B in 1 .. 2^24, K in 1 .. 64.
 */
int dlite_accept_prefix(const int32_t *candidates, const int32_t *target_tokens,
                        int32_t B, int32_t K, int32_t *accept_len,
                        int32_t *next_anchor, hipStream_t stream);

/*
 * dlite_accept_window — greedy verification of a window shorter than the
 * drafted block.
 *
 * [W] "草稿块长与验证块长不是一个参数": the drafter predicts its whole block
 * of K candidates, and a verify window of W inputs (anchor included) sends
 * only the first W - 1 of them to the target; the rest are dropped.  A is the
 * number of leading matches among those W - 1 (0 .. W - 1) and next_anchor
 * the target token at verify index A.  W = K + 1 is dlite_accept_prefix.
 *
 * candidates    [B, K] int32 (rows of K; only the first W - 1 are read)
 * target_tokens [B, W] int32 target greedy token at each of the W inputs
 * K in 1 .. 64, W in 1 .. K + 1; accept_len [B] (out); next_anchor [B] (out,
 * may be NULL).  Integer only; bit-exact.
 */
int dlite_accept_window(const int32_t *candidates, int32_t K, const int32_t *target_tokens, int32_t B,
                        int32_t W, int32_t *accept_len, int32_t *next_anchor, hipStream_t stream);

/*
 * Sampling at a positive temperature ([W] "贪心模式与随机模式要分别说明").
 *
 * Random numbers come from Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011): the uniform for counter
 * (a, b, stream, 0) under key (seed low 32 bits, seed high 32 bits) is
 * (x0 + 1/2) / 2^32.  The same (seed, stream) always gives the same draws.
 * Probabilities are evaluated in fp64 from the fp32 logits scaled by
 * 1 / (double)temperature.
 *
 * dlite_sampling_workspace_bytes(rows): scratch for rows = N of
 * dlite_sample_tokens or rows = B (2K + 1) of dlite_accept_sampled; 0 with an
 * error for rows < 1.
 */
size_t dlite_sampling_workspace_bytes(int32_t rows);

/*
 * dlite_sample_tokens — one token per row drawn from softmax(logits / T):
 * tokens[n] = argmax_v (logits[n, v] / T - log(-log u(v, n))), u from counter
 * (v, n, stream_id) (the Gumbel-max rule; ties to the lowest index).  With the
 * draft's logits (taps.logits of dlite_draft_block, rows b K + i) it samples
 * the candidates; with the target's logits it gives match mode's target
 * tokens (then dlite_accept_prefix applies the greedy prefix rule).
 *
 * logits [N, V] fp32 (device); N in 1 .. 65535; temperature > 0 and finite;
 * tokens [N] int32 (out); workspace: dlite_sampling_workspace_bytes(N) bytes,
 * 16-byte aligned.
 */
int dlite_sample_tokens(const float *logits, int32_t N, int32_t V, float temperature, uint64_t seed,
                        uint32_t stream_id, int32_t *tokens, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * dlite_accept_sampled — speculative rejection sampling of one round.
 *
 * With p_i = softmax(target_logits[b, i] / T), q_i = softmax(draft_logits[b,
 * i] / T) and d_i = candidates[b, i] (drawn from q_i): for i = 0, 1, .. the
 * candidate is kept when u q_i(d_i) < p_i(d_i), u from counter (i, b, 1); at
 * the first rejection next_token is drawn from the normalised residual
 * [p_i - q_i]_+ (from p_i if that vanishes), else, after K acceptances, from
 * p_K (the target's distribution after the last candidate); the draw is the
 * inverse CDF at u from counter (i, b, 2).  accept_len[b] = number kept, so
 * the committed token at every position is distributed as the target's
 * ([W]: the accepted mass min(p, q) plus the residual mass [p - q]_+ is p).
 * A candidate outside [0, V) is rejected.
 *
 * candidates [B, K] int32; draft_logits [B, K, V] fp32 (the logits the
 * candidates were drawn from); target_logits [B, K + 1, V] fp32 (the
 * target's at the verify inputs [a, d_1 .. d_K]); K in 1 .. 64;
 * accept_len, next_token [B] int32 (out); workspace:
 * dlite_sampling_workspace_bytes(B (2K + 1)) bytes, 16-byte aligned.
 */
int dlite_accept_sampled(const int32_t *candidates, const float *draft_logits, const float *target_logits,
                         int32_t B, int32_t K, int32_t V, float temperature, uint64_t seed,
                         int32_t *accept_len, int32_t *next_token, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Instrumentation for timing one stage of the draft step with HIP events.
 * After this call, every draft call made from the same thread attaches
 * `before` to the dispatch of the first kernel of `stage` and `after` to the
 * dispatch of its last kernel (hipExtLaunchKernel events: they carry the
 * kernels' own start and end times, as a kernel trace does; for per-layer
 * stages, in the first backbone layer).  A stage that launches no kernel in
 * that call records both events back to back on the stream; the gated head's
 * cooperative launch is bracketed by event records instead.  The events are
 * owned by the caller; pass NULL for both to switch recording off.  Returns
 * DLITE_ERR_SHAPE for an unknown stage, DLITE_ERR_NULL if exactly one event is
 * NULL.
 */
enum {
  DLITE_STAGE_FEATURES = 0,   /* feature slots, anchor and placeholder rows     */
  DLITE_STAGE_QKV = 1,        /* RMSNorm + q, k, v projections                   */
  DLITE_STAGE_ATTENTION = 2,  /* non-causal block attention                      */
  DLITE_STAGE_OPROJ = 3,      /* output projection + residual                    */
  DLITE_STAGE_GATE_UP = 4,    /* RMSNorm + gate/up projection + SwiGLU           */
  DLITE_STAGE_DOWN = 5,       /* down projection + residual                      */
  DLITE_STAGE_FINAL_NORM = 6, /* RMSNorm of the placeholder rows                 */
  DLITE_STAGE_SEQ_PROJ = 7,   /* hidden part of the sequential head's input      */
  DLITE_STAGE_SCAN = 8,       /* the K-step recurrence                           */
  DLITE_STAGE_LM_HEAD = 9,    /* vocabulary projection + argmax                  */
  DLITE_NUM_STAGES = 10
};
int dlite_set_stage_events(int stage, hipEvent_t before, hipEvent_t after);

/* Message describing the calling thread's last error ("" if none). */
const char *dlite_last_error(void);

/* Library version string. */
const char *dlite_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DLITE_H */
