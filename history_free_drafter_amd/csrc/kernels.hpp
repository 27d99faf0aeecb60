// Launch interfaces of the DLite kernels (host side).  Each launcher enqueues
// one or more kernels on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <hip/hip_ext.h>

#include <tuple>
#include <type_traits>
#include <utility>

#include "common.hpp"

namespace dlite {

// ------------------------------------------------------------- launching --
// Stage timing of the calling thread (dlite_set_stage_events).  While a stage
// is armed, every kernel launch carries the stage's stop event and the first
// one its start event, attached to the dispatch itself (hipExtLaunchKernel),
// so the events bracket the stage's kernels exactly as a kernel trace does,
// without marker packets of their own.
struct StageTimer {
  hipEvent_t start = nullptr, stop = nullptr;
  bool active = false, started = false;
};
StageTimer& stage_timer();

// Launches kernel<<<grid, block, sm, st>>>(args...), with the armed stage's
// events if any.
template <typename... Params, typename... Args>
inline void launch_k(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t sm, hipStream_t st,
                     Args&&... args) {
  std::tuple<std::decay_t<Params>...> tup(std::forward<Args>(args)...);
  void* ptrs[sizeof...(Params) > 0 ? sizeof...(Params) : 1];
  std::apply([&ptrs](auto&... e) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&e)), ...);
  }, tup);
  StageTimer& t = stage_timer();
  if (t.active) {
    (void)hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, sm, st,
                             t.started ? nullptr : t.start, t.stop, 0);
    t.started = true;
  } else {
    (void)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, sm, st);
  }
}

// Workspace counters, zeroed by the first kernel of every draft step.
// CNT_LM_DONE: XCD groups of a streaming vocabulary launch whose workgroups
// have all published (counter_lm_xcd(): the per-group arrivals); both levels
// reset themselves, so consecutive 32-token launches reuse them.
// counter_seq_done(): scan team members that have published their states
// (fused scan + vocabulary kernel), on a 256-byte line of its own.
// counter_gemm(): arrival counters of the weight-streaming GEMMs' k slices.
enum Counter { CNT_LM_DONE = 0, CNT_STATUS = 2 };
size_t scan_scratch_floats(int B, int r);   // size of ScanArgs::U
inline int counter_seq_done() { return 64; }
inline int counter_gemm() { return counter_seq_done() + 64; }
inline int counter_lm_xcd() { return counter_gemm() + 2 * 128; }   // [8 XCDs] x 16 words
inline int counter_words() { return counter_lm_xcd() + 8 * 16; }
enum Status { STATUS_BARRIER_TIMEOUT = 1 };

// Partial sums of squares per activation row: one slot per producing
// workgroup (at most kSsqParts), summed in fixed order by the consumer.
constexpr int kSsqParts = 256;
constexpr int kMaxLayers = 16;

// ------------------------------------------------------------ feature build --
struct FeatureArgs {
  // context row (b, l) = H + b h_sb + l h_sl + pos_b h_st elements, with
  // pos_b = h_pos[b] when h_pos is given (rows outside [0, h_T) read position
  // 0; their requests are reported as invalid by the argmax), else 0
  const void* H;
  long h_sb, h_sl, h_st;
  const int32_t* h_pos;
  int h_T;
  const void* depth_emb;  // [m, D]
  const void* feat_norm;  // [D]
  const void* tok_emb;    // [V, D]
  const void* ph_emb;     // [D]
  const void* attn_norm[kMaxLayers];  // [D] per layer
  const int32_t* anchors; // [B]
  float* X;               // [B, S, D] slot buffer (fp32)
  void* XB;               // [n_layers + 1][B, S, D] pre-gained GEMM inputs
  float* ssq;             // [B S, kSsqParts] row sums of squares (slot 0)
  float* tap_z;           // [B, m, D] or null
  unsigned* counters;     // counter_words() words, zeroed here
  int n_counters;
  uint4* clear;           // scan exchange slots, zeroed here (n_clear 16-byte words)
  long n_clear;
  int B, m, K, D, V, n_layers;
  float eps;
  int G = 1;                        // local token group length (slots m .. m + G - 1)
  const int32_t* gids = nullptr;    // [B, G - 1] the tokens before the anchor (G > 1)
};
hipError_t launch_feature(const FeatureArgs& a, bool bf16, hipStream_t st);

// ---------------------------------------------------------------- GEMMs ----
// out[token, n] = epilogue( s_tok * sum_k W[n, k] * in[token, k] ), tokens
// 0..M-1 (offset tok0), logical output rows n in [0, N); s_tok = 1/rms of
// the token when `ssq` is given, else 1.
enum Epi { EPI_STORE_F32 = 0, EPI_STORE_ACT = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_ARGMAX = 4 };

struct GemmArgs {
  const void* W; long ldw; int N; int K;
  long pair_off;                 // SwiGLU: up rows start pair_off rows after gate rows
  const void* src; long ld_src; RowMap smap;   // pre-gained input rows (storage type)
  int M; int tok0;
  // RMSNorm scale: partial sums at ssq[qmap.row(tok) * kSsqParts + j]; rows
  // with (row % ssq_group) < ssq_split have np_lo parts, the others np_hi
  const float* ssq; RowMap qmap; int ssq_group, ssq_split, np_lo, np_hi; int norm_len; float eps;
  void* out; long ld_out; RowMap omap;
  // EPI_RESID: x += y, then xb_out = bf16(next_gain * x) and one partial
  // sum of squares of x per workgroup into ssq_out (rows of omap)
  const void* next_gain; void* xb_out; long ld_xb; RowMap xmap; float* ssq_out;
  float* tap; long ld_tap; RowMap tmap;   // RESID: copy of the updated row; ARGMAX: logits
  // EPI_ARGMAX (tiled path only): per token and output tile a (max, index)
  // partial at part_*[(tok0 + token) * G_part + tile]
  float* part_max; int* part_idx; int G_part;
};
// Scratch of the GEMM launches: partial tiles of the tiled path, k-slice
// partials and arrival counters of the weight-streaming path.
constexpr int kStreamRowBlocks = 128;   // arrival counters per problem
struct StreamScratch {
  float* tile_part;      // gemm_tile_scratch bytes (or null: no split K)
  float* part;           // gemm_stream_scratch bytes
  size_t part_floats;
  unsigned* counters;    // 2 * kStreamRowBlocks words, zero between launches
};
// Enqueues the GEMM; M > 32 is split into launches of 32 tokens on the
// weight-streaming path, or handled in one launch by the tiled path.
hipError_t launch_gemm(const GemmArgs& a, int epi, bool bf16, const StreamScratch& ss, hipStream_t st);
// Two problems with the same K and epilogue (e.g. query rows of the local
// tokens and key/value rows of every slot), in one launch where the paths allow.
hipError_t launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, int epi, bool bf16,
                            const StreamScratch& ss, hipStream_t st);
// Bytes of k-slice partials one weight-streaming launch needs (M0, M1 <= 32).
size_t gemm_stream_scratch(int M0, int M1, int N0, int N1, int K, int epi, bool bf16);
// Number of partial sums of squares per row that an EPI_RESID launch writes.
int gemm_resid_parts(const GemmArgs& a, bool bf16);


// Tiled MFMA path for many token rows: up to two independent problems with
// the same epilogue in one launch.
// Launches with few output tiles split K over several workgroups: each writes
// an fp32 partial tile, and a second pass adds the partials in fixed order and
// applies the epilogue.
constexpr int kTileMinRows = 64;
struct TileArgs {
  GemmArgs seg[2];
  int nbm[2];          // token tiles per problem
  int tiles0, total;   // output tiles of problem 0, of the launch
  int per_xcd;         // work items handed to each of the 8 XCDs
  int ksplit;          // k slices per output tile
  int nsum;            // slices the epilogue pass adds (ksplit, or 1 once pre-added)
  float* part;         // [total * ksplit][kTileFloats] partial tiles (ksplit > 1)
};
bool gemm_tiled(const GemmArgs& a, bool bf16);
int gemm_tile_groups(int N);   // output tiles of an EPI_ARGMAX problem of N rows
// Scratch bytes a tiled launch needs for its partial tiles (0 without split).
size_t gemm_tile_scratch(int M0, int M1, int N0, int N1, int K, int epi);
// `part` is the scratch area (at least gemm_tile_scratch bytes).
hipError_t launch_gemm_tiled(const GemmArgs* segs, int nseg, int epi, float* part, hipStream_t st);
// Vocabulary projection + argmax for a few hundred token rows (bf16, K a
// multiple of 32, contiguous token rows): one persistent launch leaves
// vocab_slots(M) (max, index) partials per token at part_*[(tok0 + t) *
// vocab_slots(M) + slot], and the logits in tap when given.
bool vocab_tiled(int M, int N, int K, bool bf16);
int vocab_slots(int M);
hipError_t launch_vocab(const GemmArgs& g, hipStream_t st);

// ------------------------------------------------------------- attention --
struct AttnArgs {
  const float* Q;   // [B, L, n_q d_h]
  const float* KV;  // [B, S, 2 n_kv d_h] (k heads, then v heads)
  void* out;        // [B, L, n_q d_h] storage type
  int B, m, K, n_q, n_kv, d_h, q0;  // local rows j = q0 .. G + K - 1 are computed
  float theta;
  int G = 1;                        // local token group length
  const int32_t* gids = nullptr;    // [B, G - 1] the tokens before the anchor (G > 1)
};
hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t st);
size_t attention_smem(const AttnArgs& a);   // dynamic LDS bytes of one workgroup

// ------------------------------------------------------------ hidden tap ----
// fp32 copy of h_k = RMSNorm(x_k; gain) for the placeholder rows (checking only).
struct NormArgs {
  const float* X;     // [B, S, D]
  const void* gain;   // [D]
  float* tap;         // [B, K, D]
  int B, m, K, D; float eps;
  int G = 1;          // local token group length (placeholders from slot m + G)
};
hipError_t launch_hidden_tap(const NormArgs& a, bool bf16, hipStream_t st);

// ------------------------------------------------------ sequential head ----
struct ScanArgs {
  const float* P;        // [B, K, r]  seq_w_down[:, :D] h_k
  const void* w_down;    // [r, D + r] (state columns used)
  const void* w_up;      // [r, r]
  float* U;              // scan_scratch_floats(B, r) floats of scratch, zeroed before the launch
  float* Sf;             // [B, K, r] states (fp32)
  void* Sb;              // [B, K, r] states (storage type) for the vocabulary GEMM
  float* tap;            // [B, K, r] or null
  unsigned* counters;
  int B, K, D, r;
  unsigned tag0;         // steps run by earlier launches of this call (offsets the exchange tags)
  int rpt;               // requests per team (set by the launcher)
  int stage;             // byte offset of the weight staging area in dynamic LDS (0: none)
  // P from tagged k-slice partials instead of P (fused kernel): the value of
  // token t, row n is the sum over slices q < Pslices of the word at
  // Pw[(q * B K + t) * r + n] (value bits low, tag 1 high), in slice order
  const uint64_t* Pw;
  int Pslices;
};
hipError_t launch_scan(const ScanArgs& a, bool bf16, hipStream_t st);

// ------------------------------------------- vocabulary GEMM + argmax ----
struct LmArgs {
  const void* W;         // [V, r]
  const void* src;       // [T, r] storage type, T = B K tokens
  int V, r, M, tok0;     // this launch covers tokens tok0 .. tok0 + M - 1
  float* part_max;       // [T, G] partial maxima
  int* part_idx;         // [T, G]
  int G;                 // workgroups of every launch (partials per token)
  int32_t* cand;         // [T]
  float* max_logit;      // [T] or null
  float* tap;            // [T, V] or null
  const int32_t* anchors; // [B]: requests with an out-of-range anchor get -1
  const int32_t* pos;    // [B] or null: feature positions; outside [0, pos_n) also gives -1
  int pos_n;
  RowMap omap;           // launch token -> row of cand / max_logit / tap (request = row / K)
  int32_t* raw;          // [M] or null: the argmax of each launch token, before validity
  int K;                 // tokens per request (token t belongs to request t / K)
  unsigned* counters;
  unsigned* xcd_counters; // counter_lm_xcd() words: arrivals per XCD (64-byte apart)
  float* part;           // partial-tile scratch of the tiled path (gemm_tile_scratch)
  int G_cap;             // partials per token that part_max / part_idx hold
};
hipError_t launch_lmhead(const LmArgs& a, bool bf16, hipStream_t st);
int lmhead_groups(int V);
// Fused scan + vocabulary pass for a few requests (B * K <= 16, bf16,
// r in {320, 512}): one launch replaces launch_scan + launch_lmhead.  Needs
// kFuseMaxHelpers partials per token in LmArgs::part_max / part_idx.
constexpr int kFuseMaxHelpers = 1024;
bool seqhead_fused(int B, int K, int r, bool bf16);
// px: seqhead_fold_bytes(B K) of zeroed scratch (the helpers' tagged words);
// sw: seqhead_sw_bytes(B K, r) of zeroed scratch (the teams' tagged states).
size_t seqhead_fold_bytes(int M);
size_t seqhead_sw_bytes(int M, int r);
// The fused kernel can also compute the scan's input P = W_down[:, :D] h
// itself (ph: the GEMM arguments of the separate launch, EPI_STORE_F32): its
// first helpers each take a 16-row tile and a k slice and publish tagged
// partials into pw, which the team sums before its first step.  Returns the
// number of k slices (0: P must come from the separate launch).
int seqhead_p_slices(int B, int K, int r, int D);
size_t seqhead_pw_bytes(int M, int r, int slices);   // zeroed scratch for pw
hipError_t launch_seqhead(const ScanArgs& s, const LmArgs& l, uint64_t* px, uint64_t* sw, const GemmArgs* ph,
                          uint64_t* pw, hipStream_t st);

// ------------------------------------------------- gated sequential head ----
constexpr int kGatedMaxRank = 512;
struct GatedArgs {
  const void* emb;        // E_R [V, R]
  const void* w_s;        // [2R, 2R]: rows g then c, columns state then embedding
  const void* b_s;        // [2R]
  const void* w_h;        // [R, R + D]: columns state then backbone row
  const void* b_h;        // [R]
  const int32_t* tok;     // [B] d_{i-1}; ids outside [0, V) read a zero row
  const float* s_prev;    // row b at s_prev + b ld_sp; null: s_0 = 0
  float* s_out;           // row b at s_out + b ld_s
  long ld_s, ld_sp;
  int warm;               // warm-up update: a token outside [0, V) leaves s = 0
  const float* qh;        // W_h[:, R:] u_i: row b at qh + b ld_q
  long ld_q;
  void* r_out;            // [B, R] storage type
  int B, R, V, D;
};
// One step: the state update, then r_i (two launches).
hipError_t launch_gated_step(const GatedArgs& a, bool bf16, hipStream_t st);

// All K positions in one persistent launch for a few requests (bf16, R = 512,
// B <= 8): W_o stays on chip across the positions.
struct GatedFuseArgs {
  const void* emb; const void* w_s; const void* b_s; const void* w_h; const void* b_h;
  const int32_t* anchors;   // [B] d_0
  const float* s_init;      // [B, R] state before position 1 (warm-up) or null: 0
  const float* qh;          // [B K, R] W_h[:, R:] u
  float* s_out;             // [B K, R] states
  uint64_t* sx;             // [B, R]   tagged state words (team exchange)
  uint64_t* rx;             // [B, R/2] tagged r_i words (two bf16 each)
  uint64_t* dx;             // [B]      tagged d_i words
  uint64_t* px;             // [B, G]   tagged (max, index) words of the helpers
  LmArgs la;                // W = W_o; outputs and the status word
  int B, K, D;
};
bool gatedhead_fused(int B, int K, int r, int V, bool bf16);
size_t gatedhead_exchange_bytes(int B, int r);
hipError_t launch_gatedhead(const GatedFuseArgs& f, hipStream_t st);

// ------------------------------------------------ sampling at temperature ----
size_t sampling_scratch_bytes(long rows);
hipError_t launch_sample_tokens(const float* logits, int N, int V, float T, unsigned long long seed,
                                unsigned stream, int32_t* tokens, void* scratch, hipStream_t st);
hipError_t launch_accept_sampled(const int32_t* cand, const float* draft, const float* target, int B, int K, int V,
                                 float T, unsigned long long seed, int32_t* A, int32_t* next, void* scratch,
                                 hipStream_t st);

// --------------------------------------------------------------- accept ----
// Verify window of W inputs (anchor included, W <= K + 1): the first W - 1
// of the K drafted candidates (rows K apart) against target rows of W.
hipError_t launch_accept_window(const int32_t* cand, int K, const int32_t* tgt, int B, int W,
                                int32_t* A, int32_t* next, hipStream_t st);
// Copies the workspace status word (counters + CNT_STATUS) to `out` on the stream.
hipError_t launch_status_copy(const unsigned* word, uint32_t* out, hipStream_t st);
hipError_t launch_accept(const int32_t* cand, const int32_t* tgt, int B, int K,
                         int32_t* A, int32_t* next, hipStream_t st);

}  // namespace dlite
