// C ABI of the DLite draft step: argument validation, workspace plan and the
// launch sequence.  Nothing here allocates device memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "dlite.h"
#include "kernels.hpp"

using namespace dlite;

namespace {

thread_local std::string g_err;

struct StageEvents {
  int stage = -1;
  hipEvent_t before = nullptr, after = nullptr;
};
thread_local StageEvents g_ev;
thread_local StageTimer g_timer;

// Arms (begin) or disarms (end) the stage timer for `stage` (layer 0 for
// per-layer stages): the launches in between carry the events.  A stage that
// launched nothing records both events back to back.
hipError_t mark(int stage, bool begin, hipStream_t st, int layer = 0) {
  if (g_ev.stage != stage || layer != 0) return hipSuccess;
  if (begin) {
    g_timer = StageTimer{g_ev.before, g_ev.after, true, false};
    return hipSuccess;
  }
  const bool launched = g_timer.started;
  g_timer = StageTimer{};
  if (launched) return hipSuccess;
  const hipError_t e = hipEventRecord(g_ev.before, st);
  return e != hipSuccess ? e : hipEventRecord(g_ev.after, st);
}

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DLITE_OK;
}

size_t esize(const dlite_dims& d) { return d.dtype == DLITE_BF16 ? 2 : 4; }

// Options of one draft step (dlite_block_options, checked).
struct Opts {
  int G = 1;                         // local token group length
  const int32_t* gids = nullptr;     // [B, G - 1] the tokens before the anchor
  const int32_t* warm = nullptr;     // [B] gated head: warm-up tokens, or null
};

// NULL options: the defaults; a group of 0 means 1.
void read_opts(const dlite_block_options* o, Opts* out) {
  *out = Opts{};
  if (!o) return;
  out->G = o->group == 0 ? 1 : o->group;
  out->gids = out->G > 1 ? o->group_ids : nullptr;
  out->warm = o->warmup_ids;
}

// Workspace regions, each 256-byte aligned.
struct Plan {
  size_t counters, X, XB, XF, SSQ, Q, KV, AO, ACT, P, U, Sf, Sb, GR, GT, WS, pmax, pidx, TP, SP, total;
  int G;
  int Gcap;   // partials per token in pmax / pidx
};

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Partial-tile scratch of the tiled GEMMs: the largest need of any launch of
// the step (the same tile plan the launches use).
size_t tile_scratch_bytes(const dlite_dims& d, int G) {
  if (d.dtype != DLITE_BF16) return 0;
  const int B = d.B, S = d.m + G + d.K, L = G + d.K, K = d.K, D = d.D, F = d.ffn, r = d.rank;
  const int Hq = d.n_q * d.d_h, Hkv2 = 2 * d.n_kv * d.d_h;
  auto one = [&](int M0, int M1, int N0, int N1, int Kd, int epi) -> size_t {
    const int mx = M0 > M1 ? M0 : M1;
    if (mx < kTileMinRows || Kd % 64) return 0;
    return gemm_tile_scratch(M0, M1, N0, N1, Kd, epi);
  };
  size_t need = 0;
  auto keep = [&](size_t v) { need = v > need ? v : need; };
  for (int Lr : {L, K}) {
    const int Mq = B * Lr, Mkv = B * S;
    if (Mq >= kTileMinRows) keep(one(Mq, Mkv, Hq, Hkv2, D, EPI_STORE_F32));
    else keep(one(Mkv, 0, Hkv2, 0, D, EPI_STORE_F32));
    keep(one(Mq, 0, D, 0, Hq, EPI_RESID));
    keep(one(Mq, 0, F, 0, D, EPI_SWIGLU));
    keep(one(Mq, 0, D, 0, F, EPI_RESID));
  }
  keep(one(B * K, 0, r, 0, D, EPI_STORE_F32));
  keep(one(B * K, 0, d.vocab, 0, r, EPI_ARGMAX));
  return need;
}

// k-slice partials of the weight-streaming GEMMs: the largest need of any
// launch of the step (launches of at most 32 tokens, the same decisions the
// launchers take).
size_t stream_scratch_bytes(const dlite_dims& d, int G) {
  const bool bf16 = d.dtype == DLITE_BF16;
  const int B = d.B, S = d.m + G + d.K, L = G + d.K, K = d.K, D = d.D, F = d.ffn, r = d.rank;
  const int Hq = d.n_q * d.d_h, Hkv2 = 2 * d.n_kv * d.d_h;
  auto tiled = [&](int M, int Kd) { GemmArgs g{}; g.M = M; g.K = Kd; return gemm_tiled(g, bf16); };
  auto c32 = [](int M) { return M < 32 ? M : 32; };
  size_t need = 0;
  auto keep = [&](size_t v) { need = v > need ? v : need; };
  for (int Lr : {L, K}) {
    const int Mq = B * Lr, Mkv = B * S;
    if (!tiled(Mq, D) && !tiled(Mkv, D) && Mq <= 32 && Mkv <= 32) {
      keep(gemm_stream_scratch(Mq, Mkv, Hq, Hkv2, D, EPI_STORE_F32, bf16));
    } else {
      if (!tiled(Mq, D)) keep(gemm_stream_scratch(c32(Mq), 0, Hq, 0, D, EPI_STORE_F32, bf16));
      if (!tiled(Mkv, D)) keep(gemm_stream_scratch(c32(Mkv), 0, Hkv2, 0, D, EPI_STORE_F32, bf16));
    }
    if (!tiled(Mq, Hq)) keep(gemm_stream_scratch(c32(Mq), 0, D, 0, Hq, EPI_RESID, bf16));
    if (!tiled(Mq, D)) keep(gemm_stream_scratch(c32(Mq), 0, F, 0, D, EPI_SWIGLU, bf16));
    if (!tiled(Mq, F)) keep(gemm_stream_scratch(c32(Mq), 0, D, 0, F, EPI_RESID, bf16));
  }
  if (!tiled(B * K, D)) keep(gemm_stream_scratch(c32(B * K), 0, r, 0, D, EPI_STORE_F32, bf16));
  return need;
}

Plan make_plan(const dlite_dims& d, int G = 1) {
  const size_t B = d.B, S = d.m + G + d.K, L = G + d.K, D = d.D;
  const size_t Hq = static_cast<size_t>(d.n_q) * d.d_h, Hkv = static_cast<size_t>(d.n_kv) * d.d_h;
  const size_t F = d.ffn, K = d.K, r = d.rank, es = esize(d);
  Plan p{};
  p.G = lmhead_groups(d.vocab);
  const int Gt = gemm_tile_groups(d.vocab);
  size_t Gmax = p.G > Gt ? p.G : Gt;
  if (seqhead_fused(d.B, d.K, d.rank, d.dtype == DLITE_BF16) && Gmax < kFuseMaxHelpers) Gmax = kFuseMaxHelpers;
  // the persistent vocabulary pass (all B K tokens, or B per position of the
  // gated head) leaves vocab_slots partials per token
  for (const int M : {static_cast<int>(B * K), static_cast<int>(B)})
    if (vocab_tiled(M, d.vocab, d.rank, d.dtype == DLITE_BF16) && static_cast<size_t>(vocab_slots(M)) > Gmax)
      Gmax = vocab_slots(M);
  p.Gcap = static_cast<int>(Gmax);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  p.counters = take(counter_words() * sizeof(unsigned));
  p.X = take(B * S * D * 4);
  p.XB = take((d.n_layers + 1) * B * S * D * es);
  p.XF = take(B * L * D * es);
  p.SSQ = take(B * S * kSsqParts * 4);
  p.Q = take(B * L * Hq * 4);
  p.KV = take(B * S * 2 * Hkv * 4);
  p.AO = take(B * L * Hq * es);
  p.ACT = take(B * L * F * es);
  p.P = take(B * K * r * 4);
  // scan exchange slots, then (fused head) the helpers' tagged words: both
  // zeroed by the feature kernel
  // (and the P partials when the fused kernel computes P: at most 16 slices)
  p.U = take(scan_scratch_floats(d.B, d.rank) * 4 +
             (seqhead_fused(d.B, d.K, d.rank, d.dtype == DLITE_BF16)
                  ? seqhead_fold_bytes(d.B * d.K) + seqhead_sw_bytes(d.B * d.K, d.rank) +
                        seqhead_pw_bytes(d.B * d.K, d.rank, 16)
                  : 0));
  p.Sf = take(B * K * r * 4);
  p.Sb = take(B * K * r * es);
  p.GR = take(B * r * es);        // gated head: r_i of the current step
  p.GT = take(B * 4);             // gated head: d_i of the current step
  p.WS = take(B * r * 4);         // gated head: warm-up state
  p.pmax = take(B * K * Gmax * 4);
  p.pidx = take(B * K * Gmax * 4);
  p.TP = take(tile_scratch_bytes(d, G));
  p.SP = take(stream_scratch_bytes(d, G));
  p.total = off;
  return p;
}

int check_dims(const dlite_dims* dp, int G = 1) {
  if (!dp) return fail(DLITE_ERR_NULL, "dims is NULL");
  if (G < 1 || G > 16) return fail(DLITE_ERR_SHAPE, "group=%d not in [1, 16]", G);
  const dlite_dims& d = *dp;
  if (d.dtype != DLITE_F32 && d.dtype != DLITE_BF16)
    return fail(DLITE_ERR_DTYPE, "dtype %d is neither DLITE_F32 nor DLITE_BF16", d.dtype);
  if (d.B < 1 || d.B > 4096) return fail(DLITE_ERR_SHAPE, "B=%d not in [1, 4096]", d.B);
  if (d.m < 1 || d.m > 64) return fail(DLITE_ERR_SHAPE, "m=%d not in [1, 64]", d.m);
  if (d.D < 64 || d.D > 16384 || d.D % 64)
    return fail(DLITE_ERR_SHAPE, "D=%d must be a multiple of 64 in [64, 16384]", d.D);
  if (d.n_layers < 1 || d.n_layers > 16)
    return fail(DLITE_ERR_SHAPE, "n_layers=%d not in [1, 16]", d.n_layers);
  if (d.n_q < 1 || d.n_kv < 1 || d.n_q % d.n_kv || d.n_q / d.n_kv > 16)
    return fail(DLITE_ERR_SHAPE, "n_q=%d, n_kv=%d: need n_q %% n_kv == 0 and n_q / n_kv <= 16",
                d.n_q, d.n_kv);
  if (d.d_h != 64 && d.d_h != 128) return fail(DLITE_ERR_SHAPE, "d_h=%d not in {64, 128}", d.d_h);
  if (static_cast<long>(d.n_q) * d.d_h > 65536 || static_cast<long>(d.n_kv) * d.d_h > 65536)
    return fail(DLITE_ERR_SHAPE, "too many heads");
  if (d.ffn < 32 || d.ffn % 32 || d.ffn > 262144)
    return fail(DLITE_ERR_SHAPE, "ffn=%d must be a multiple of 32 in [32, 262144]", d.ffn);
  if (d.K < 1 || d.K > 16) return fail(DLITE_ERR_SHAPE, "K=%d not in [1, 16]", d.K);
  const int rmax = d.dtype == DLITE_BF16 ? 512 : 256;
  if (d.rank < 32 || d.rank % 32 || d.rank > rmax)
    return fail(DLITE_ERR_SHAPE, "rank=%d must be a multiple of 32 in [32, %d]", d.rank, rmax);
  if (d.vocab < 1 || d.vocab > (1 << 30)) return fail(DLITE_ERR_SHAPE, "vocab=%d not in [1, 2^30]", d.vocab);
  if (d.D > 8 * 256 * (d.dtype == DLITE_BF16 ? 8 : 4))
    return fail(DLITE_ERR_UNSUPPORTED, "D=%d too large for the feature kernel", d.D);
  {
    AttnArgs aa{};
    aa.n_q = d.n_q; aa.n_kv = d.n_kv; aa.m = d.m; aa.K = d.K; aa.d_h = d.d_h; aa.G = G;
    if (attention_smem(aa) > 160 * 1024)
      return fail(DLITE_ERR_UNSUPPORTED, "attention block too large for LDS (m=%d, G=%d, K=%d, n_q/n_kv=%d)",
                  d.m, G, d.K, d.n_q / d.n_kv);
  }
  if (!(d.rms_eps >= 0.f) || !std::isfinite(d.rms_eps))
    return fail(DLITE_ERR_SHAPE, "rms_eps must be finite and >= 0");
  if (!(d.rope_theta > 0.f) || !std::isfinite(d.rope_theta))
    return fail(DLITE_ERR_SHAPE, "rope_theta must be finite and > 0");
  return DLITE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(DLITE_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(DLITE_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  return DLITE_OK;
}

#define DLITE_TRY(x)              \
  do {                            \
    const int rc_ = (x);          \
    if (rc_ != DLITE_OK) return rc_; \
  } while (0)

#define DLITE_LAUNCH(x)                                                        \
  do {                                                                         \
    const hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess)                                                      \
      return fail(DLITE_ERR_HIP, "%s: %s", #x, hipGetErrorString(e_));         \
  } while (0)

const char* at(const void* base, size_t bytes) { return static_cast<const char*>(base) + bytes; }

struct FeatureSource {
  const void* H;
  long sb, sl, st;          // element strides: request, layer slot, position
  const int32_t* pos;       // [B] positions or null
  int T;                    // positions per request
};

// The draft step with the boundary features read through `fs` (both entry
// points; dims and the feature pointer are checked by the caller).
int draft_impl(const dlite_dims* dims, const dlite_weights* w, const FeatureSource& fs,
               const dlite_gated_head* gh, const Opts& op, const int32_t* anchor_ids, int32_t* candidates,
               float* max_logit, const dlite_taps* taps, void* workspace, size_t workspace_bytes,
               hipStream_t st) {
  const dlite_dims& d = *dims;
  if (!w) return fail(DLITE_ERR_NULL, "weights is NULL");
  DLITE_TRY(check_ptr(w->depth_emb, "weights.depth_emb"));
  DLITE_TRY(check_ptr(w->feat_norm, "weights.feat_norm"));
  DLITE_TRY(check_ptr(w->tok_emb, "weights.tok_emb"));
  DLITE_TRY(check_ptr(w->ph_emb, "weights.ph_emb"));
  DLITE_TRY(check_ptr(w->final_norm, "weights.final_norm"));
  if (gh) {
    DLITE_TRY(check_ptr(gh->emb, "head.emb"));
    DLITE_TRY(check_ptr(gh->w_s, "head.w_s"));
    DLITE_TRY(check_ptr(gh->b_s, "head.b_s"));
    DLITE_TRY(check_ptr(gh->w_h, "head.w_h"));
    DLITE_TRY(check_ptr(gh->b_h, "head.b_h"));
    DLITE_TRY(check_ptr(gh->w_o, "head.w_o"));
    if (d.rank > kGatedMaxRank || d.rank % 8)
      return fail(DLITE_ERR_UNSUPPORTED, "gated head: rank %d must be a multiple of 8 up to %d", d.rank,
                  kGatedMaxRank);
  } else {
    DLITE_TRY(check_ptr(w->seq_w_down, "weights.seq_w_down"));
    DLITE_TRY(check_ptr(w->seq_w_up, "weights.seq_w_up"));
    DLITE_TRY(check_ptr(w->lm_head, "weights.lm_head"));
  }
  if (!w->layers) return fail(DLITE_ERR_NULL, "weights.layers is NULL");
  for (int l = 0; l < d.n_layers; ++l) {
    const dlite_layer_weights& lw = w->layers[l];
    DLITE_TRY(check_ptr(lw.attn_norm, "layer.attn_norm"));
    DLITE_TRY(check_ptr(lw.wqkv, "layer.wqkv"));
    DLITE_TRY(check_ptr(lw.wo, "layer.wo"));
    DLITE_TRY(check_ptr(lw.ffn_norm, "layer.ffn_norm"));
    DLITE_TRY(check_ptr(lw.w_gate_up, "layer.w_gate_up"));
    DLITE_TRY(check_ptr(lw.w_down, "layer.w_down"));
  }
  if (!anchor_ids) return fail(DLITE_ERR_NULL, "anchor_ids is NULL");
  if (!candidates) return fail(DLITE_ERR_NULL, "candidates is NULL");
  if (!workspace) return fail(DLITE_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DLITE_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  if (op.G > 1 && !op.gids) return fail(DLITE_ERR_NULL, "options.group_ids is NULL with group=%d", op.G);
  if (op.warm && !gh) return fail(DLITE_ERR_UNSUPPORTED, "a warm-up token needs the gated head");
  const Plan p = make_plan(d, op.G);
  if (workspace_bytes < p.total)
    return fail(DLITE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, p.total);

  const bool bf16 = d.dtype == DLITE_BF16;
  const size_t es = esize(d);
  const int G = op.G;
  const int B = d.B, m = d.m, K = d.K, D = d.D, S = m + G + K, L = G + K;
  const int Hq = d.n_q * d.d_h, Hkv = d.n_kv * d.d_h, F = d.ffn, r = d.rank;
  char* ws = static_cast<char*>(workspace);
  unsigned* counters = reinterpret_cast<unsigned*>(ws + p.counters);
  float* X = reinterpret_cast<float*>(ws + p.X);
  char* XB = ws + p.XB;                      // [n_layers + 1][B S, D] GEMM inputs
  void* XF = ws + p.XF;                      // [B L, D] FFN inputs
  float* SSQ = reinterpret_cast<float*>(ws + p.SSQ);
  float* Qb = reinterpret_cast<float*>(ws + p.Q);
  float* KVb = reinterpret_cast<float*>(ws + p.KV);
  void* AO = ws + p.AO;
  void* ACT = ws + p.ACT;
  float* P = reinterpret_cast<float*>(ws + p.P);
  float* U = reinterpret_cast<float*>(ws + p.U);
  float* Sf = reinterpret_cast<float*>(ws + p.Sf);
  void* Sb = ws + p.Sb;
  float* pmax = reinterpret_cast<float*>(ws + p.pmax);
  int* pidx = reinterpret_cast<int*>(ws + p.pidx);
  float* TPs = p.TP != p.SP ? reinterpret_cast<float*>(ws + p.TP) : nullptr;
  const StreamScratch gs{TPs, reinterpret_cast<float*>(ws + p.SP), (p.total - p.SP) / sizeof(float),
                         counters + counter_gemm()};
  const dlite_taps no_taps{};
  const dlite_taps& tp = taps ? *taps : no_taps;
  const size_t xb_layer = static_cast<size_t>(B) * S * D * es;
  // partial sums of squares per local row left by the last residual update
  // (the feature kernel writes one)
  int local_parts = 1;

  // 1. feature slots, group (anchor) and placeholder rows, first GEMM inputs
  //    (also clears the counters)
  FeatureArgs fa{};
  fa.H = fs.H; fa.h_sb = fs.sb; fa.h_sl = fs.sl; fa.h_st = fs.st; fa.h_pos = fs.pos; fa.h_T = fs.T;
  fa.depth_emb = w->depth_emb; fa.feat_norm = w->feat_norm;
  fa.tok_emb = w->tok_emb; fa.ph_emb = w->ph_emb;
  for (int l = 0; l < d.n_layers; ++l) fa.attn_norm[l] = w->layers[l].attn_norm;
  fa.anchors = anchor_ids; fa.X = X; fa.XB = XB; fa.ssq = SSQ; fa.tap_z = tp.z;
  fa.counters = counters; fa.n_counters = counter_words();
  fa.clear = reinterpret_cast<uint4*>(U);
  // the fused sequential-head kernel computes P itself when it can (then its
  // tagged partials follow the helpers' words in the cleared region)
  const int p_slices = !gh ? seqhead_p_slices(B, K, r, D) : 0;
  const size_t fold_bytes = seqhead_fused(B, K, r, bf16) ? seqhead_fold_bytes(B * K) : 0;
  const size_t sw_bytes = seqhead_fused(B, K, r, bf16) ? seqhead_sw_bytes(B * K, r) : 0;
  const size_t pw_bytes = p_slices ? seqhead_pw_bytes(B * K, r, p_slices) : 0;
  fa.n_clear = static_cast<long>((scan_scratch_floats(B, r) * sizeof(float) + fold_bytes + sw_bytes + pw_bytes) / 16);
  fa.B = B; fa.m = m; fa.K = K; fa.D = D; fa.V = d.vocab; fa.n_layers = d.n_layers;
  fa.eps = d.rms_eps; fa.G = G; fa.gids = op.gids;
  DLITE_LAUNCH(mark(DLITE_STAGE_FEATURES, true, st));
  DLITE_LAUNCH(launch_feature(fa, bf16, st));
  DLITE_LAUNCH(mark(DLITE_STAGE_FEATURES, false, st));

  // 2. backbone layers
  for (int l = 0; l < d.n_layers; ++l) {
    const dlite_layer_weights& lw = w->layers[l];
    // the group rows of the last layer feed nothing downstream
    const int q0 = (l == d.n_layers - 1) ? G : 0;
    const int Lr = L - q0;
    const RowMap slot_rows{Lr, S, m + q0}, local_rows{Lr, L, q0}, all_slots{S, S, 0};
    const void* xb = XB + l * xb_layer;

    GemmArgs q{};
    q.W = lw.wqkv; q.ldw = D; q.N = Hq; q.K = D;
    q.src = xb; q.ld_src = D; q.smap = slot_rows; q.M = B * Lr;
    q.ssq = SSQ; q.qmap = slot_rows; q.ssq_group = S; q.ssq_split = m; q.np_lo = 1;
    q.np_hi = local_parts; q.norm_len = D; q.eps = d.rms_eps;
    q.out = Qb; q.ld_out = Hq; q.omap = local_rows;
    DLITE_LAUNCH(mark(DLITE_STAGE_QKV, true, st, l));
    GemmArgs kv = q;
    kv.W = at(lw.wqkv, static_cast<size_t>(Hq) * D * es); kv.N = 2 * Hkv;
    kv.smap = all_slots; kv.qmap = all_slots; kv.M = B * S;
    kv.out = KVb; kv.ld_out = 2 * Hkv; kv.omap = all_slots;
    DLITE_LAUNCH(launch_gemm_pair(q, kv, EPI_STORE_F32, bf16, gs, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_QKV, false, st, l));

    AttnArgs aa{Qb, KVb, AO, B, m, K, d.n_q, d.n_kv, d.d_h, q0, d.rope_theta};
    aa.G = G; aa.gids = op.gids;
    DLITE_LAUNCH(mark(DLITE_STAGE_ATTENTION, true, st, l));
    DLITE_LAUNCH(launch_attention(aa, bf16, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_ATTENTION, false, st, l));

    GemmArgs o{};
    o.W = lw.wo; o.ldw = Hq; o.N = D; o.K = Hq;
    o.src = AO; o.ld_src = Hq; o.smap = local_rows; o.M = B * Lr;
    o.out = X; o.ld_out = D; o.omap = slot_rows;
    o.next_gain = lw.ffn_norm; o.xb_out = XF; o.ld_xb = D; o.xmap = local_rows; o.ssq_out = SSQ;
    DLITE_LAUNCH(mark(DLITE_STAGE_OPROJ, true, st, l));
    DLITE_LAUNCH(launch_gemm(o, EPI_RESID, bf16, gs, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_OPROJ, false, st, l));

    GemmArgs gu{};
    gu.W = lw.w_gate_up; gu.ldw = D; gu.N = F; gu.K = D; gu.pair_off = F;
    gu.src = XF; gu.ld_src = D; gu.smap = local_rows; gu.M = B * Lr;
    gu.ssq = SSQ; gu.qmap = slot_rows; gu.ssq_group = S; gu.ssq_split = 0; gu.np_lo = gemm_resid_parts(o, bf16);
    gu.np_hi = gu.np_lo; gu.norm_len = D; gu.eps = d.rms_eps;
    gu.out = ACT; gu.ld_out = F; gu.omap = local_rows;
    DLITE_LAUNCH(mark(DLITE_STAGE_GATE_UP, true, st, l));
    DLITE_LAUNCH(launch_gemm(gu, EPI_SWIGLU, bf16, gs, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_GATE_UP, false, st, l));

    GemmArgs dn{};
    dn.W = lw.w_down; dn.ldw = F; dn.N = D; dn.K = F;
    dn.src = ACT; dn.ld_src = F; dn.smap = local_rows; dn.M = B * Lr;
    dn.out = X; dn.ld_out = D; dn.omap = slot_rows;
    dn.next_gain = (l + 1 < d.n_layers) ? w->layers[l + 1].attn_norm : w->final_norm;
    dn.xb_out = XB + (l + 1) * xb_layer; dn.ld_xb = D; dn.xmap = slot_rows; dn.ssq_out = SSQ;
    if (tp.x) {
      dn.tap = tp.x + static_cast<size_t>(l) * B * L * D;
      dn.ld_tap = D; dn.tmap = local_rows;
    }
    DLITE_LAUNCH(mark(DLITE_STAGE_DOWN, true, st, l));
    DLITE_LAUNCH(launch_gemm(dn, EPI_RESID, bf16, gs, st));
    local_parts = gemm_resid_parts(dn, bf16);
    DLITE_LAUNCH(mark(DLITE_STAGE_DOWN, false, st, l));
  }

  // 3. final RMSNorm: folded into the down projection (pre-gained rows and
  //    partial sums of squares) and the next GEMM's epilogue; fp32 copy on request
  DLITE_LAUNCH(mark(DLITE_STAGE_FINAL_NORM, true, st));
  if (tp.hidden) {
    NormArgs na{X, w->final_norm, tp.hidden, B, m, K, D, d.rms_eps};
    na.G = G;
    DLITE_LAUNCH(launch_hidden_tap(na, bf16, st));
  }
  DLITE_LAUNCH(mark(DLITE_STAGE_FINAL_NORM, false, st));

  // 4. hidden part of the sequential head's input projection, all B*K rows at once
  const RowMap ph_rows{K, S, m + G};
  GemmArgs ph{};
  // fixed head: W_down[:, :D] h (hidden columns first); gated head:
  // W_h[:, R:] u (state columns first)
  if (gh) {
    ph.W = static_cast<const char*>(gh->w_h) + static_cast<size_t>(r) * es;
  } else {
    ph.W = w->seq_w_down;
  }
  ph.ldw = static_cast<long>(D) + r; ph.N = r; ph.K = D;
  ph.src = XB + d.n_layers * xb_layer; ph.ld_src = D; ph.smap = ph_rows; ph.M = B * K;
  ph.ssq = SSQ; ph.qmap = ph_rows; ph.ssq_group = S; ph.ssq_split = 0; ph.np_lo = local_parts;
  ph.np_hi = local_parts; ph.norm_len = D; ph.eps = d.rms_eps;
  ph.out = P; ph.ld_out = r; ph.omap = RowMap{K, K, 0};
  DLITE_LAUNCH(mark(DLITE_STAGE_SEQ_PROJ, true, st));
  if (!p_slices) DLITE_LAUNCH(launch_gemm(ph, EPI_STORE_F32, bf16, gs, st));
  DLITE_LAUNCH(mark(DLITE_STAGE_SEQ_PROJ, false, st));

  // 5. the K-step recurrence, 6. vocabulary projection + argmax (one fused
  //    launch for a few requests)
  ScanArgs sa{P, w->seq_w_down, w->seq_w_up, U, Sf, Sb, tp.state, counters, B, K, D, r, 0u, 0};
  LmArgs la{};
  la.W = w->lm_head; la.src = Sb; la.V = d.vocab; la.r = r; la.M = B * K; la.tok0 = 0;
  la.part_max = pmax; la.part_idx = pidx; la.G = p.G; la.G_cap = p.Gcap;
  la.cand = candidates; la.max_logit = max_logit; la.tap = tp.logits;
  la.anchors = anchor_ids; la.pos = fs.pos; la.pos_n = fs.T; la.K = K; la.counters = counters; la.part = TPs;
  la.xcd_counters = counters + counter_lm_xcd();
  if (gh) {
    // the walkthrough's gated head: K dependent steps, each a state update,
    // its output r_i and one vocabulary pass over the B requests whose greedy
    // tokens feed the next step (stage events: the first step)
    float* Sst = tp.state ? tp.state : Sf;
    int32_t* GT = reinterpret_cast<int32_t*>(ws + p.GT);
    float* Sw = op.warm ? reinterpret_cast<float*>(ws + p.WS) : nullptr;
    // warm-up: one state update from s = 0 with the token before the anchor
    // (no output), so that position 1 starts from that state
    GatedArgs gw{};
    gw.emb = gh->emb; gw.w_s = gh->w_s; gw.b_s = gh->b_s; gw.w_h = gh->w_h; gw.b_h = gh->b_h;
    gw.tok = op.warm; gw.s_prev = nullptr; gw.s_out = Sw; gw.ld_s = r; gw.ld_sp = r; gw.warm = 1;
    gw.B = B; gw.R = r; gw.V = d.vocab; gw.D = D;
    const bool fused = gatedhead_fused(B, K, r, d.vocab, bf16) &&
                       gatedhead_exchange_bytes(B, r) <= scan_scratch_floats(B, r) * sizeof(float);
    if (fused) {
      // all K positions in one persistent launch, W_o held on chip
      uint64_t* xw = reinterpret_cast<uint64_t*>(U);   // zeroed by the feature kernel
      GatedFuseArgs gf{};
      gf.emb = gh->emb; gf.w_s = gh->w_s; gf.b_s = gh->b_s; gf.w_h = gh->w_h; gf.b_h = gh->b_h;
      gf.anchors = anchor_ids; gf.qh = P; gf.s_out = Sst;
      gf.sx = xw; gf.rx = xw + static_cast<size_t>(B) * r; gf.dx = xw + static_cast<size_t>(B) * (r + r / 2);
      gf.px = xw + static_cast<size_t>(B) * (r + r / 2 + 1);
      gf.la = la;
      gf.la.W = gh->w_o; gf.la.M = B; gf.la.tok0 = 0;
      gf.B = B; gf.K = K; gf.D = D;
      gf.s_init = Sw;
      DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, true, st));
      if (Sw) DLITE_LAUNCH(launch_gated_step(gw, bf16, st));
      DLITE_LAUNCH(launch_gatedhead(gf, st));
      DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, false, st));
      DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, true, st));
      DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, false, st));
    }
    for (int i = 0; i < K && !fused; ++i) {
      GatedArgs ga{};
      ga.emb = gh->emb; ga.w_s = gh->w_s; ga.b_s = gh->b_s; ga.w_h = gh->w_h; ga.b_h = gh->b_h;
      ga.tok = i == 0 ? anchor_ids : GT;
      ga.s_prev = i == 0 ? Sw : Sst + static_cast<size_t>(i - 1) * r;
      ga.s_out = Sst + static_cast<size_t>(i) * r;
      ga.ld_s = static_cast<long>(K) * r;
      ga.ld_sp = i == 0 ? r : ga.ld_s;
      ga.qh = P + static_cast<size_t>(i) * r;
      ga.ld_q = static_cast<long>(K) * r;
      ga.r_out = ws + p.GR;
      ga.B = B; ga.R = r; ga.V = d.vocab; ga.D = D;
      DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, true, st, i));
      if (i == 0 && Sw) DLITE_LAUNCH(launch_gated_step(gw, bf16, st));
      DLITE_LAUNCH(launch_gated_step(ga, bf16, st));
      DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, false, st, i));
      LmArgs lg = la;
      lg.W = gh->w_o; lg.src = ws + p.GR; lg.M = B; lg.tok0 = 0;
      lg.omap = RowMap{1, K, i};
      lg.raw = GT;
      DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, true, st, i));
      DLITE_LAUNCH(launch_lmhead(lg, bf16, st));
      DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, false, st, i));
    }
  } else if (seqhead_fused(B, K, r, bf16)) {
    DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, true, st));
    uint64_t* px = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(U) + scan_scratch_floats(B, r) * sizeof(float));
    uint64_t* sw = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(px) + fold_bytes);
    uint64_t* pw = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(sw) + sw_bytes);
    DLITE_LAUNCH(launch_seqhead(sa, la, px, sw, p_slices ? &ph : nullptr, p_slices ? pw : nullptr, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, false, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, true, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, false, st));
  } else {
    DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, true, st));
    DLITE_LAUNCH(launch_scan(sa, bf16, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_SCAN, false, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, true, st));
    DLITE_LAUNCH(launch_lmhead(la, bf16, st));
    DLITE_LAUNCH(mark(DLITE_STAGE_LM_HEAD, false, st));
  }
  return ok();
}

// The allocation-free entry point's scratch: one array per GPU, held until the
// process ends.  Host code never uses its name as an address (that is a host
// stand-in); each device's address is looked up once with that device current.
constexpr size_t kStaticScratchBytes = size_t{64} << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on first use).
int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DLITE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DLITE_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DLITE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DLITE_OK;
}

}  // namespace

namespace dlite {
StageTimer& stage_timer() { return g_timer; }
}  // namespace dlite

extern "C" {

const char* dlite_last_error(void) { return g_err.c_str(); }

int dlite_set_stage_events(int stage, hipEvent_t before, hipEvent_t after) {
  if (!before && !after) {
    g_ev = StageEvents{};
    return ok();
  }
  if (!before || !after) return fail(DLITE_ERR_NULL, "both events are needed");
  if (stage < 0 || stage >= DLITE_NUM_STAGES) return fail(DLITE_ERR_SHAPE, "unknown stage %d", stage);
  g_ev.stage = stage;
  g_ev.before = before;
  g_ev.after = after;
  return ok();
}

const char* dlite_version(void) { return "dlite-mi355x 0.1 (gfx950)"; }

size_t dlite_workspace_bytes(const dlite_dims* dims) {
  if (check_dims(dims) != DLITE_OK) return 0;
  ok();
  return make_plan(*dims).total;
}

int dlite_draft_block(const dlite_dims* dims, const dlite_weights* w, const void* features,
                      const int32_t* anchor_ids, int32_t* candidates, float* max_logit,
                      const dlite_taps* taps, void* workspace, size_t workspace_bytes,
                      hipStream_t st) {
  DLITE_TRY(check_dims(dims));
  DLITE_TRY(check_ptr(features, "features"));
  const long D = dims->D;
  const FeatureSource fs{features, static_cast<long>(dims->m) * D, D, 0, nullptr, 1};
  return draft_impl(dims, w, fs, nullptr, Opts{}, anchor_ids, candidates, max_logit, taps, workspace,
                    workspace_bytes, st);
}

int dlite_draft_block_noalloc(const dlite_dims* dims, const dlite_weights* w, const void* features,
                              const int32_t* anchor_ids, int32_t* candidates, float* max_logit,
                              const dlite_taps* taps, uint32_t* status, hipStream_t st) {
  DLITE_TRY(check_dims(dims));
  DLITE_TRY(check_ptr(features, "features"));
  const size_t need = make_plan(*dims).total;
  if (need > kStaticScratchBytes)
    return fail(DLITE_ERR_WORKSPACE,
                "these dimensions need %zu bytes of scratch; the allocation-free entry point has %zu "
                "(use dlite_draft_block with a workspace)", need, kStaticScratchBytes);
  void* ws = nullptr;
  DLITE_TRY(static_scratch(&ws));
  const long D = dims->D;
  const FeatureSource fs{features, static_cast<long>(dims->m) * D, D, 0, nullptr, 1};
  DLITE_TRY(draft_impl(dims, w, fs, nullptr, Opts{}, anchor_ids, candidates, max_logit, taps, ws,
                       kStaticScratchBytes, st));
  if (status) DLITE_LAUNCH(launch_status_copy(static_cast<const unsigned*>(ws) + CNT_STATUS, status, st));
  return ok();
}

int dlite_draft_block_gated(const dlite_dims* dims, const dlite_weights* w, const dlite_gated_head* head,
                            const void* features, const int32_t* anchor_ids, int32_t* candidates,
                            float* max_logit, const dlite_taps* taps, void* workspace,
                            size_t workspace_bytes, hipStream_t st) {
  DLITE_TRY(check_dims(dims));
  if (!head) return fail(DLITE_ERR_NULL, "head is NULL");
  DLITE_TRY(check_ptr(features, "features"));
  const long D = dims->D;
  const FeatureSource fs{features, static_cast<long>(dims->m) * D, D, 0, nullptr, 1};
  return draft_impl(dims, w, fs, head, Opts{}, anchor_ids, candidates, max_logit, taps, workspace,
                    workspace_bytes, st);
}

size_t dlite_workspace_bytes_ex(const dlite_dims* dims, const dlite_block_options* opts) {
  Opts op;
  read_opts(opts, &op);
  if (check_dims(dims, op.G) != DLITE_OK) return 0;
  ok();
  return make_plan(*dims, op.G).total;
}

int dlite_draft_block_ex(const dlite_dims* dims, const dlite_weights* w, const dlite_gated_head* head,
                         const dlite_block_options* opts, const void* features, const int32_t* anchor_ids,
                         int32_t* candidates, float* max_logit, const dlite_taps* taps, void* workspace,
                         size_t workspace_bytes, hipStream_t st) {
  Opts op;
  read_opts(opts, &op);
  DLITE_TRY(check_dims(dims, op.G));
  DLITE_TRY(check_ptr(features, "features"));
  const long D = dims->D;
  const FeatureSource fs{features, static_cast<long>(dims->m) * D, D, 0, nullptr, 1};
  return draft_impl(dims, w, fs, head, op, anchor_ids, candidates, max_logit, taps, workspace,
                    workspace_bytes, st);
}

int dlite_draft_block_at(const dlite_dims* dims, const dlite_weights* w, const void* verify_hidden,
                         int32_t T, const int32_t* accept_len, const int32_t* anchor_ids,
                         int32_t* candidates, float* max_logit, const dlite_taps* taps,
                         void* workspace, size_t workspace_bytes, hipStream_t st) {
  DLITE_TRY(check_dims(dims));
  DLITE_TRY(check_ptr(verify_hidden, "verify_hidden"));
  if (!accept_len) return fail(DLITE_ERR_NULL, "accept_len is NULL");
  if (T < 1 || T > 65) return fail(DLITE_ERR_SHAPE, "T=%d not in [1, 65]", T);
  const long D = dims->D;
  // [m, B, T, D]: layer l of request b at verify index A_b
  const FeatureSource fs{verify_hidden, static_cast<long>(T) * D, static_cast<long>(dims->B) * T * D, D,
                         accept_len, T};
  return draft_impl(dims, w, fs, nullptr, Opts{}, anchor_ids, candidates, max_logit, taps, workspace,
                    workspace_bytes, st);
}

int dlite_draft_status(const void* workspace, size_t workspace_bytes, uint32_t* status, hipStream_t st) {
  if (!workspace) return fail(DLITE_ERR_NULL, "workspace is NULL");
  if (!status) return fail(DLITE_ERR_NULL, "status is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DLITE_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  // the counters are the workspace's first region in every plan
  if (workspace_bytes < counter_words() * sizeof(unsigned))
    return fail(DLITE_ERR_WORKSPACE, "workspace has %zu bytes, no draft step fits", workspace_bytes);
  DLITE_LAUNCH(launch_status_copy(static_cast<const unsigned*>(workspace) + CNT_STATUS, status, st));
  return ok();
}

int dlite_accept_window(const int32_t* candidates, int32_t K, const int32_t* target_tokens, int32_t B,
                        int32_t W, int32_t* accept_len, int32_t* next_anchor, hipStream_t st) {
  if (!candidates) return fail(DLITE_ERR_NULL, "candidates is NULL");
  if (!target_tokens) return fail(DLITE_ERR_NULL, "target_tokens is NULL");
  if (!accept_len) return fail(DLITE_ERR_NULL, "accept_len is NULL");
  if (B < 1 || B > (1 << 24)) return fail(DLITE_ERR_SHAPE, "B=%d not in [1, 2^24]", B);
  if (K < 1 || K > 64) return fail(DLITE_ERR_SHAPE, "K=%d not in [1, 64]", K);
  if (W < 1 || W > K + 1) return fail(DLITE_ERR_SHAPE, "W=%d not in [1, K + 1 = %d]", W, K + 1);
  DLITE_LAUNCH(launch_accept_window(candidates, K, target_tokens, B, W, accept_len, next_anchor, st));
  return ok();
}

size_t dlite_sampling_workspace_bytes(int32_t rows) {
  if (rows < 1) {
    fail(DLITE_ERR_SHAPE, "rows=%d must be positive", rows);
    return 0;
  }
  ok();
  return align256(sampling_scratch_bytes(rows));
}

int dlite_sample_tokens(const float* logits, int32_t N, int32_t V, float temperature, uint64_t seed,
                        uint32_t stream_id, int32_t* tokens, void* workspace, size_t workspace_bytes,
                        hipStream_t st) {
  if (!logits) return fail(DLITE_ERR_NULL, "logits is NULL");
  if (!tokens) return fail(DLITE_ERR_NULL, "tokens is NULL");
  if (!workspace) return fail(DLITE_ERR_NULL, "workspace is NULL");
  if (N < 1 || N > 65535) return fail(DLITE_ERR_SHAPE, "N=%d not in [1, 65535]", N);
  if (V < 1) return fail(DLITE_ERR_SHAPE, "V=%d must be positive", V);
  if (!(temperature > 0.f) || !(temperature < INFINITY))
    return fail(DLITE_ERR_SHAPE, "temperature must be positive and finite");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(DLITE_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  if (workspace_bytes < sampling_scratch_bytes(N))
    return fail(DLITE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, sampling_scratch_bytes(N));
  DLITE_LAUNCH(launch_sample_tokens(logits, N, V, temperature, seed, stream_id, tokens, workspace, st));
  return ok();
}

int dlite_accept_sampled(const int32_t* candidates, const float* draft_logits, const float* target_logits,
                         int32_t B, int32_t K, int32_t V, float temperature, uint64_t seed, int32_t* accept_len,
                         int32_t* next_token, void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (!candidates) return fail(DLITE_ERR_NULL, "candidates is NULL");
  if (!draft_logits) return fail(DLITE_ERR_NULL, "draft_logits is NULL");
  if (!target_logits) return fail(DLITE_ERR_NULL, "target_logits is NULL");
  if (!accept_len) return fail(DLITE_ERR_NULL, "accept_len is NULL");
  if (!next_token) return fail(DLITE_ERR_NULL, "next_token is NULL");
  if (!workspace) return fail(DLITE_ERR_NULL, "workspace is NULL");
  if (B < 1 || K < 1 || K > 64 || static_cast<long>(B) * (2 * K + 1) > 65535)
    return fail(DLITE_ERR_SHAPE, "B=%d, K=%d: need K in [1, 64] and B (2K + 1) <= 65535", B, K);
  if (V < 1) return fail(DLITE_ERR_SHAPE, "V=%d must be positive", V);
  if (!(temperature > 0.f) || !(temperature < INFINITY))
    return fail(DLITE_ERR_SHAPE, "temperature must be positive and finite");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(DLITE_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  const size_t need = sampling_scratch_bytes(static_cast<long>(B) * (2 * K + 1));
  if (workspace_bytes < need) return fail(DLITE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  DLITE_LAUNCH(launch_accept_sampled(candidates, draft_logits, target_logits, B, K, V, temperature, seed, accept_len,
                                     next_token, workspace, st));
  return ok();
}

int dlite_accept_prefix(const int32_t* candidates, const int32_t* target_tokens, int32_t B,
                        int32_t K, int32_t* accept_len, int32_t* next_anchor, hipStream_t st) {
  if (!candidates) return fail(DLITE_ERR_NULL, "candidates is NULL");
  if (!target_tokens) return fail(DLITE_ERR_NULL, "target_tokens is NULL");
  if (!accept_len) return fail(DLITE_ERR_NULL, "accept_len is NULL");
  if (B < 1 || B > (1 << 24)) return fail(DLITE_ERR_SHAPE, "B=%d not in [1, 2^24]", B);
  if (K < 1 || K > 64) return fail(DLITE_ERR_SHAPE, "K=%d not in [1, 64]", K);
  DLITE_LAUNCH(launch_accept(candidates, target_tokens, B, K, accept_len, next_anchor, st));
  return ok();
}

}  // extern "C"
