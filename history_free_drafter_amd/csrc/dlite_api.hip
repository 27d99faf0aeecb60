// C ABI of the DLite draft step: argument validation, workspace plan and the
// launch sequence.  Nothing here allocates device memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "dlite.h"
#include "kernels.hpp"

using namespace dlite;

namespace {

thread_local std::string g_err;

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

// Workspace regions, each 256-byte aligned.
struct Plan {
  size_t counters, X, Q, KV, AO, ACT, Hn, P, U, Sf, Sb, pmax, pidx, total;
  int G;
};

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

Plan make_plan(const dlite_dims& d) {
  const size_t B = d.B, S = d.m + 1 + d.K, L = 1 + d.K, D = d.D;
  const size_t Hq = static_cast<size_t>(d.n_q) * d.d_h, Hkv = static_cast<size_t>(d.n_kv) * d.d_h;
  const size_t F = d.ffn, K = d.K, r = d.rank, es = esize(d);
  Plan p{};
  p.G = lmhead_groups(d.vocab);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  p.counters = take(CNT_COUNT * sizeof(unsigned));
  p.X = take(B * S * D * 4);
  p.Q = take(B * L * Hq * 4);
  p.KV = take(B * S * 2 * Hkv * 4);
  p.AO = take(B * L * Hq * es);
  p.ACT = take(B * L * F * es);
  p.Hn = take(B * K * D * es);
  p.P = take(B * K * r * 4);
  p.U = take(B * r * 4);
  p.Sf = take(B * K * r * 4);
  p.Sb = take(B * K * r * es);
  p.pmax = take(B * K * static_cast<size_t>(p.G) * 4);
  p.pidx = take(B * K * static_cast<size_t>(p.G) * 4);
  p.total = off;
  return p;
}

int check_dims(const dlite_dims* dp) {
  if (!dp) return fail(DLITE_ERR_NULL, "dims is NULL");
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

}  // namespace

extern "C" {

const char* dlite_last_error(void) { return g_err.c_str(); }

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
  const dlite_dims& d = *dims;
  if (!w) return fail(DLITE_ERR_NULL, "weights is NULL");
  DLITE_TRY(check_ptr(w->depth_emb, "weights.depth_emb"));
  DLITE_TRY(check_ptr(w->feat_norm, "weights.feat_norm"));
  DLITE_TRY(check_ptr(w->tok_emb, "weights.tok_emb"));
  DLITE_TRY(check_ptr(w->ph_emb, "weights.ph_emb"));
  DLITE_TRY(check_ptr(w->final_norm, "weights.final_norm"));
  DLITE_TRY(check_ptr(w->seq_w_down, "weights.seq_w_down"));
  DLITE_TRY(check_ptr(w->seq_w_up, "weights.seq_w_up"));
  DLITE_TRY(check_ptr(w->lm_head, "weights.lm_head"));
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
  DLITE_TRY(check_ptr(features, "features"));
  if (!anchor_ids) return fail(DLITE_ERR_NULL, "anchor_ids is NULL");
  if (!candidates) return fail(DLITE_ERR_NULL, "candidates is NULL");
  if (!workspace) return fail(DLITE_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DLITE_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  const Plan p = make_plan(d);
  if (workspace_bytes < p.total)
    return fail(DLITE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, p.total);

  const bool bf16 = d.dtype == DLITE_BF16;
  const size_t es = esize(d);
  const int B = d.B, m = d.m, K = d.K, D = d.D, S = m + 1 + K, L = 1 + K;
  const int Hq = d.n_q * d.d_h, Hkv = d.n_kv * d.d_h, F = d.ffn, r = d.rank;
  unsigned* counters = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + p.counters);
  float* X = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.X);
  float* Qb = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.Q);
  float* KVb = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.KV);
  void* AO = static_cast<char*>(workspace) + p.AO;
  void* ACT = static_cast<char*>(workspace) + p.ACT;
  void* Hn = static_cast<char*>(workspace) + p.Hn;
  float* P = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.P);
  float* U = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.U);
  float* Sf = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.Sf);
  void* Sb = static_cast<char*>(workspace) + p.Sb;
  float* pmax = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.pmax);
  int* pidx = reinterpret_cast<int*>(static_cast<char*>(workspace) + p.pidx);
  const dlite_taps no_taps{};
  const dlite_taps& tp = taps ? *taps : no_taps;

  // 1. feature slots, anchor and placeholder rows (also clears the counters)
  FeatureArgs fa{features, w->depth_emb, w->feat_norm, w->tok_emb, w->ph_emb, anchor_ids,
                 X, tp.z, counters, B, m, K, D, d.vocab, d.rms_eps};
  DLITE_LAUNCH(launch_feature(fa, bf16, st));

  // 2. backbone layers
  for (int l = 0; l < d.n_layers; ++l) {
    const dlite_layer_weights& lw = w->layers[l];
    // the anchor row of the last layer feeds nothing downstream
    const int q0 = (l == d.n_layers - 1) ? 1 : 0;
    const int Lr = L - q0;
    const RowMap slot_rows{Lr, S, m + q0}, local_rows{Lr, L, q0}, all_slots{S, S, 0};

    GemmArgs q{};
    q.W = lw.wqkv; q.ldw = D; q.N = Hq; q.K = D;
    q.src = X; q.src_f32 = 1; q.ld_src = D; q.smap = slot_rows; q.M = B * Lr;
    q.gain = lw.attn_norm; q.eps = d.rms_eps;
    q.out = Qb; q.ld_out = Hq; q.omap = local_rows;
    DLITE_LAUNCH(launch_gemm(q, EPI_STORE_F32, bf16, st));

    GemmArgs kv{};
    kv.W = at(lw.wqkv, static_cast<size_t>(Hq) * D * es); kv.ldw = D; kv.N = 2 * Hkv; kv.K = D;
    kv.src = X; kv.src_f32 = 1; kv.ld_src = D; kv.smap = all_slots; kv.M = B * S;
    kv.gain = lw.attn_norm; kv.eps = d.rms_eps;
    kv.out = KVb; kv.ld_out = 2 * Hkv; kv.omap = all_slots;
    DLITE_LAUNCH(launch_gemm(kv, EPI_STORE_F32, bf16, st));

    AttnArgs aa{Qb, KVb, AO, B, m, K, d.n_q, d.n_kv, d.d_h, q0, d.rope_theta};
    DLITE_LAUNCH(launch_attention(aa, bf16, st));

    GemmArgs o{};
    o.W = lw.wo; o.ldw = Hq; o.N = D; o.K = Hq;
    o.src = AO; o.src_f32 = 0; o.ld_src = Hq; o.smap = local_rows; o.M = B * Lr;
    o.out = X; o.ld_out = D; o.omap = slot_rows;
    DLITE_LAUNCH(launch_gemm(o, EPI_RESID, bf16, st));

    GemmArgs gu{};
    gu.W = lw.w_gate_up; gu.ldw = D; gu.N = F; gu.K = D; gu.pair_off = F;
    gu.src = X; gu.src_f32 = 1; gu.ld_src = D; gu.smap = slot_rows; gu.M = B * Lr;
    gu.gain = lw.ffn_norm; gu.eps = d.rms_eps;
    gu.out = ACT; gu.ld_out = F; gu.omap = local_rows;
    DLITE_LAUNCH(launch_gemm(gu, EPI_SWIGLU, bf16, st));

    GemmArgs dn{};
    dn.W = lw.w_down; dn.ldw = F; dn.N = D; dn.K = F;
    dn.src = ACT; dn.src_f32 = 0; dn.ld_src = F; dn.smap = local_rows; dn.M = B * Lr;
    dn.out = X; dn.ld_out = D; dn.omap = slot_rows;
    if (tp.x) {
      dn.tap = tp.x + static_cast<size_t>(l) * B * L * D;
      dn.ld_tap = D; dn.tmap = local_rows;
    }
    DLITE_LAUNCH(launch_gemm(dn, EPI_RESID, bf16, st));
  }

  // 3. final norm of the placeholder rows
  NormArgs na{X, w->final_norm, Hn, tp.hidden, B, m, K, D, d.rms_eps};
  DLITE_LAUNCH(launch_final_norm(na, bf16, st));

  // 4. hidden part of the sequential head's input projection, all B*K rows at once
  GemmArgs ph{};
  ph.W = w->seq_w_down; ph.ldw = static_cast<long>(D) + r; ph.N = r; ph.K = D;
  ph.src = Hn; ph.src_f32 = 0; ph.ld_src = D; ph.smap = RowMap{K, K, 0}; ph.M = B * K;
  ph.out = P; ph.ld_out = r; ph.omap = RowMap{K, K, 0};
  DLITE_LAUNCH(launch_gemm(ph, EPI_STORE_F32, bf16, st));

  // 5. the K-step recurrence
  ScanArgs sa{P, w->seq_w_down, w->seq_w_up, U, Sf, Sb, tp.state, counters, B, K, D, r};
  DLITE_LAUNCH(launch_scan(sa, bf16, st));

  // 6. vocabulary projection + argmax
  LmArgs la{};
  la.W = w->lm_head; la.src = Sb; la.V = d.vocab; la.r = r; la.M = B * K; la.tok0 = 0;
  la.part_max = pmax; la.part_idx = pidx; la.G = p.G;
  la.cand = candidates; la.max_logit = max_logit; la.tap = tp.logits;
  la.anchors = anchor_ids; la.K = K; la.counters = counters;
  DLITE_LAUNCH(launch_lmhead(la, bf16, st));
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
