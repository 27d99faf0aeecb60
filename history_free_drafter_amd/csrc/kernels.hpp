// Launch interfaces of the DLite kernels (host side).  Each launcher enqueues
// one or more kernels on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dlite {

// Workspace counters, zeroed by the first kernel of every draft step.
enum Counter { CNT_LM_DONE = 0, CNT_SCAN_BAR = 1, CNT_STATUS = 2, CNT_COUNT = 16 };
enum Status { STATUS_BARRIER_TIMEOUT = 1 };

// ------------------------------------------------------------ feature build --
struct FeatureArgs {
  const void* H;          // [B, m, D] storage type
  const void* depth_emb;  // [m, D]
  const void* feat_norm;  // [D]
  const void* tok_emb;    // [V, D]
  const void* ph_emb;     // [D]
  const int32_t* anchors; // [B]
  float* X;               // [B, S, D] slot buffer (fp32)
  float* tap_z;           // [B, m, D] or null
  unsigned* counters;     // CNT_COUNT words, zeroed here
  int B, m, K, D, V;
  float eps;
};
hipError_t launch_feature(const FeatureArgs& a, bool bf16, hipStream_t st);

// ---------------------------------------------------------------- GEMMs ----
// out[token, n] = epilogue( sum_k W[n, k] * in[token, k] ), tokens 0..M-1
// (offset tok0), logical output rows n in [0, N).
enum Epi { EPI_STORE_F32 = 0, EPI_STORE_ACT = 1, EPI_RESID = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  const void* W; long ldw; int N; int K;
  long pair_off;                 // SwiGLU: up rows start pair_off rows after gate rows
  const void* src; int src_f32; long ld_src; RowMap smap;
  int M; int tok0;
  const void* gain; float eps;   // RMSNorm prologue over the K inputs (null: none)
  void* out; long ld_out; RowMap omap;
  float* tap; long ld_tap; RowMap tmap;   // RESID: copy of the updated row
};
hipError_t launch_gemm(const GemmArgs& a, int epi, bool bf16, hipStream_t st);

// ------------------------------------------------------------- attention --
struct AttnArgs {
  const float* Q;   // [B, L, n_q d_h]
  const float* KV;  // [B, S, 2 n_kv d_h] (k heads, then v heads)
  void* out;        // [B, L, n_q d_h] storage type
  int B, m, K, n_q, n_kv, d_h, q0;  // rows j = q0..K of each request are computed
  float theta;
};
hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t st);

// ----------------------------------------------------------- final norm ----
struct NormArgs {
  const float* X;     // [B, S, D]
  const void* gain;   // [D]
  void* out;          // [B, K, D] storage type
  float* tap;         // [B, K, D] or null
  int B, m, K, D; float eps;
};
hipError_t launch_final_norm(const NormArgs& a, bool bf16, hipStream_t st);

// ------------------------------------------------------ sequential head ----
struct ScanArgs {
  const float* P;        // [B, K, r]  seq_w_down[:, :D] h_k
  const void* w_down;    // [r, D + r] (state columns used)
  const void* w_up;      // [r, r]
  float* U;              // [B, r] scratch
  float* Sf;             // [B, K, r] states (fp32)
  void* Sb;              // [B, K, r] states (storage type) for the vocabulary GEMM
  float* tap;            // [B, K, r] or null
  unsigned* counters;
  int B, K, D, r;
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
  int K;                 // tokens per request (token t belongs to request t / K)
  unsigned* counters;
};
hipError_t launch_lmhead(const LmArgs& a, bool bf16, hipStream_t st);
int lmhead_groups(int V);

// --------------------------------------------------------------- accept ----
hipError_t launch_accept(const int32_t* cand, const int32_t* tgt, int B, int K,
                         int32_t* A, int32_t* next, hipStream_t st);

}  // namespace dlite
