// The gated sequential head of the DLite walkthrough, section "官方顺序头具体
// 算了什么": the previous token enters through an R-wide embedding
// (d_0 = a, v_i = E_R(d_{i-1})), a gate mixes the old state with a tanh
// candidate, and r_i = W_h [s_i ; u_i] + b_h feeds the per-step vocabulary
// projection, whose greedy choice d_i is the next step's input.
//
// The u-part of W_h does not depend on any token and is applied to all K
// positions at once by the GEMM before the loop (qh_i = W_h[:, R:] u_i).  Each
// step then runs two small launches before its vocabulary pass:
//   state:  [g ; c] = W_s [s_{i-1} ; v_i] + b_s,
//           s_i = sigmoid(g) * s_{i-1} + (1 - sigmoid(g)) * tanh(c)   (fp32)
//   output: r_i = W_h[:, :R] s_i + qh_i + b_h   (storage type, the
//           vocabulary pass's input)
// A warm-up update (the token before the anchor, same section) runs the state
// launch alone from s = 0, before position 1.
// One wave per output element (rows j and R + j of W_s; row j of W_h) holds
// its weight rows in registers and serves a chunk of requests whose inputs
// are staged in LDS; weights are read once per request chunk.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kThreads = 256;   // four waves, four output elements
constexpr int kChunk = 8;       // requests staged in LDS per workgroup

template <typename T>
__global__ __launch_bounds__(kThreads) void gated_state_kernel(GatedArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int MAXC = 2 * kGatedMaxRank / PER / 64;   // 16-byte chunks per lane of a 2R row
  extern __shared__ float xs[];                        // [kChunk][2R]
  const int R = a.R, R2 = 2 * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + wave;
  const int b0 = blockIdx.y * kChunk;
  const int nb = (a.B - b0) < kChunk ? (a.B - b0) : kChunk;
  const T* emb = static_cast<const T*>(a.emb);
  for (int e = threadIdx.x; e < nb * R2; e += blockDim.x) {
    const int bb = e / R2, k = e % R2, b = b0 + bb;
    float v = 0.f;
    if (k < R) {
      if (a.s_prev) v = a.s_prev[b * a.ld_sp + k];
    } else {
      const int d = a.tok[b];
      if (d >= 0 && d < a.V) v = Elem<T>::to_f32(emb[static_cast<long>(d) * R + (k - R)]);
    }
    xs[bb * R2 + k] = v;
  }
  __syncthreads();
  if (j >= R) return;

  const T* W = static_cast<const T*>(a.w_s);
  const int nch = R2 / PER;
  float wg[MAXC][PER], wc[MAXC][PER];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int t = 0; t < PER; ++t) wg[c][t] = wc[c][t] = 0.f;
    if (ch < nch) {
      load16_f32(W + static_cast<long>(j) * R2 + ch * PER, wg[c]);
      load16_f32(W + static_cast<long>(R + j) * R2 + ch * PER, wc[c]);
    }
  }
  const float bg = Elem<T>::to_f32(static_cast<const T*>(a.b_s)[j]);
  const float bc = Elem<T>::to_f32(static_cast<const T*>(a.b_s)[R + j]);
  for (int bb = 0; bb < nb; ++bb) {
    float dg = 0.f, dc = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
#pragma unroll
        for (int t = 0; t < PER; ++t) {
          const float x = xs[bb * R2 + ch * PER + t];
          dg += wg[c][t] * x;
          dc += wc[c][t] * x;
        }
      }
    }
    dg = wave_sum(dg);
    dc = wave_sum(dc);
    if (lane == 0) {
      const int b = b0 + bb;
      const float f = 1.0f / (1.0f + expf(-(dg + bg)));
      const float sp = a.s_prev ? a.s_prev[b * a.ld_sp + j] : 0.f;
      const bool skip = a.warm && !(a.tok[b] >= 0 && a.tok[b] < a.V);   // no token to warm up with
      a.s_out[b * a.ld_s + j] = skip ? 0.f : f * sp + (1.0f - f) * tanhf(dc + bc);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void gated_out_kernel(GatedArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int MAXC = (kGatedMaxRank / PER + 63) / 64;
  extern __shared__ float xs[];                        // [kChunk][R]
  const int R = a.R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + wave;
  const int b0 = blockIdx.y * kChunk;
  const int nb = (a.B - b0) < kChunk ? (a.B - b0) : kChunk;
  for (int e = threadIdx.x; e < nb * R; e += blockDim.x) {
    const int bb = e / R, k = e % R;
    xs[bb * R + k] = a.s_out[(b0 + bb) * a.ld_s + k];
  }
  __syncthreads();
  if (j >= R) return;

  const T* W = static_cast<const T*>(a.w_h) + static_cast<long>(j) * (R + a.D);   // state columns first
  const int nch = R / PER;
  float w[MAXC][PER];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int t = 0; t < PER; ++t) w[c][t] = 0.f;
    if (ch < nch) load16_f32(W + ch * PER, w[c]);
  }
  const float bh = Elem<T>::to_f32(static_cast<const T*>(a.b_h)[j]);
  T* out = static_cast<T*>(a.r_out);
  for (int bb = 0; bb < nb; ++bb) {
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
#pragma unroll
        for (int t = 0; t < PER; ++t) d += w[c][t] * xs[bb * R + ch * PER + t];
      }
    }
    d = wave_sum(d);
    if (lane == 0) {
      const int b = b0 + bb;
      out[static_cast<long>(b) * R + j] = Elem<T>::from_f32(d + a.qh[b * a.ld_q + j] + bh);
    }
  }
}

}  // namespace

hipError_t launch_gated_step(const GatedArgs& a, bool bf16, hipStream_t st) {
  if (a.R < 1 || a.R > kGatedMaxRank || a.R % 8 || a.B < 1) return hipErrorInvalidValue;
  const dim3 grid((a.R + 3) / 4, (a.B + kChunk - 1) / kChunk), block(kThreads);
  const size_t sm_state = static_cast<size_t>(kChunk) * 2 * a.R * sizeof(float);
  const size_t sm_out = static_cast<size_t>(kChunk) * a.R * sizeof(float);
  if (bf16) {
    launch_k(gated_state_kernel<uint16_t>, grid, block, sm_state, st, a);
    if (!a.warm) launch_k(gated_out_kernel<uint16_t>, grid, block, sm_out, st, a);
  } else {
    launch_k(gated_state_kernel<float>, grid, block, sm_state, st, a);
    if (!a.warm) launch_k(gated_out_kernel<float>, grid, block, sm_out, st, a);
  }
  return hipGetLastError();
}

}  // namespace dlite
