// Row-wise kernels of the draft step: building the slot buffer (depth-embedded,
// RMS-normalised context features, anchor embedding, placeholders) and the
// final RMSNorm in front of the sequential head.
//
// Feature slots follow the DLite walkthrough, section "历史并没有消失，而是由目标
// 模型编码" (z = Norm(h^(l) + e_depth^(l))), kept as m separate sequence slots
// ("沿序列维拼接，保留各层的独立身份").  The anchor enters through its token
// embedding and the K placeholders through one shared input vector.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += sh[w];
  __syncthreads();
  return t;
}

template <typename T>
__device__ __forceinline__ float ld(const void* p, long i) {
  return Elem<T>::to_f32(static_cast<const T*>(p)[i]);
}

// One workgroup per slot (b, s).
template <typename T>
__global__ __launch_bounds__(kThreads) void feature_kernel(FeatureArgs a) {
  __shared__ float sh[kThreads / 64];
  const int S = a.m + 1 + a.K;
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  float* x = a.X + static_cast<long>(blockIdx.x) * a.D;
  if (blockIdx.x == 0 && threadIdx.x < CNT_COUNT) a.counters[threadIdx.x] = 0u;
  if (s < a.m) {
    const long hrow = (static_cast<long>(b) * a.m + s) * a.D;
    float ss = 0.f;
    for (int e = threadIdx.x; e < a.D; e += blockDim.x) {
      const float y = ld<T>(a.H, hrow + e) + ld<T>(a.depth_emb, static_cast<long>(s) * a.D + e);
      ss += y * y;
    }
    const float inv = 1.0f / sqrtf(block_sum(ss, sh) / static_cast<float>(a.D) + a.eps);
    for (int e = threadIdx.x; e < a.D; e += blockDim.x) {
      const float y = ld<T>(a.H, hrow + e) + ld<T>(a.depth_emb, static_cast<long>(s) * a.D + e);
      const float z = ld<T>(a.feat_norm, e) * (y * inv);
      x[e] = z;
      if (a.tap_z) a.tap_z[hrow + e] = z;
    }
  } else if (s == a.m) {
    const int tok = a.anchors[b];
    const bool ok = tok >= 0 && tok < a.V;   // out of range: zero input row
    for (int e = threadIdx.x; e < a.D; e += blockDim.x)
      x[e] = ok ? ld<T>(a.tok_emb, static_cast<long>(tok) * a.D + e) : 0.f;
  } else {
    for (int e = threadIdx.x; e < a.D; e += blockDim.x) x[e] = ld<T>(a.ph_emb, e);
  }
}

// h_k = RMSNorm(x_k; gain) for the placeholder rows; one workgroup per row.
template <typename T>
__global__ __launch_bounds__(kThreads) void final_norm_kernel(NormArgs a) {
  __shared__ float sh[kThreads / 64];
  const int S = a.m + 1 + a.K;
  const int b = blockIdx.x / a.K, k = blockIdx.x % a.K;
  const float* x = a.X + (static_cast<long>(b) * S + a.m + 1 + k) * a.D;
  float ss = 0.f;
  for (int e = threadIdx.x; e < a.D; e += blockDim.x) ss += x[e] * x[e];
  const float inv = 1.0f / sqrtf(block_sum(ss, sh) / static_cast<float>(a.D) + a.eps);
  const long orow = static_cast<long>(blockIdx.x) * a.D;
  for (int e = threadIdx.x; e < a.D; e += blockDim.x) {
    const float h = ld<T>(a.gain, e) * (x[e] * inv);
    static_cast<T*>(a.out)[orow + e] = Elem<T>::from_f32(h);
    if (a.tap) a.tap[orow + e] = h;
  }
}

}  // namespace

hipError_t launch_feature(const FeatureArgs& a, bool bf16, hipStream_t st) {
  const dim3 grid(a.B * (a.m + 1 + a.K)), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL(feature_kernel<uint16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(feature_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_final_norm(const NormArgs& a, bool bf16, hipStream_t st) {
  const dim3 grid(a.B * a.K), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL(final_norm_kernel<uint16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(final_norm_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dlite
