// Row-wise kernels of the draft step: building the slot buffer (depth-embedded,
// RMS-normalised context features, anchor or local token group embeddings,
// placeholders) with the first GEMM inputs, and the optional fp32 copy of the
// final-normed hidden rows.
//
// Feature slots follow the DLite walkthrough, section "历史并没有消失，而是由目标
// 模型编码" (z = Norm(h^(l) + e_depth^(l))), kept as m separate sequence slots
// ("沿序列维拼接，保留各层的独立身份").  The anchor (or a local group of G
// tokens ending at it, section "锚点是已经确定、尚待目标前向处理的输入") enters
// through its token embeddings and the K placeholders through one shared input
// vector.  Slot order per request: m features, G group tokens, K placeholders.
#include <type_traits>

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

// One workgroup per slot (b, s).  Writes the row's sum of squares (slot 0 of
// the row's partials), the fp32 residual row of group and placeholder slots
// (context slots are key/value inputs only and never updated), and the
// pre-gained GEMM input rows:
// context slots for every layer (they do not change between layers), group
// and placeholder rows for the first layer.  Each thread holds its share of
// the row in registers (16-byte loads, all issued before the reduction).
constexpr int kMaxVec = 8;   // 16-byte vectors per thread: D <= 8 * 256 * 8 (NV: as many as D needs)

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& v, float* out) {
  load16_f32(reinterpret_cast<const T*>(&v), out);
}

template <typename T, int NV>
__global__ __launch_bounds__(kThreads) void feature_kernel(FeatureArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  __shared__ float sh[kThreads / 64];
  const int S = a.m + a.G + a.K;
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  const long row = blockIdx.x;
  float* x = a.X + row * a.D;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.n_counters; i += blockDim.x) a.counters[i] = 0u;
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < a.n_clear;
       i += static_cast<long>(gridDim.x) * blockDim.x)
    a.clear[i] = make_uint4(0u, 0u, 0u, 0u);
  const int nvec = a.D / PER;

  const T* src;
  const T* add = nullptr;
  if (s < a.m) {
    int pos = 0;
    if (a.h_pos) {
      const int pb = a.h_pos[b];
      pos = (pb >= 0 && pb < a.h_T) ? pb : 0;
    }
    src = static_cast<const T*>(a.H) + static_cast<long>(b) * a.h_sb + static_cast<long>(s) * a.h_sl +
          static_cast<long>(pos) * a.h_st;
    add = static_cast<const T*>(a.depth_emb) + static_cast<long>(s) * a.D;
  } else if (s < a.m + a.G) {
    // group token j (j = G - 1: the anchor); padding and out-of-range ids: zero row
    const int j = s - a.m;
    const int32_t* ids = a.gids + static_cast<long>(b) * (a.G - 1);
    const int tok = j == a.G - 1 ? a.anchors[b] : (j >= group_pad(ids, a.G) ? ids[j] : -1);
    src = (tok >= 0 && tok < a.V) ? static_cast<const T*>(a.tok_emb) + static_cast<long>(tok) * a.D
                                  : nullptr;
  } else {
    src = static_cast<const T*>(a.ph_emb);
  }
  const T* g0 = static_cast<const T*>(a.attn_norm[0]);
  const T* gf = static_cast<const T*>(a.feat_norm);
  uint4 hv[NV], dv[NV], gv[NV], av[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int idx = threadIdx.x + q * kThreads;
    hv[q] = dv[q] = gv[q] = av[q] = make_uint4(0, 0, 0, 0);
    if (idx < nvec) {
      av[q] = *reinterpret_cast<const uint4*>(g0 + idx * PER);   // first layer's gain, with the rest
      if (src) hv[q] = *reinterpret_cast<const uint4*>(src + idx * PER);
      if (add) {
        dv[q] = *reinterpret_cast<const uint4*>(add + idx * PER);
        gv[q] = *reinterpret_cast<const uint4*>(gf + idx * PER);
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    float h[PER], e[PER];
    unpack16<T>(hv[q], h);
    unpack16<T>(dv[q], e);
#pragma unroll
    for (int t = 0; t < PER; ++t) ss += (h[t] + e[t]) * (h[t] + e[t]);
  }
  float inv = 1.f;
  if (add) inv = 1.0f / sqrtf(block_sum(ss, sh) / static_cast<float>(a.D) + a.eps);
  ss = 0.f;
  // final slot values (fp32), their sum of squares, the first layer's inputs
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int idx = threadIdx.x + q * kThreads;
    if (idx < nvec) {
      float h[PER], e[PER], gz[PER], v[PER], g[PER];
      unpack16<T>(hv[q], h);
      unpack16<T>(dv[q], e);
      unpack16<T>(gv[q], gz);
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        v[t] = add ? gz[t] * ((h[t] + e[t]) * inv) : h[t];
        ss += v[t] * v[t];
      }
      if (!add) {   // residual stream: group and placeholder rows only
        float* xo = x + idx * PER;
#pragma unroll
        for (int t = 0; t < PER; t += 4)
          *reinterpret_cast<float4*>(xo + t) = make_float4(v[t], v[t + 1], v[t + 2], v[t + 3]);
      }
      if (add && a.tap_z) {
        float* tz = a.tap_z + (static_cast<long>(b) * a.m + s) * a.D + idx * PER;
#pragma unroll
        for (int t = 0; t < PER; t += 4)
          *reinterpret_cast<float4*>(tz + t) = make_float4(v[t], v[t + 1], v[t + 2], v[t + 3]);
      }
      unpack16<T>(av[q], g);
      float o[PER];
#pragma unroll
      for (int t = 0; t < PER; ++t) o[t] = g[t] * v[t];
      *reinterpret_cast<uint4*>(static_cast<T*>(a.XB) + row * a.D + idx * PER) = pack16(o, T());
      // context slots feed every layer's keys and values with that layer's gain
      if (add) {
        for (int l = 1; l < a.n_layers; ++l) {
          load16_f32(static_cast<const T*>(a.attn_norm[l]) + idx * PER, g);
#pragma unroll
          for (int t = 0; t < PER; ++t) o[t] = g[t] * v[t];
          *reinterpret_cast<uint4*>(static_cast<T*>(a.XB) +
                                    (l * static_cast<long>(a.B) * S + row) * a.D + idx * PER) =
              pack16(o, T());
        }
      }
    }
  }
  ss = block_sum(ss, sh);
  if (threadIdx.x == 0) a.ssq[row * kSsqParts] = ss;
}

// fp32 h_k = RMSNorm(x_k; gain) of the placeholder rows; one workgroup per row.
template <typename T>
__global__ __launch_bounds__(kThreads) void hidden_tap_kernel(NormArgs a) {
  __shared__ float sh[kThreads / 64];
  const int S = a.m + a.G + a.K;
  const int b = blockIdx.x / a.K, k = blockIdx.x % a.K;
  const float* x = a.X + (static_cast<long>(b) * S + a.m + a.G + k) * a.D;
  float ss = 0.f;
  for (int e = threadIdx.x; e < a.D; e += blockDim.x) ss += x[e] * x[e];
  const float inv = 1.0f / sqrtf(block_sum(ss, sh) / static_cast<float>(a.D) + a.eps);
  const long orow = static_cast<long>(blockIdx.x) * a.D;
  for (int e = threadIdx.x; e < a.D; e += blockDim.x) a.tap[orow + e] = ld<T>(a.gain, e) * (x[e] * inv);
}

}  // namespace

hipError_t launch_feature(const FeatureArgs& a, bool bf16, hipStream_t st) {
  if (a.G < 1 || (a.G > 1 && !a.gids)) return hipErrorInvalidValue;
  const dim3 grid(a.B * (a.m + a.G + a.K)), block(kThreads);
  // 16-byte vectors per thread for this width (registers sized to it)
  const int nvec = a.D / (bf16 ? 8 : 4);
  const int need = (nvec + kThreads - 1) / kThreads;
  if (need > kMaxVec) return hipErrorInvalidValue;
  auto go = [&](auto t, auto nv) {
    using TT = decltype(t);
    launch_k(feature_kernel<TT, decltype(nv)::value>, grid, block, 0, st, a);
  };
  auto pick = [&](auto t) {
    if (need <= 1) go(t, std::integral_constant<int, 1>{});
    else if (need <= 2) go(t, std::integral_constant<int, 2>{});
    else if (need <= 4) go(t, std::integral_constant<int, 4>{});
    else go(t, std::integral_constant<int, 8>{});
  };
  if (bf16) pick(uint16_t{});
  else pick(float{});
  return hipGetLastError();
}

hipError_t launch_hidden_tap(const NormArgs& a, bool bf16, hipStream_t st) {
  const dim3 grid(a.B * a.K), block(kThreads);
  if (bf16)
    launch_k(hidden_tap_kernel<uint16_t>, grid, block, 0, st, a);
  else
    launch_k(hidden_tap_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dlite
