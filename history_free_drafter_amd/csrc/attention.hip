// Non-causal block attention over the m + 1 + K slots of one request.
//
// One workgroup per (request, key/value head); its G = n_q / n_kv waves are the
// query heads that share that key/value head.  The block is tiny (at most 81
// keys), so keys and values are rotated and staged once in LDS and each wave
// handles its head's query rows: one lane per key for the scores, a wave-wide
// softmax in fp32, and one lane per output element for the weighted sum.
// Local RoPE positions: context slots and the anchor sit at 0, placeholder k
// at k (DLite walkthrough, Figure 3 layout); nothing is kept after the call.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kMaxSlots = 81;   // m <= 64, K <= 16
constexpr int kMaxD = 128;

__device__ __forceinline__ float inv_freq(int i, int d, float theta) {
  return powf(theta, -2.0f * static_cast<float>(i) / static_cast<float>(d));
}

template <typename T>
__global__ __launch_bounds__(1024) void attention_kernel(AttnArgs a) {
  __shared__ float Ks[kMaxSlots][kMaxD + 1];
  __shared__ float Vs[kMaxSlots][kMaxD + 1];
  __shared__ float qs[16][kMaxD];
  __shared__ float ps[16][kMaxSlots + 3];

  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = a.n_q / a.n_kv;
  const int d = a.d_h, half = d / 2;
  const int S = a.m + 1 + a.K, L = 1 + a.K;
  const int Hq = a.n_q * d, Hkv = a.n_kv * d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // stage rotated keys and values of this head
  for (int idx = threadIdx.x; idx < S * half; idx += blockDim.x) {
    const int s = idx / half, i = idx % half;
    const float* kv = a.KV + (static_cast<long>(b) * S + s) * 2 * Hkv;
    const float k1 = kv[kvh * d + i], k2 = kv[kvh * d + i + half];
    const int pos = s <= a.m ? 0 : s - a.m;
    float sn, cs;
    sincosf(static_cast<float>(pos) * inv_freq(i, d, a.theta), &sn, &cs);
    Ks[s][i] = k1 * cs - k2 * sn;
    Ks[s][i + half] = k1 * sn + k2 * cs;
    Vs[s][i] = kv[Hkv + kvh * d + i];
    Vs[s][i + half] = kv[Hkv + kvh * d + i + half];
  }
  __syncthreads();

  const int h = kvh * G + wave;
  const float scale = 1.0f / sqrtf(static_cast<float>(d));
  for (int j = a.q0; j < L; ++j) {
    const float* q = a.Q + (static_cast<long>(b) * L + j) * Hq + h * d;
    if (lane < half) {
      float sn, cs;
      sincosf(static_cast<float>(j) * inv_freq(lane, d, a.theta), &sn, &cs);
      const float q1 = q[lane], q2 = q[lane + half];
      qs[wave][lane] = q1 * cs - q2 * sn;
      qs[wave][lane + half] = q1 * sn + q2 * cs;
    }
    __syncthreads();
    // scores: lane handles keys lane and lane + 64
    float sc[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int s = lane + 64 * r;
      if (s < S) {
        float acc = 0.f;
        for (int e = 0; e < d; ++e) acc += qs[wave][e] * Ks[s][e];
        sc[r] = acc * scale;
      }
    }
    const float mx = wave_max(fmaxf(sc[0], sc[1]));
    float p[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) p[r] = (lane + 64 * r < S) ? expf(sc[r] - mx) : 0.f;
    const float sum = wave_sum(p[0] + p[1]);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (lane + 64 * r < S) ps[wave][lane + 64 * r] = p[r] * inv;
    __syncthreads();
    // output: lane handles elements lane and lane + 64
    T* o = static_cast<T*>(a.out) + (static_cast<long>(b) * L + j) * Hq + h * d;
    for (int e = lane; e < d; e += 64) {
      float acc = 0.f;
      for (int s = 0; s < S; ++s) acc += ps[wave][s] * Vs[s][e];
      o[e] = Elem<T>::from_f32(acc);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t st) {
  const int G = a.n_q / a.n_kv;
  const dim3 grid(a.n_kv, a.B), block(64 * G);
  if (bf16)
    hipLaunchKernelGGL(attention_kernel<uint16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(attention_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dlite
