// Non-causal block attention over the m + 1 + K slots of one request.
//
// One workgroup per (request, key/value head); its G = n_q / n_kv waves are the
// query heads that share that key/value head.  The block is tiny (at most 81
// keys), so the rotated keys, the values and the rotated queries of all local
// rows are staged once in LDS (every global load issued up front), and each
// query head's rows are split over two waves: one lane per key for the scores
// (query rows read as broadcasts), one lane per row for the fp32 softmax, and
// one lane per output element for the weighted sums.  Local RoPE positions:
// context slots and the anchor sit at 0, placeholder k at k (DLite walkthrough,
// Figure 3 layout); nothing is kept after the call.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kMaxD = 128;
constexpr int kLd = kMaxD + 4;  // padded LDS row: 16-byte aligned, banks spread
constexpr int kRows = 4;        // query rows per register block

__device__ __forceinline__ float inv_freq(int i, int d, float theta) {
  return powf(theta, -2.0f * static_cast<float>(i) / static_cast<float>(d));
}

template <typename T>
__global__ __launch_bounds__(1024) void attention_kernel(AttnArgs a) {
  extern __shared__ __align__(16) float sm[];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = a.n_q / a.n_kv;
  const int d = a.d_h, half = d / 2;
  const int S = a.m + 1 + a.K, L = 1 + a.K;
  const int Hq = a.n_q * d, Hkv = a.n_kv * d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int RG = nw / G;                  // row groups per head

  float* Ks = sm;                         // [S][kLd]
  float* Vs = Ks + S * kLd;               // [S][kLd]
  float* Qs = Vs + S * kLd;               // [G][L][kLd]
  float* Ps = Qs + G * L * kLd;           // [G][L][S + 1] scores, then probabilities
  float* rc = Ps + G * L * (S + 1);       // [L][half] cos
  float* rs = rc + L * half;              // [L][half] sin

  // every global load up front: keys, values and the G heads' query rows
  const int vd = d / 4;
  const int nkv = 2 * S * vd, nq = G * L * vd, nv = nkv + nq;
  constexpr int kBatch = 16;
  for (int base = threadIdx.x; base < nv; base += kBatch * blockDim.x) {
    float4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int idx = base + u * blockDim.x;
      idx = idx < nv ? idx : nv - 1;   // clamped: every load is issued unconditionally
      const float* src;
      if (idx < nkv) {
        const int which = idx / (S * vd), s = (idx / vd) % S, e = (idx % vd) * 4;
        src = a.KV + (static_cast<long>(b) * S + s) * 2 * Hkv + which * Hkv + kvh * d + e;
      } else {
        const int t = idx - nkv, hq = t / (L * vd), j = (t / vd) % L, e = (t % vd) * 4;
        src = a.Q + (static_cast<long>(b) * L + j) * Hq + (kvh * G + hq) * d + e;
      }
      v[u] = *reinterpret_cast<const float4*>(src);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = base + u * blockDim.x;
      if (idx < nkv) {
        const int which = idx / (S * vd), s = (idx / vd) % S, e = (idx % vd) * 4;
        *reinterpret_cast<float4*>((which ? Vs : Ks) + s * kLd + e) = v[u];
      } else if (idx < nv) {
        const int t = idx - nkv, hq = t / (L * vd), j = (t / vd) % L, e = (t % vd) * 4;
        *reinterpret_cast<float4*>(Qs + (hq * L + j) * kLd + e) = v[u];
      }
    }
  }
  // rotation table for local positions 0..K
  for (int idx = threadIdx.x; idx < L * half; idx += blockDim.x) {
    const int p = idx / half, i = idx % half;
    float sn, cs;
    sincosf(static_cast<float>(p) * inv_freq(i, d, a.theta), &sn, &cs);
    rc[idx] = cs;
    rs[idx] = sn;
  }
  __syncthreads();
  // rotate keys (slot positions) and queries (row j sits at position j) in
  // place: one row per wave, lane = rotation pair
  for (int row = wave; row < S + G * L; row += nw) {
    const int pos = row < S ? (row <= a.m ? 0 : row - a.m) : (row - S) % L;
    float* p = row < S ? Ks + row * kLd : Qs + (row - S) * kLd;
    for (int i = lane; i < half; i += 64) {
      const float cs = rc[pos * half + i], sn = rs[pos * half + i];
      const float x1 = p[i], x2 = p[i + half];
      p[i] = x1 * cs - x2 * sn;
      p[i + half] = x1 * sn + x2 * cs;
    }
  }
  __syncthreads();

  // this wave: head g, rows j = rg, rg + RG, ... in blocks of kRows
  const int g = wave % G, rg = wave / G;
  const int h = kvh * G + g;
  const float scale = 1.0f / sqrtf(static_cast<float>(d));
  const float* Qh = Qs + g * L * kLd;
  float* Ph = Ps + g * L * (S + 1);
  const int nrow = (L - rg + RG - 1) / RG;   // rows of this wave

  // scores: lane = key (passes of 64)
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    const bool ok = s < S;
    const float* kr = Ks + (ok ? s : 0) * kLd;
    for (int r0 = 0; r0 < nrow; r0 += kRows) {
      float acc[kRows][2];
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) acc[jj][0] = acc[jj][1] = 0.f;
      for (int e = 0; e < d; e += 8) {
        const float4 k0 = *reinterpret_cast<const float4*>(kr + e);
        const float4 k1 = *reinterpret_cast<const float4*>(kr + e + 4);
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj) {
          const int ri = r0 + jj < nrow ? r0 + jj : nrow - 1;
          const float* qr = Qh + (rg + ri * RG) * kLd + e;
          const float4 q0 = *reinterpret_cast<const float4*>(qr);
          const float4 q1 = *reinterpret_cast<const float4*>(qr + 4);
          acc[jj][0] += (q0.x * k0.x + q0.y * k0.y) + (q0.z * k0.z + q0.w * k0.w);
          acc[jj][1] += (q1.x * k1.x + q1.y * k1.y) + (q1.z * k1.z + q1.w * k1.w);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj)
        if (r0 + jj < nrow && ok)
          Ph[(rg + (r0 + jj) * RG) * (S + 1) + s] = (acc[jj][0] + acc[jj][1]) * scale;
    }
  }
  __syncthreads();
  // softmax: one lane per row, serial over the S keys (no cross-lane traffic)
  if (lane < nrow) {
    float* pr = Ph + (rg + lane * RG) * (S + 1);
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, pr[s]);
    float sum = 0.f;
    for (int s = 0; s < S; ++s) {
      const float p = expf(pr[s] - mx);
      pr[s] = p;
      sum += p;
    }
    const float inv = 1.0f / sum;
    for (int s = 0; s < S; ++s) pr[s] *= inv;
  }
  __syncthreads();
  // outputs: lane = element e (two per lane at d = 128), rows in blocks of kRows
  for (int e = lane; e < d; e += 64) {
    for (int r0 = 0; r0 < nrow; r0 += kRows) {
      float acc[kRows];
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) acc[jj] = 0.f;
      for (int s = 0; s < S; ++s) {
        const float vv = Vs[s * kLd + e];
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj) {
          const int ri = r0 + jj < nrow ? r0 + jj : nrow - 1;
          acc[jj] += Ph[(rg + ri * RG) * (S + 1) + s] * vv;
        }
      }
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) {
        const int j = rg + (r0 + jj) * RG;
        if (r0 + jj < nrow && j >= a.q0)
          static_cast<T*>(a.out)[(static_cast<long>(b) * L + j) * Hq + h * d + e] =
              Elem<T>::from_f32(acc[jj]);
      }
    }
  }
}

}  // namespace

size_t attention_smem(const AttnArgs& a) {
  const int G = a.n_q / a.n_kv, S = a.m + 1 + a.K, L = 1 + a.K;
  return (static_cast<size_t>(2 * S * kLd) + G * L * kLd + G * L * (S + 1) + L * a.d_h) * 4;
}

hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t st) {
  const int G = a.n_q / a.n_kv;
  const int RG = G <= 8 ? 2 : 1;          // split each head's rows over RG waves
  const dim3 grid(a.n_kv, a.B), block(64 * G * RG);
  const size_t sm = attention_smem(a);
  const void* fn = bf16 ? reinterpret_cast<const void*>(&attention_kernel<uint16_t>)
                        : reinterpret_cast<const void*>(&attention_kernel<float>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(sm));
  if (e != hipSuccess) return e;
  if (bf16)
    hipLaunchKernelGGL(attention_kernel<uint16_t>, grid, block, sm, st, a);
  else
    hipLaunchKernelGGL(attention_kernel<float>, grid, block, sm, st, a);
  return hipGetLastError();
}

}  // namespace dlite
