// Vocabulary projection of the sequential-head states fused with the greedy
// choice: logits_k = W_lm s_k for all B*K states at once (the projection is
// applied once, after the head), argmax with ties to the lowest index.
//
// Pass 1: workgroup g streams vocabulary rows [g V / G, (g+1) V / G) through
// 16x16 MFMA tiles against the token block held in registers and keeps a
// running (max, index) per token; the full logits are never written (unless
// the logits tap is requested).  Pass 2 runs in whichever workgroup finishes
// last: it reduces the G partials of every token in a fixed order, so the
// result does not depend on scheduling.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kWaves = 8;
constexpr int kMaxSteps = 16;   // r <= 512 (bf16) / 256 (fp32)

template <typename T, int MT>
__global__ __launch_bounds__(kWaves * 64) void lmhead_kernel(LmArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int KS = PER * 4;
  __shared__ float sv[kWaves][32];
  __shared__ int si[kWaves][32];
  __shared__ int is_last;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const long G = gridDim.x, g = blockIdx.x;
  const int r0 = static_cast<int>((g * a.V) / G), r1 = static_cast<int>(((g + 1) * a.V) / G);
  const int ntile = (r1 - r0 + 15) >> 4;
  const int nsteps = a.r / KS;
  const T* W = static_cast<const T*>(a.W);
  const T* X = static_cast<const T*>(a.src);

  uint4 b[MT][kMaxSteps];
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int tok = u * 16 + c16;
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
      if (s < nsteps && tok < a.M)
        b[u][s] = *reinterpret_cast<const uint4*>(
            X + static_cast<long>(a.tok0 + tok) * a.r + s * KS + grp * PER);
      else
        b[u][s] = make_uint4(0, 0, 0, 0);
    }
  }

  float bv[MT];
  int bi[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) { bv[u] = -INFINITY; bi[u] = 0x7fffffff; }

  for (int t = wave; t < ntile; t += kWaves) {
    const int row = r0 + t * 16 + c16;
    const bool rok = row < r1;
    uint4 av[kMaxSteps];
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
      if (s < nsteps && rok)
        av[s] = ld_stream(W + static_cast<long>(row) * a.r + s * KS + grp * PER);
      else
        av[s] = make_uint4(0, 0, 0, 0);
    }
    floatx4 acc[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
      if (s < nsteps)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[u] = mma_step(av[s], b[u][s], acc[u], T());
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int tok = u * 16 + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vr = r0 + t * 16 + grp * 4 + i;
        if (vr < r1 && tok < a.M) {
          const float v = acc[u][i];
          if (better(v, vr, bv[u], bi[u])) { bv[u] = v; bi[u] = vr; }
          if (a.tap) a.tap[static_cast<long>(a.tok0 + tok) * a.V + vr] = v;
        }
      }
    }
  }

  // combine the four row groups of each token column, then the waves
#pragma unroll
  for (int u = 0; u < MT; ++u) {
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv[u], o, kWave);
      const int oi = __shfl_xor(bi[u], o, kWave);
      if (better(ov, oi, bv[u], bi[u])) { bv[u] = ov; bi[u] = oi; }
    }
    if (grp == 0) { sv[wave][u * 16 + c16] = bv[u]; si[wave][u * 16 + c16] = bi[u]; }
  }
  __syncthreads();
  if (threadIdx.x < MT * 16 && static_cast<int>(threadIdx.x) < a.M) {
    float v = sv[0][threadIdx.x];
    int i = si[0][threadIdx.x];
    for (int w = 1; w < kWaves; ++w)
      if (better(sv[w][threadIdx.x], si[w][threadIdx.x], v, i)) { v = sv[w][threadIdx.x]; i = si[w][threadIdx.x]; }
    const long o = static_cast<long>(a.tok0 + threadIdx.x) * G + g;
    a.part_max[o] = v;
    a.part_idx[o] = i;
  }

  // pass 2 in the last workgroup to finish
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(a.counters + CNT_LM_DONE, 1u);
    is_last = (prev == static_cast<unsigned>(G - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int tok = wave; tok < a.M; tok += kWaves) {
    const long base = static_cast<long>(a.tok0 + tok) * G;
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (long j = lane; j < G; j += 64) {
      const float pv = a.part_max[base + j];
      const int pi = a.part_idx[base + j];
      if (better(pv, pi, v, i)) { v = pv; i = pi; }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(v, o, kWave);
      const int oi = __shfl_xor(i, o, kWave);
      if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
    if (lane == 0) {
      const int gt = a.tok0 + tok;
      const int anchor = a.anchors[gt / a.K];
      const bool ok = anchor >= 0 && anchor < a.V;
      a.cand[gt] = ok ? i : -1;
      if (a.max_logit) a.max_logit[gt] = ok ? v : 0.f;
    }
  }
  if (threadIdx.x == 0) a.counters[CNT_LM_DONE] = 0u;
}

}  // namespace

int lmhead_groups(int V) {
  const int tiles = (V + 15) / 16;
  return tiles < 256 ? tiles : 256;
}

hipError_t launch_lmhead(const LmArgs& a0, bool bf16, hipStream_t st) {
  const dim3 grid(a0.G), block(kWaves * 64);
  for (int t0 = 0; t0 < a0.M; t0 += 32) {
    LmArgs a = a0;
    a.tok0 = a0.tok0 + t0;
    a.M = (a0.M - t0) < 32 ? (a0.M - t0) : 32;
    if (bf16) {
      if (a.M <= 16) hipLaunchKernelGGL((lmhead_kernel<uint16_t, 1>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((lmhead_kernel<uint16_t, 2>), grid, block, 0, st, a);
    } else {
      if (a.M <= 16) hipLaunchKernelGGL((lmhead_kernel<float, 1>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((lmhead_kernel<float, 2>), grid, block, 0, st, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dlite
