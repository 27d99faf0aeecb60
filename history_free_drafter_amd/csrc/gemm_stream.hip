// Weight-streaming GEMM for few activation rows (M <= 32 per launch).
//
// In the small-batch draft step every linear map is read-bound: each weight
// byte is used by at most 32 token rows.  The kernel therefore streams each
// weight row exactly once from HBM straight into registers (16 bytes per lane,
// no LDS staging) and feeds it to 16x16 MFMA tiles whose other operand is the
// token block, built in registers from the activation rows (L2-resident).
//
// Work split: workgroup g owns logical output rows [g N / G, (g+1) N / G) in
// 16-row tiles; its waves split the K dimension, and partial tiles are summed
// through LDS in a fixed order (deterministic).  An optional RMSNorm prologue
// multiplies inputs by the gain while the waves accumulate each row's sum of
// squares; the 1/rms factor is applied to the finished dot products, which is
// exact algebra (the factor is constant along k).
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kMaxWaves = 8;
constexpr int kMaxTiles = 4;    // 16-row tiles per workgroup
constexpr int kChunk = 8;       // k-steps held in registers at once

template <typename T, int MT, int EPI, bool NORM>
__global__ __launch_bounds__(512) void gemm_stream_kernel(GemmArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int KS = PER * 4;                        // k per MFMA step
  constexpr int NP = (EPI == EPI_SWIGLU) ? 2 : 1;    // gate/up pairs

  __shared__ float red[2][kMaxWaves * NP * MT * 256];
  __shared__ float ssq_part[kMaxWaves][32];
  __shared__ float inv_rms[32];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;

  const long G = gridDim.x, g = blockIdx.x;
  const int r0 = static_cast<int>((g * a.N) / G);
  const int r1 = static_cast<int>(((g + 1) * a.N) / G);
  const int ntile = (r1 - r0 + 15) >> 4;

  const int nsteps = a.K / KS;
  const int s0 = (wave * nsteps) / nwaves, s1 = ((wave + 1) * nsteps) / nwaves;

  const T* W = static_cast<const T*>(a.W);
  const T* gain = static_cast<const T*>(a.gain);

  floatx4 acc[kMaxTiles][NP][MT];
#pragma unroll
  for (int t = 0; t < kMaxTiles; ++t)
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[t][p][u] = floatx4{0.f, 0.f, 0.f, 0.f};
  float ssq[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) ssq[u] = 0.f;

  // physical source rows of this lane's tokens
  long srow[MT];
  bool tok_ok[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int tok = u * 16 + c16;
    tok_ok[u] = tok < a.M;
    srow[u] = tok_ok[u] ? a.smap.row(a.tok0 + tok) : 0;
  }

  for (int c0 = s0; c0 < s1; c0 += kChunk) {
    // token block for this chunk of k-steps
    uint4 b[MT][kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int s = c0 + i;
      const int k = s * KS + grp * PER;
      float gv[PER];
      if (NORM && s < s1) {
        load16_f32(gain + k, gv);
      }
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        float v[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) v[e] = 0.f;
        if (s < s1 && tok_ok[u]) {
          if (a.src_f32) {
            const float* sp = static_cast<const float*>(a.src) + srow[u] * a.ld_src + k;
            if constexpr (PER == 8) {
              load16_f32(sp, v);
              load16_f32(sp + 4, v + 4);
            } else {
              load16_f32(sp, v);
            }
          } else {
            load16_f32(static_cast<const T*>(a.src) + srow[u] * a.ld_src + k, v);
          }
          if (NORM) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
              ssq[u] += v[e] * v[e];
              v[e] *= gv[e];
            }
          }
        }
        b[u][i] = pack16(v, T());
      }
    }
    // stream the weight tiles of this workgroup through the MFMAs
#pragma unroll
    for (int t = 0; t < kMaxTiles; ++t) {
      if (t < ntile) {
        const int row = r0 + t * 16 + c16;
        const bool rok = row < r1;
        uint4 av[NP][kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          const int s = c0 + i;
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            if (s < s1 && rok)
              av[p][i] = ld_stream(W + (row + p * a.pair_off) * a.ldw + s * KS + grp * PER);
            else
              av[p][i] = make_uint4(0, 0, 0, 0);
          }
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int u = 0; u < MT; ++u)
              acc[t][p][u] = mma_step(av[p][i], b[u][i], acc[t][p][u], T());
      }
    }
  }

  if (NORM) {
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      float v = ssq[u];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      if (grp == 0) ssq_part[wave][u * 16 + c16] = v;
    }
    __syncthreads();
    if (threadIdx.x < MT * 16) {
      float s = 0.f;
      for (int w = 0; w < nwaves; ++w) s += ssq_part[w][threadIdx.x];
      inv_rms[threadIdx.x] = 1.0f / sqrtf(s / static_cast<float>(a.K) + a.eps);
    }
  }

  // cross-wave reduction and epilogue, one 16-row tile at a time
  const int per_wave = NP * MT * 256;
#pragma unroll
  for (int t = 0; t < kMaxTiles; ++t) {
    if (t < ntile) {
      float* buf = red[t & 1];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int u = 0; u < MT; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            buf[wave * per_wave + ((p * MT + u) * 4 + i) * 64 + lane] = acc[t][p][u][i];
      __syncthreads();
      for (int e = threadIdx.x; e < MT * 256; e += blockDim.x) {
        // e = (token, row16) with row16 fastest so stores run along n
        const int row16 = e & 15, tokl = e >> 4;
        const int u = tokl >> 4, c = tokl & 15;
        const int i = row16 & 3, gq = row16 >> 2;
        const int ln = gq * 16 + c;
        const int row = r0 + t * 16 + row16;
        if (row >= r1 || tokl >= a.M) continue;
        float v0 = 0.f, v1 = 0.f;
        for (int w = 0; w < nwaves; ++w) {
          v0 += buf[w * per_wave + ((0 * MT + u) * 4 + i) * 64 + ln];
          if (NP == 2) v1 += buf[w * per_wave + ((1 * MT + u) * 4 + i) * 64 + ln];
        }
        if (NORM) {
          v0 *= inv_rms[tokl];
          v1 *= inv_rms[tokl];
        }
        const long orow = a.omap.row(a.tok0 + tokl);
        if (EPI == EPI_STORE_F32) {
          static_cast<float*>(a.out)[orow * a.ld_out + row] = v0;
        } else if (EPI == EPI_STORE_ACT) {
          static_cast<T*>(a.out)[orow * a.ld_out + row] = Elem<T>::from_f32(v0);
        } else if (EPI == EPI_RESID) {
          float* x = static_cast<float*>(a.out) + orow * a.ld_out + row;
          const float nv = *x + v0;
          *x = nv;
          if (a.tap) a.tap[a.tmap.row(a.tok0 + tokl) * a.ld_tap + row] = nv;
        } else {  // SwiGLU: silu(gate) * up
          const float act = v0 / (1.0f + expf(-v0)) * v1;
          static_cast<T*>(a.out)[orow * a.ld_out + row] = Elem<T>::from_f32(act);
        }
      }
    }
  }
}

template <typename T, int MT>
hipError_t dispatch_epi(const GemmArgs& a, int epi, dim3 grid, dim3 block, hipStream_t st) {
  const bool norm = a.gain != nullptr;
#define DLITE_GS(E, NRM) \
  hipLaunchKernelGGL((gemm_stream_kernel<T, MT, E, NRM>), grid, block, 0, st, a)
  switch (epi) {
    case EPI_STORE_F32: if (norm) DLITE_GS(EPI_STORE_F32, true); else DLITE_GS(EPI_STORE_F32, false); break;
    case EPI_STORE_ACT: if (norm) DLITE_GS(EPI_STORE_ACT, true); else DLITE_GS(EPI_STORE_ACT, false); break;
    case EPI_RESID:     if (norm) DLITE_GS(EPI_RESID, true);     else DLITE_GS(EPI_RESID, false); break;
    case EPI_SWIGLU:    if (norm) DLITE_GS(EPI_SWIGLU, true);    else DLITE_GS(EPI_SWIGLU, false); break;
    default: return hipErrorInvalidValue;
  }
#undef DLITE_GS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a0, int epi, bool bf16, hipStream_t st) {
  const int KS = bf16 ? 32 : 16;
  const int nsteps = a0.K / KS;
  const int nwaves = nsteps < kMaxWaves ? nsteps : kMaxWaves;
  // rows per workgroup <= 16 * kMaxTiles; about 256 workgroups when possible
  long G = a0.N < 256 ? a0.N : 256;
  const long min_g = (a0.N + 16 * kMaxTiles - 1) / (16 * kMaxTiles);
  if (G < min_g) G = min_g;
  const dim3 grid(static_cast<unsigned>(G)), block(nwaves * 64);
  for (int t0 = 0; t0 < a0.M; t0 += 32) {
    GemmArgs a = a0;
    a.tok0 = a0.tok0 + t0;
    a.M = (a0.M - t0) < 32 ? (a0.M - t0) : 32;
    hipError_t e;
    if (bf16)
      e = a.M <= 16 ? dispatch_epi<uint16_t, 1>(a, epi, grid, block, st)
                    : dispatch_epi<uint16_t, 2>(a, epi, grid, block, st);
    else
      e = a.M <= 16 ? dispatch_epi<float, 1>(a, epi, grid, block, st)
                    : dispatch_epi<float, 2>(a, epi, grid, block, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dlite
