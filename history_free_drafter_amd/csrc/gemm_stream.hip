// Weight-streaming GEMM for few activation rows (M <= 32 per launch).
//
// In the small-batch draft step every linear map is read-bound: each weight
// byte meets at most 32 token rows.  Each weight row is therefore streamed
// once from HBM straight into registers (16 bytes per lane, non-temporal) and
// fed to 16x16 MFMA tiles; the other operand, the token block, is read from
// the (L2-resident) activation rows alongside.  Workgroup g owns logical output
// rows [g N / G, (g+1) N / G) in 16-row tiles; its waves split K.  Each wave
// walks (tile, k-chunk) units through a two-stage register pipeline, so the
// loads of the next unit are in flight while the current one is multiplied.
// Partial tiles are summed through LDS in a fixed order (deterministic).
//
// Inputs are pre-gained rows bf16(gamma * x) written by the producing kernel;
// when the map is preceded by an RMSNorm, each token's 1/rms is rebuilt from
// the producer's partial sums of squares and applied to the finished dot
// products (the factor is constant along k, so this is exact algebra).
#include "kernels.hpp"

namespace dlite {

namespace {

// residual tiles whose elements are fetched at kernel start
constexpr int kResTiles = 2;

template <typename T, int NP, int MT, int NS>
struct Stage {
  uint4 a[NP][NS];
  uint4 b[MT][NS];
};

// BL: the token rows are staged once in LDS (row stride K + 8 elements keeps
// 16-byte alignment and spreads banks) and every wave reads its fragments
// from there; otherwise fragments are loaded per unit from global memory.
template <typename T, int MT, int NS, int EPI, bool BL>
__global__ __launch_bounds__(512) void gemm_stream_kernel(StreamArgs sa) {
  // workgroups [0, g0) serve problem 0, the rest problem 1
  const int seg = static_cast<int>(blockIdx.x) < sa.g0 ? 0 : 1;
  const GemmArgs& a = sa.seg[seg];
  extern __shared__ __align__(16) unsigned char bsm[];
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int KS = PER * 4;                        // k per MFMA step
  constexpr int NP = (EPI == EPI_SWIGLU) ? 2 : 1;    // gate/up pairs

  // per tile: nwaves * NP * MT * 256 partials, nwaves <= 8
  __shared__ float red[2][8 * NP * MT * 256];
  __shared__ float inv_rms[32];
  __shared__ uint4 wbuf[8 * 16 * NS * 4];   // per wave: 16 rows x NS * 4 chunks

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;

  const long G = seg ? static_cast<long>(gridDim.x) - sa.g0 : sa.g0;
  const long g = static_cast<long>(blockIdx.x) - (seg ? sa.g0 : 0);
  const int r0 = static_cast<int>((g * a.N) / G);
  const int r1 = static_cast<int>(((g + 1) * a.N) / G);
  const int ntile = (r1 - r0 + 15) >> 4;

  const int nsteps = a.K / KS;
  const int s0 = (wave * nsteps) / nwaves, s1 = ((wave + 1) * nsteps) / nwaves;
  const int per_max = (nsteps + nwaves - 1) / nwaves;
  const int nchunk = (per_max + NS - 1) / NS;        // same for every wave
  const int nunit = ntile * nchunk;

  const T* W = static_cast<const T*>(a.W);
  const T* X = static_cast<const T*>(a.src);

  // token rows of this lane (invalid tokens read token 0's row, masked later)
  long srow[MT];
  bool tok_ok[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int tok = u * 16 + c16;
    tok_ok[u] = tok < a.M;
    srow[u] = a.smap.row(a.tok0 + (tok_ok[u] ? tok : 0));
  }

  const int ldb = a.K + 8;
  const T* Bs = reinterpret_cast<const T*>(bsm);
  auto stage_tokens = [&]() {
    // stage the M real token rows: 16-byte loads, all issued before the stores
    T* bw = reinterpret_cast<T*>(bsm);
    const int vk = a.K / PER, nv = a.M * vk;
    for (int base = threadIdx.x; base < nv; base += 8 * blockDim.x) {
      uint4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int idx = base + q * blockDim.x;
        idx = idx < nv ? idx : nv - 1;   // clamped: every load is issued unconditionally
        v[q] = *reinterpret_cast<const uint4*>(X + a.smap.row(a.tok0 + idx / vk) * a.ld_src +
                                               (idx % vk) * PER);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int idx = base + q * blockDim.x;
        if (idx < nv) *reinterpret_cast<uint4*>(bw + (idx / vk) * ldb + (idx % vk) * PER) = v[q];
      }
    }
    __syncthreads();
  };

  // chunk order rotated by workgroup so that workgroups read different
  // activation lines at any moment
  const int crot = static_cast<int>(g % nchunk);
  // Weight loads are row-contiguous: raw load i of a unit covers rows
  // i * RPI + lane / LPR of the 16-row tile, 16 bytes at chunk lane % LPR of
  // the unit's k range (NS k-steps); compute() turns them into MFMA fragments
  // through the wave's LDS buffer.
  constexpr int LPR = NS * 4;           // 16-byte chunks of one row per unit
  constexpr int RPI = 64 / LPR;         // rows per load instruction
  const int rt = lane / LPR, cl = lane % LPR;
  auto issue = [&](int p, Stage<T, NP, MT, NS>& st) {
    const int t = p / nchunk, c = (p % nchunk + crot) % nchunk;
    const int slast = s1 > 0 ? s1 - 1 : 0;
    {
      int s = s0 + c * NS + (cl >> 2);
      s = s < s1 ? s : slast;
      const long ka = static_cast<long>(s) * KS + (cl & 3) * PER;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        int row = r0 + t * 16 + i * RPI + rt;
        row = row < r1 ? row : r1 - 1;
#pragma unroll
        for (int q = 0; q < NP; ++q) st.a[q][i] = ld_stream(W + (row + q * a.pair_off) * a.ldw + ka);
      }
    }
    if (!BL) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        int s = s0 + c * NS + i;
        s = s < s1 ? s : slast;
        const long k = static_cast<long>(s) * KS + grp * PER;
#pragma unroll
        for (int u = 0; u < MT; ++u)
          if (tok_ok[u]) st.b[u][i] = *reinterpret_cast<const uint4*>(X + srow[u] * a.ld_src + k);
      }
    }
  };

  floatx4 acc[NP][MT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[q][u] = floatx4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  // the wave's 16 x LPR chunk buffer; chunk j of tile row r sits at
  // position j ^ r, so both the row-wise writes and the column-wise fragment
  // reads (16 rows, one chunk) hit distinct banks
  uint4* wb = wbuf + wave * (16 * LPR);
  auto compute = [&](int p, const Stage<T, NP, MT, NS>& st) {
    const int c = (p % nchunk + crot) % nchunk;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int rr = i * RPI + rt;
        wb[rr * LPR + (cl ^ rr)] = st.a[q][i];
      }
      uint4 fa[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) fa[i] = wb[c16 * LPR + ((i * 4 + grp) ^ c16)];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bool ok = s0 + c * NS + i < s1;
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          uint4 bv;
          if (BL) {
            const int s = s0 + c * NS + i;
            const int sc = s < s1 ? s : (s1 > 0 ? s1 - 1 : 0);
            const int tok = tok_ok[u] ? u * 16 + c16 : 0;
            bv = *reinterpret_cast<const uint4*>(Bs + tok * ldb + sc * KS + grp * PER);
          } else {
            bv = st.b[u][i];
          }
          bv = (ok && tok_ok[u]) ? bv : make_uint4(0, 0, 0, 0);
          acc[q][u] = mma_step(fa[i], bv, acc[q][u], T());
        }
      }
    }
  };

  // per-thread running sum of squares of the updated residual rows
  float ssq_loc = 0.f;
  float xres[kResTiles];
  const int per_wave = NP * MT * 256;

  auto finish_tile = [&](int t) {
    float* buf = red[t & 1];
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          buf[wave * per_wave + ((q * MT + u) * 4 + i) * 64 + lane] = acc[q][u][i];
    __syncthreads();
    const int e = threadIdx.x;   // one (token, row) element per thread
    if (e < MT * 256) {
      const int row16 = e & 15, tokl = e >> 4;
      const int u = tokl >> 4, cc = tokl & 15;
      const int i = row16 & 3, gq = row16 >> 2;
      const int ln = gq * 16 + cc;
      const int row = r0 + t * 16 + row16;
      if (row < r1 && tokl < a.M) {
        float v0 = 0.f, v1 = 0.f;
        for (int w = 0; w < nwaves; ++w) {
          v0 += buf[w * per_wave + ((0 * MT + u) * 4 + i) * 64 + ln];
          if (NP == 2) v1 += buf[w * per_wave + ((1 * MT + u) * 4 + i) * 64 + ln];
        }
        if (a.ssq) {
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
          float xo = 0.f;
#pragma unroll
          for (int tt = 0; tt < kResTiles; ++tt) xo = tt == t ? xres[tt] : xo;
          const float nv = (t < kResTiles ? xo : *x) + v0;
          *x = nv;
          ssq_loc += nv * nv;
          const T* ng = static_cast<const T*>(a.next_gain);
          static_cast<T*>(a.xb_out)[a.xmap.row(a.tok0 + tokl) * a.ld_xb + row] =
              Elem<T>::from_f32(Elem<T>::to_f32(ng[row]) * nv);
          if (a.tap) a.tap[a.tmap.row(a.tok0 + tokl) * a.ld_tap + row] = nv;
        } else {  // SwiGLU: silu(gate) * up
          const float act = v0 / (1.0f + expf(-v0)) * v1;
          static_cast<T*>(a.out)[orow * a.ld_out + row] = Elem<T>::from_f32(act);
        }
      }
    }
  };

  // 1/rms of each token from the producer's partial sums of squares
  auto token_scales = [&]() {
    if (!a.ssq) return;
    for (int tl = wave; tl < MT * 16; tl += nwaves) {
      float v = 0.f;
      if (tl < a.M) {
        const long prow = a.qmap.row(a.tok0 + tl);
        const int np = (prow % a.ssq_group) < a.ssq_split ? a.np_lo : a.np_hi;
        const float* sp = a.ssq + prow * kSsqParts;
        for (int j = lane; j < np; j += 64) v += sp[j];
      }
      v = wave_sum(v);
      if (lane == 0) inv_rms[tl] = 1.0f / sqrtf(v / static_cast<float>(a.norm_len) + a.eps);
    }
  };

  // two-stage pipeline over (tile, chunk) units
  // the first two stages of weights are requested before anything else (token
  // rows, residual elements, sums of squares), so all those round trips overlap
  Stage<T, NP, MT, NS> st0, st1;
  if (nunit > 0) issue(0, st0);
  if (nunit > 1) issue(1, st1);
  // the residual elements this thread updates, requested behind the weights
  if (EPI == EPI_RESID) {
    const int e = threadIdx.x;
#pragma unroll
    for (int t = 0; t < kResTiles; ++t) {
      xres[t] = 0.f;
      const int row = r0 + t * 16 + (e & 15), tokl = e >> 4;
      if (t < ntile && e < MT * 256 && row < r1 && tokl < a.M)
        xres[t] = static_cast<const float*>(a.out)[a.omap.row(a.tok0 + tokl) * a.ld_out + row];
    }
  }
  if (BL) stage_tokens();
  token_scales();
  for (int p = 0; p < nunit; p += 2) {
    if (p + 1 < nunit && p > 0) issue(p + 1, st1);
    compute(p, st0);
    if (p % nchunk == nchunk - 1) { finish_tile(p / nchunk); zero_acc(); }
    if (p + 1 < nunit) {
      if (p + 2 < nunit) issue(p + 2, st0);
      compute(p + 1, st1);
      if ((p + 1) % nchunk == nchunk - 1) { finish_tile((p + 1) / nchunk); zero_acc(); }
    }
  }

  if (EPI == EPI_RESID && a.ssq_out) {
    // combine the 16 rows of each token (consecutive lanes), one partial per workgroup
    float v = ssq_loc;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, kWave);
    const int e = threadIdx.x;
    if (e < MT * 256 && (e & 15) == 0 && (e >> 4) < a.M)
      a.ssq_out[a.omap.row(a.tok0 + (e >> 4)) * kSsqParts + g] = v;
  }
}

// Workgroups of one launch are meant to be resident together: a second round
// would repeat the whole load latency for a sliver of the rows.  When the
// wanted grid exceeds what the device holds at once, the rows are spread over
// fewer workgroups, shared between the two problems in proportion to their
// rows.  Residual epilogues keep their grid: it fixes how many partial sums of
// squares the next map reads (at most kSsqParts, one per workgroup, which fits
// on the device in one round).
void fit_resident(const void* fn, int threads, size_t sm, const StreamArgs& a, int& g0, int& g1) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, threads, sm) != hipSuccess || per < 1)
    return;
  const long cap = static_cast<long>(cus) * per;
  if (g0 + g1 <= cap) return;
  if (g1 == 0) {
    g0 = static_cast<int>(cap);
    return;
  }
  const long n0 = a.seg[0].N, n1 = a.seg[1].N;
  long c0 = cap * n0 / (n0 + n1);
  c0 = c0 < 1 ? 1 : (c0 > cap - 1 ? cap - 1 : c0);
  g0 = static_cast<int>(c0 < g0 ? c0 : g0);
  g1 = static_cast<int>(cap - c0 < g1 ? cap - c0 : g1);
}

template <typename T, int MT, int NS0, bool BL>
hipError_t dispatch_epi(StreamArgs a, int epi, int g1, dim3 block, size_t sm, hipStream_t st) {
  // register budget: two token tiles without LDS staging keep 4-step stages,
  // and so does the gate/up pair unless its token rows sit in LDS with one tile
  constexpr int NS = (!BL && MT == 2) ? 4 : NS0;
  constexpr int NSG = ((MT == 2 || !BL) && NS == 8) ? 4 : NS;
  const void* fn = nullptr;
  switch (epi) {
    case EPI_STORE_F32: fn = reinterpret_cast<const void*>(&gemm_stream_kernel<T, MT, NS, EPI_STORE_F32, BL>); break;
    case EPI_STORE_ACT: fn = reinterpret_cast<const void*>(&gemm_stream_kernel<T, MT, NS, EPI_STORE_ACT, BL>); break;
    case EPI_RESID:     fn = reinterpret_cast<const void*>(&gemm_stream_kernel<T, MT, NS, EPI_RESID, BL>); break;
    case EPI_SWIGLU:    fn = reinterpret_cast<const void*>(&gemm_stream_kernel<T, MT, NSG, EPI_SWIGLU, BL>); break;
    default: return hipErrorInvalidValue;
  }
  if (BL) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
    if (e != hipSuccess) return e;
  }
  int g0 = a.g0;
  if (epi != EPI_RESID) fit_resident(fn, static_cast<int>(block.x), sm, a, g0, g1);
  a.g0 = g0;
  const dim3 grid(static_cast<unsigned>(g0 + g1));
  switch (epi) {
    case EPI_STORE_F32: hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NS, EPI_STORE_F32, BL>), grid, block, sm, st, a); break;
    case EPI_STORE_ACT: hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NS, EPI_STORE_ACT, BL>), grid, block, sm, st, a); break;
    case EPI_RESID:     hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NS, EPI_RESID, BL>), grid, block, sm, st, a); break;
    case EPI_SWIGLU:    hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NSG, EPI_SWIGLU, BL>), grid, block, sm, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int MT, int NS>
hipError_t dispatch_bl(const StreamArgs& a, int epi, int g1, dim3 block, hipStream_t st) {
  // stage the token rows in LDS when they fit beside the reduction buffers
  const size_t es = sizeof(T);
  const size_t red = 2ull * 8 * (epi == EPI_SWIGLU ? 2 : 1) * MT * 256 * 4 +
                     8ull * 16 * NS * 4 * 16;   // + weight transposition buffers
  int mmax = a.seg[0].M;
  if (g1 > 0 && a.seg[1].M > mmax) mmax = a.seg[1].M;
  const size_t sm = static_cast<size_t>(mmax) * (a.seg[0].K + 8) * es;
  // staging pays off only when a workgroup owns at least one full tile of
  // weight rows; with fewer, the token loads are better overlapped with them
  const bool full_tiles = a.seg[0].N >= 16 * static_cast<int>(a.g0);
  if (full_tiles && sm + red + 1024 <= 160 * 1024)
    return dispatch_epi<T, MT, NS, true>(a, epi, g1, block, sm, st);
  return dispatch_epi<T, MT, NS, false>(a, epi, g1, block, 0, st);
}

// Waves per workgroup: the first count in {8, 4, 2, 1} that splits the k-steps
// into equal whole chunks, else 8 with a masked tail.
int pick_waves(int nsteps, int ns) {
  const int cand[] = {8, 4, 2, 1};
  for (int w : cand)
    if (nsteps % w == 0 && (nsteps / w) % ns == 0) return w;
  return 8;
}

}  // namespace

int gemm_resid_parts(const GemmArgs& a, bool bf16) {
  if (gemm_tiled(a, bf16)) return (a.N + 127) / 128;
  return a.N < kSsqParts ? a.N : kSsqParts;
}

namespace {

// One launch for up to two problems with the same K and epilogue and at most
// 32 tokens each; problem 1's workgroups follow problem 0's.
hipError_t launch_stream(const GemmArgs* segs, int nseg, int epi, bool bf16, hipStream_t st) {
  const int KS = bf16 ? 32 : 16;
  const int nsteps = segs[0].K / KS;
  // pipeline depth: 8 k-steps per stage when the split allows it, else 4
  int ns = 8;
  int nw8 = pick_waves(nsteps, 8);
  if (!(nsteps % nw8 == 0 && (nsteps / nw8) % 8 == 0)) ns = 4;
  StreamArgs sa{};
  sa.seg[0] = segs[0];
  sa.seg[1] = nseg > 1 ? segs[1] : segs[0];
  const int g0 = segs[0].N < kSsqParts ? segs[0].N : kSsqParts;
  const int g1 = nseg > 1 ? (segs[1].N < kSsqParts ? segs[1].N : kSsqParts) : 0;
  sa.g0 = g0;
  int mmax = segs[0].M;
  if (nseg > 1 && segs[1].M > mmax) mmax = segs[1].M;
  // one epilogue element per thread: at least 4 waves per 16-token tile
  int nwaves = pick_waves(nsteps, ns);
  const int minw = mmax <= 16 ? 4 : 8;
  if (nwaves < minw) nwaves = minw;
  const dim3 block(nwaves * 64);
  const bool one = mmax <= 16;
  if (bf16) {
    if (ns == 8) return one ? dispatch_bl<uint16_t, 1, 8>(sa, epi, g1, block, st)
                            : dispatch_bl<uint16_t, 2, 8>(sa, epi, g1, block, st);
    return one ? dispatch_bl<uint16_t, 1, 4>(sa, epi, g1, block, st)
               : dispatch_bl<uint16_t, 2, 4>(sa, epi, g1, block, st);
  }
  if (ns == 8) return one ? dispatch_bl<float, 1, 8>(sa, epi, g1, block, st)
                          : dispatch_bl<float, 2, 8>(sa, epi, g1, block, st);
  return one ? dispatch_bl<float, 1, 4>(sa, epi, g1, block, st)
             : dispatch_bl<float, 2, 4>(sa, epi, g1, block, st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a0, int epi, bool bf16, float* part, hipStream_t st) {
  if (gemm_tiled(a0, bf16)) return launch_gemm_tiled(&a0, 1, epi, part, st);
  if (epi == EPI_ARGMAX) return hipErrorInvalidValue;
  for (int t0 = 0; t0 < a0.M; t0 += 32) {
    GemmArgs a = a0;
    a.tok0 = a0.tok0 + t0;
    a.M = (a0.M - t0) < 32 ? (a0.M - t0) : 32;
    const hipError_t e = launch_stream(&a, 1, epi, bf16, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, int epi, bool bf16, float* part,
                            hipStream_t st) {
  if (a.K != b.K) return hipErrorInvalidValue;
  if (gemm_tiled(a, bf16) && gemm_tiled(b, bf16)) {
    const GemmArgs segs[2] = {a, b};
    return launch_gemm_tiled(segs, 2, epi, part, st);
  }
  if (!gemm_tiled(a, bf16) && !gemm_tiled(b, bf16) && a.M <= 32 && b.M <= 32 && epi != EPI_ARGMAX) {
    const GemmArgs segs[2] = {a, b};
    return launch_stream(segs, 2, epi, bf16, st);
  }
  const hipError_t e = launch_gemm(a, epi, bf16, part, st);
  if (e != hipSuccess) return e;
  return launch_gemm(b, epi, bf16, part, st);
}

}  // namespace dlite
