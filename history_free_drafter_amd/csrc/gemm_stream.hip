// Weight-streaming GEMM for few activation rows (M <= 32 per launch).
//
// In the small-batch draft step every linear map is read-bound: each weight
// byte meets at most 32 token rows, so the kernel is built around streaming
// the weight matrix from HBM exactly once while touching the token rows as
// little as possible.
//
// Work split.  Workgroup = (row block of R output rows, k slice).  Its eight
// waves form a WR x WK grid: wave (wr, wk) owns the 16-row tiles wr, wr + WR,
// ... of the block and the k sub-range wk of the slice.  Because a wave's k
// range never changes, its token fragments (16 bytes per lane per k-step and
// token tile) are loaded once into registers and reused for every tile; only
// weights move in the main loop.
//
// Weight loads are row-contiguous (each load instruction covers whole
// 64..512-byte runs of a few rows, non-temporal) and turned into MFMA
// fragments through a small per-wave LDS buffer; a two-stage register
// pipeline keeps the next loads in flight while the current ones are
// multiplied (16x16x32 bf16 MFMA; fp32 storage uses 16x16x4 steps).
//
// Reduction.  Finished tiles are parked in LDS; the WK waves of a tile are
// added in wave order.  When K is split over workgroups, each writes its
// [rows x tokens] partial with device-scope stores and counts itself in on the
// row block's arrival counter; the workgroup that arrives last adds all slices
// in slice order (so the sum does not depend on which workgroup finishes last)
// and applies the epilogue.  Nothing waits on another workgroup.
//
// Inputs are pre-gained rows bf16(gamma * x) written by the producing kernel;
// when the map is preceded by an RMSNorm, each token's 1/rms is rebuilt from
// the producer's partial sums of squares and applied to the finished dot
// products (the factor is constant along k, so this is exact algebra).
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kWaves = 8;
constexpr int kRes = 2;                   // residual elements prefetched per thread
constexpr int kPolicyDev = 16;            // buffer cache policy: device scope (sc1)
constexpr int kRsrcWord3 = 0x00020000;    // raw 32-bit buffer resource

struct Layout {
  int R;      // rows per workgroup (multiple of 16)
  int nrb;    // row blocks
  int nks;    // k slices (workgroups per row block)
  int g0;     // first workgroup of the problem
};

struct SArgs {
  GemmArgs seg[2];
  Layout lay[2];
  int nseg;
  int WR, WK;             // wave grid
  float* part[2];         // k-split partials [nks][nrb][NP][M][R] per problem
  unsigned* cnt[2];       // arrival counters [nrb] per problem (self-resetting)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const float* p, long floats) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, static_cast<int>(floats * 4), kRsrcWord3);
}

template <typename T, int MT, int KW, int NS, int EPI>
__global__ __launch_bounds__(kWaves * 64) void gemm_stream_kernel(SArgs sa) {
  constexpr int NP = (EPI == EPI_SWIGLU) ? 2 : 1;    // gate/up pairs
  constexpr int NG = KW / NS;                        // k groups per tile
  static_assert(NG % 2 == 0, "two stage buffers alternate over the k groups of a tile");
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int KS = PER * 4;                        // k per MFMA step
  constexpr int LPR = NS * 4;                        // 16-byte chunks of one row per unit
  constexpr int RPI = 64 / LPR;                      // rows per load instruction
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float inv_rms[32];
  __shared__ int last;

  const int seg = (sa.nseg > 1 && static_cast<int>(blockIdx.x) >= sa.lay[1].g0) ? 1 : 0;
  const GemmArgs& a = sa.seg[seg];
  const Layout ly = sa.lay[seg];
  const int wg = static_cast<int>(blockIdx.x) - ly.g0;
  const int rb = wg / ly.nks, ks = wg % ly.nks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int WR = sa.WR, WK = sa.WK;
  const int wr = wave % WR, wk = wave / WR;
  const int M = a.M;

  const int row0 = rb * ly.R;
  const int nrow = (a.N - row0) < ly.R ? (a.N - row0) : ly.R;   // multiple of 16
  const int ntw = (nrow / 16 - wr + WR - 1) / WR;               // tiles of this wave

  // k steps: slice ks of the problem, sub-range wk of the slice (<= KW steps)
  const int nst = a.K / KS;
  const int k0 = static_cast<int>(static_cast<long>(ks) * nst / ly.nks);
  const int k1 = static_cast<int>(static_cast<long>(ks + 1) * nst / ly.nks);
  const int s0 = k0 + wk * (k1 - k0) / WK, s1 = k0 + (wk + 1) * (k1 - k0) / WK;
  const int slast = s1 > s0 ? s1 - 1 : (s0 < nst ? s0 : nst - 1);   // in-range clamp

  // LDS: per-wave weight transposition buffers, then parked tiles [WK][NP][M][R]
  uint4* wb = reinterpret_cast<uint4*>(smem) + wave * (16 * LPR);
  float* Y = reinterpret_cast<float*>(smem + static_cast<size_t>(nwaves) * 16 * LPR * 16);
  const int R = ly.R;

  const T* W = static_cast<const T*>(a.W);
  const T* X = static_cast<const T*>(a.src);

  // ---- token fragments of this wave's k range, kept in registers
  uint4 tf[MT][KW];
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int tok = u * 16 + c16;
    const bool ok = tok < M;
    const long srow = a.smap.row(a.tok0 + (ok ? tok : 0));
#pragma unroll
    for (int s = 0; s < KW; ++s) {
      const bool sv = s0 + s < s1;
      const int ss = sv ? s0 + s : slast;
      const uint4 v = *reinterpret_cast<const uint4*>(X + srow * a.ld_src + static_cast<long>(ss) * KS + grp * PER);
      tf[u][s] = (ok && sv) ? v : make_uint4(0, 0, 0, 0);
    }
  }

  // ---- weight units: (tile ti of this wave, k group g)
  const int rt = lane / LPR, cl = lane % LPR;
  auto issue = [&](int ti, int g, uint4 (&st)[NP][NS]) {
    const int rowt = row0 + (wr + ti * WR) * 16;
    int s = s0 + g * NS + (cl >> 2);
    s = s < s1 ? s : slast;
    const long ka = static_cast<long>(s) * KS + (cl & 3) * PER;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const long row = rowt + i * RPI + rt;
#pragma unroll
      for (int q = 0; q < NP; ++q) st[q][i] = ld_stream(W + (row + q * a.pair_off) * a.ldw + ka);
    }
  };

  floatx4 acc[NP][MT];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[q][u] = floatx4{0.f, 0.f, 0.f, 0.f};

  // chunk j of tile row rr sits at position j ^ (rr mod LPR): the row-wise
  // writes and the column-wise fragment reads both spread over the banks
  auto compute = [&](int g, const uint4 (&st)[NP][NS]) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int rr = i * RPI + rt;
        wb[rr * LPR + (cl ^ (rr & (LPR - 1)))] = st[q][i];
      }
      uint4 fa[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) fa[i] = wb[c16 * LPR + ((i * 4 + grp) ^ (c16 & (LPR - 1)))];
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[q][u] = mma_step(fa[i], tf[u][g * NS + i], acc[q][u], T());
    }
  };

  // park a finished tile: lane holds rows 4 grp .. 4 grp + 3 of token c16
  auto park = [&](int ti) {
    const int t = wr + ti * WR;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const int tok = u * 16 + c16;
        if (tok < M)
          *reinterpret_cast<floatx4*>(Y + ((static_cast<long>(wk) * NP + q) * M + tok) * R + t * 16 + grp * 4) =
              acc[q][u];
        acc[q][u] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
  };

  uint4 st0[NP][NS], st1[NP][NS];
  if (ntw > 0) {
    issue(0, 0, st0);
    issue(0, 1, st1);
  }

  // behind the first weight loads: each token's 1/rms, and the residual
  // elements the epilogue updates with their next-norm gains (kRes per
  // thread), so that their round trips overlap the stream
  if (a.ssq) {
    for (int tl = wave; tl < M; tl += nwaves) {
      const long prow = a.qmap.row(a.tok0 + tl);
      const int np = (prow % a.ssq_group) < a.ssq_split ? a.np_lo : a.np_hi;
      const float* sp = a.ssq + prow * kSsqParts;
      float v = 0.f;
      for (int j = lane; j < np; j += 64) v += sp[j];
      v = wave_sum(v);
      if (lane == 0) inv_rms[tl] = 1.0f / sqrtf(v / static_cast<float>(a.norm_len) + a.eps);
    }
  }
  float xres[kRes], gres[kRes];
#pragma unroll
  for (int j = 0; j < kRes; ++j) {
    xres[j] = 0.f;
    gres[j] = 0.f;
    const int e = threadIdx.x + j * blockDim.x;
    if (EPI == EPI_RESID && e < M * nrow) {
      const int tok = e / nrow, row = e % nrow;
      xres[j] = static_cast<const float*>(a.out)[a.omap.row(a.tok0 + tok) * a.ld_out + row0 + row];
      gres[j] = Elem<T>::to_f32(static_cast<const T*>(a.next_gain)[row0 + row]);
    }
  }
  for (int ti = 0; ti < ntw; ++ti) {
#pragma unroll
    for (int g = 0; g < NG; g += 2) {
      compute(g, st0);
      if (g + 2 < NG) issue(ti, g + 2, st0);
      else if (ti + 1 < ntw) issue(ti + 1, 0, st0);
      compute(g + 1, st1);
      if (g + 3 < NG) issue(ti, g + 3, st1);
      else if (ti + 1 < ntw) issue(ti + 1, 1, st1);
    }
    park(ti);
  }
  __syncthreads();

  // ---- add the WK k sub-ranges (wave order) into slot 0
  const int nel = NP * M * R;      // [NP][M][R], rows past nrow unused
  if (WK > 1) {
    for (int e = threadIdx.x; e < nel; e += blockDim.x) {
      float v = Y[e];
      for (int w = 1; w < WK; ++w) v += Y[static_cast<long>(w) * nel + e];
      Y[e] = v;
    }
    __syncthreads();
  }

  // ---- k split over workgroups: publish, count in, the last one adds all
  if (ly.nks > 1) {
    float* part = sa.part[seg];
    const long blk = static_cast<long>(nel);
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(part, static_cast<long>(ly.nks) * ly.nrb * blk);
    const long mine = (static_cast<long>(ks) * ly.nrb + rb) * blk;
    for (int e4 = threadIdx.x; e4 < nel / 4; e4 += blockDim.x) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(Y + e4 * 4);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                             static_cast<int>((mine + e4 * 4) * 4), 0, kPolicyDev);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's partial stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* c = sa.cnt[seg] + rb;
      const unsigned prev = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = prev + 1 == static_cast<unsigned>(ly.nks);
      // the last arrival resets the counter for the next launch on the stream
      if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    for (int e4 = threadIdx.x; e4 < nel / 4; e4 += blockDim.x) {
      // up to kBatch slices requested at once, then added in slice order
      constexpr int kBatch = 8;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < ly.nks; k0 += kBatch) {
        floatx4 pv[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int k = k0 + b < ly.nks ? k0 + b : ly.nks - 1;
          const long o = (static_cast<long>(k) * ly.nrb + rb) * blk + e4 * 4;
          pv[b] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(o * 4), 0, kPolicyDev));
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (k0 + b < ly.nks) v += pv[b];
      }
      *reinterpret_cast<floatx4*>(Y + e4 * 4) = v;
    }
    __syncthreads();
  }

  // ---- epilogue on Y[NP][M][R] (inv_rms is published by the barriers above)
  for (int j = 0; j * static_cast<int>(blockDim.x) < M * nrow; ++j) {
    const int e = threadIdx.x + j * blockDim.x;
    if (e >= M * nrow) break;
    const int tok = e / nrow, row = e % nrow;
    const float sc = a.ssq ? inv_rms[tok] : 1.f;
    const float v0 = Y[tok * R + row] * sc;
    const long orow = a.omap.row(a.tok0 + tok);
    const int grow = row0 + row;
    if (EPI == EPI_STORE_F32) {
      static_cast<float*>(a.out)[orow * a.ld_out + grow] = v0;
    } else if (EPI == EPI_STORE_ACT) {
      static_cast<T*>(a.out)[orow * a.ld_out + grow] = Elem<T>::from_f32(v0);
    } else if (EPI == EPI_RESID) {
      float* x = static_cast<float*>(a.out) + orow * a.ld_out + grow;
      float xo = 0.f, go = 0.f;
#pragma unroll
      for (int jj = 0; jj < kRes; ++jj) {
        xo = jj == j ? xres[jj] : xo;
        go = jj == j ? gres[jj] : go;
      }
      const float nv = (j < kRes ? xo : *x) + v0;
      *x = nv;
      const float gain = j < kRes ? go : Elem<T>::to_f32(static_cast<const T*>(a.next_gain)[grow]);
      static_cast<T*>(a.xb_out)[a.xmap.row(a.tok0 + tok) * a.ld_xb + grow] = Elem<T>::from_f32(gain * nv);
      if (a.tap) a.tap[a.tmap.row(a.tok0 + tok) * a.ld_tap + grow] = nv;
      Y[tok * R + row] = nv * nv;
    } else {  // SwiGLU: silu(gate) * up
      const float v1 = Y[(M + tok) * R + row] * sc;
      const float act = v0 / (1.0f + expf(-v0)) * v1;
      static_cast<T*>(a.out)[orow * a.ld_out + grow] = Elem<T>::from_f32(act);
    }
  }
  if (EPI == EPI_RESID && a.ssq_out) {
    // one partial sum of squares per token and row block, fixed order
    __syncthreads();
    for (int tok = wave; tok < M; tok += nwaves) {
      float v = 0.f;
      for (int row = lane; row < nrow; row += 64) v += Y[tok * R + row];
      v = wave_sum(v);
      if (lane == 0) a.ssq_out[a.omap.row(a.tok0 + tok) * kSsqParts + rb] = v;
    }
  }
}

// ------------------------------------------------------------ launch plan --

struct LaunchPlan {
  int MT, KW, NS, WR, WK;
  Layout lay[2];
  int G;
};

int ceil_div(long a, long b) { return static_cast<int>((a + b - 1) / b); }

// Work split: every wave streams all tiles of its workgroup's row block over
// one eighth of the workgroup's k slice (WR = 1, WK = 8), so a wave holds the
// token fragments of at most KW = 16 k-steps.  K is split over workgroups only
// when K exceeds 8 x 16 steps, or to give tiny launches (fewer than 128
// workgroups) more parallelism.  Row blocks then grow, largest problem first,
// until the launch fits one resident round of at most 256 workgroups.
LaunchPlan plan_launch(const GemmArgs* segs, int nseg, int epi, bool bf16) {
  LaunchPlan p{};
  const int KS = bf16 ? 32 : 16;
  const int nst = segs[0].K / KS;
  int mmax = 0, ttot = 0, tiles[2] = {0, 0};
  for (int s = 0; s < nseg; ++s) {
    mmax = segs[s].M > mmax ? segs[s].M : mmax;
    tiles[s] = segs[s].N / 16;
    ttot += tiles[s];
  }
  p.MT = mmax > 16 ? 2 : 1;
  p.WR = 1;
  p.WK = kWaves;
  p.KW = 16;
  int nks = ceil_div(nst, kWaves * p.KW);
  while (p.KW > 4 && static_cast<long>(ttot) * nks < 128 && ceil_div(nst, kWaves * (p.KW / 2)) > nks) {
    p.KW /= 2;
    nks = ceil_div(nst, kWaves * p.KW);
  }
  int tpb[2] = {1, 1};
  auto blocks = [&](int s) { return ceil_div(tiles[s], tpb[s]); };
  for (;;) {
    long g = 0;
    int big = 0;
    for (int s = 0; s < nseg; ++s) {
      g += static_cast<long>(blocks(s)) * nks;
      if (blocks(s) > blocks(big)) big = s;
    }
    if (g <= 256 || blocks(big) <= 1) break;
    ++tpb[big];
  }
  int g = 0;
  for (int s = 0; s < nseg; ++s) {
    Layout& l = p.lay[s];
    l.R = 16 * tpb[s];
    l.nrb = ceil_div(segs[s].N, l.R);
    l.nks = nks;
    l.g0 = g;
    g += l.nrb * l.nks;
  }
  p.G = g;
  if (p.KW == 16) p.NS = (epi == EPI_SWIGLU || p.MT == 2) ? 4 : 8;
  else p.NS = p.KW / 2;
  return p;
}

size_t plan_lds(const LaunchPlan& p, const GemmArgs* segs, int nseg, int epi) {
  const int NP = epi == EPI_SWIGLU ? 2 : 1;
  size_t y = 0;
  for (int s = 0; s < nseg; ++s) {
    const size_t v = static_cast<size_t>(p.WK) * NP * segs[s].M * p.lay[s].R * sizeof(float);
    y = v > y ? v : y;
  }
  return static_cast<size_t>(kWaves) * 16 * p.NS * 4 * 16 + y;
}

size_t plan_scratch_floats(const LaunchPlan& p, const GemmArgs* segs, int nseg, int epi) {
  const int NP = epi == EPI_SWIGLU ? 2 : 1;
  size_t n = 0;
  for (int s = 0; s < nseg; ++s) {
    const Layout& l = p.lay[s];
    if (l.nks > 1) n += static_cast<size_t>(l.nks) * l.nrb * NP * segs[s].M * l.R;
  }
  return n;
}

template <typename T, int MT, int KW, int NS, int EPI>
hipError_t launch_variant(const SArgs& sa, int G, size_t sm, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&gemm_stream_kernel<T, MT, KW, NS, EPI>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
  if (e != hipSuccess) return e;
  launch_k((gemm_stream_kernel<T, MT, KW, NS, EPI>), dim3(G), dim3(kWaves * 64), sm, st, sa);
  return hipGetLastError();
}

template <typename T, int MT, int EPI>
hipError_t launch_kw(const SArgs& sa, const LaunchPlan& p, size_t sm, hipStream_t st) {
  if (p.KW == 4) return launch_variant<T, MT, 4, 2, EPI>(sa, p.G, sm, st);
  if (p.KW == 8) return launch_variant<T, MT, 8, 4, EPI>(sa, p.G, sm, st);
  if (p.KW == 16 && p.NS == 4) return launch_variant<T, MT, 16, 4, EPI>(sa, p.G, sm, st);
  if constexpr (MT == 1 && EPI != EPI_SWIGLU) {
    if (p.KW == 16 && p.NS == 8) return launch_variant<T, MT, 16, 8, EPI>(sa, p.G, sm, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int MT>
hipError_t launch_epi(const SArgs& sa, const LaunchPlan& p, int epi, size_t sm, hipStream_t st) {
  switch (epi) {
    case EPI_STORE_F32: return launch_kw<T, MT, EPI_STORE_F32>(sa, p, sm, st);
    case EPI_STORE_ACT: return launch_kw<T, MT, EPI_STORE_ACT>(sa, p, sm, st);
    case EPI_RESID: return launch_kw<T, MT, EPI_RESID>(sa, p, sm, st);
    case EPI_SWIGLU: return launch_kw<T, MT, EPI_SWIGLU>(sa, p, sm, st);
    default: return hipErrorInvalidValue;
  }
}

// One launch for up to two problems with the same K and epilogue and at most
// 32 tokens each; problem 1's workgroups follow problem 0's.
hipError_t launch_stream(const GemmArgs* segs, int nseg, int epi, bool bf16, const StreamScratch& ss,
                         hipStream_t st) {
  const LaunchPlan p = plan_launch(segs, nseg, epi, bf16);
  if (p.G == 0) return hipSuccess;
  SArgs sa{};
  sa.nseg = nseg;
  sa.WR = p.WR;
  sa.WK = p.WK;
  size_t off = 0;
  for (int s = 0; s < nseg; ++s) {
    sa.seg[s] = segs[s];
    sa.lay[s] = p.lay[s];
    if (p.lay[s].nks > 1) {
      if (p.lay[s].nrb > kStreamRowBlocks) return hipErrorInvalidValue;
      sa.part[s] = ss.part + off;
      sa.cnt[s] = ss.counters + s * kStreamRowBlocks;
      off += static_cast<size_t>(p.lay[s].nks) * p.lay[s].nrb * (epi == EPI_SWIGLU ? 2 : 1) * segs[s].M * p.lay[s].R;
    }
  }
  if (off > ss.part_floats) return hipErrorInvalidValue;
  const size_t sm = plan_lds(p, segs, nseg, epi);
  if (sm > 160 * 1024) return hipErrorInvalidValue;
  if (bf16) return p.MT == 1 ? launch_epi<uint16_t, 1>(sa, p, epi, sm, st) : launch_epi<uint16_t, 2>(sa, p, epi, sm, st);
  return p.MT == 1 ? launch_epi<float, 1>(sa, p, epi, sm, st) : launch_epi<float, 2>(sa, p, epi, sm, st);
}

}  // namespace

int gemm_resid_parts(const GemmArgs& a, bool bf16) {
  if (gemm_tiled(a, bf16)) return (a.N + 127) / 128;
  GemmArgs c = a;
  c.M = a.M < 32 ? a.M : 32;
  return plan_launch(&c, 1, EPI_RESID, bf16).lay[0].nrb;
}

size_t gemm_stream_scratch(int M0, int M1, int N0, int N1, int K, int epi, bool bf16) {
  GemmArgs s[2]{};
  s[0].M = M0; s[0].N = N0; s[0].K = K;
  s[1].M = M1; s[1].N = N1; s[1].K = K;
  const int nseg = M1 > 0 ? 2 : 1;
  return plan_scratch_floats(plan_launch(s, nseg, epi, bf16), s, nseg, epi) * sizeof(float);
}

hipError_t launch_gemm(const GemmArgs& a0, int epi, bool bf16, const StreamScratch& ss, hipStream_t st) {
  if (gemm_tiled(a0, bf16)) return launch_gemm_tiled(&a0, 1, epi, ss.tile_part, st);
  if (epi == EPI_ARGMAX) return hipErrorInvalidValue;
  for (int t0 = 0; t0 < a0.M; t0 += 32) {
    GemmArgs a = a0;
    a.tok0 = a0.tok0 + t0;
    a.M = (a0.M - t0) < 32 ? (a0.M - t0) : 32;
    const hipError_t e = launch_stream(&a, 1, epi, bf16, ss, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, int epi, bool bf16, const StreamScratch& ss,
                            hipStream_t st) {
  if (a.K != b.K) return hipErrorInvalidValue;
  if (gemm_tiled(a, bf16) && gemm_tiled(b, bf16)) {
    const GemmArgs segs[2] = {a, b};
    return launch_gemm_tiled(segs, 2, epi, ss.tile_part, st);
  }
  if (!gemm_tiled(a, bf16) && !gemm_tiled(b, bf16) && a.M <= 32 && b.M <= 32 && epi != EPI_ARGMAX) {
    const GemmArgs segs[2] = {a, b};
    return launch_stream(segs, 2, epi, bf16, ss, st);
  }
  const hipError_t e = launch_gemm(a, epi, bf16, ss, st);
  if (e != hipSuccess) return e;
  return launch_gemm(b, epi, bf16, ss, st);
}

}  // namespace dlite
