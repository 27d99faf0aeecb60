// Vocabulary projection of the sequential-head states fused with the greedy
// choice: logits_k = W_lm s_k for all B*K states at once (the projection is
// applied once, after the head), argmax with ties to the lowest index.
//
// Pass 1: workgroup g streams vocabulary rows [g V / G, (g+1) V / G) through
// 16x16 MFMA tiles against the token block held in registers and keeps a
// running (max, index) per token; the full logits are never written (unless
// the logits tap is requested).  Pass 2 reduces the G partials of every token
// in a fixed order, so the result does not depend on scheduling: done by the
// last workgroup to finish pass 1, or by a second small kernel after the
// tiled path.
#include "scan_team.hpp"

namespace dlite {

namespace {

constexpr int kWaves = 8;
constexpr int kMaxSteps = 16;   // r <= 512 (bf16) / 256 (fp32)

// Pass 2 for one token (one wave), after each lane has folded its strided
// share of the G partials: a butterfly, then the candidate (ties resolve to
// the lowest index throughout).
__device__ __forceinline__ void finish_token(const LmArgs& a, int tok, int lane, float v, int i) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
  if (lane == 0) {
    const int gt = a.tok0 + tok;
    const long orow = a.omap.row(gt);
    const int b = static_cast<int>(orow / a.K);
    const int anchor = a.anchors[b];
    bool ok = anchor >= 0 && anchor < a.V;
    if (a.pos) {
      const int pb = a.pos[b];
      ok = ok && pb >= 0 && pb < a.pos_n;
    }
    a.cand[orow] = ok ? i : -1;
    if (a.max_logit) a.max_logit[orow] = ok ? v : 0.f;
    if (a.raw) a.raw[gt] = i;
  }
}

// Pass 2 as its own launch (after the tiled path): the kernel boundary orders
// it after every partial.
__global__ __launch_bounds__(256) void lmhead_reduce_kernel(LmArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.M) return;
  const long G = a.G;
  const long base = static_cast<long>(a.tok0 + tok) * G;
  float v = -INFINITY;
  int i = 0x7fffffff;
  for (long j = lane; j < G; j += 64) {
    const float pv = a.part_max[base + j];
    const int pi = a.part_idx[base + j];
    if (better(pv, pi, v, i)) { v = pv; i = pi; }
  }
  finish_token(a, tok, lane, v, i);
}

// Pass 2 inside the streaming kernels: every workgroup stores its partials
// with device-coherent (agent-scope atomic) stores, waits for them to
// complete and counts itself in; the workgroup that arrives last reads all
// partials back with device-coherent loads and reduces them, one wave per
// token.  Only the partials and the counter cross workgroups, so no cache
// write-back or invalidate is needed.  Nothing waits on another workgroup,
// so nothing depends on which workgroups are resident; the counter is
// cleared by the step's first kernel.
__device__ __forceinline__ void publish_partial(const LmArgs& a, long o, float v, int i) {
  __hip_atomic_store(a.part_max + o, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(a.part_idx + o, i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival is counted in two levels so that no counter takes more than about
// 32 atomics: per XCD of the workgroup (blockIdx % 8; n_xcd = workgroups of
// this launch that publish on that XCD), then the last one of each XCD counts
// in globally (n_busy = XCDs with at least one such workgroup).
__device__ __forceinline__ void reduce_if_last(const LmArgs& a, long G, int* last, int n_xcd, int n_busy) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    // the last arrival at each level puts its counter back to zero for the
    // next launch on the stream (a step may run several 32-token launches)
    unsigned* cx = a.xcd_counters + static_cast<int>(blockIdx.x & 7) * 16;
    const unsigned px = __hip_atomic_fetch_add(cx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool lg = false;
    if (px + 1 == static_cast<unsigned>(n_xcd)) {
      __hip_atomic_store(cx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned* cnt = a.counters + CNT_LM_DONE;
      const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lg = prev + 1 == static_cast<unsigned>(n_busy);
      if (lg) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *last = lg;
  }
  __syncthreads();
  if (!*last) return;
  const int lane = threadIdx.x & 63;
  for (int tok = threadIdx.x >> 6; tok < a.M; tok += static_cast<int>(blockDim.x >> 6)) {
    const long base = static_cast<long>(a.tok0 + tok) * G;
    float v = -INFINITY;
    int i = 0x7fffffff;
    // kBatch partials per lane requested at once, then folded in index order
    constexpr int kBatch = 8;
    for (long j0 = lane; j0 < G; j0 += 64 * kBatch) {
      float pv[kBatch];
      int pi[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const long j = j0 + 64 * q < G ? j0 + 64 * q : j0;
        pv[q] = __hip_atomic_load(a.part_max + base + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pi[q] = __hip_atomic_load(a.part_idx + base + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (better(pv[q], pi[q], v, i)) { v = pv[q]; i = pi[q]; }
    }
    finish_token(a, tok, lane, v, i);
  }
}

template <typename T, int MT>
__global__ __launch_bounds__(kWaves * 64) void lmhead_kernel(LmArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int KS = PER * 4;
  __shared__ float sv[kWaves][32];
  __shared__ int si[kWaves][32];
  __shared__ int last;

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
      const int sc = s < nsteps ? s : nsteps - 1;
      b[u][s] = *reinterpret_cast<const uint4*>(
          X + static_cast<long>(a.tok0 + (tok < a.M ? tok : 0)) * a.r + sc * KS + grp * PER);
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
    const int rowc = rok ? row : r1 - 1;
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
      const int sc = s < nsteps ? s : nsteps - 1;
      av[s] = ld_stream(W + static_cast<long>(rowc) * a.r + sc * KS + grp * PER);
    }
    floatx4 acc[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
      if (s < nsteps)
#pragma unroll
        for (int u = 0; u < MT; ++u)
          acc[u] = mma_step(av[s], (u * 16 + c16 < a.M) ? b[u][s] : make_uint4(0, 0, 0, 0), acc[u], T());
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int tok = u * 16 + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vr = r0 + t * 16 + grp * 4 + i;
        if (vr < r1 && tok < a.M) {
          const float v = acc[u][i];
          if (better(v, vr, bv[u], bi[u])) { bv[u] = v; bi[u] = vr; }
          if (a.tap) a.tap[a.omap.row(a.tok0 + tok) * a.V + vr] = v;
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
    publish_partial(a, static_cast<long>(a.tok0 + threadIdx.x) * G + g, v, i);
  }
  {
    const int gw = static_cast<int>(G), x = static_cast<int>(blockIdx.x & 7);
    reduce_if_last(a, G, &last, (gw - x + 7) / 8, gw < 8 ? gw : 8);
  }
}

// Pipelined variant for at most 16 tokens: each wave streams its tiles
// (16 vocabulary rows, all r columns) through a two-stage register pipeline
// so that the next tile's 16 KB is in flight while the current one is
// multiplied and reduced.  Rows are read whole (one contiguous row per load
// instruction) and transposed into MFMA fragments through LDS.
template <typename T>
__global__ __launch_bounds__(kWaves * 64) void lmhead_pipe_kernel(LmArgs a) {
  constexpr int PER = Elem<T>::kPerLane;
  constexpr int KS = PER * 4;
  static_assert(kMaxSteps == 16, "one raw load per tile row");
  __shared__ float sv[kWaves][16];
  __shared__ int si[kWaves][16];
  __shared__ int last;
  __shared__ uint4 wbuf[kWaves][16 * 64];   // per wave: 16 rows x 64 chunks

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const long G = gridDim.x, g = blockIdx.x;
  const int r0 = static_cast<int>((g * a.V) / G), r1 = static_cast<int>(((g + 1) * a.V) / G);
  const int ntile = (r1 - r0 + 15) >> 4;
  const int nsteps = a.r / KS;
  const T* W = static_cast<const T*>(a.W);
  const T* X = static_cast<const T*>(a.src);

  // token block: all loads issued unconditionally (clamped addresses); the
  // mask for missing tokens is applied where the values are used
  const bool tok_ok = c16 < a.M;
  const long xrow = static_cast<long>(a.tok0 + (tok_ok ? c16 : 0)) * a.r;
  uint4 b[kMaxSteps];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    const int sc = s < nsteps ? s : nsteps - 1;
    b[s] = *reinterpret_cast<const uint4*>(X + xrow + sc * KS + grp * PER);
  }

  // Weight rows are loaded whole: raw load i of a tile is vocabulary row
  // t * 16 + i, lane j holding its 16-byte chunk j (rows are at most 64
  // chunks); consume() turns the chunks into MFMA fragments through the
  // wave's LDS buffer, chunk j of tile row i at position j ^ i.
  const int lpr = nsteps * 4;                       // chunks per row
  const int jc = lane < lpr ? lane : lpr - 1;
  auto issue = [&](int t, uint4 (&st)[kMaxSteps]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int row = r0 + t * 16 + i;
      row = row < r1 ? row : r1 - 1;
      st[i] = ld_stream(W + static_cast<long>(row) * a.r + jc * PER);
    }
  };

  float bv = -INFINITY;
  int bi = 0x7fffffff;
  uint4* wb = wbuf[wave];
  auto consume = [&](int t, const uint4 (&st)[kMaxSteps]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (lane < lpr) wb[i * 64 + (lane ^ i)] = st[i];
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
      if (s < nsteps) {
        const uint4 fa = wb[c16 * 64 + ((s * 4 + grp) ^ c16)];
        acc = mma_step(fa, tok_ok ? b[s] : make_uint4(0, 0, 0, 0), acc, T());
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = r0 + t * 16 + grp * 4 + i;
      if (vr < r1 && tok_ok) {
        const float v = acc[i];
        if (better(v, vr, bv, bi)) { bv = v; bi = vr; }
        if (a.tap) a.tap[a.omap.row(a.tok0 + c16) * a.V + vr] = v;
      }
    }
  };

  uint4 st0[kMaxSteps], st1[kMaxSteps];
  int t = wave;
  if (t < ntile) issue(t, st0);
  for (; t < ntile; t += 2 * kWaves) {
    if (t + kWaves < ntile) issue(t + kWaves, st1);
    consume(t, st0);
    if (t + kWaves < ntile) {
      if (t + 2 * kWaves < ntile) issue(t + 2 * kWaves, st0);
      consume(t + kWaves, st1);
    }
  }

  // combine the four row groups of each token column, then the waves
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (grp == 0) { sv[wave][c16] = bv; si[wave][c16] = bi; }
  __syncthreads();
  if (threadIdx.x < 16 && static_cast<int>(threadIdx.x) < a.M) {
    float v = sv[0][threadIdx.x];
    int i = si[0][threadIdx.x];
    for (int w = 1; w < kWaves; ++w)
      if (better(sv[w][threadIdx.x], si[w][threadIdx.x], v, i)) { v = sv[w][threadIdx.x]; i = si[w][threadIdx.x]; }
    publish_partial(a, static_cast<long>(a.tok0 + threadIdx.x) * G + g, v, i);
  }
  {
    const int gw = static_cast<int>(G), x = static_cast<int>(blockIdx.x & 7);
    reduce_if_last(a, G, &last, (gw - x + 7) / 8, gw < 8 ? gw : 8);
  }
}


// ------------------------------------------ fused scan + vocabulary pass --
//
// For a few requests the sequential scan keeps one team of 8 workgroups busy
// for K dependent steps while the rest of the chip idles, and the vocabulary
// projection after it is a pure stream of V x r weights.  The fused kernel
// overlaps the two: team workgroups run the scan (scan_team), every other
// workgroup ("helper") owns a contiguous range of 16-row vocabulary tiles and,
// while the scan runs, pulls its tiles on chip: TR tiles per wave into
// registers as ready MFMA fragments, TL tiles per workgroup into LDS
// (global_load_lds, row-contiguous).  The team publishes every state as
// tagged words; helpers read them, stage the states in LDS, multiply the
// resident tiles, stream the few tiles that did not fit, and publish one
// tagged (max, index) word per token, which the team folds.  The team waits
// on the first helpers (the scan's input P) and on all helpers (the fold), the
// helpers on the team (the states): the launch is one workgroup per CU (at
// most 256, all resident at once), and every wait is bounded and flags the
// status word on time-out, so the kernel always drains.
constexpr int kFuseRegs = 192;            // VGPRs per lane for resident fragments
constexpr int kFuseLdsTiles = 144 * 1024; // LDS bytes for resident tiles (gated head)
// Sequential head: LDS bytes for resident tiles and rows of staged states.
// Up to 8 states (one request) the states take 8 rows and the tiles 144 KB,
// else 16 rows and 128 KB (one tile per wave).
__host__ __device__ constexpr int seq_state_rows(int M) { return M <= 8 ? 8 : 16; }
__host__ __device__ constexpr int seq_lds_tiles(int M, int RK) { return (M <= 8 ? 144 : 128) / RK; }
constexpr int kTouchLds = 256;            // LDS bytes that receive the touch loads (never read)
constexpr int kStatePad = 32;             // bf16 elements after each staged state row (spreads banks)

struct FuseArgs {
  ScanArgs sa;
  LmArgs la;
  int nteam;        // scan teams (one request each): blocks xq * 8 + t, t < nteam, xq < team size
  uint64_t* sw;     // [M][r / 2] tagged bf16 state pairs published by the teams (zero at launch)
  uint64_t* px;     // [M, G] tagged (max, index) words of the helpers (zero at launch)
  GemmArgs ph;      // P = W_down[:, :D] h, when the helpers compute it (nps > 0)
  int nps;          // its k slices: helper q * nps + p takes row tile q, slice p
};

constexpr int kPSteps = 4;   // k-steps of 32 per wave and P slice (at most)

// One helper's share of P: the 16 rows pt * 16 .. of W_down[:, :D] times the
// M pre-gained token rows over k slice ps, scaled by each token's 1/rms (the
// slices add up to P), published as tagged words (tag 1) for the team.  The
// eight waves split the slice's k-steps and are added in wave order.
__device__ void seqhead_p_partial(const FuseArgs& f, int hp, unsigned char* smem) {
  const GemmArgs& g = f.ph;
  const int r = f.la.r, M = g.M;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int pt = hp / f.nps, ps = hp % f.nps;
  const int nst = g.K / 32;
  const int k0 = static_cast<int>(static_cast<long>(ps) * nst / f.nps);
  const int k1 = static_cast<int>(static_cast<long>(ps + 1) * nst / f.nps);
  const int s0 = k0 + wave * (k1 - k0) / kWaves, s1 = k0 + (wave + 1) * (k1 - k0) / kWaves;
  const uint16_t* W = static_cast<const uint16_t*>(g.W);
  const uint16_t* X = static_cast<const uint16_t*>(g.src);
  const bool tok_ok = c16 < M;
  const long xrow = g.smap.row(tok_ok ? c16 : 0);
  const long wrow = static_cast<long>(pt) * 16 + c16;
  uint4 av[kPSteps], bv[kPSteps];
#pragma unroll
  for (int i = 0; i < kPSteps; ++i) {
    const int s = s0 + i < s1 ? s0 + i : k0;   // in-range clamp
    av[i] = ld_stream(W + wrow * g.ldw + s * 32 + grp * 8);
    bv[i] = *reinterpret_cast<const uint4*>(X + xrow * g.ld_src + s * 32 + grp * 8);
  }
  float* red = reinterpret_cast<float*>(smem);          // [8 waves][64 lanes][4]
  float* inv = red + kWaves * 64 * 4;                   // [16]
  // each token's 1/rms from the producer's partial sums of squares
  for (int t = wave; t < M; t += kWaves) {
    const float* sp = g.ssq + g.qmap.row(t) * kSsqParts;
    float v = 0.f;
    for (int j = lane; j < g.np_hi; j += 64) v += sp[j];
    v = wave_sum(v);
    if (lane == 0) inv[t] = 1.0f / sqrtf(v / static_cast<float>(g.norm_len) + g.eps);
  }
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kPSteps; ++i)
    if (s0 + i < s1) acc = mma_step(av[i], tok_ok ? bv[i] : make_uint4(0, 0, 0, 0), acc, uint16_t());
  *reinterpret_cast<floatx4*>(red + (wave * 64 + lane) * 4) = acc;
  __syncthreads();
  // lane (row group q, token c) holds rows 4 q .. 4 q + 3 of token c
  for (int e = threadIdx.x; e < 16 * M; e += blockDim.x) {
    const int t = e >> 4, rr = e & 15;
    const int src = ((rr >> 2) * 16 + t) * 4 + (rr & 3);
    float v = 0.f;
    for (int w = 0; w < kWaves; ++w) v += red[w * 256 + src];
    v *= inv[t];
    const long o = (static_cast<long>(ps) * M + t) * r + pt * 16 + rr;
    __hip_atomic_store(const_cast<uint64_t*>(f.sa.Pw) + o, (uint64_t{1} << 32) | __float_as_uint(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();   // the LDS is reused for the resident tiles
}

// A helper's (max, index) for one token as one word: the value's bits in the
// high half, the index in the low 24 bits, a tag (1) in the top 8 bits of
// the low half; a zeroed slot has tag 0.
__device__ __forceinline__ uint64_t pack_best(float v, int i) {
  return (static_cast<uint64_t>(__float_as_uint(v)) << 32) | (static_cast<uint32_t>(i) & 0xffffffu) | (1u << 24);
}

// Team workgroup q of nq folds tokens q, q + nq, ..: waits for the G words of
// the token (bounded), folds them in index order per thread and then in
// wave order (the result does not depend on arrival order), writes the
// candidate.
__device__ void fold_tokens(const FuseArgs& f, int q, int nq, int G, unsigned char* smem) {
  const LmArgs& a = f.la;
  unsigned* status = a.counters + CNT_STATUS;
  float* rv = reinterpret_cast<float*>(smem);
  int* ri = reinterpret_cast<int*>(rv + kWaves);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = q; t < a.M; t += nq) {
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int e = threadIdx.x; e < G; e += blockDim.x) {
      const uint64_t* p = f.px + static_cast<long>(t) * G + e;
      uint64_t w = scan_detail::ld_tagged(p);
      unsigned spins = 0;
      while (((static_cast<uint32_t>(w) >> 24) & 0xffu) != 1u) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > scan_detail::kSpinLimit) {
          atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
          break;
        }
        w = scan_detail::ld_tagged(p);
      }
      const float pv = __uint_as_float(static_cast<uint32_t>(w >> 32));
      const int pi = static_cast<int>(static_cast<uint32_t>(w) & 0xffffffu);
      if (better(pv, pi, v, ix)) { v = pv; ix = pi; }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(v, o, kWave);
      const int oi = __shfl_xor(ix, o, kWave);
      if (better(ov, oi, v, ix)) { v = ov; ix = oi; }
    }
    if (lane == 0) { rv[wave] = v; ri[wave] = ix; }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kWaves; ++w)
        if (better(rv[w], ri[w], v, ix)) { v = rv[w]; ix = ri[w]; }
      const int b = t / a.K;
      bool ok = a.anchors[b] >= 0 && a.anchors[b] < a.V;
      if (a.pos) ok = ok && a.pos[b] >= 0 && a.pos[b] < a.pos_n;
      a.cand[t] = ok ? ix : -1;
      if (a.max_logit) a.max_logit[t] = ok ? v : 0.f;
    }
    __syncthreads();
  }
}

template <int RK>   // k-steps of 32 (r / 32)
__global__ __launch_bounds__(kWaves * 64) void seqhead_kernel(FuseArgs f) {
  using namespace scan_detail;
  constexpr int TR = kFuseRegs / (4 * RK);         // register tiles per wave
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float sv[kWaves][16];
  __shared__ int si[kWaves][16];

  const int bx = blockIdx.x, xq = bx >> 3, x = bx & 7;
  const int nteam = f.nteam;
  constexpr int kTeam = (RK * 32) % 256 == 0 ? 16 : 8;   // members per scan team (team_size(r, B), B <= 8)
  if (xq < kTeam && x < nteam) {
    scan_team<uint16_t, kTeam>(f.sa, reinterpret_cast<float*>(smem), x, xq, f.sw);
    // then the argmax of the tokens from the helpers' words
    __syncthreads();
    fold_tokens(f, x * kTeam + xq, kTeam * nteam, static_cast<int>(gridDim.x) - kTeam * nteam, smem);
    return;
  }

  const LmArgs& a = f.la;
  const int h = bx < 8 * kTeam ? xq * (8 - nteam) + (x - nteam) : bx - kTeam * nteam;
  const int G = static_cast<int>(gridDim.x) - kTeam * nteam;
  // the scan's input first: the team waits for it before its first step
  if (f.nps > 0 && h < (a.r / 16) * f.nps) seqhead_p_partial(f, h, smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int r = a.r, V = a.V, M = a.M;
  const int NT = (V + 15) / 16;
  const int t0 = static_cast<int>(static_cast<long>(h) * NT / G);
  const int t1 = static_cast<int>(static_cast<long>(h + 1) * NT / G);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  // fragment (tile t, k-step s) of this lane: row t*16 + c16, 16 bytes at s*32 + grp*8
  auto frag_ptr = [&](int t, int s) {
    int row = t * 16 + c16;
    row = row < V ? row : V - 1;
    return W + static_cast<long>(row) * r + s * 32 + grp * 8;
  };

  const int TL = seq_lds_tiles(M, RK);            // LDS tiles per workgroup
  const int SR = seq_state_rows(M);               // staged state rows (zeros past M)
  uint4* lds_w = reinterpret_cast<uint4*>(smem);                                   // [TL][RK][64]
  uint16_t* lds_s = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(TL) * RK * 1024);  // [SR][r + pad]
  unsigned char* lds_touch = smem + static_cast<size_t>(TL) * RK * 1024 + static_cast<size_t>(SR) * (r + kStatePad) * 2;

  // ---- while the scan runs: resident tiles.  Register tiles are loaded in
  //      fragment order (16 bytes of each of 16 rows per instruction, the
  //      two halves of a 128-byte line by consecutive instructions).  LDS
  //      tiles are loaded row-contiguous (each instruction covers whole
  //      lines, which streams faster), chunk c of tile row i stored at
  //      c ^ (i & kSwz) so that the fragment reads spread over the banks.
  const int treg = t0 + wave * TR;             // this wave's register tiles
  uint4 wr[TR][RK];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int s = 0; s < RK; ++s) wr[i][s] = ld_stream(frag_ptr(treg + i, s));
  constexpr int CPR = 4 * RK;                  // 16-byte chunks per row
  constexpr int kSwz = (CPR % 16 == 0) ? 15 : 7;
  const int tlds = t0 + kWaves * TR;           // first LDS tile
  for (int j = wave; j < TL; j += kWaves)
#pragma unroll
    for (int q = 0; q < RK; ++q) {
      const int g = q * 64 + lane, i = g / CPR, c = g % CPR;
      int row = (tlds + j) * 16 + i;
      row = row < V ? row : V - 1;
      load_lds16_nt(W + static_cast<long>(row) * r + (c ^ (i & kSwz)) * 8, lds_w + (j * RK + q) * 64);
    }

  // ---- the tiles that do not fit: touched once now (one dword per 128-byte
  //      line, temporal loads) so that they sit in L2 when they are streamed
  //      after the scan.  The touches are direct-to-LDS loads into a scratch
  //      area that is never read, so no register waits for them and they
  //      queue behind the resident tiles without stalling the wave.
  const int tstream = tlds + TL;
  for (int t = tstream + wave; t < t1; t += kWaves) {
    const uint32_t* base = reinterpret_cast<const uint32_t*>(W + static_cast<long>(t) * 16 * r);
    const int lines = (t * 16 + 16 <= V ? 16 : V - t * 16) * r / 64;   // 128-byte lines of the tile
    for (int l = lane; l < lines; l += 64)
      __builtin_amdgcn_global_load_lds(base + l * 32, (__attribute__((address_space(3))) void*)(lds_touch), 4, 0, 0);
  }

  // ---- the team's states: tagged words of two bf16 values, the word of
  //      token t carrying tag (t mod K) + 1 once that step is published;
  //      every word is requested at once and re-read until its tag is right
  //      (bounded), then staged in LDS
  {
    const int hw = r / 2, nw = M * hw;         // M <= 16, r <= 512: at most 8 words per thread
    constexpr int kWpt = 4;                    // words per thread and pass (two passes past 8 tokens)
    for (int base = 0; base < nw; base += kWpt * kWaves * 64) {
      uint64_t wv[kWpt];
      auto want = [&](int i) {
        const int e = base + threadIdx.x + i * kWaves * 64;
        return static_cast<uint32_t>((e / hw) % a.K + 1);
      };
      auto valid = [&](int i) { return base + static_cast<int>(threadIdx.x) + i * kWaves * 64 < nw; };
#pragma unroll
      for (int i = 0; i < kWpt; ++i) wv[i] = valid(i) ? ld_tagged(f.sw + base + threadIdx.x + i * kWaves * 64) : 0;
      unsigned spins = 0;
      for (;;) {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < kWpt; ++i) bad = bad || (valid(i) && static_cast<uint32_t>(wv[i] >> 32) != want(i));
        if (!bad) break;
        if (++spins > kSpinLimit) {
          atomicOr(a.counters + CNT_STATUS, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
          break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int i = 0; i < kWpt; ++i)
          if (valid(i) && static_cast<uint32_t>(wv[i] >> 32) != want(i))
            wv[i] = ld_tagged(f.sw + base + threadIdx.x + i * kWaves * 64);
      }
#pragma unroll
      for (int i = 0; i < kWpt; ++i) {
        const int e = base + threadIdx.x + i * kWaves * 64;
        if (valid(i))
          *reinterpret_cast<uint32_t*>(lds_s + (e / hw) * (r + kStatePad) + (e % hw) * 2) = static_cast<uint32_t>(wv[i]);
      }
    }
    // token columns past M read zeros (no select in the fragment reads)
    for (int e = nw + threadIdx.x; e < SR * hw; e += blockDim.x)
      *reinterpret_cast<uint32_t*>(lds_s + (e / hw) * (r + kStatePad) + (e % hw) * 2) = 0u;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): register and LDS tiles have landed
  __syncthreads();

  const bool tok_ok = c16 < M;
  auto bfrag = [&](int s) {
    return *reinterpret_cast<const uint4*>(lds_s + (c16 & (SR - 1)) * (r + kStatePad) + s * 32 + grp * 8);
  };
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  float* const tap = a.tap;
  auto take = [&](int t, const floatx4& acc) {
    const bool ok_t = t < t1 && tok_ok;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = t * 16 + grp * 4 + i;
      if (ok_t && vr < V && better(acc[i], vr, bv, bi)) { bv = acc[i]; bi = vr; }
    }
    if (tap && ok_t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t * 16 + grp * 4 + i < V) tap[static_cast<long>(c16) * V + t * 16 + grp * 4 + i] = acc[i];
    }
  };

  // register tiles (state fragments requested two steps ahead)
  {
    floatx4 acc[TR];
#pragma unroll
    for (int i = 0; i < TR; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint4 bb[3];
    bb[0] = bfrag(0);
    if (RK > 1) bb[1] = bfrag(1);
#pragma unroll
    for (int s = 0; s < RK; ++s) {
      if (s + 2 < RK) bb[(s + 2) % 3] = bfrag(s + 2);
#pragma unroll
      for (int i = 0; i < TR; ++i) acc[i] = mma_step(wr[i][s], bb[s % 3], acc[i], uint16_t());
    }
#pragma unroll
    for (int i = 0; i < TR; ++i) take(treg + i, acc[i]);
  }
  // the register file is free again: the first tile that did not fit
  // (touched into L2 above) is requested, then the LDS tiles are multiplied
  // while it arrives; one wave per streamed tile
  int t = tstream + wave;
  uint4 nx[RK];
  if (t < t1) {
#pragma unroll
    for (int s = 0; s < RK; ++s) nx[s] = ld_stream(frag_ptr(t, s));
  }
  uint4 bq[RK];
#pragma unroll
  for (int s = 0; s < RK; ++s) bq[s] = bfrag(s);
  // one LDS tile per wave: every fragment read is issued before the first
  // multiply, and the k-steps alternate between two accumulators
  for (int j = wave; j < TL; j += kWaves) {
    uint4 af[RK];
#pragma unroll
    for (int s = 0; s < RK; ++s) af[s] = lds_w[j * RK * 64 + c16 * CPR + ((4 * s + grp) ^ (c16 & kSwz))];
    // all reads in flight before the first multiply (one LDS latency per tile)
#pragma unroll
    for (int s = 0; s < RK; ++s) asm volatile("" ::"v"(af[s].x), "v"(af[s].y), "v"(af[s].z), "v"(af[s].w));
    floatx4 acc0 = floatx4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
    for (int s = 0; s < RK; s += 2) {
      acc0 = mma_step(af[s], bq[s], acc0, uint16_t());
      if (s + 1 < RK) acc1 = mma_step(af[s + 1], bq[s + 1], acc1, uint16_t());
    }
    take(tlds + j, acc0 + acc1);
  }
  for (; t < t1; t += kWaves) {
    floatx4 acc0 = floatx4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
    for (int s = 0; s < RK; s += 2) {
      acc0 = mma_step(nx[s], bq[s], acc0, uint16_t());
      if (s + 1 < RK) acc1 = mma_step(nx[s + 1], bq[s + 1], acc1, uint16_t());
    }
    take(t, acc0 + acc1);
    if (t + kWaves < t1) {
#pragma unroll
      for (int s = 0; s < RK; ++s) nx[s] = ld_stream(frag_ptr(t + kWaves, s));
    }
  }

  // combine the four row groups of each token column, then the waves
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (grp == 0) { sv[wave][c16] = bv; si[wave][c16] = bi; }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < M) {
    float v = sv[0][threadIdx.x];
    int i = si[0][threadIdx.x];
    for (int w = 1; w < kWaves; ++w)
      if (better(sv[w][threadIdx.x], si[w][threadIdx.x], v, i)) { v = sv[w][threadIdx.x]; i = si[w][threadIdx.x]; }
    // one word per token for the team to fold (a helper without tiles
    // reports index 0 at -inf: never better)
    __hip_atomic_store(f.px + static_cast<long>(threadIdx.x) * G + h, pack_best(v, i < V ? i : 0),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int RK>
size_t seqhead_lds(int M, int r) {
  return static_cast<size_t>(seq_lds_tiles(M, RK)) * RK * 1024 +
         static_cast<size_t>(seq_state_rows(M)) * (r + kStatePad) * 2 + kTouchLds;
}

// --------------------------------------------- fused gated head (few requests) --
//
// The walkthrough's gated head ("官方顺序头具体算了什么") runs one vocabulary
// pass per position, each over the same 155.6 MB W_o.  For a few requests
// this launch keeps W_o on chip for all K positions instead of streaming it K
// times: helper workgroup h owns a contiguous range of 16-row tiles and holds
// TR of them per wave in registers and TL per workgroup in LDS for the whole
// launch; only the remainder (touched into L2 before the first position) is
// re-read at each position.  Sixteen team workgroups run the state updates.
// Per position i (tag i + 1; s_0 = 0, or the warm-up state computed before
// the launch):
//   team     d_{i-1} (the anchor at i = 0) -> v_i = E_R(d_{i-1});
//            [g; c] = W_s [s_{i-1}; v_i] + b_s and the gate for its 32 state
//            elements, published as tagged words; all R read back;
//            r_i = W_h[:, :R] s_i + qh_i + b_h for its 32 elements, published
//            as tagged words (two bf16 each);
//   helpers  wait for every r_i word, multiply their tiles, publish one
//            tagged (max, index) word per request;
//   team     member b < B waits for request b's G words, reduces them in
//            fixed order, writes its candidate and publishes d_i as a tagged
//            word for the whole team.
// A word is rewritten only for a later position, after all its readers have
// passed the dependency that the later position needs, so tags alone order
// everything.  The launch is cooperative (every workgroup resident: the team
// and the helpers wait on each other); every wait is bounded and flags the
// status word on time-out, so the kernel always drains.
constexpr int kGTeam = 16;       // team workgroups (blocks 0 .. 15)
constexpr int kGR = 512;         // state width of the fused path

__device__ __forceinline__ float dot8(const uint4& w, const float* x) {
  return __uint_as_float(w.x << 16) * x[0] + __uint_as_float(w.x & 0xffff0000u) * x[1] +
         __uint_as_float(w.y << 16) * x[2] + __uint_as_float(w.y & 0xffff0000u) * x[3] +
         __uint_as_float(w.z << 16) * x[4] + __uint_as_float(w.z & 0xffff0000u) * x[5] +
         __uint_as_float(w.w << 16) * x[6] + __uint_as_float(w.w & 0xffff0000u) * x[7];
}

// N (8 or 4) sums over the 64 lanes at once: butterfly steps that halve the
// number of values per lane (lanes above the step's bit keep the upper
// half), then a plain butterfly over the remaining lanes.  Lane l ends with
// the total of value l >> (6 - log2 N): 10 (N = 8) or 6 (N = 4) lane swaps
// instead of 6 N.
template <int N>
__device__ __forceinline__ float wave_sums(float (&v)[N], int lane) {
  static_assert(N == 8 || N == 4, "N = 8 or 4");
#pragma unroll
  for (int o = 32, n = N; n > 1; o >>= 1, n >>= 1) {
    const bool hi = (lane & o) != 0;
#pragma unroll
    for (int k = 0; k < n / 2; ++k) {
      const float send = hi ? v[k] : v[k + n / 2];
      const float keep = hi ? v[k + n / 2] : v[k];
      v[k] = keep + __shfl_xor(send, o, kWave);
    }
  }
  float t = v[0];
#pragma unroll
  for (int o = 32 / N; o > 0; o >>= 1) t += __shfl_xor(t, o, kWave);
  return t;
}

__device__ __forceinline__ uint64_t wait_tag(const uint64_t* p, unsigned tag, unsigned* status) {
  uint64_t w = scan_detail::ld_tagged(p);
  unsigned spins = 0;
  while (static_cast<unsigned>(w >> 32) != tag) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > scan_detail::kSpinLimit) {
      atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
      break;
    }
    w = scan_detail::ld_tagged(p);
  }
  return w;
}

__device__ __forceinline__ void put_tag(uint64_t* p, uint32_t v, unsigned tag) {
  __hip_atomic_store(p, static_cast<uint64_t>(v) | (static_cast<uint64_t>(tag) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// The argmax of request b at position i: every helper's (max, index) for
// the position arrives as one tagged word (value in the high half, index in
// the low 24 bits, tag in the top 8); fold them (each thread a strided
// share in index order, then the waves in order: the same result for any
// arrival order), write the candidate and publish d_i.
__device__ __forceinline__ void gated_finish(const GatedFuseArgs& f, unsigned char* smem, int b, int i,
                                             unsigned* status) {
  const LmArgs& a = f.la;
  const int G = a.G, K = f.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* rv = reinterpret_cast<float*>(smem + static_cast<size_t>(f.B) * 3 * kGR * 4 + 64);   // after xs, ss, dsh
  int* ri = reinterpret_cast<int*>(rv + kWaves);
  const unsigned tag = static_cast<unsigned>(i + 1) & 0xffu;
  float v = -INFINITY;
  int ix = 0x7fffffff;
  for (int e = threadIdx.x; e < G; e += blockDim.x) {
    const uint64_t* p = f.px + static_cast<long>(b) * G + e;
    uint64_t w = scan_detail::ld_tagged(p);
    unsigned spins = 0;
    while ((static_cast<uint32_t>(w) >> 24) != tag) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > scan_detail::kSpinLimit) {
        atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
        break;
      }
      w = scan_detail::ld_tagged(p);
    }
    const float pv = __uint_as_float(static_cast<uint32_t>(w >> 32));
    const int pi = static_cast<int>(static_cast<uint32_t>(w) & 0xffffffu);
    if (better(pv, pi, v, ix)) { v = pv; ix = pi; }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(ix, o, kWave);
    if (better(ov, oi, v, ix)) { v = ov; ix = oi; }
  }
  if (lane == 0) { rv[wave] = v; ri[wave] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w)
      if (better(rv[w], ri[w], v, ix)) { v = rv[w]; ix = ri[w]; }
    const int anchor = a.anchors[b];
    bool ok = anchor >= 0 && anchor < a.V;
    if (a.pos) ok = ok && a.pos[b] >= 0 && a.pos[b] < a.pos_n;
    const long orow = static_cast<long>(b) * K + i;
    a.cand[orow] = ok ? ix : -1;
    if (a.max_logit) a.max_logit[orow] = ok ? v : 0.f;
    put_tag(f.dx + b, static_cast<uint32_t>(ix), static_cast<unsigned>(i + 1));
  }
  __syncthreads();
}

// Team member m: state elements [32 m, 32 m + 32), wave w the four from
// 32 m + 4 w; its rows of W_s (g and c) and W_h (state columns) stay in
// registers, lane l holding columns 8 l .. 8 l + 7 of each half.
__device__ __forceinline__ void gated_team(const GatedFuseArgs& f, unsigned char* smem, int m) {
  constexpr int R = kGR, R2 = 2 * kGR;
  const int B = f.B, K = f.K, V = f.la.V, D = f.D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = m * 32 + wave * 4;
  unsigned* status = f.la.counters + CNT_STATUS;
  const uint16_t* Ws = static_cast<const uint16_t*>(f.w_s);
  const uint16_t* Wh = static_cast<const uint16_t*>(f.w_h);
  const uint16_t* E = static_cast<const uint16_t*>(f.emb);
  uint4 wg[4][2], wc[4][2], wh[4];
  float bg[4], bc[4], bh[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint16_t* rg = Ws + static_cast<long>(j0 + q) * R2 + lane * 8;
    const uint16_t* rc = Ws + static_cast<long>(R + j0 + q) * R2 + lane * 8;
    wg[q][0] = *reinterpret_cast<const uint4*>(rg);
    wg[q][1] = *reinterpret_cast<const uint4*>(rg + R);
    wc[q][0] = *reinterpret_cast<const uint4*>(rc);
    wc[q][1] = *reinterpret_cast<const uint4*>(rc + R);
    wh[q] = *reinterpret_cast<const uint4*>(Wh + static_cast<long>(j0 + q) * (R + D) + lane * 8);
    bg[q] = bf16_to_f32(static_cast<const uint16_t*>(f.b_s)[j0 + q]);
    bc[q] = bf16_to_f32(static_cast<const uint16_t*>(f.b_s)[R + j0 + q]);
    bh[q] = bf16_to_f32(static_cast<const uint16_t*>(f.b_h)[j0 + q]);
  }
  float* xs = reinterpret_cast<float*>(smem);      // [B][2R]: s_{i-1}, v_i
  float* ss = xs + B * R2;                         // [B][R]:  s_i
  int* dsh = reinterpret_cast<int*>(ss + B * R);   // [B]:     d_{i-1}
  auto pick = [](const float (&v)[4], int q) { return q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3]; };

  for (int i = 0; i < K; ++i) {
    const unsigned tag = static_cast<unsigned>(i + 1);
    if (static_cast<int>(threadIdx.x) < B)
      dsh[threadIdx.x] = i == 0 ? f.anchors[threadIdx.x]
                                : static_cast<int>(static_cast<uint32_t>(wait_tag(f.dx + threadIdx.x, tag - 1, status)));
    __syncthreads();
    for (int e = threadIdx.x; e < B * R; e += blockDim.x) {
      const int b = e / R, k = e % R;
      const int d = dsh[b];
      xs[b * R2 + k] = i == 0 ? (f.s_init ? f.s_init[e] : 0.f) : ss[e];
      xs[b * R2 + R + k] = (d >= 0 && d < V) ? bf16_to_f32(E[static_cast<long>(d) * R + k]) : 0.f;
    }
    __syncthreads();
    // gate of this wave's four elements, every request
    for (int b = 0; b < B; ++b) {
      const float* x = xs + b * R2;
      float x0[8], x1[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) { x0[t] = x[lane * 8 + t]; x1[t] = x[R + lane * 8 + t]; }
      float d8[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        d8[q] = dot8(wg[q][0], x0) + dot8(wg[q][1], x1);
        d8[4 + q] = dot8(wc[q][0], x0) + dot8(wc[q][1], x1);
      }
      // lane 8 q holds the g sum of element q, lane 8 q + 32 its c sum
      const float sum = wave_sums<8>(d8, lane);
      const float csum = __shfl_xor(sum, 32, kWave);
      if (lane < 32 && (lane & 7) == 0) {
        const int q = lane >> 3, j = j0 + q;
        const float g = sum + pick(bg, q), c = csum + pick(bc, q);
        const float fg = 1.0f / (1.0f + expf(-g));
        const float sn = fg * x[j] + (1.0f - fg) * tanhf(c);
        f.s_out[(static_cast<long>(b) * K + i) * R + j] = sn;
        put_tag(f.sx + b * R + j, __float_as_uint(sn), tag);
      }
    }
    // the whole s_i from the team's words
    for (int e = threadIdx.x; e < B * R; e += blockDim.x)
      ss[e] = __uint_as_float(static_cast<uint32_t>(wait_tag(f.sx + e, tag, status)));
    __syncthreads();
    // r_i of this wave's four elements, published in pairs
    for (int b = 0; b < B; ++b) {
      float s8[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) s8[t] = ss[b * R + lane * 8 + t];
      float d4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) d4[q] = dot8(wh[q], s8);
      // lane 16 q holds element q's sum; pairs (0, 1) and (2, 3) meet at
      // lanes 0 and 32
      const float sum = wave_sums<4>(d4, lane);
      const float odd = __shfl_xor(sum, 16, kWave);
      if ((lane & 31) == 0) {
        const int q = lane >> 4;   // 0 or 2
        const float* qrow = f.qh + (static_cast<long>(b) * K + i) * R + j0;
        const float ra = sum + qrow[q] + pick(bh, q);
        const float rb = odd + qrow[q + 1] + pick(bh, q + 1);
        const uint32_t pk = static_cast<uint32_t>(f32_to_bf16(ra)) | (static_cast<uint32_t>(f32_to_bf16(rb)) << 16);
        put_tag(f.rx + b * (R / 2) + j0 / 2 + q / 2, pk, tag);
      }
    }
    // member m < B: the argmax of request m once every helper has counted in
    if (m < B) gated_finish(f, smem, m, i, status);
  }
}

template <int RK>   // k-steps of 32 (R / 32)
__global__ __launch_bounds__(kWaves * 64) void gatedhead_kernel(GatedFuseArgs f) {
  constexpr int TR = kFuseRegs / (4 * RK);
  constexpr int TL = kFuseLdsTiles / (RK * 1024);
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float sv[kWaves][16];
  __shared__ int si[kWaves][16];

  if (static_cast<int>(blockIdx.x) < kGTeam) {
    gated_team(f, smem, static_cast<int>(blockIdx.x));
    return;
  }
  const LmArgs& a = f.la;
  unsigned* status = a.counters + CNT_STATUS;
  const int h = static_cast<int>(blockIdx.x) - kGTeam;
  const int G = static_cast<int>(gridDim.x) - kGTeam;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  constexpr int r = RK * 32;
  const int V = a.V, B = f.B, K = f.K;
  const int NT = (V + 15) / 16;
  const int t0 = static_cast<int>(static_cast<long>(h) * NT / G);
  const int t1 = static_cast<int>(static_cast<long>(h + 1) * NT / G);
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  auto frag_ptr = [&](int t, int s) {
    int row = t * 16 + c16;
    row = row < V ? row : V - 1;
    return W + static_cast<long>(row) * r + s * 32 + grp * 8;
  };
  uint4* lds_w = reinterpret_cast<uint4*>(smem);                                   // [TL][RK][64]
  uint16_t* lds_r = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(TL) * RK * 1024);  // [B][r + pad]

  const int treg = t0 + wave * TR;
  uint4 wr[TR][RK];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int s = 0; s < RK; ++s) wr[i][s] = ld_stream(frag_ptr(treg + i, s));
  const int tlds = t0 + kWaves * TR;
  for (int j = wave; j < TL; j += kWaves)
#pragma unroll
    for (int s = 0; s < RK; ++s) load_lds16(frag_ptr(tlds + j, s), lds_w + (j * RK + s) * 64);
  const int tstream = tlds + TL;
  unsigned touch = 0;
  for (int t = tstream + (kWaves - 1 - wave); t < t1; t += kWaves) {
    const uint32_t* base = reinterpret_cast<const uint32_t*>(W + static_cast<long>(t) * 16 * r);
    const int lines = (t * 16 + 16 <= V ? 16 : V - t * 16) * r / 64;
    for (int l = lane; l < lines; l += 64) touch ^= base[l * 32];
  }
  const bool tok_ok = c16 < B;

  for (int i = 0; i < K; ++i) {
    const unsigned tag = static_cast<unsigned>(i + 1);
    for (int e = threadIdx.x; e < B * (r / 2); e += blockDim.x) {
      const uint64_t w = wait_tag(f.rx + e, tag, status);
      const int b = e / (r / 2), jj = e % (r / 2);
      *reinterpret_cast<uint32_t*>(lds_r + b * (r + kStatePad) + 2 * jj) = static_cast<uint32_t>(w);
    }
    if (i == 0) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): resident tiles have landed
    __syncthreads();

    // state fragment: columns of absent requests read request 0's row (their
    // logits are never taken)
    auto bfrag = [&](int s) {
      return *reinterpret_cast<const uint4*>(lds_r + (tok_ok ? c16 : 0) * (r + kStatePad) + s * 32 + grp * 8);
    };
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    auto take = [&](int t, const floatx4& acc) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int vr = t * 16 + grp * 4 + q;
        if (t < t1 && vr < V && tok_ok) {
          const float v = acc[q];
          if (better(v, vr, bv, bi)) { bv = v; bi = vr; }
          if (a.tap) a.tap[(static_cast<long>(c16) * K + i) * V + vr] = v;
        }
      }
    };
    // the register tiles hold nearly the whole register file: the state
    // fragments are read from LDS two k-steps at a time (the empty asm with
    // a memory clobber keeps the compiler from hoisting all of them at once)
    {
      floatx4 acc[TR];
#pragma unroll
      for (int q = 0; q < TR; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < RK; s0 += 2) {
        asm volatile("" ::: "memory");
        uint4 b4[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) b4[s] = bfrag(s0 + s);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int q = 0; q < TR; ++q) acc[q] = mma_step(wr[q][s0 + s], b4[s], acc[q], uint16_t());
      }
#pragma unroll
      for (int q = 0; q < TR; ++q) take(treg + q, acc[q]);
    }
    for (int j = wave; j < TL; j += kWaves) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
      int toff = j * RK * 64 + lane;   // opaque: one base per tile, k-steps as immediate offsets
      asm volatile("" : "+v"(toff));
#pragma unroll
      for (int s0 = 0; s0 < RK; s0 += 2) {
        asm volatile("" ::: "memory");
        uint4 af[2], b4[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          af[s] = lds_w[toff + (s0 + s) * 64];
          b4[s] = bfrag(s0 + s);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mma_step(af[s], b4[s], acc, uint16_t());
      }
      take(tlds + j, acc);
    }
    // streamed tiles from the last wave down: wave 0 already has the
    // ninth LDS tile
    for (int t = tstream + (kWaves - 1 - wave); t < t1; t += kWaves) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < RK; s0 += 2) {
        asm volatile("" ::: "memory");
        uint4 nx[2], b4[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          nx[s] = *reinterpret_cast<const uint4*>(frag_ptr(t, s0 + s));
          b4[s] = bfrag(s0 + s);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mma_step(nx[s], b4[s], acc, uint16_t());
      }
      take(t, acc);
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (grp == 0) { sv[wave][c16] = bv; si[wave][c16] = bi; }
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < B) {
      float v = sv[0][threadIdx.x];
      int ix = si[0][threadIdx.x];
      for (int w = 1; w < kWaves; ++w)
        if (better(sv[w][threadIdx.x], si[w][threadIdx.x], v, ix)) { v = sv[w][threadIdx.x]; ix = si[w][threadIdx.x]; }
      // (a helper without tiles reports index 0 at -inf: never better)
      const uint32_t lo = (static_cast<uint32_t>(ix < V ? ix : 0) & 0xffffffu) | ((tag & 0xffu) << 24);
      __hip_atomic_store(f.px + static_cast<long>(threadIdx.x) * G + h,
                         (static_cast<uint64_t>(__float_as_uint(v)) << 32) | lo, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (touch == 0x9e3779b9u && B < 0) a.cand[0] = 0;   // keeps the touch loads
}

template <int RK>
size_t gatedhead_lds(int B, int r) {
  constexpr int TL = kFuseLdsTiles / (RK * 1024);
  const size_t helper = static_cast<size_t>(TL) * RK * 1024 + static_cast<size_t>(B) * (r + kStatePad) * 2;
  const size_t team = static_cast<size_t>(B) * (3 * r) * 4 + 64 + 2 * kWaves * 4;
  return helper > team ? helper : team;
}

}  // namespace

int lmhead_groups(int V) {
  const int tiles = (V + 15) / 16;
  return tiles < 256 ? tiles : 256;
}

bool seqhead_fused(int B, int K, int r, bool bf16) {
  if (!bf16 || B * K > 16 || B > 8 || (r != 320 && r != 512)) return false;
  const size_t lds = r == 512 ? seqhead_lds<16>(B * K, r) : seqhead_lds<10>(B * K, r);
  return lds + 2048 <= 160 * 1024;   // + static LDS of the kernel
}

size_t seqhead_fold_bytes(int M) { return static_cast<size_t>(M) * kFuseMaxHelpers * sizeof(uint64_t); }
size_t seqhead_sw_bytes(int M, int r) { return static_cast<size_t>(M) * (r / 2) * sizeof(uint64_t); }

namespace {
// Grid of the fused kernel (one workgroup per CU, at least 8 per team member).
int seqhead_grid(int B, int r) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int team = scan_detail::team_size(r, B);
  return cus > team * 8 ? cus : team * 8;
}
}  // namespace

int seqhead_p_slices(int B, int K, int r, int D) {
  if (!seqhead_fused(B, K, r, true) || D % 32) return 0;
  const int G = seqhead_grid(B, r) - scan_detail::team_size(r, B) * B;
  const int tiles = r / 16, nst = D / 32;
  // few slices: fewer words for the team to sum, and the helpers without a
  // share start their vocabulary loads at once (4 measured best at the 8B
  // shape); at least as many as keep every wave's share within its kPSteps
  // registers, at most one helper per (row tile, slice)
  const int need = (nst + kWaves * kPSteps - 1) / (kWaves * kPSteps);
  int nps = need > 4 ? need : 4;
  if (nps > G / tiles || nps > 16) return 0;
  return nps;
}

size_t seqhead_pw_bytes(int M, int r, int slices) {
  return static_cast<size_t>(slices) * M * r * sizeof(uint64_t);
}

hipError_t launch_seqhead(const ScanArgs& s0, const LmArgs& l0, uint64_t* px, uint64_t* sw, const GemmArgs* ph,
                          uint64_t* pw,
                          hipStream_t st) {
  using namespace scan_detail;
  if (!seqhead_fused(s0.B, s0.K, s0.r, true) || l0.M != s0.B * s0.K || l0.tok0 != 0) return hipErrorInvalidValue;
  FuseArgs f{};
  f.sa = s0;
  f.sa.rpt = 1;
  f.sa.tag0 = 0;
  f.nteam = s0.B;
  f.sw = sw;
  f.px = px;
  if (ph) {
    f.nps = seqhead_p_slices(s0.B, s0.K, s0.r, ph->K);
    if (f.nps == 0 || !pw || ph->M != l0.M || ph->N != s0.r) return hipErrorInvalidValue;
    f.ph = *ph;
    f.sa.Pw = pw;
    f.sa.Pslices = f.nps;
  }
  const int team = team_size(s0.r, s0.B);
  const int grid = seqhead_grid(s0.B, s0.r);
  if (grid == 0) return hipErrorInvalidDevice;
  f.la = l0;
  f.la.G = grid - team * f.nteam;
  if (f.la.G > kFuseMaxHelpers) return hipErrorInvalidValue;
  if (f.nps * (s0.r / 16) > f.la.G) return hipErrorInvalidValue;
  const int RK = s0.r / 32;
  const size_t sm_scan = team_lds(s0.r, team, 1, s0.K, true, &f.sa.stage);
  const void* fn = RK == 16 ? reinterpret_cast<const void*>(&seqhead_kernel<16>)
                            : reinterpret_cast<const void*>(&seqhead_kernel<10>);
  size_t sm = RK == 16 ? seqhead_lds<16>(l0.M, s0.r) : seqhead_lds<10>(l0.M, s0.r);
  sm = sm > sm_scan ? sm : sm_scan;
  const size_t sm_p = (kWaves * 64 * 4 + 16) * sizeof(float);   // the P partial's reduction
  sm = sm > sm_p ? sm : sm_p;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
  if (e != hipSuccess) return e;
  if (RK == 16) launch_k(seqhead_kernel<16>, dim3(grid), dim3(kWaves * 64), sm, st, f);
  else launch_k(seqhead_kernel<10>, dim3(grid), dim3(kWaves * 64), sm, st, f);
  return hipGetLastError();
}

bool gatedhead_fused(int B, int K, int r, int V, bool bf16) {
  if (!bf16 || r != kGR || B < 1 || B > 8 || K < 1 || K > 255 || V < 1 || V >= (1 << 24)) return false;
  int dev = 0, coop = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (cus - kGTeam < 64 || cus - kGTeam > kFuseMaxHelpers) return false;
  return gatedhead_lds<16>(B, r) + 2048 <= 160 * 1024;
}

size_t gatedhead_exchange_bytes(int B, int r) {
  return static_cast<size_t>(B) * (r + r / 2 + 1 + kFuseMaxHelpers) * sizeof(uint64_t);
}

hipError_t launch_gatedhead(const GatedFuseArgs& f0, hipStream_t st) {
  if (!gatedhead_fused(f0.B, f0.K, f0.la.r, f0.la.V, true)) return hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  GatedFuseArgs f = f0;
  f.la.G = cus - kGTeam;
  const size_t sm = gatedhead_lds<16>(f.B, f.la.r);
  const void* fn = reinterpret_cast<const void*>(&gatedhead_kernel<16>);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
  if (e != hipSuccess) return e;
  void* args[] = {&f};
  // a cooperative launch takes no dispatch events: an armed stage is timed
  // by markers around it
  StageTimer& t = stage_timer();
  if (t.active && !t.started) {
    e = hipEventRecord(t.start, st);
    if (e != hipSuccess) return e;
  }
  e = hipLaunchCooperativeKernel(fn, dim3(cus), dim3(kWaves * 64), args, static_cast<unsigned>(sm), st);
  if (e != hipSuccess) return e;
  if (t.active) {
    t.started = true;
    e = hipEventRecord(t.stop, st);
  }
  return e;
}

hipError_t launch_lmhead(const LmArgs& a0, bool bf16, hipStream_t st) {
  // many tokens: one tiled MFMA launch writes per-tile partials
  GemmArgs g{};
  g.W = a0.W; g.ldw = a0.r; g.N = a0.V; g.K = a0.r;
  g.src = a0.src; g.ld_src = a0.r; g.smap = RowMap{1, 1, 0}; g.M = a0.M; g.tok0 = a0.tok0;
  g.tap = a0.tap; g.ld_tap = a0.V; g.tmap = a0.omap;
  g.part_max = a0.part_max; g.part_idx = a0.part_idx; g.G_part = gemm_tile_groups(a0.V);
  if (vocab_tiled(a0.M, a0.V, a0.r, bf16) && vocab_slots(a0.M) <= a0.G_cap) {
    hipError_t e = launch_vocab(g, st);
    if (e != hipSuccess) return e;
    LmArgs a = a0;
    a.G = vocab_slots(a0.M);
    launch_k(lmhead_reduce_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (gemm_tiled(g, bf16)) {
    hipError_t e = launch_gemm_tiled(&g, 1, EPI_ARGMAX, a0.part, st);
    if (e != hipSuccess) return e;
    LmArgs a = a0;
    a.G = g.G_part;
    launch_k(lmhead_reduce_kernel, dim3((a.M + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(a0.G), block(kWaves * 64);
  for (int t0 = 0; t0 < a0.M; t0 += 32) {
    LmArgs a = a0;
    a.tok0 = a0.tok0 + t0;
    a.M = (a0.M - t0) < 32 ? (a0.M - t0) : 32;
    if (bf16) {
      if (a.M <= 16) launch_k((lmhead_pipe_kernel<uint16_t>), grid, block, 0, st, a);
      else launch_k((lmhead_kernel<uint16_t, 2>), grid, block, 0, st, a);
    } else {
      if (a.M <= 16) launch_k((lmhead_pipe_kernel<float>), grid, block, 0, st, a);
      else launch_k((lmhead_kernel<float, 2>), grid, block, 0, st, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dlite
