// LDS-tiled bf16 MFMA GEMM for many activation rows (batched draft steps).
//
// Once a linear map meets hundreds of token rows, each weight byte carries
// hundreds of multiply-adds and the maps become MFMA-bound, so the weights are
// no longer streamed past a tiny token block.  The output is cut into tiles of
// 256 weight rows x 128 tokens; four waves each own a 128 x 64 block of one
// tile and compute it with 32x32x16 MFMAs whose fragments come from LDS.  K is
// walked in 64-wide stages fetched with 16-byte loads into registers.  LDS
// rows are 128 bytes with the 16-byte chunks of row R stored at position
// (chunk ^ ((R >> 1) & 7)), so each 16-lane group of a fragment load (16
// consecutive rows) hits distinct banks without padding.
//
// Launches of at most 256 work items run the pipelined loop, one workgroup
// per CU: two register stages in flight and two 48 KB LDS buffers, one
// barrier per stage, the next stage's stores interleaved with the MFMAs and
// the fragments read one k step ahead.  Its steady-state loads are
// unconditional: with conditional loads the compiler's wait counting loses
// track of which register stage is older and waits for every load.  Larger
// launches keep one register stage and one buffer, with two workgroups per CU
// so that one's loads and barriers overlap the other's MFMAs.
//
// SwiGLU (gate/up) tiles are sized so that the launch fills one pipelined
// round: 128 outputs (four 32-row blocks per wave, gate and up rows in
// alternate 64-row halves), 96 outputs (three blocks) when 128-output tiles
// would leave CUs idle, 192 outputs (six blocks) when they would need a
// second round; in the three- and six-block shapes each 32-row block holds
// the gate rows and then the up rows of the same 16 outputs.
//
// Launches with fewer output tiles than CUs split K (rounded down, so the
// slices stay one round): work item (tile, slice) stores its fp32
// accumulators as a partial tile, and a second launch of the same kernel adds
// the slices of each tile in slice order (deterministic) and runs the
// epilogue, one wave per (128-row quarter, 32-token block) of a tile.

// Tiles are numbered with the token tile fastest and handed out per XCD in
// contiguous ranges, so the token tiles that share a weight tile run side by
// side on one XCD and read the weight tile through one L2.  Up to two
// independent problems with the same K (e.g. query rows of the local tokens
// and key/value rows of every slot) share one launch.
//
// Epilogues match the weight-streaming kernel (same argument block): plain
// stores, residual update with pre-gained copy and partial sums of squares,
// SwiGLU pairs, and for the vocabulary projection a per-tile (max, index)
// partial with ties to the lower index.
#include <type_traits>

#include "kernels.hpp"

namespace dlite {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBN = 256;        // weight rows per workgroup tile
constexpr int kBK = 64;         // k per stage
constexpr int kRowB = kBK * 2;  // bytes of one LDS row
constexpr int kBM = 128;        // tokens per workgroup tile
constexpr int kTileFloats = kBN * kBM;   // one fp32 partial tile
constexpr int kSplitTarget = 256;        // work items wanted per launch
constexpr int kSplitBelow = 128;         // split K only for launches with fewer tiles
constexpr int kMinSlice = 4;             // stages per k slice, at least
constexpr int kDirectSum = 2;            // slices the epilogue pass adds itself
constexpr int kPipeItems = 256;          // work items up to which the main loop is pipelined

// MODE_REDUCE1: the reduce pass with one wave per workgroup (8 workgroups
// per output tile) for epilogues that need no exchange between waves.
enum Mode { MODE_FULL = 0, MODE_SLICE = 1, MODE_REDUCE = 2, MODE_REDUCE1 = 3 };

__device__ __forceinline__ floatx16 mma32(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-byte chunk c of LDS row r sits at position c ^ ((r >> 1) & 7): the 16
// rows read by each 16-lane group of a fragment load cover all 64 banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Weight row behind LDS row l of output tile nb (SwiGLU: 64-row blocks
// alternate gate and up rows of the same 64 outputs).
template <int EPI, int WTN>
__device__ __forceinline__ long weight_row(const GemmArgs& a, int nb, int l) {
  if (EPI == EPI_SWIGLU && WTN != 4) {
    // 32 WTN rows per wave: each 32-row block holds the gate rows (first 16)
    // and the up rows (last 16) of the same 16 outputs
    const int w = l / (32 * WTN), r = l % (32 * WTN), i = r >> 5, h = r & 31;
    int n = nb * (32 * WTN) + w * (16 * WTN) + i * 16 + (h & 15);
    n = n < a.N ? n : a.N - 1;
    return n + ((h & 16) ? a.pair_off : 0);
  }
  if (EPI == EPI_SWIGLU) {
    const int q = l >> 6;
    int n = nb * (kBN / 2) + (q >> 1) * 64 + (l & 63);
    n = n < a.N ? n : a.N - 1;
    return n + ((q & 1) ? a.pair_off : 0);
  }
  int n = nb * kBN + l;
  return n < a.N ? n : a.N - 1;
}

template <int EPI, int MODE, int PIPE, int WTN>
__global__ __launch_bounds__(256, PIPE ? 1 : 2) void gemm_tile_kernel(TileArgs ta) {
  static_assert(WTN == 4 || EPI == EPI_SWIGLU, "three- and six-block waves only for SwiGLU");
  constexpr int WTM = 2;                      // 32-token blocks per wave
  constexpr int kBN = 64 * WTN;               // weight rows per tile (WTN 32-row blocks per wave)
  constexpr int WR = 32 * WTN;                // weight rows per wave
  constexpr int NT = 256;                     // four waves, 2 x 2 over the tile
  constexpr int BM = kBM;
  constexpr int ROWS = kBN + BM;              // LDS rows per stage
  constexpr int NLD = ROWS * 8 / NT;          // 16-byte loads per thread per stage
  constexpr int NLA = kBN * 8 / NT;           // of which weight loads
  constexpr int TPT = NT / BM;                // threads per token for the norm sums
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* lds = reinterpret_cast<uint4*>(smem);                      // [ROWS * 8] chunks
  constexpr int NBUF = MODE == MODE_FULL || MODE == MODE_SLICE ? 1 + PIPE : 0;   // LDS stage buffers
  float* red = reinterpret_cast<float*>(smem + NBUF * ROWS * kRowB);   // [TPT][BM]
  float* bv_s = red + TPT * BM;                                     // [2][BM] argmax values
  int* bi_s = reinterpret_cast<int*>(bv_s + 2 * BM);                // [2][BM] argmax indices

  // ---- work item: XCD x (workgroups x, x + 8, ...) owns items
  //      [x per_xcd, (x+1) per_xcd); within a problem the token tile is
  //      fastest, then the k slice, then the weight tile, so the token tiles
  //      of one weight slice run side by side on one XCD
  const int S = MODE == MODE_SLICE ? ta.ksplit : 1;
  // MODE_REDUCE1: eight one-wave workgroups per tile, one per (wave
  // quarter, 32-token block)
  constexpr int Q4 = MODE == MODE_REDUCE1 ? 8 : 1;   // workgroups per tile
  const int bid = blockIdx.x;
  int t = (bid & 7) * ta.per_xcd + (bid >> 3);
  if (t >= ta.total * S * Q4) return;
  const int quarter = t % Q4;
  t /= Q4;
  const int sg = t < ta.tiles0 * S ? 0 : 1;
  if (sg) t -= ta.tiles0 * S;
  const GemmArgs& a = ta.seg[sg];
  const int nbm = ta.nbm[sg];
  const int mb = t % nbm, rest = t / nbm;
  const int slice = rest % S, nb = rest / S;
  const int m0 = mb * BM;
  const int tile = (sg ? ta.tiles0 : 0) + nb * nbm + mb;   // index of the output tile

  // tid: the thread's place in the 4-wave tile layout (one wave per
  // workgroup in MODE_REDUCE1)
  const int tid = MODE == MODE_REDUCE1 ? (quarter >> 1) * 64 + static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x);
  const int uq = MODE == MODE_REDUCE1 ? (quarter & 1) : -1;   // the one token block of a reduce wave
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int fr = lane & 31, fk = lane >> 5;

  floatx16 acc[WTN][WTM];
#pragma unroll
  for (int i = 0; i < WTN; ++i)
#pragma unroll
    for (int u = 0; u < WTM; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][u][e] = 0.f;

  // partial tile layout: float4 j of thread tid at (j * 256 + tid) * 4
  auto part_at = [&](int sl) { return ta.part + (static_cast<long>(tile) * ta.ksplit + sl) * kTileFloats; };

  if (MODE == MODE_FULL || MODE == MODE_SLICE) {
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    const uint16_t* X = static_cast<const uint16_t*>(a.src);
    // ---- stage loads: thread covers rows (tid / 8) + 32 i, 16-byte chunk tid % 8
    const int kc = tid & 7;
    const uint16_t* gp[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int row = (tid >> 3) + i * (NT / 8);
      if (i < NLA) {
        gp[i] = W + weight_row<EPI, WTN>(a, nb, row) * a.ldw + kc * 8;
      } else {
        int tk = m0 + row - kBN;
        tk = tk < a.M ? tk : a.M - 1;
        gp[i] = X + a.smap.row(a.tok0 + tk) * a.ld_src + kc * 8;
      }
    }
    const int nk = a.K / kBK;
    const int k0 = (slice * nk) / S, k1 = ((slice + 1) * nk) / S;
    // two register stages and two LDS buffers: while stage kt is multiplied
    // out of one buffer, stage kt + 1 waits in registers for the other and
    // stage kt + 2 is on its way from memory
    uint4 ra[NLD], rb[NLD];
    auto load_stage = [&](uint4 (&r)[NLD], int kt) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint16_t* q = gp[i] + static_cast<long>(kt) * kBK;
        r[i] = i < NLA ? ld_stream(q) : *reinterpret_cast<const uint4*>(q);
      }
    };
    auto store_stage = [&](const uint4 (&r)[NLD], int buf) {
      uint4* l = lds + buf * (ROWS * 8);
#pragma unroll
      for (int i = 0; i < NLD; ++i) l[swz((tid >> 3) + i * (NT / 8), kc)] = r[i];
    };
    auto compute = [&](int buf) {
      const uint4* l = lds + buf * (ROWS * 8);
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        const int ch = 2 * ks + fk;
        uint4 af[WTN], bf[WTM];
#pragma unroll
        for (int i = 0; i < WTN; ++i) af[i] = l[swz(wn * WR + i * 32 + fr, ch)];
#pragma unroll
        for (int u = 0; u < WTM; ++u) bf[u] = l[swz(kBN + wm * (BM / 2) + u * 32 + fr, ch)];
#pragma unroll
        for (int i = 0; i < WTN; ++i)
#pragma unroll
          for (int u = 0; u < WTM; ++u) acc[i][u] = mma32(af[i], bf[u], acc[i][u]);
      }
    };
    // the pipelined step: the fragments of k step ks + 1 are read while the
    // MFMAs of ks run, and the next stage's registers go into the other
    // buffer between them (a quarter per k step)
    auto compute_store = [&](int buf, const uint4 (&r)[NLD]) {
      const uint4* l = lds + buf * (ROWS * 8);
      uint4* lw = lds + (buf ^ 1) * (ROWS * 8);
      uint4 af[2][WTN], bf[2][WTM];
      auto rd = [&](int ks, int h) {
        const int ch = 2 * ks + fk;
#pragma unroll
        for (int i = 0; i < WTN; ++i) af[h][i] = l[swz(wn * WR + i * 32 + fr, ch)];
#pragma unroll
        for (int u = 0; u < WTM; ++u) bf[h][u] = l[swz(kBN + wm * (BM / 2) + u * 32 + fr, ch)];
      };
      rd(0, 0);
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        if (ks + 1 < kBK / 16) rd(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = ks * NLD / (kBK / 16); i < (ks + 1) * NLD / (kBK / 16); ++i)
          lw[swz((tid >> 3) + i * (NT / 8), kc)] = r[i];
#pragma unroll
        for (int i = 0; i < WTN; ++i)
#pragma unroll
          for (int u = 0; u < WTM; ++u) acc[i][u] = mma32(af[ks & 1][i], bf[ks & 1][u], acc[i][u]);
        __builtin_amdgcn_sched_barrier(0);   // keep the reads a k step ahead
      }
    };
    int kt = k0;
    if (PIPE && k1 - k0 >= 4) {
      load_stage(ra, k0);
      load_stage(rb, k0 + 1);
      store_stage(ra, 0);
      __syncthreads();
      load_stage(ra, k0 + 2);
      // steady state: buffer 0 holds stage kt, rb stage kt + 1, ra stage
      // kt + 2.  The loads here are unconditional so that the wait before
      // each buffer store covers only the older register stage.
      for (; kt + 4 < k1; kt += 2) {
        compute_store(0, rb);
        __syncthreads();
        load_stage(rb, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute_store(1, ra);
        __syncthreads();
        load_stage(ra, kt + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the last three or four stages
      auto step = [&](int k, int b, uint4 (&r)[NLD]) {
        compute(b);
        if (k + 1 < k1) store_stage(r, b ^ 1);
        __syncthreads();
        if (k + 3 < k1) load_stage(r, k + 3);
      };
      for (; kt < k1; kt += 2) {
        step(kt, 0, rb);
        if (kt + 1 < k1) step(kt + 1, 1, ra);
      }
    } else {
      // one register stage, one buffer (two workgroups per CU, or short k slices)
      load_stage(ra, k0);
      store_stage(ra, 0);
      __syncthreads();
      for (; kt < k1; ++kt) {
        if (kt + 1 < k1) load_stage(ra, kt + 1);
        compute(0);
        __syncthreads();
        if (kt + 1 < k1) {
          store_stage(ra, 0);
          __syncthreads();
        }
      }
    }
    if (MODE == MODE_SLICE) {
      float4* pp = reinterpret_cast<float4*>(part_at(slice));
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int u = 0; u < WTM; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pp[((i * WTM + u) * 4 + q) * NT + tid] =
                make_float4(acc[i][u][4 * q], acc[i][u][4 * q + 1], acc[i][u][4 * q + 2], acc[i][u][4 * q + 3]);
      return;
    }
  } else {
    // ---- add the k slices of this tile in slice order (or read slice 0
    //      when a parallel pass has already added them there)
    for (int sl = 0; sl < ta.nsum; ++sl) {
      const float4* pp = reinterpret_cast<const float4*>(part_at(sl));
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int u = 0; u < WTM; ++u) {
          if (MODE == MODE_REDUCE1 && u != uq) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = pp[((i * WTM + u) * 4 + q) * NT + tid];
            acc[i][u][4 * q] += v.x;
            acc[i][u][4 * q + 1] += v.y;
            acc[i][u][4 * q + 2] += v.z;
            acc[i][u][4 * q + 3] += v.w;
          }
        }
    }
  }

  // ---- partial sums of squares of this tile's tokens (TPT threads per token;
  //      in MODE_REDUCE1 one thread per token of the wave's half)
  if (a.ssq && MODE == MODE_REDUCE1) {
    const int tl = wm * (BM / 2) + lane;
    float v = 0.f;
    const int tk = m0 + tl;
    if (tk < a.M) {
      const long prow = a.qmap.row(a.tok0 + tk);
      const int np = (prow % a.ssq_group) < a.ssq_split ? a.np_lo : a.np_hi;
      const float* sp = a.ssq + prow * kSsqParts;
      for (int j = 0; j < np; ++j) v += sp[j];
    }
    red[tl] = v;
    red[BM + tl] = 0.f;
  } else if (a.ssq) {
    const int tl = tid % BM, part = tid / BM;
    float v = 0.f;
    const int tk = m0 + tl;
    if (tk < a.M) {
      const long prow = a.qmap.row(a.tok0 + tk);
      const int np = (prow % a.ssq_group) < a.ssq_split ? a.np_lo : a.np_hi;
      const float* sp = a.ssq + prow * kSsqParts;
      for (int j = part; j < np; j += TPT) v += sp[j];
    }
    red[part * BM + tl] = v;
  }
  __syncthreads();

  // ---- epilogue: lane holds token column fr of each 32x32 block and rows
  //      8 q + 4 fk + (0..3) of it
  float inv[WTM];
  int tk[WTM];
  bool tok_ok[WTM];
#pragma unroll
  for (int u = 0; u < WTM; ++u) {
    const int tloc = wm * (BM / 2) + u * 32 + fr;
    tk[u] = m0 + tloc;
    tok_ok[u] = tk[u] < a.M;
    inv[u] = 1.f;
    if (a.ssq) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < TPT; ++q) v += red[q * BM + tloc];
      inv[u] = 1.0f / sqrtf(v / static_cast<float>(a.norm_len) + a.eps);
    }
  }

  if (EPI == EPI_ARGMAX && MODE != MODE_REDUCE1) {
    // a lane's values come in increasing row order, so "strictly greater"
    // keeps the lowest index among equal maxima; rows past N only exist in
    // the last weight tile
    const int nbase = nb * kBN + wn * WR + 4 * fk;
    const bool full = nb * kBN + kBN <= a.N;
#pragma unroll
    for (int u = 0; u < WTM; ++u) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      if (full) {
#pragma unroll
        for (int i = 0; i < WTN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = acc[i][u][4 * q + e];
              const bool gt = v > bv;
              bv = gt ? v : bv;
              bi = gt ? nbase + i * 32 + 8 * q + e : bi;
            }
      } else {
#pragma unroll
        for (int i = 0; i < WTN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int n = nbase + i * 32 + 8 * q + e;
              const float v = acc[i][u][4 * q + e];
              const bool gt = v > bv && n < a.N;
              bv = gt ? v : bv;
              bi = gt ? n : bi;
            }
      }
      const float ov = __shfl_xor(bv, 32, kWave);
      const int oi = __shfl_xor(bi, 32, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      if (fk == 0) {
        const int tloc = wm * (BM / 2) + u * 32 + fr;
        bv_s[wn * BM + tloc] = bv;
        bi_s[wn * BM + tloc] = bi;
      }
    }
    if (a.tap) {   // logits copy (the sampled path reads it)
      // four consecutive rows per (i, q): one 16-byte store when the rows
      // exist and the row stride keeps them aligned
      const bool vec = full && (a.ld_tap & 3) == 0 && (reinterpret_cast<uintptr_t>(a.tap) & 15) == 0;
#pragma unroll
      for (int u = 0; u < WTM; ++u) {
        if (!tok_ok[u]) continue;
        float* trow = a.tap + a.tmap.row(a.tok0 + tk[u]) * a.ld_tap;
#pragma unroll
        for (int i = 0; i < WTN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = nbase + i * 32 + 8 * q;
            if (vec) {
              *reinterpret_cast<float4*>(trow + n) =
                  make_float4(acc[i][u][4 * q], acc[i][u][4 * q + 1], acc[i][u][4 * q + 2], acc[i][u][4 * q + 3]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < a.N) trow[n + e] = acc[i][u][4 * q + e];
            }
          }
      }
    }
    __syncthreads();
    if (tid < BM && m0 + tid < a.M) {
      float v = bv_s[tid];
      int ix = bi_s[tid];
      if (better(bv_s[BM + tid], bi_s[BM + tid], v, ix)) { v = bv_s[BM + tid]; ix = bi_s[BM + tid]; }
      const long o = static_cast<long>(a.tok0 + m0 + tid) * a.G_part + nb;
      a.part_max[o] = v;
      a.part_idx[o] = ix;
    }
    return;
  }

  // stores of token block u; CHK: rows past N possible (last weight tile)
  auto store_u = [&](int u, auto chk) {
    constexpr bool CHK = decltype(chk)::value;
    const long orow = a.omap.row(a.tok0 + tk[u]);
    if (EPI == EPI_SWIGLU && WTN != 4) {
      // gate rows 8 q + 4 fk + e (q < 2) and up rows 16 + the same of each block
      uint16_t* out = static_cast<uint16_t*>(a.out) + orow * a.ld_out;
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int n = nb * (32 * WTN) + wn * (16 * WTN) + i * 16 + 8 * q + 4 * fk;
          if (CHK && n >= a.N) continue;
          uint32_t h[2];
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            float r2[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const float gt = acc[i][u][4 * q + e + f] * inv[u];
              const float up = acc[i][u][4 * (q + 2) + e + f] * inv[u];
              r2[f] = gt / (1.0f + expf(-gt)) * up;
            }
            h[e / 2] = static_cast<uint32_t>(f32_to_bf16(r2[0])) |
                       (static_cast<uint32_t>(f32_to_bf16(r2[1])) << 16);
          }
          *reinterpret_cast<uint2*>(out + n) = make_uint2(h[0], h[1]);
        }
    } else if (EPI == EPI_SWIGLU) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + orow * a.ld_out;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb * (kBN / 2) + wn * 64 + i * 32 + 8 * q + 4 * fk;
          if (CHK && n >= a.N) continue;
          uint32_t h[2];
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            float r2[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const float gt = acc[i][u][4 * q + e + f] * inv[u];
              const float up = acc[i + 2 < WTN ? i + 2 : 0][u][4 * q + e + f] * inv[u];
              r2[f] = gt / (1.0f + expf(-gt)) * up;
            }
            h[e / 2] = static_cast<uint32_t>(f32_to_bf16(r2[0])) |
                       (static_cast<uint32_t>(f32_to_bf16(r2[1])) << 16);
          }
          *reinterpret_cast<uint2*>(out + n) = make_uint2(h[0], h[1]);
        }
    } else {
      float ssq = 0.f;
      // residual epilogue of the reduce pass: the residual and gain loads of
      // a 32-row block go out together before any of its stores (a load
      // issued after a store the compiler cannot tell apart waits a round
      // trip; the full-K kernel keeps its registers for the main loop)
      constexpr bool kBatch = EPI == EPI_RESID && MODE == MODE_REDUCE1;
      float4 xr[4];
      uint2 gr[4];
      auto fetch = [&](int i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int n = nb * kBN + wn * WR + i * 32 + 8 * q + 4 * fk;
          n = (CHK && n >= a.N) ? nb * kBN : n;   // in range; unused
          xr[q] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.out) + orow * a.ld_out + n);
          gr[q] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.next_gain) + n);
        }
      };
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (kBatch && q == 0) fetch(i);
          const int n = nb * kBN + wn * WR + i * 32 + 8 * q + 4 * fk;
          if (CHK && n >= a.N) continue;
          const float4 y = make_float4(acc[i][u][4 * q] * inv[u], acc[i][u][4 * q + 1] * inv[u],
                                       acc[i][u][4 * q + 2] * inv[u], acc[i][u][4 * q + 3] * inv[u]);
          if (EPI == EPI_STORE_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * a.ld_out + n) = y;
          } else if (EPI == EPI_STORE_ACT) {
            const uint32_t h0 = static_cast<uint32_t>(f32_to_bf16(y.x)) | (static_cast<uint32_t>(f32_to_bf16(y.y)) << 16);
            const uint32_t h1 = static_cast<uint32_t>(f32_to_bf16(y.z)) | (static_cast<uint32_t>(f32_to_bf16(y.w)) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow * a.ld_out + n) = make_uint2(h0, h1);
          } else {  // residual
            float4* xp = reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * a.ld_out + n);
            float4 x = kBatch ? xr[q] : *xp;
            x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
            *xp = x;
            ssq += (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w);
            const uint2 gw = kBatch ? gr[q] : *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.next_gain) + n);
            const float g0 = __uint_as_float(gw.x << 16), g1 = __uint_as_float(gw.x & 0xffff0000u);
            const float g2 = __uint_as_float(gw.y << 16), g3 = __uint_as_float(gw.y & 0xffff0000u);
            const uint32_t h0 = static_cast<uint32_t>(f32_to_bf16(g0 * x.x)) | (static_cast<uint32_t>(f32_to_bf16(g1 * x.y)) << 16);
            const uint32_t h1 = static_cast<uint32_t>(f32_to_bf16(g2 * x.z)) | (static_cast<uint32_t>(f32_to_bf16(g3 * x.w)) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.xb_out) + a.xmap.row(a.tok0 + tk[u]) * a.ld_xb + n) =
                make_uint2(h0, h1);
            if (a.tap)
              *reinterpret_cast<float4*>(a.tap + a.tmap.row(a.tok0 + tk[u]) * a.ld_tap + n) = x;
          }
        }
      if (EPI == EPI_RESID && a.ssq_out) {
        // the two row halves of this token's 128 rows sit in lanes fr, fr + 32
        ssq += __shfl_xor(ssq, 32, kWave);
        if (fk == 0) a.ssq_out[orow * kSsqParts + (nb * kBN + wn * WR) / 128] = ssq;
      }
    }
  };
  const int bno = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const bool full = (nb + 1) * bno <= a.N;
#pragma unroll
  for (int u = 0; u < WTM; ++u) {
    // the ssq shuffle pairs lanes fr and fr + 32, which share tok_ok
    if (!tok_ok[u] || (MODE == MODE_REDUCE1 && u != uq)) continue;
    if (full) store_u(u, std::integral_constant<bool, false>());
    else store_u(u, std::integral_constant<bool, true>());
  }
}

// Adds the k slices of every partial tile into slice 0, in slice order; one
// thread per 4 floats, spread over the whole chip.
__global__ __launch_bounds__(256) void slice_sum_kernel(float* part, int tiles, int ksplit) {
  const long q = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;   // float4 index within all tiles
  const long per = kTileFloats / 4;
  if (q >= static_cast<long>(tiles) * per) return;
  const long t = q / per, i = q % per;
  float4* base = reinterpret_cast<float4*>(part) + t * ksplit * per + i;
  float4 acc = base[0];
  for (int sl = 1; sl < ksplit; ++sl) {
    const float4 v = base[sl * per];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  base[0] = acc;
}

template <int EPI, int MODE, int PIPE, int WTN>
hipError_t launch_tile_t1(const TileArgs& ta, int items, hipStream_t st) {
  const size_t nbuf = MODE == MODE_FULL || MODE == MODE_SLICE ? 1 + PIPE : 0;
  const size_t sm = nbuf * (64 * WTN + kBM) * kRowB + (256ull + 4ull * kBM) * 4;
  const void* fn = reinterpret_cast<const void*>(&gemm_tile_kernel<EPI, MODE, PIPE, WTN>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
  if (e != hipSuccess) return e;
  const int per_xcd = (items + 7) / 8;
  TileArgs t = ta;
  t.per_xcd = per_xcd;
  launch_k((gemm_tile_kernel<EPI, MODE, PIPE, WTN>), dim3(8 * per_xcd), dim3(MODE == MODE_REDUCE1 ? 64 : 256), sm, st, t);
  return hipGetLastError();
}

// Main-loop passes with at most one work item per CU take the two-stage
// pipeline (one workgroup per CU); larger ones keep two workgroups per CU.
template <int EPI, int MODE, int WTN>
hipError_t launch_tile_t(const TileArgs& ta, int items, hipStream_t st) {
  if constexpr (MODE == MODE_FULL || MODE == MODE_SLICE) {
    if (items <= kPipeItems) return launch_tile_t1<EPI, MODE, 1, WTN>(ta, items, st);
  }
  return launch_tile_t1<EPI, MODE, 0, WTN>(ta, items, st);
}

template <int EPI, int WTN = 4>
hipError_t launch_tile_e(const TileArgs& ta, hipStream_t st) {
  if (ta.ksplit == 1) return launch_tile_t<EPI, MODE_FULL, WTN>(ta, ta.total, st);
  hipError_t e = launch_tile_t<EPI, MODE_SLICE, WTN>(ta, ta.total * ta.ksplit, st);
  if (e != hipSuccess) return e;
  TileArgs tr = ta;
  tr.nsum = ta.ksplit;
  if (ta.ksplit > kDirectSum) {
    // many slices: add them with the whole chip first, the epilogue pass reads one
    const long f4 = static_cast<long>(ta.total) * (kTileFloats / 4);
    launch_k(slice_sum_kernel, dim3(static_cast<unsigned>((f4 + 255) / 256)), dim3(256), 0, st,
                       ta.part, ta.total, ta.ksplit);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    tr.nsum = 1;
  }
  if constexpr (EPI == EPI_ARGMAX) return launch_tile_t<EPI, MODE_REDUCE, WTN>(tr, ta.total, st);
  else return launch_tile_t<EPI, MODE_REDUCE1, WTN>(tr, ta.total * 8, st);
}

// Output tiles of each problem and the k split of the launch.
struct TilePlan {
  int nbm[2], tiles[2], total, ksplit, wtn;
};

TilePlan plan_tiles(const int* M, const int* N, int nseg, int K, int epi) {
  TilePlan p{};
  auto count = [&](int bno) {
    p.total = 0;
    for (int s = 0; s < nseg; ++s) {
      p.nbm[s] = (M[s] + kBM - 1) / kBM;
      p.tiles[s] = M[s] > 0 ? ((N[s] + bno - 1) / bno) * p.nbm[s] : 0;
      p.total += p.tiles[s];
    }
  };
  // SwiGLU whose 128-output tiles leave CUs idle takes 96-output tiles
  // (three 32-row blocks per wave) when those still fit one pipelined round
  // without a k split
  p.wtn = 4;
  count(epi == EPI_SWIGLU ? kBN / 2 : kBN);
  if (epi == EPI_SWIGLU && p.total < kPipeItems) {
    count(96);
    if (p.total > kPipeItems || p.total < kSplitBelow) count(kBN / 2);
    else p.wtn = 3;
  } else if (epi == EPI_SWIGLU && p.total > kPipeItems) {
    // too many for one pipelined round: 192-output tiles (six blocks per wave)
    count(192);
    if (p.total > kPipeItems) count(kBN / 2);
    else p.wtn = 6;
  }
  // split K when the tiles leave CUs idle, keeping at least kMinSlice stages a slice
  p.ksplit = 1;
  const int nk = K / kBK;
  if (p.total > 0 && p.total < kSplitBelow) {
    int sp = kSplitTarget / p.total;   // rounded down: the slices stay one pipelined round
    const int smax = nk / kMinSlice;
    sp = sp < smax ? sp : smax;
    p.ksplit = sp > 1 ? sp : 1;
  }
  return p;
}

}  // namespace

bool gemm_tiled(const GemmArgs& a, bool bf16) {
  return bf16 && a.M >= kTileMinRows && a.K % kBK == 0;
}

int gemm_tile_groups(int N) { return (N + kBN - 1) / kBN; }

size_t gemm_tile_scratch(int M0, int M1, int N0, int N1, int K, int epi) {
  const int M[2] = {M0, M1}, N[2] = {N0, N1};
  const TilePlan p = plan_tiles(M, N, M1 > 0 ? 2 : 1, K, epi);
  return p.ksplit > 1 ? static_cast<size_t>(p.total) * p.ksplit * kTileFloats * sizeof(float) : 0;
}

hipError_t launch_gemm_tiled(const GemmArgs* segs, int nseg, int epi, float* part, hipStream_t st) {
  if (nseg < 1 || nseg > 2) return hipErrorInvalidValue;
  for (int s = 1; s < nseg; ++s)
    if (segs[s].K != segs[0].K) return hipErrorInvalidValue;
  int M[2] = {0, 0}, N[2] = {0, 0};
  for (int s = 0; s < nseg; ++s) { M[s] = segs[s].M; N[s] = segs[s].N; }
  const TilePlan p = plan_tiles(M, N, nseg, segs[0].K, epi);
  if (p.total == 0) return hipSuccess;
  TileArgs ta{};
  for (int s = 0; s < nseg; ++s) { ta.seg[s] = segs[s]; ta.nbm[s] = p.nbm[s]; }
  ta.tiles0 = p.tiles[0];
  ta.total = p.total;
  ta.ksplit = part ? p.ksplit : 1;
  ta.part = part;
  switch (epi) {
    case EPI_STORE_F32: return launch_tile_e<EPI_STORE_F32>(ta, st);
    case EPI_STORE_ACT: return launch_tile_e<EPI_STORE_ACT>(ta, st);
    case EPI_RESID: return launch_tile_e<EPI_RESID>(ta, st);
    case EPI_SWIGLU:
      if (p.wtn == 3) return launch_tile_e<EPI_SWIGLU, 3>(ta, st);
      if (p.wtn == 6) return launch_tile_t1<EPI_SWIGLU, MODE_FULL, 1, 6>(ta, ta.total, st);   // one round, never split
      return launch_tile_e<EPI_SWIGLU, 4>(ta, st);
    case EPI_ARGMAX: return launch_tile_e<EPI_ARGMAX>(ta, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dlite
