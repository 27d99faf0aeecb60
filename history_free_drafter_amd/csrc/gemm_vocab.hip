// Vocabulary projection with argmax for a few hundred token rows (batched
// draft steps), as one persistent MFMA launch.
//
// The projection is applied once, to every drafted position after the
// sequential head (DLite walkthrough, section "官方顺序头具体算了什么"), so at
// many requests it is one [tokens x r] by [r x V] product whose only output is
// a (max, index) per token.  With r = 512 every weight row is read once and
// meets every token row; the work is MFMA-bound once there are a few hundred
// tokens.
//
// One workgroup per CU.  An item is 256 vocabulary rows x 112 tokens.  The
// workgroup keeps one 112-token tile for all its items, resident in LDS
// (112 KB at r = 512, 16-byte chunks XOR-swizzled by row so each 16-lane
// fragment read hits distinct banks), and walks the vocabulary tiles of its
// XCD's range together with the workgroups of the other token tiles (the four
// token tiles of one vocabulary tile run side by side on one XCD and read the
// weights through one L2).  Each of the four waves owns 64 vocabulary rows:
// their MFMA fragments (16x16x32) are loaded straight into registers, eight
// 32-wide k steps ahead, so the main loop has no barrier and no LDS writes;
// the token fragments come from the resident tile.  Each lane keeps a running
// (max, index) of its own rows per token column over all its items; the
// workgroup's partials go out once, at the end, and a second launch reduces
// them per token with ties to the lower index.
#include "kernels.hpp"

namespace dlite {

namespace {


constexpr int kVN = 256;                      // vocabulary rows per item (64 per wave)
constexpr int kVT = 7;                        // token blocks of 16 per item
constexpr int kVM = 16 * kVT;                 // tokens per item (and per workgroup)
constexpr int kVKs = 32;                      // k per step
// weight steps in flight per wave (fewer with the logits copy, whose stores
// need registers of their own)
template <bool TAP> constexpr int kVD = TAP ? 4 : 8;
constexpr int kVWg = 256;                     // workgroups

struct VocabArgs {
  const uint16_t* W;   // [N, K]
  const uint16_t* X;   // token rows at (tok0 + t) * ld_src
  long ld_src;
  int N, K, M, tok0, mt;
  float* tap; long ld_tap; RowMap tmap;   // optional logits copy
  float* part_max; int* part_idx;         // [(tok0 + t) * slots + slot]
  int slots;
};

// 16 bytes per lane from global address g straight into LDS at byte address
// lds + 16 lane (lds is the same for the whole wave; inactive lanes write
// nothing).  Written as assembly so that the compiler does not treat every
// later LDS read as waiting on it (the kernel waits once, with wait_vm0 and a
// barrier).  The compiler does not look inside the assembly for hazards, so
// the address is a VGPR pair (no scalar operand that a VALU instruction may
// have just written) and five wait states separate the load from the write
// of M0 before it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <bool TAP, int KS>
__global__ __launch_bounds__(256, 1) void vocab_kernel(VocabArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* xs = reinterpret_cast<uint4*>(smem);   // [kVM rows][K / 8 chunks]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int c16 = lane & 15, grp = lane >> 4;

  // ---- this workgroup's token tile and vocabulary tiles
  const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
  const int wpx = gridDim.x >> 3;
  const int m = l % a.mt, p = l / a.mt, np = wpx / a.mt;
  const int NT = (a.N + kVN - 1) / kVN;
  const int nx0 = xcd * NT / 8, nx1 = (xcd + 1) * NT / 8;
  const int items = nx1 - nx0 > p ? (nx1 - nx0 - p + np - 1) / np : 0;
  constexpr int D = kVD<TAP>;
  static_assert(KS % D == 0, "whole prefetch rounds per item");   // KS = K / kVKs steps per item
  const int cpr = a.K / 8;                      // 16-byte chunks per token row

  // ---- weight fragments of step g: lane holds row c16 of each 16-row block
  //      i and the 8 k elements at grp * 8 of the step
  uint4 wv[D][4];
  auto issue = [&](int g, uint4 (&w)[4]) {
    const int it = g / KS, kk = g - it * KS;
    const int n = nx0 + p + it * np;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = n * kVN + wave * 64 + i * 16 + c16;
      row = row < a.N ? row : a.N - 1;
      w[i] = *reinterpret_cast<const uint4*>(a.W + static_cast<long>(row) * a.K + kk * kVKs + grp * 8);
    }
  };
  // (issued unconditionally, past the last step too: rows are clamped to the
  // matrix, and without branches the compiler's waits stay exact)
#pragma unroll
  for (int h = 0; h < D; ++h) issue(h, wv[h]);

  // ---- the token tile into LDS (direct loads, all in flight at once), chunk
  //      c of row R at position c ^ (R & 15)
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(smem))));
  for (int R = wave; R < kVM; R += 4) {
    int tk = m * kVM + R;
    tk = tk < a.M ? tk : a.M - 1;
    const uint16_t* xr = a.X + static_cast<long>(a.tok0 + tk) * a.ld_src;
    for (int c0 = 0; c0 < cpr; c0 += 64)
      if (c0 + lane < cpr)
        dma16(xr + ((c0 + lane) ^ (R & 15)) * 8, lds0 + static_cast<uint32_t>((R * cpr + c0) * 16));
  }
  wait_vm0();
  __syncthreads();

  float rv[kVT];
  int ri[kVT];
#pragma unroll
  for (int u = 0; u < kVT; ++u) { rv[u] = -INFINITY; ri[u] = 0x7fffffff; }

  // one step: 4 x kVT MFMAs; token fragment u is row u * 16 + c16 (so R & 15
  // = c16), k chunk kk * 4 + grp
  // (the item's first step starts its sums from zero).  Position of chunk
  // kk * 4 + grp of row u * 16 + c16: (kk / 4) * 16 + (((kk % 4) * 4 + grp) ^ c16),
  // so four per-lane bases and compile-time offsets cover every step
  constexpr int kCpr = KS * kVKs / 8;
  int xb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) xb[j] = c16 * kCpr + ((j * 4 + grp) ^ c16);
  auto load_b = [&](int kk, int u) { return xs[xb[kk & 3] + u * 16 * kCpr + (kk >> 2) * 16]; };
  // token fragments of step kk are in cur; those of the next step (the next
  // item's first for the last) are read into nxt between the MFMAs
  auto compute = [&](int kk, const uint4 (&w)[4], floatx4 (&acc)[4][kVT], const uint4 (&cur)[kVT],
                     uint4 (&nxt)[kVT]) {
    const int kn = kk + 1 < KS ? kk + 1 : 0;
#pragma unroll
    for (int u = 0; u < kVT; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][u] = mma_step(w[i], cur[u], kk == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[i][u], uint16_t());
      nxt[u] = load_b(kn, u);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // four MFMAs,
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then one LDS read
    }
  };

  // end of an item: lane (c16, grp) of block (i, u) holds token u * 16 + c16
  // at rows nb + i * 16 + e, nb = item rows + wave * 64 + 4 grp
  auto argmax_rows = [&](const floatx4 (&acc)[4][kVT], int nb, auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;   // rows past N only in the last tile
#pragma unroll
    for (int u = 0; u < kVT; ++u) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (FULL || nb + i * 16 + e < a.N) mx = fmaxf(mx, acc[i][u][e]);
      // a later item's rows are higher: equal maxima keep the earlier index
      if (mx > rv[u]) {
        int ix = 0x7fffffff;
#pragma unroll
        for (int i = 3; i >= 0; --i)
#pragma unroll
          for (int e = 3; e >= 0; --e)
            ix = (acc[i][u][e] == mx && (FULL || nb + i * 16 + e < a.N)) ? nb + i * 16 + e : ix;
        rv[u] = mx;
        ri[u] = ix;
      }
    }
  };
  auto finish_item = [&](const floatx4 (&acc)[4][kVT], int n) {
    const int nb = n * kVN + wave * 64 + 4 * grp;
    const bool full = n * kVN + kVN <= a.N;
    if (full) argmax_rows(acc, nb, std::true_type());
    else argmax_rows(acc, nb, std::false_type());
    if (TAP) {
      // through LDS, one 16-token block at a time, so that each token's 256
      // logits of the item go out as one contiguous kilobyte: the waves put
      // their rows in place (rows padded by 4 floats: the 16 tokens of a
      // 16-byte write hit distinct banks), then wave w writes tokens
      // 4 w .. 4 w + 3
      const bool vec = full && (a.ld_tap & 3) == 0 && (reinterpret_cast<uintptr_t>(a.tap) & 15) == 0;
      float* st = reinterpret_cast<float*>(smem + static_cast<size_t>(kVM) * kCpr * 16);   // [16][kVN + 4]
      const int row0 = n * kVN;
#pragma unroll
      for (int u = 0; u < kVT; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(st + c16 * (kVN + 4) + wave * 64 + i * 16 + 4 * grp) =
              make_float4(acc[i][u][0], acc[i][u][1], acc[i][u][2], acc[i][u][3]);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = wave * 4 + q;
          const int tk = m * kVM + u * 16 + t;
          if (tk < a.M) {
            const float4 v = *reinterpret_cast<const float4*>(st + t * (kVN + 4) + lane * 4);
            float* trow = a.tap + a.tmap.row(a.tok0 + tk) * a.ld_tap + row0 + lane * 4;
            if (vec) {
              *reinterpret_cast<float4*>(trow) = v;
            } else {
              const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row0 + lane * 4 + e < a.N) trow[e] = f[e];
            }
          }
        }
        __syncthreads();
      }
    }
  };

  // ---- items one after another; the weight slot of step kk is refilled
  //      with the step D later (the next item's for the last steps) once
  //      its MFMAs are issued
  uint4 bf[2][kVT];
#pragma unroll
  for (int u = 0; u < kVT; ++u) bf[0][u] = load_b(0, u);
  for (int it = 0; it < items; ++it) {
    floatx4 acc[4][kVT];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      compute(kk, wv[kk % D], acc, bf[kk & 1], bf[(kk + 1) & 1]);   // KS even
      issue(it * KS + kk + D, wv[kk % D]);
      __builtin_amdgcn_sched_barrier(0);   // one step at a time (register pressure)
    }
    finish_item(acc, nx0 + p + it * np);
  }

  // ---- the workgroup's partial per token: the four row groups of a token
  //      column sit in lanes c16, c16 + 16, c16 + 32, c16 + 48; the waves hold
  //      disjoint rows
#pragma unroll
  for (int u = 0; u < kVT; ++u) {
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(rv[u], o, kWave);
      const int oi = __shfl_xor(ri[u], o, kWave);
      if (better(ov, oi, rv[u], ri[u])) { rv[u] = ov; ri[u] = oi; }
    }
  }
  __syncthreads();   // every wave is done with the token tile
  float* sv = reinterpret_cast<float*>(smem);        // [4][kVM]
  int* si = reinterpret_cast<int*>(sv + 4 * kVM);    // [4][kVM]
  if (grp == 0) {
#pragma unroll
    for (int u = 0; u < kVT; ++u) {
      sv[wave * kVM + u * 16 + c16] = rv[u];
      si[wave * kVM + u * 16 + c16] = ri[u];
    }
  }
  __syncthreads();
  const int slot = xcd * np + p;
  for (int t = threadIdx.x; t < kVM; t += blockDim.x) {
    const int tk = m * kVM + t;
    if (tk >= a.M) continue;
    float v = sv[t];
    int ix = si[t];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (better(sv[w * kVM + t], si[w * kVM + t], v, ix)) { v = sv[w * kVM + t]; ix = si[w * kVM + t]; }
    const long o = static_cast<long>(a.tok0 + tk) * a.slots + slot;
    a.part_max[o] = v;
    a.part_idx[o] = ix;
  }
}

int token_tiles(int M) { return (M + kVM - 1) / kVM; }

}  // namespace

bool vocab_tiled(int M, int N, int K, bool bf16) {
  if (!bf16 || M < 1 || N < 1) return false;
  if (K != 256 && K != 512) return false;   // steps per item: 8 or 16
  const int mt = token_tiles(M);
  // the token tiles split each XCD's workgroups evenly, and are mostly full
  if ((kVWg / 8) % mt != 0) return false;
  return static_cast<long>(M) * 10 >= static_cast<long>(mt) * kVM * 7;
}

int vocab_slots(int M) { return kVWg / token_tiles(M); }

hipError_t launch_vocab(const GemmArgs& g, hipStream_t st) {
  if (!vocab_tiled(g.M, g.N, g.K, true)) return hipErrorInvalidValue;
  if (g.smap.g != 1 || g.smap.stride != 1 || g.smap.off != 0) return hipErrorInvalidValue;   // contiguous rows
  VocabArgs a{};
  a.W = static_cast<const uint16_t*>(g.W);
  a.X = static_cast<const uint16_t*>(g.src);
  a.ld_src = g.ld_src;
  a.N = g.N; a.K = g.K; a.M = g.M; a.tok0 = g.tok0; a.mt = token_tiles(g.M);
  a.tap = g.tap; a.ld_tap = g.ld_tap; a.tmap = g.tmap;
  a.part_max = g.part_max; a.part_idx = g.part_idx;
  a.slots = vocab_slots(g.M);
  // the resident token tile, and with the logits copy its staging block
  const size_t sm = static_cast<size_t>(kVM) * g.K * 2 + (g.tap ? 16 * (kVN + 4) * sizeof(float) : 0);
  auto go = [&](auto kern) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
    if (e != hipSuccess) return e;
    launch_k(kern, dim3(kVWg), dim3(256), static_cast<uint32_t>(sm), st, a);
    return hipGetLastError();
  };
  if (g.K == 512) return a.tap ? go(vocab_kernel<true, 16>) : go(vocab_kernel<false, 16>);
  return a.tap ? go(vocab_kernel<true, 8>) : go(vocab_kernel<false, 8>);
}

}  // namespace dlite
