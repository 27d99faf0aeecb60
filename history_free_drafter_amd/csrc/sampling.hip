// Sampling at a positive temperature and speculative rejection sampling
// (DLite walkthrough, section "贪心模式与随机模式要分别说明").
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator computed
// where it is needed, so no generator state exists.  The uniform with index
// a of row b in a stream is word a mod 4 of the generator at counter
// (a div 4, b, stream, 0) under key (seed low, seed high), as
// (word + 1/2) / 2^32 in fp64: one call serves four consecutive indices.
//
// Draws from softmax(l / T) use the Gumbel-max rule, argmax_v (l_v / T -
// log(-log u_v)), with the (value, index) reduction of the vocabulary pass.
// Verification follows the page: candidate d ~ q is kept when u q(d) < p(d);
// at the first rejection the token is drawn from the positive residual
// [p - q]_+ (inverse CDF), after K acceptances from the target's last row.
// Three passes over the vocabulary, each spread over 64 chunks: log-sum-exp
// partials of every row (one pass each), the deciding row's chunk sums, and
// the draw (chunk, then index inside it).  A draw's perturbed scores are
// formed in fp32 and only the near-maximal ones again in fp64, which finds
// the same token as an fp64 evaluation of every score.
// Probabilities, exponentials and logarithms are fp64: the decisions are the
// ones an exact evaluation would make except within rounding of a threshold.
#include "gumbel_bounds.hpp"
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kSampleChunks = 64;   // vocabulary chunks per row
constexpr int kThreads = 256;

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint2 k) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // full 64-bit products: one multiply instruction each for both halves
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    c = make_uint4(static_cast<uint32_t>(p1 >> 32) ^ c.y ^ k.x, static_cast<uint32_t>(p1),
                   static_cast<uint32_t>(p0 >> 32) ^ c.w ^ k.y, static_cast<uint32_t>(p0));
    k.x += 0x9E3779B9u;
    k.y += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ uint4 philox_group(unsigned long long seed, unsigned stream, unsigned g, unsigned b) {
  return philox4x32_10(make_uint4(g, b, stream, 0u),
                       make_uint2(static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32)));
}
__device__ __forceinline__ uint32_t pick_word(const uint4& x, unsigned w) {
  return w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
}
__device__ __forceinline__ double to_uniform(uint32_t x) { return (static_cast<double>(x) + 0.5) * (1.0 / 4294967296.0); }
__device__ __forceinline__ double uniform01(unsigned long long seed, unsigned stream, unsigned a, unsigned b) {
  return to_uniform(pick_word(philox_group(seed, stream, a >> 2, b), a & 3u));
}

struct Best {
  double v;
  int i;
};
__device__ __forceinline__ bool better_d(double v, int i, double bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide (value, index) maximum in a fixed order; result in thread 0.
__device__ Best block_best(double v, int i, Best* sh) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    if (better_d(ov, oi, v, i)) { v = ov; i = oi; }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = Best{v, i};
  __syncthreads();
  Best b = sh[0];
  if (threadIdx.x == 0)
    for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w)
      if (better_d(sh[w].v, sh[w].i, b.v, b.i)) b = sh[w];
  __syncthreads();
  return b;
}


// Pass 1 of a draw: the best perturbed score of chunk c of row n, exactly
// as an fp64 evaluation of every score would find it; one wave per chunk
// (CPB chunks per workgroup).  The chunk is walked in groups of four
// consecutive indices (one generator call and, for rows of a multiple of
// four, one 16-byte load each).  The Gumbel term of a word lies between the
// bounds of its bucket (kGumbelBounds, staged in LDS), so every score has an
// fp32 interval [lo, hi] that holds its fp64 value (rounding covered by a
// relative margin of 4e-7).  No index whose hi is below the largest lo of the
// chunk can win, so only the others (a few per chunk) are formed in fp64 (the
// costly logarithms) and compared as (value, index) with ties to the lower
// index.  The first phase takes a lane's groups kSB at a time, the next
// batch's loads issued (at addresses clamped into the chunk) before the
// current batch's generator words and intervals are formed; a lane keeps the
// largest hi of each of its first kKeep groups, later groups are formed again
// to find their candidates.
constexpr int kSB = 5;                  // groups per lane and batch
constexpr int kKeepB = 4;               // batches whose groups' bounds are kept
constexpr int kKeep = kSB * kKeepB;
static_assert(kKeep <= 32, "candidate groups of a lane as a 32-bit mask");
constexpr int kChunksPerBlock = 4;      // waves (chunks) per workgroup of the large passes
constexpr float kBoundMargin = 4e-7f;
template <int CPB, bool VEC>   // VEC: rows of a multiple of four values at a 16-byte aligned address
__global__ __launch_bounds__(64 * CPB) void sample_partial_kernel(const float* logits, int V, double invT,
                                                                  unsigned long long seed, unsigned stream,
                                                                  Best* part) {
  __shared__ float2 gb[kGumbelBuckets];
  for (int i = threadIdx.x; i < kGumbelBuckets; i += 64 * CPB)
    gb[i] = make_float2(kGumbelBounds[2 * i], kGumbelBounds[2 * i + 1]);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * CPB + wave, n = blockIdx.y;
  const int v0 = static_cast<int>(static_cast<long>(c) * V / kSampleChunks);
  const int v1 = static_cast<int>(static_cast<long>(c + 1) * V / kSampleChunks);
  const float* row = logits + static_cast<long>(n) * V;
  const float invTf = static_cast<float>(invT);
  const int g0 = v0 >> 2, g1 = v1 > v0 ? ((v1 - 1) >> 2) + 1 : g0;   // groups touching the chunk
  // group g: its logits, words, and score intervals (empty outside the chunk)
  auto group = [&](int g, float (&lv)[4], uint32_t (&wd)[4], float (&lo)[4], float (&hi)[4]) {
    const uint4 x = philox_group(seed, stream, static_cast<unsigned>(g), static_cast<unsigned>(n));
    wd[0] = x.x; wd[1] = x.y; wd[2] = x.z; wd[3] = x.w;
    const int vb = 4 * g;
    if (VEC && vb >= v0 && vb + 3 < v1) {
      const float4 q = *reinterpret_cast<const float4*>(row + vb);
      lv[0] = q.x; lv[1] = q.y; lv[2] = q.z; lv[3] = q.w;
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) lv[w] = (vb + w >= v0 && vb + w < v1) ? row[vb + w] : 0.f;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bool in = vb + w >= v0 && vb + w < v1;
      const float lt = lv[w] * invTf;
      const float2 bd = gb[wd[w] >> kGumbelShift];
      const float l0 = lt + bd.x, h0 = lt + bd.y;
      lo[w] = in ? l0 - (fabsf(lt) + fabsf(bd.x)) * kBoundMargin : -INFINITY;
      hi[w] = in ? h0 + (fabsf(lt) + fabsf(bd.y)) * kBoundMargin : -INFINITY;
    }
  };
  // batch loads: group b0 + lane + 64 q, clamped to the chunk's last group
  auto load = [&](int b0, float (&f)[kSB][4]) {
#pragma unroll
    for (int q = 0; q < kSB; ++q) {
      const int g = min(b0 + lane + q * 64, g1 - 1);
      if constexpr (VEC) {
        const float4 t4 = *reinterpret_cast<const float4*>(row + 4 * g);
        f[q][0] = t4.x; f[q][1] = t4.y; f[q][2] = t4.z; f[q][3] = t4.w;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) f[q][w] = row[min(max(4 * g + w, v0), v1 - 1)];
      }
    }
  };
  // the batch's intervals: the largest lo into mlo, each group's largest hi
  float mlo = -INFINITY;
  auto bounds = [&](int b0, const float (&f)[kSB][4], float* gh) {
#pragma unroll
    for (int q = 0; q < kSB; ++q) {
      const int g = b0 + lane + q * 64;
      const uint4 x = philox_group(seed, stream, static_cast<unsigned>(g), static_cast<unsigned>(n));
      const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
      float h = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int v = 4 * g + w;
        const float lt = f[q][w] * invTf;
        const float2 bd = gb[wd[w] >> kGumbelShift];
        const float lo = lt + bd.x - (fabsf(lt) + fabsf(bd.x)) * kBoundMargin;
        const float hi = lt + bd.y + (fabsf(lt) + fabsf(bd.y)) * kBoundMargin;
        const bool in = v >= v0 && v < v1;
        mlo = fmaxf(mlo, in ? lo : -INFINITY);
        h = fmaxf(h, in ? hi : -INFINITY);
      }
      if (gh) gh[q] = h;
    }
  };
  float ghi[kKeep];
  float cur[kSB][4], nxt[kSB][4];
  if (g1 > g0) load(g0, cur);
#pragma unroll
  for (int kb = 0; kb < kKeepB; ++kb) {
    const int b0 = g0 + kb * kSB * 64;
#pragma unroll
    for (int q = 0; q < kSB; ++q) ghi[kb * kSB + q] = -INFINITY;
    if (b0 < g1) {
      load(b0 + kSB * 64, nxt);
      bounds(b0, cur, ghi + kb * kSB);
#pragma unroll
      for (int q = 0; q < kSB; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) cur[q][w] = nxt[q][w];
    }
  }
  for (int b0 = g0 + kKeep * 64; b0 < g1; b0 += kSB * 64) {
    load(b0 + kSB * 64, nxt);
    bounds(b0, cur, nullptr);
#pragma unroll
    for (int q = 0; q < kSB; ++q)
#pragma unroll
      for (int w = 0; w < 4; ++w) cur[q][w] = nxt[q][w];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mlo = fmaxf(mlo, __shfl_xor(mlo, o, kWave));
  // the candidates, in fp64 (each lane visits its indices in ascending
  // order, so strictly greater keeps the lower index on ties)
  double bv = -INFINITY;
  int bi = 0x7fffffff;
  auto candidates = [&](int g) {
    float lv[4], lo[4], hi[4];
    uint32_t wd[4];
    group(g, lv, wd, lo, hi);
    uint32_t em = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (hi[w] >= mlo && hi[w] != -INFINITY) em |= 1u << w;
    while (em) {   // one fp64 evaluation per lane and iteration
      const int w = __builtin_ctz(em);
      em &= em - 1;
      const float l = w == 0 ? lv[0] : w == 1 ? lv[1] : w == 2 ? lv[2] : lv[3];
      const uint32_t x = w == 0 ? wd[0] : w == 1 ? wd[1] : w == 2 ? wd[2] : wd[3];
      const double sv = static_cast<double>(l) * invT - log(-log(to_uniform(x)));
      if (sv > bv) { bv = sv; bi = 4 * g + w; }
    }
  };
  if (mlo != -INFINITY) {
    // a lane's candidate groups among its first kKeep, visited in ascending
    // order (typically one per lane: the loads wait once per wave)
    uint32_t cm = 0;
#pragma unroll
    for (int k = 0; k < kKeep; ++k)
      if (g0 + lane + k * 64 < g1 && ghi[k] >= mlo) cm |= 1u << k;
    while (cm) {
      const int k = __builtin_ctz(cm);
      cm &= cm - 1;
      candidates(g0 + lane + k * 64);
    }
    for (int g = g0 + lane + kKeep * 64; g < g1; g += 64) candidates(g);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (better_d(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (lane == 0) part[static_cast<long>(n) * kSampleChunks + c] = Best{bv, bi};
}

// Pass 2: the chunks of a row (one wave per row, a lane per chunk; the
// (value, index) order makes the result independent of the reduction order).
static_assert(kSampleChunks == 64, "one lane per chunk");
__global__ __launch_bounds__(256) void sample_final_kernel(const Best* part, int N, int32_t* tokens) {
  const int n = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  if (n >= N) return;
  const int lane = threadIdx.x & 63;
  const Best o = part[static_cast<long>(n) * kSampleChunks + lane];
  double v = o.v;
  int i = o.i;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const double ov = __shfl_xor(v, s, kWave);
    const int oi = __shfl_xor(i, s, kWave);
    if (better_d(ov, oi, v, i)) { v = ov; i = oi; }
  }
  if (lane == 0) tokens[n] = i;
}

// log-sum-exp partials of l / T: (chunk maximum, sum of exp(x - maximum)).
struct Lse {
  double m, s;
};

// exp(d) in fp64 for the probabilities of the verification passes (d <= 0
// there), four at a time: d = (256 k + j) ln2 / 256 + r with |r| <= ln2 / 512,
// so exp(d) = 2^k 2^(j/256) e^r.  n = 256 k + j is d 256 / ln2 rounded to an
// integer (added to 1.5 2^52, so the sum's low word holds it), r follows by a
// Cody-Waite reduction (ln2 / 256 as a head of 29 significant bits, whose
// products with n are exact, plus the fp64 remainder), e^r by its Taylor
// polynomial through r^4 (truncation below 4e-17 relative), 2^(j/256) from a
// 256-entry table in LDS (exp_table).  About 3 ulp in all.  The four table
// reads are issued before the polynomials, so their latency is covered.
// Arguments below -1000 (and -inf) give exactly 0 through the final scaling;
// a NaN stays NaN.  Valid for d up to 700.
constexpr int kExpTab = 256;
constexpr double kInvLn2xT = 0x1.71547652b82fep+8;     // 256 / ln 2
constexpr double kLn2xTHi = 0x1.62e42ffp-9;            // ln 2 / 256, head
constexpr double kLn2xTLo = -0x1.718432a1b0e26p-43;    // ln 2 / 256 - head
constexpr double kRound52 = 0x1.8p52;
__device__ __forceinline__ void exp_table(double* tab) {   // then a barrier
  for (int i = threadIdx.x; i < kExpTab; i += blockDim.x) tab[i] = exp2(static_cast<double>(i) / kExpTab);
}
__device__ __forceinline__ void exp4(const double (&d4)[4], const double* tab, double (&e)[4]) {
  double r[4], tv[4];
  int n[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const double d = d4[w] < -1000.0 ? -1000.0 : d4[w];   // (a NaN stays NaN)
    const double t = fma(d, kInvLn2xT, kRound52);
    n[w] = __double2loint(t);
    const double nf = t - kRound52;
    r[w] = fma(-nf, kLn2xTLo, fma(-nf, kLn2xTHi, d));
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) tv[w] = tab[n[w] & (kExpTab - 1)];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    double p = fma(r[w], 1.0 / 24.0, 1.0 / 6.0);
    p = fma(p, r[w], 0.5);
    p = fma(p, r[w], 1.0);
    p = fma(p, r[w], 1.0);
    e[w] = ldexp(tv[w] * p, n[w] >> 8);
  }
}

// One wave per chunk (four chunks per workgroup).  A lane takes its groups of
// four consecutive values kLseGroups at a time (16-byte loads for rows of a
// multiple of four, all issued before any is used; a group straddling the
// chunk's edge is masked): their maximum (in fp32 on the raw logits: scaling
// by 1/T > 0 keeps the order), the running maximum m rescaling the sum s
// once per batch when it grows, then the batch's exp(y - m).  The lanes'
// (m, s) pairs are merged in a fixed order.
constexpr int kLseGroups = 10;   // one batch covers chunks of up to 2560 values
template <bool VEC>   // rows of a multiple of four values at 16-byte aligned addresses
__global__ __launch_bounds__(64 * kChunksPerBlock) void lse_partial_kernel(const float* draft, const float* target,
                                                                           int BK, int V, double invT, Lse* part) {
  __shared__ double tab[kExpTab];
  exp_table(tab);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * kChunksPerBlock + wave, row = blockIdx.y;
  const float* x = row < BK ? draft + static_cast<long>(row) * V : target + static_cast<long>(row - BK) * V;
  const int v0 = static_cast<int>(static_cast<long>(c) * V / kSampleChunks);
  const int v1 = static_cast<int>(static_cast<long>(c + 1) * V / kSampleChunks);
  const int g0 = v0 >> 2, g1 = v1 > v0 ? ((v1 - 1) >> 2) + 1 : g0;
  double m = -INFINITY, s = 0.0;
  for (int b0 = g0; b0 < g1; b0 += kLseGroups * 64) {
    // addresses clamped into the chunk's groups, values outside it masked
    float f[kLseGroups * 4];
#pragma unroll
    for (int q = 0; q < kLseGroups; ++q) {
      const int g = min(b0 + lane + q * 64, g1 - 1);
      if constexpr (VEC) {
        const float4 t4 = *reinterpret_cast<const float4*>(x + 4 * g);
        f[q * 4] = t4.x; f[q * 4 + 1] = t4.y; f[q * 4 + 2] = t4.z; f[q * 4 + 3] = t4.w;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) f[q * 4 + w] = x[min(max(4 * g + w, v0), v1 - 1)];
        __builtin_amdgcn_sched_barrier(0);   // (registers)
      }
    }
    float xm = -INFINITY;
#pragma unroll
    for (int q = 0; q < kLseGroups; ++q)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int v = 4 * (b0 + lane + q * 64) + w;
        if (v < v0 || v >= v1) f[q * 4 + w] = -INFINITY;
        xm = fmaxf(xm, f[q * 4 + w]);
      }
    const double bm = static_cast<double>(xm) * invT;
    if (bm > m) {
      s = m == -INFINITY ? 0.0 : s * exp(m - bm);
      m = bm;
    }
    if (m != -INFINITY) {
      double t = 0.0;
#pragma unroll
      for (int q = 0; q < kLseGroups; ++q) {
        double d4[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) d4[w] = static_cast<double>(f[q * 4 + w]) * invT - m;
        double e[4];
        exp4(d4, tab, e);
        t += ((e[0] + e[1]) + e[2]) + e[3];
        __builtin_amdgcn_sched_barrier(0);   // one group at a time (registers)
      }
      s += t;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double om = __shfl_xor(m, o, kWave), os = __shfl_xor(s, o, kWave);
    const double M = fmax(m, om);
    const double a = m == -INFINITY ? 0.0 : s * exp(m - M);
    const double b = om == -INFINITY ? 0.0 : os * exp(om - M);
    m = M;
    s = a + b;
  }
  if (lane == 0) part[static_cast<long>(row) * kSampleChunks + c] = Lse{m, s};
}

constexpr int kMaxRows = 2 * 64 + 1;   // rows of one request: K draft + K + 1 target (K <= 64)

// log-sum-exp of the 2K + 1 rows of request b from the chunk partials
// (draft rows b K + i, then target rows b (K + 1) + i): one wave per row, a
// lane per chunk (64 chunks), wave reductions in a fixed order.
static_assert(kSampleChunks == 64, "one lane per chunk");
__device__ void request_lse(const Lse* part, int b, int B, int K, double* lse) {
  const int BK = B * K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = static_cast<int>(blockDim.x >> 6);
  for (int j = wave; j < 2 * K + 1; j += nw) {
    const long row = j < K ? static_cast<long>(b) * K + j : BK + static_cast<long>(b) * (K + 1) + (j - K);
    const Lse pc = part[row * kSampleChunks + lane];
    double M = pc.m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmax(M, __shfl_xor(M, o, kWave));
    double S = pc.s > 0.0 ? pc.s * exp(pc.m - M) : 0.0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) S += __shfl_xor(S, o, kWave);
    if (lane == 0) lse[j] = M + log(S);
  }
}

// The acceptance tests of all positions at once (wave 0, lane i tests
// position i; K <= 64), then the first rejection by a ballot: the number
// kept, and whether the deciding draw is from the residual (else from the
// target's row K).  Result in *out_i / *out_res (shared), valid after a
// barrier.
__device__ void decide(const int32_t* cand, const float* draft, const float* target, const double* lse, int b,
                       int K, int V, double invT, unsigned long long seed, int* out_i, int* out_res) {
  if (threadIdx.x >= 64) return;
  const int i = static_cast<int>(threadIdx.x);
  bool keep = true;
  if (i < K) {
    const int d = cand[static_cast<long>(b) * K + i];
    keep = false;
    if (d >= 0 && d < V) {
      const double q = exp(static_cast<double>(draft[(static_cast<long>(b) * K + i) * V + d]) * invT - lse[i]);
      const double p =
          exp(static_cast<double>(target[(static_cast<long>(b) * (K + 1) + i) * V + d]) * invT - lse[K + i]);
      const double u = uniform01(seed, 1u, static_cast<unsigned>(i), static_cast<unsigned>(b));
      keep = u * q < p;
    }
  }
  const unsigned long long rejected = __ballot(!keep);
  if (i == 0) {
    const int first = rejected ? __builtin_ctzll(rejected) : K;
    *out_i = first < K ? first : K;
    *out_res = first < K;
  }
}

// The decision of request b, made once: the deciding position, whether its
// draw is from the residual, and the log-sum-exps its weights need.
struct Decision {
  double lp, lq;   // lse of the target row at the position (and of the draft row, residual)
  int i, res;
};
__global__ __launch_bounds__(kThreads) void decide_kernel(const int32_t* cand, const float* draft,
                                                          const float* target, const Lse* part, int B, int K,
                                                          int V, double invT, unsigned long long seed,
                                                          Decision* dec) {
  __shared__ double lse[kMaxRows];
  __shared__ int di, dres;
  const int b = blockIdx.x;
  request_lse(part, b, B, K, lse);
  __syncthreads();
  decide(cand, draft, target, lse, b, K, V, invT, seed, &di, &dres);
  __syncthreads();
  if (threadIdx.x == 0) dec[b] = Decision{lse[K + di], dres ? lse[di] : 0.0, di, dres};
}

// Pass 2: per (chunk, request), the deciding row's chunk sums of the
// residual weights and of the target probabilities (the fallback when the
// residual vanishes); four consecutive values per thread and step.
__global__ __launch_bounds__(kThreads) void chunk_sum_kernel(const float* draft, const float* target,
                                                             const Decision* dec, int K, int V, double invT,
                                                             double* csum) {
  __shared__ double shr[kThreads / 64], shp[kThreads / 64];
  __shared__ double tab[kExpTab];
  exp_table(tab);
  __syncthreads();
  const int c = blockIdx.x, b = blockIdx.y;
  const Decision d = dec[b];
  const int i = d.i;
  const bool res = d.res != 0;
  const float* tp = target + (static_cast<long>(b) * (K + 1) + i) * V;
  const float* dp = draft + (static_cast<long>(b) * K + (res ? i : 0)) * V;
  const double lp = d.lp, lq = d.lq;
  const int v0 = static_cast<int>(static_cast<long>(c) * V / kSampleChunks);
  const int v1 = static_cast<int>(static_cast<long>(c + 1) * V / kSampleChunks);
  double sr = 0.0, sp = 0.0;
  for (int v = v0 + 4 * static_cast<int>(threadIdx.x); v < v1; v += 4 * kThreads) {
    double dpv[4], dqv[4], p[4], q[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int u = min(v + w, v1 - 1);
      dpv[w] = static_cast<double>(tp[u]) * invT - lp;
      dqv[w] = res ? static_cast<double>(dp[u]) * invT - lq : 0.0;
    }
    exp4(dpv, tab, p);
    if (res) exp4(dqv, tab, q);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (v + w < v1) {
        sp += p[w];
        if (res) sr += p[w] > q[w] ? p[w] - q[w] : 0.0;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    sr += __shfl_xor(sr, o, kWave);
    sp += __shfl_xor(sp, o, kWave);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { shr[wave] = sr; shp[wave] = sp; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double tr = 0.0, tq = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) { tr += shr[w]; tq += shp[w]; }
    csum[(static_cast<long>(b) * kSampleChunks + c) * 2] = tr;
    csum[(static_cast<long>(b) * kSampleChunks + c) * 2 + 1] = tq;
  }
}

// Pass 3: per request, the chunk whose running range holds the draw, then
// the index inside it: each thread a contiguous piece of the chunk, the
// pieces' sums scanned in thread order, the piece holding the draw rescanned.
__global__ __launch_bounds__(kThreads) void pick_kernel(const float* draft, const float* target,
                                                        const Decision* dec, const double* csum, int K, int V,
                                                        double invT, unsigned long long seed, int32_t* A_out,
                                                        int32_t* next_out) {
  __shared__ double pre[kThreads + 1];
  __shared__ int di, dres, chunk;
  __shared__ double tloc;
  __shared__ double tab[kExpTab];
  exp_table(tab);
  const int b = blockIdx.x;
  const Decision d = dec[b];
  if (threadIdx.x == 0) { di = d.i; dres = d.res; }
  __syncthreads();
  if (threadIdx.x < 64) {
    // wave 0, lane = chunk: the chunk sums scanned in chunk order, the chunk
    // holding the draw found by a ballot
    const int lane = static_cast<int>(threadIdx.x);
    const int i = di;
    const double* cs = csum + static_cast<long>(b) * kSampleChunks * 2;
    const double xr = cs[lane * 2], xp = cs[lane * 2 + 1];
    auto scan = [&](double x) {   // inclusive, fixed order
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      return x;
    };
    const double ir = scan(xr), ip = scan(xp);
    bool r = dres != 0;
    double Z = __shfl(ir, 63, kWave);
    if (r && !(Z > 0.0)) r = false;   // the residual vanishes (p == q): draw from p
    const double incl = r ? ir : ip, x = r ? xr : xp;
    Z = __shfl(incl, 63, kWave);
    const double t = uniform01(seed, 2u, static_cast<unsigned>(i), static_cast<unsigned>(b)) * Z;
    const unsigned long long hit = __ballot(t < incl && x > 0.0);
    const unsigned long long pos = __ballot(x > 0.0);
    // rounding past the end: the last chunk with mass, drawn at its top
    const int ch = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
    if (lane == ch) tloc = hit ? fmax(t - (incl - x), 0.0) : x;
    if (lane == 0) {
      dres = r;
      chunk = ch;
      A_out[b] = i;
    }
  }
  __syncthreads();
  const int i = di;
  const bool res = dres != 0;
  const float* tp = target + (static_cast<long>(b) * (K + 1) + i) * V;
  const float* dp = draft + (static_cast<long>(b) * K + (res ? i : 0)) * V;
  const double lp = d.lp, lq = res ? d.lq : 0.0;
  // the weights of v .. v + 3 (0 from a1 on; requires v < a1)
  auto weights4 = [&](int v, int a1, double (&wt)[4]) {
    double dpv[4], dqv[4], p[4], q[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int u = min(v + w, a1 - 1);
      dpv[w] = static_cast<double>(tp[u]) * invT - lp;
      dqv[w] = res ? static_cast<double>(dp[u]) * invT - lq : 0.0;
    }
    exp4(dpv, tab, p);
    if (res) exp4(dqv, tab, q);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      wt[w] = v + w >= a1 ? 0.0 : !res ? p[w] : p[w] > q[w] ? p[w] - q[w] : 0.0;
  };
  const int c = chunk;
  const int v0 = static_cast<int>(static_cast<long>(c) * V / kSampleChunks);
  const int v1 = static_cast<int>(static_cast<long>(c + 1) * V / kSampleChunks);
  const int per = (v1 - v0 + kThreads - 1) / kThreads;
  const int a0 = v0 + static_cast<int>(threadIdx.x) * per;
  const int a1 = a0 + per < v1 ? a0 + per : v1;
  double mine = 0.0;
  for (int v = a0; v < a1; v += 4) {
    double wt[4];
    weights4(v, a1, wt);
#pragma unroll
    for (int w = 0; w < 4; ++w) mine += wt[w];   // (+0 past a1 leaves it unchanged)
  }
  pre[threadIdx.x + 1] = mine;
  if (threadIdx.x == 0) pre[0] = 0.0;
  __syncthreads();
  // inclusive scan of pre[1..kThreads] (Hillis-Steele, fixed order)
  for (int o = 1; o < kThreads; o <<= 1) {
    const double add = static_cast<int>(threadIdx.x) >= o ? pre[threadIdx.x + 1 - o] : 0.0;
    __syncthreads();
    pre[threadIdx.x + 1] += add;
    __syncthreads();
  }
  const double total = pre[kThreads];
  double t = tloc;
  if (!(t < total)) t = nextafter(total, 0.0);   // rounding between the two sums of the chunk
  const double lo = pre[threadIdx.x], hi = pre[threadIdx.x + 1];
  if (lo <= t && t < hi) {
    double run = lo;
    int pick = -1, lastpos = a0;
    for (int v = a0; v < a1 && pick < 0; v += 4) {
      double wt[4];
      weights4(v, a1, wt);
      for (int w = 0; w < 4 && v + w < a1; ++w) {
        if (wt[w] > 0.0) lastpos = v + w;
        run += wt[w];
        if (run > t) { pick = v + w; break; }
      }
    }
    next_out[b] = pick >= 0 ? pick : lastpos;
  }
}

}  // namespace

size_t sampling_scratch_bytes(long rows) {
  // partials of every row, then two chunk sums per chunk of at most `rows`
  // requests (accept: rows = B (2K + 1) >= B)
  return static_cast<size_t>(rows) * kSampleChunks * 16 * 2;
}

hipError_t launch_sample_tokens(const float* logits, int N, int V, float T, unsigned long long seed,
                                unsigned stream, int32_t* tokens, void* scratch, hipStream_t st) {
  Best* part = static_cast<Best*>(scratch);
  // few rows: one wave per workgroup, so that the chunks spread over more CUs
  const bool few = N * kSampleChunks < 4096;
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  const dim3 grid = few ? dim3(kSampleChunks, N) : dim3(kSampleChunks / kChunksPerBlock, N);
  const dim3 block = few ? dim3(64) : dim3(64 * kChunksPerBlock);
  const double invT = 1.0 / static_cast<double>(T);
  auto go = [&](auto kern) { launch_k(kern, grid, block, 0, st, logits, V, invT, seed, stream, part); };
  if (few) {
    if (vec) go(sample_partial_kernel<1, true>);
    else go(sample_partial_kernel<1, false>);
  } else {
    if (vec) go(sample_partial_kernel<kChunksPerBlock, true>);
    else go(sample_partial_kernel<kChunksPerBlock, false>);
  }
  launch_k(sample_final_kernel, dim3((N + 3) / 4), dim3(256), 0, st, part, N, tokens);
  return hipGetLastError();
}

hipError_t launch_accept_sampled(const int32_t* cand, const float* draft, const float* target, int B, int K, int V,
                                 float T, unsigned long long seed, int32_t* A, int32_t* next, void* scratch,
                                 hipStream_t st) {
  if (K > 64) return hipErrorInvalidValue;
  Lse* part = static_cast<Lse*>(scratch);
  double* csum = reinterpret_cast<double*>(part + static_cast<long>(B) * (2 * K + 1) * kSampleChunks);
  const double invT = 1.0 / static_cast<double>(T);
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(draft) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(target) & 15) == 0;
  const dim3 lgrid(kSampleChunks / kChunksPerBlock, B * (2 * K + 1)), lblock(64 * kChunksPerBlock);
  if (vec)
    launch_k(lse_partial_kernel<true>, lgrid, lblock, 0, st, draft, target, B * K, V, invT, part);
  else
    launch_k(lse_partial_kernel<false>, lgrid, lblock, 0, st, draft, target, B * K, V, invT, part);
  Decision* dec = reinterpret_cast<Decision*>(csum + static_cast<long>(B) * kSampleChunks * 2);
  launch_k(decide_kernel, dim3(B), dim3(kThreads), 0, st, cand, draft, target, part, B, K, V, invT, seed, dec);
  launch_k(chunk_sum_kernel, dim3(kSampleChunks, B), dim3(kThreads), 0, st, draft, target, dec, K, V, invT,
           csum);
  launch_k(pick_kernel, dim3(B), dim3(kThreads), 0, st, draft, target, dec, csum, K, V, invT, seed, A, next);
  return hipGetLastError();
}

}  // namespace dlite
