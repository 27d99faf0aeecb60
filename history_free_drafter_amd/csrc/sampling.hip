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
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k.x, lo1, hi0 ^ c.w ^ k.y, lo0);
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
// index.  A lane keeps the largest hi of each of its first kKeep groups;
// later groups are formed again to find their candidates.
constexpr int kKeep = 16;
constexpr int kChunksPerBlock = 4;      // waves (chunks) per workgroup of the large passes
constexpr float kBoundMargin = 4e-7f;
template <int CPB>
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
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  const float invTf = static_cast<float>(invT);
  const int g0 = v0 >> 2, g1 = v1 > v0 ? ((v1 - 1) >> 2) + 1 : g0;   // groups touching the chunk
  // group g: its logits, words, and score intervals (empty outside the chunk)
  auto group = [&](int g, float (&lv)[4], uint32_t (&wd)[4], float (&lo)[4], float (&hi)[4]) {
    const uint4 x = philox_group(seed, stream, static_cast<unsigned>(g), static_cast<unsigned>(n));
    wd[0] = x.x; wd[1] = x.y; wd[2] = x.z; wd[3] = x.w;
    const int vb = 4 * g;
    if (vec && vb >= v0 && vb + 3 < v1) {
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
  float ghi[kKeep];
  float mlo = -INFINITY;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const int g = g0 + lane + k * 64;
    ghi[k] = -INFINITY;
    if (g < g1) {
      float lv[4], lo[4], hi[4];
      uint32_t wd[4];
      group(g, lv, wd, lo, hi);
      ghi[k] = fmaxf(fmaxf(hi[0], hi[1]), fmaxf(hi[2], hi[3]));
      mlo = fmaxf(mlo, fmaxf(fmaxf(lo[0], lo[1]), fmaxf(lo[2], lo[3])));
    }
  }
  for (int g = g0 + lane + kKeep * 64; g < g1; g += 64) {
    float lv[4], lo[4], hi[4];
    uint32_t wd[4];
    group(g, lv, wd, lo, hi);
    mlo = fmaxf(mlo, fmaxf(fmaxf(lo[0], lo[1]), fmaxf(lo[2], lo[3])));
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
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (hi[w] >= mlo && hi[w] != -INFINITY) {
        const double sv = static_cast<double>(lv[w]) * invT - log(-log(to_uniform(wd[w])));
        if (sv > bv) { bv = sv; bi = 4 * g + w; }
      }
    }
  };
  if (mlo != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
      const int g = g0 + lane + k * 64;
      if (g < g1 && ghi[k] >= mlo) candidates(g);
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

// One wave per chunk (four chunks per workgroup): a single pass over the
// chunk in batches of eight values per lane (two 16-byte loads), with a
// running maximum m and sum s of exp(y - m) rescaled once per batch when the
// maximum grows; the eight exponentials of a batch are independent.  The
// lanes' (m, s) pairs are merged in a fixed order.
__global__ __launch_bounds__(64 * kChunksPerBlock) void lse_partial_kernel(const float* draft, const float* target,
                                                                           int BK, int V, double invT, Lse* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * kChunksPerBlock + wave, row = blockIdx.y;
  const float* x = row < BK ? draft + static_cast<long>(row) * V : target + static_cast<long>(row - BK) * V;
  const int v0 = static_cast<int>(static_cast<long>(c) * V / kSampleChunks);
  const int v1 = static_cast<int>(static_cast<long>(c + 1) * V / kSampleChunks);
  // groups of four consecutive values (one 16-byte load for rows of a
  // multiple of four), two groups per lane and batch; the next batch is
  // loaded while the current one is summed
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  const int g0 = v0 >> 2, g1 = v1 > v0 ? ((v1 - 1) >> 2) + 1 : g0;
  constexpr int kGB = 2;
  auto load = [&](int gb, float (&f)[kGB * 4]) {
#pragma unroll
    for (int q = 0; q < kGB; ++q) {
      const int vb = 4 * (gb + q * 64);
      if (vec && vb >= v0 && vb + 3 < v1) {
        const float4 t4 = *reinterpret_cast<const float4*>(x + vb);
        f[q * 4] = t4.x; f[q * 4 + 1] = t4.y; f[q * 4 + 2] = t4.z; f[q * 4 + 3] = t4.w;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int v = vb + w;
          f[q * 4 + w] = (v >= v0 && v < v1) ? x[v] : -INFINITY;
        }
      }
    }
  };
  double m = -INFINITY, s = 0.0;
  float cur[kGB * 4];
  int gb = g0 + lane;
  if (gb < g1) load(gb, cur);
  for (; gb < g1; gb += kGB * 64) {
    float nxt[kGB * 4];
    if (gb + kGB * 64 < g1) load(gb + kGB * 64, nxt);
    double y[kGB * 4];
    double bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kGB * 4; ++j) {
      y[j] = static_cast<double>(cur[j]) * invT;
      bm = fmax(bm, y[j]);
    }
    if (bm > m) {
      s = m == -INFINITY ? 0.0 : s * exp(m - bm);
      m = bm;
    }
    if (m != -INFINITY) {
      double t = 0.0;
#pragma unroll
      for (int j = 0; j < kGB * 4; ++j) t += exp(y[j] - m);   // exp(-inf) = 0
      s += t;
    }
#pragma unroll
    for (int j = 0; j < kGB * 4; ++j) cur[j] = nxt[j];
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
// residual vanishes).
__global__ __launch_bounds__(kThreads) void chunk_sum_kernel(const float* draft, const float* target,
                                                             const Decision* dec, int K, int V, double invT,
                                                             double* csum) {
  __shared__ double shr[kThreads / 64], shp[kThreads / 64];
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
  for (int v = v0 + static_cast<int>(threadIdx.x); v < v1; v += kThreads) {
    const double p = exp(static_cast<double>(tp[v]) * invT - lp);
    sp += p;
    if (res) {
      const double q = exp(static_cast<double>(dp[v]) * invT - lq);
      sr += p > q ? p - q : 0.0;
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
  auto weight = [&](int v) {
    const double p = exp(static_cast<double>(tp[v]) * invT - lp);
    if (!res) return p;
    const double q = exp(static_cast<double>(dp[v]) * invT - lq);
    return p > q ? p - q : 0.0;
  };
  const int c = chunk;
  const int v0 = static_cast<int>(static_cast<long>(c) * V / kSampleChunks);
  const int v1 = static_cast<int>(static_cast<long>(c + 1) * V / kSampleChunks);
  const int per = (v1 - v0 + kThreads - 1) / kThreads;
  const int a0 = v0 + static_cast<int>(threadIdx.x) * per;
  const int a1 = a0 + per < v1 ? a0 + per : v1;
  double mine = 0.0;
  for (int v = a0; v < a1; ++v) mine += weight(v);
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
    for (int v = a0; v < a1; ++v) {
      const double w = weight(v);
      if (w > 0.0) lastpos = v;
      run += w;
      if (run > t) { pick = v; break; }
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
  if (N * kSampleChunks < 4096)
    launch_k(sample_partial_kernel<1>, dim3(kSampleChunks, N), dim3(64), 0, st, logits, V,
             1.0 / static_cast<double>(T), seed, stream, part);
  else
    launch_k(sample_partial_kernel<kChunksPerBlock>, dim3(kSampleChunks / kChunksPerBlock, N),
             dim3(64 * kChunksPerBlock), 0, st, logits, V, 1.0 / static_cast<double>(T), seed, stream, part);
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
  launch_k(lse_partial_kernel, dim3(kSampleChunks / kChunksPerBlock, B * (2 * K + 1)), dim3(64 * kChunksPerBlock), 0, st, draft,
                     target, B * K, V, invT, part);
  Decision* dec = reinterpret_cast<Decision*>(csum + static_cast<long>(B) * kSampleChunks * 2);
  launch_k(decide_kernel, dim3(B), dim3(kThreads), 0, st, cand, draft, target, part, B, K, V, invT, seed, dec);
  launch_k(chunk_sum_kernel, dim3(kSampleChunks, B), dim3(kThreads), 0, st, draft, target, dec, K, V, invT,
           csum);
  launch_k(pick_kernel, dim3(B), dim3(kThreads), 0, st, draft, target, dec, csum, K, V, invT, seed, A, next);
  return hipGetLastError();
}

}  // namespace dlite
