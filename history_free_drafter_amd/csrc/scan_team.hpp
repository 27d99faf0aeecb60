// Sequential head: K dependent steps of a rank-r recurrent state.  The team
// routine here is shared by the stand-alone scan kernel and the fused
// scan + vocabulary kernel.
//
//   s_0 = 0,  s_k = s_{k-1} + W_up silu(P_k + W_s s_{k-1}),
//   P_k = W_down[:, :D] h_k (one batched GEMM before this kernel),
//   W_s = W_down[:, D:].
//
// Both r x r matrices are re-applied at every step, so one workgroup would
// re-read them from L2 K times.  Instead a team of TEAM workgroups (16 when r
// is a multiple of 256, else 8) splits the state index: workgroup j keeps rows
// [r0, r1) of W_s and the same columns of W_up in registers for the whole
// kernel.  Per step it forms its slice of the gate input t = P_k + W_s s (wave
// w multiplies its 1/8 of the columns; lane = row, or with 16 members lane =
// row + 32 h for the two halves of the wave's columns, added by a lane swap;
// the eight wave sums are added through LDS in wave order), then its
// full-length contribution W_up[:, r0:r1] silu(t[r0:r1]) (thread = output
// row).  More members means less arithmetic per member and step; the exchange
// costs about the same.  Each contribution is stored as one 64-bit word, the value
// beside a tag naming the step; every workgroup reads all kTeam contributions
// back, re-reading until every tag is the current step's, and adds them in
// the same fixed order, so each holds the identical new state without a
// second exchange and without an arrival counter.  Contributions are
// double-buffered by step parity: a slot is rewritten two steps later, after
// its readers have contributed to the step in between.  Tags are unique
// within a call (launch chunks offset them) and the slots are zeroed by the
// first kernel of every call, so no value left by an earlier call matches.
// Requests are split into teams of up to kReq requests; teams run
// independently.
//
// Latency matters more than bandwidth here: the weight slices and every
// step's P values are requested at once at the start and settled before the
// first step, the state is read from LDS as broadcasts (all reads of a slice issued
// before the first multiply), and the exchange needs no
// barrier: each 64-bit word is one device-scope atomic store and is read
// with device-scope atomic loads, so value and tag arrive together wherever
// the team members run, and no ordering between different words is needed.
//
// All workgroups of a launch are resident at once (at most 256 workgroups,
// one per CU), and every wait is bounded: a wait that does not complete
// within its spin budget is flagged in the status word and released, so the
// kernel always drains.
#pragma once

#include "kernels.hpp"

namespace dlite {

namespace scan_detail {

constexpr int kThreads = 512;
constexpr int kReq = 8;
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kPolicySc1 = 16;            // buffer-load cache policy: device scope
constexpr int kRsrcWord3 = 0x00020000;    // raw 32-bit buffer resource

// Members per team for B requests of rank r: 16 when every member's slices
// stay 16-element aligned (r a multiple of 256) and one launch still gives
// each team a single request (B <= 16), else 8 (more teams, fewer requests
// per team).
inline int team_size(int r, int B) { return r % 256 == 0 && B <= 16 ? 16 : 8; }
// Teams per launch: at most 256 workgroups (one per CU, so that every team is
// resident at once).
inline int teams_per_launch(int r, int B) { return 256 / team_size(r, B); }

// One tagged contribution (value in the low word, step tag in the high word),
// a device-scope atomic load: never served by a stale cache line, and value
// and tag always come from the same store.
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Up to CW consecutive elements (count of them, even) into fp32 registers;
// the rest are zero.  vec: 16-byte aligned rows, count a multiple of 4.
template <int CW, typename T>
__device__ __forceinline__ void load_row_f32(const T* p, int count, bool vec, float (&out)[CW]) {
  constexpr int PER = Elem<T>::kPerLane;
  if (vec) {
#pragma unroll
    for (int e = 0; e < CW; e += PER) {
      const bool ok = e < count;
      float v[PER];
      load16_f32(p + (ok ? e : 0), v);
#pragma unroll
      for (int q = 0; q < PER; ++q) out[e + q] = ok ? v[q] : 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      const bool ok = e < count;
      const float v = Elem<T>::to_f32(p[ok ? e : 0]);
      out[e] = ok ? v : 0.f;
    }
  }
}

// Up to CW consecutive bf16 elements (count of them, even) as packed pairs;
// the rest are zero.  vec: 16-byte aligned rows, count a multiple of 8.
template <int CW>
__device__ __forceinline__ void load_row_bf16(const uint16_t* p, int count, bool vec, uint32_t (&out)[CW / 2]) {
  if (vec) {
#pragma unroll
    for (int c = 0; c < CW / 8; ++c) {
      const bool ok = 8 * c < count;
      const uint4 v = *reinterpret_cast<const uint4*>(p + (ok ? 8 * c : 0));
      out[4 * c] = ok ? v.x : 0u;
      out[4 * c + 1] = ok ? v.y : 0u;
      out[4 * c + 2] = ok ? v.z : 0u;
      out[4 * c + 3] = ok ? v.w : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) {
      const bool ok = 2 * i < count;
      const uint32_t lo = p[ok ? 2 * i : 0], hi = p[ok ? 2 * i + 1 : 0];
      out[i] = ok ? (lo | (hi << 16)) : 0u;
    }
  }
}

// The first n (a multiple of 4, at most CW) bf16 values at p (8-byte
// aligned) as packed pairs, all requested before any is used; the rest zero.
template <int CW>
__device__ __forceinline__ void read_slice_bf16(const uint16_t* p, int n, uint2 (&x)[CW / 4]) {
#pragma unroll
  for (int c = 0; c < CW / 4; ++c) x[c] = 4 * c < n ? *reinterpret_cast<const uint2*>(p + 4 * c) : make_uint2(0u, 0u);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// sum_e w[e] x[e] over CW bf16 products (two per instruction, fp32
// accumulation), four independent partial sums
template <int CW>
__device__ __forceinline__ float dot_bf16(const uint32_t (&w)[CW / 2], const uint2 (&x)[CW / 4]) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CW / 4; ++c) {
    acc[c & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2 * c]),
                                                  __builtin_bit_cast(bf16x2, x[c].x), acc[c & 3], false);
    acc[c & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2 * c + 1]),
                                                  __builtin_bit_cast(bf16x2, x[c].y), acc[c & 3], false);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// The first n (a multiple of 4, at most CW) floats at p, 16 bytes at a time,
// all requested before any is used (LDS latency is paid once); the rest zero.
template <int CW>
__device__ __forceinline__ void read_slice_f32(const float* p, int n, float4 (&x)[CW / 4]) {
#pragma unroll
  for (int c = 0; c < CW / 4; ++c)
    x[c] = 4 * c < n ? *reinterpret_cast<const float4*>(p + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
}
// sum_e w[e] x[e] over CW elements, four independent partial sums
template <int CW>
__device__ __forceinline__ float dot_f32(const float (&w)[CW], const float4 (&x)[CW / 4]) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CW / 4; ++c)
    acc[c & 3] += (w[4 * c] * x[c].x + w[4 * c + 1] * x[c].y) + (w[4 * c + 2] * x[c].z + w[4 * c + 3] * x[c].w);
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// LDS layout (fp32):
//   s   [rpt][r]        state (identical in every team member)
//   u   [rpt][64]       silu(t) of this workgroup's rows
//   pk  [rpt][K][64]    P values of this workgroup's rows
//   red [8][rpt][64]    per-wave partial sums of t
// and, for bf16 weights, bf16 copies of s [rpt][r] and u [rpt][64] (the
// matrix-vector inputs: bf16 products, fp32 sums); then, at byte offset
// stage (256-aligned) when given, the staged bf16 weight slices as 16-byte
// chunks: W_up[:, r0:r1] as [r][8] (row slices padded to 8 chunks) and
// W_s[r0:r1, :] as [nr][r / 8].
// One team member: workgroup j of team `team` (requests team * rpt ...).
// sw: when given (bf16 states read by other workgroups of the launch), each
// member publishes its rows of every new state as tagged words [token][r / 2]
// (two bf16 values in the low half, the step's tag in the high half; one
// device-scope atomic store each), so readers need no counter: a word with
// the right tag carries its values.
template <typename T, int TEAM>
__device__ __forceinline__ void scan_team(const ScanArgs& a, float* sm, int team, int j, uint64_t* sw) {
  constexpr int H = TEAM / 8;                 // column halves per wave in the first product
  constexpr int CW = 64 / H;                  // register slice width (columns, inputs)
  constexpr bool kBf16 = sizeof(T) == 2;
  const int r = a.r;
  const int rpt = a.rpt;                      // requests per team
  const int b0 = team * rpt;
  const int nb = (a.B - b0) < rpt ? (a.B - b0) : rpt;
  const int nr = r / TEAM, r0 = j * nr;      // this workgroup's rows (at most CW)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane % CW, half = lane / CW;   // first product: row, column half
  const int ncol = r / (8 * H);               // its columns per lane
  const int c0 = wave * (r / 8) + half * ncol;

  float* s = sm;
  float* u = s + rpt * r;
  float* pk = u + rpt * 64;
  float* red = pk + rpt * a.K * 64;
  uint16_t* s16 = reinterpret_cast<uint16_t*>(red + 8 * rpt * 64);
  uint16_t* u16 = s16 + rpt * r;

  const T* Wd = static_cast<const T*>(a.w_down);
  const T* Wu = static_cast<const T*>(a.w_up);
  const long ldd = static_cast<long>(a.D) + r;
  // 16-byte aligned register slices
  const bool vec_u = Elem<T>::kPerLane == 4 ? nr % 4 == 0 : nr % 8 == 0;
  const bool vec_s = Elem<T>::kPerLane == 4 ? ncol % 4 == 0 : ncol % 8 == 0;

  // ---- one-shot preload: the P values, W_up columns (second product, thread
  //      = output row n) and W_s rows (first product)
  float wu_reg[CW], ws_reg[CW];               // fp32 weights
  uint32_t wu_p[CW / 2], ws_p[CW / 2];        // bf16 weights, packed pairs
  constexpr int kPMax = 8;                    // P values per thread and pass
  const int np = nb * a.K * nr;
  auto p_index = [&](int idx) {
    const int bb = idx / (a.K * nr), k = (idx / nr) % a.K, i = idx % nr;
    return (static_cast<long>(b0 + bb) * a.K + k) * r + r0 + i;
  };
  auto p_slot = [&](int idx) {
    const int bb = idx / (a.K * nr), k = (idx / nr) % a.K, i = idx % nr;
    return (bb * a.K + k) * 64 + i;
  };
  // one P value: from P, or summed from the helpers' tagged k-slice partials
  // (polled until every slice's word carries tag 1; bounded)
  unsigned* pstatus = a.counters + CNT_STATUS;
  auto load_p = [&](int idx) -> float {
    const long o = p_index(idx);
    if (!a.Pw) return a.P[o];
    const long t = o / r, n = o % r;
    const long stride = static_cast<long>(a.B) * a.K * r;
    float v = 0.f;
    for (int q = 0; q < a.Pslices; ++q) {
      const uint64_t* w = a.Pw + q * stride + t * r + n;
      uint64_t x = ld_tagged(w);
      unsigned spins = 0;
      while ((x >> 32) != 1u) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          atomicOr(pstatus, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
          break;
        }
        x = ld_tagged(w);
      }
      v += __uint_as_float(static_cast<uint32_t>(x));
    }
    return v;
  };
  const int n_own = static_cast<int>(threadIdx.x) < r ? static_cast<int>(threadIdx.x) : 0;
  const int row_c = row < nr ? row : 0;
  bool staged = false;
  if constexpr (kBf16) {
    if (a.stage > 0 && np <= kPMax * kThreads) {
      // Both slices pass through LDS: direct-to-LDS loads in which consecutive
      // lanes take consecutive 16-byte chunks of a row, so one wave
      // instruction covers whole cache lines (thread-per-row loads would touch
      // 64 lines per instruction); then each thread reads its row back.  The
      // chunk index inside a row is XOR-ed with the row's low three bits, so
      // that the read-back of one chunk by 8 consecutive rows hits 8 different
      // bank groups.
      staged = true;
      const int cpr = nr / 8, cps = r / 8;    // 16-byte chunks of a W_up row slice / of a W_s row
      uint4* su = reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(sm) + a.stage);   // [r][8]
      uint4* sw = su + r * 8;                                                                   // [nr][cps]
      for (int i = wave * 64; i < r * 8; i += kThreads) {
        const int p = i + lane, n = p >> 3, k = (p & 7) ^ (n & 7);
        if (k < cpr) load_lds16(Wu + static_cast<long>(n) * r + r0 + k * 8, su + i);
      }
      for (int i = wave * 64; i < nr * cps; i += kThreads) {
        const int p = i + lane, rw = p / cps, c = (p % cps) ^ (rw & 7);
        if (rw < nr) load_lds16(Wd + static_cast<long>(r0 + rw) * ldd + a.D + c * 8, sw + i);
      }
      // the P values behind the weight slices (in the fused kernel they are
      // still being computed by the helpers while the slices arrive)
      float pv[kPMax];
#pragma unroll
      for (int q = 0; q < kPMax; ++q) {
        const int idx = static_cast<int>(threadIdx.x) + q * kThreads;
        pv[q] = (a.Pw && idx >= np) ? 0.f : load_p(idx < np ? idx : np - 1);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      __syncthreads();
#pragma unroll
      for (int k = 0; k < CW / 8; ++k) {
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
        const uint4 vu = k < cpr ? su[n_own * 8 + (k ^ (n_own & 7))] : zero;
        const uint4 vs = k < ncol / 8 ? sw[row_c * cps + (((c0 >> 3) + k) ^ (row_c & 7))] : zero;
        wu_p[4 * k] = vu.x; wu_p[4 * k + 1] = vu.y; wu_p[4 * k + 2] = vu.z; wu_p[4 * k + 3] = vu.w;
        ws_p[4 * k] = vs.x; ws_p[4 * k + 1] = vs.y; ws_p[4 * k + 2] = vs.z; ws_p[4 * k + 3] = vs.w;
      }
#pragma unroll
      for (int q = 0; q < kPMax; ++q) {
        const int idx = static_cast<int>(threadIdx.x) + q * kThreads;
        if (idx < np) pk[p_slot(idx)] = pv[q];
      }
    }
  }
  if (!staged) {
    if constexpr (kBf16) {
      load_row_bf16<CW>(Wu + static_cast<long>(n_own) * r + r0, nr, vec_u, wu_p);
    } else {
      load_row_f32<CW>(Wu + static_cast<long>(n_own) * r + r0, nr, vec_u, wu_reg);
    }
    for (int base = threadIdx.x; base < np; base += kPMax * kThreads) {
      float pv[kPMax];
#pragma unroll
      for (int q = 0; q < kPMax; ++q) {
        const int idx = base + q * kThreads;
        pv[q] = (a.Pw && idx >= np) ? 0.f : load_p(idx < np ? idx : np - 1);   // clamped: unconditional loads
      }
#pragma unroll
      for (int q = 0; q < kPMax; ++q) {
        const int idx = base + q * kThreads;
        if (idx < np) pk[p_slot(idx)] = pv[q];
      }
    }
    if constexpr (kBf16) {
      load_row_bf16<CW>(Wd + (r0 + row_c) * ldd + a.D + c0, ncol, vec_s, ws_p);
    } else {
      load_row_f32<CW>(Wd + (r0 + row_c) * ldd + a.D + c0, ncol, vec_s, ws_reg);
    }
  }

  unsigned* status = a.counters + CNT_STATUS;
  for (int idx = threadIdx.x; idx < rpt * r; idx += kThreads) s[idx] = 0.f;
  // u past the workgroup's rows stays zero (read by the 4-wide chunks)
  for (int idx = threadIdx.x; idx < rpt * 64; idx += kThreads) u[idx] = 0.f;
  if constexpr (kBf16) {
    for (int idx = threadIdx.x; idx < rpt * r; idx += kThreads) s16[idx] = 0;
    for (int idx = threadIdx.x; idx < rpt * 64; idx += kThreads) u16[idx] = 0;
  }
  // the weight slices are used at every step: settle their loads once here,
  // so that no wait inside the loop is tied to them
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  uint64_t* U64 = reinterpret_cast<uint64_t*>(a.U);

  for (int k = 0; k < a.K; ++k) {
    // (1) t = P_k + W_s s for this workgroup's rows; the state is zero at the
    //     first step
    if (k > 0) {
      for (int bb = 0; bb < nb; ++bb) {
        float d;
        if constexpr (kBf16) {
          uint2 x[CW / 4];
          read_slice_bf16<CW>(s16 + bb * r + c0, ncol, x);
          d = dot_bf16<CW>(ws_p, x);
        } else {
          float4 x[CW / 4];
          read_slice_f32<CW>(s + bb * r + c0, ncol, x);
          d = dot_f32<CW>(ws_reg, x);
        }
        if constexpr (H == 2) d += __shfl_xor(d, 32, kWave);   // the other column half
        if (half == 0) red[(wave * rpt + bb) * 64 + row] = d;
      }
    }
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < nb * 64) {
      const int bb = threadIdx.x >> 6;
      if (lane < nr) {
        float t = pk[(bb * a.K + k) * 64 + lane];
        if (k > 0) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < 8; ++w) acc += red[(w * rpt + bb) * 64 + lane];
          t += acc;
        }
        const float sl = t / (1.0f + expf(-t));
        if constexpr (kBf16) u16[bb * 64 + lane] = f32_to_bf16(sl);
        else u[bb * 64 + lane] = sl;
      }
    }
    __syncthreads();
    // (2) this workgroup's contribution c_n = sum_i W_up[n, r0 + i] u_i,
    //     thread = output row n, stored with the step's tag beside it
    const unsigned tag = a.tag0 + static_cast<unsigned>(k) + 1u;
    uint64_t* part_out = U64 + ((static_cast<long>(k & 1) * a.B + b0) * TEAM + j) * r;
    if (static_cast<int>(threadIdx.x) < r) {
      for (int bb = 0; bb < nb; ++bb) {
        float d;
        if constexpr (kBf16) {
          uint2 x[CW / 4];
          read_slice_bf16<CW>(u16 + bb * 64, nr, x);
          d = dot_bf16<CW>(wu_p, x);
        } else {
          float4 x[CW / 4];
          read_slice_f32<CW>(u + bb * 64, nr, x);
          d = dot_f32<CW>(wu_reg, x);
        }
        const uint64_t tv = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(d);
        __hip_atomic_store(part_out + static_cast<long>(bb) * TEAM * r + threadIdx.x, tv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // (3) s += sum over the team's contributions, in workgroup order; each
    //     thread re-reads its entries until all carry this step's tag
    const long ubase = (static_cast<long>(k & 1) * a.B + b0) * TEAM * r;
    for (int q = threadIdx.x; q < nb * r; q += kThreads) {
      const int bb = q / r, n = q % r;
      const uint64_t* src = U64 + ubase + static_cast<long>(bb) * TEAM * r + n;
      uint64_t v[TEAM];
#pragma unroll
      for (int w = 0; w < TEAM; ++w) v[w] = ld_tagged(src + w * r);
      unsigned spins = 0;
      for (;;) {
        unsigned bad = 0;
#pragma unroll
        for (int w = 0; w < TEAM; ++w) bad |= static_cast<unsigned>(v[w] >> 32) ^ tag;
        if (bad == 0) break;
        if (++spins > kSpinLimit) {
          atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int w = 0; w < TEAM; ++w) v[w] = ld_tagged(src + w * r);
      }
      float acc = s[bb * r + n];
#pragma unroll
      for (int w = 0; w < TEAM; ++w) acc += __uint_as_float(static_cast<unsigned>(v[w]));
      s[bb * r + n] = acc;
      if constexpr (kBf16) s16[bb * r + n] = f32_to_bf16(acc);
      // the neighbouring element (n ^ 1: same wave, same side of every row
      // boundary since r, r0 and nr are even) for the two-value words
      const float acc_pair = (kBf16 && sw) ? __shfl_xor(acc, 1, kWave) : 0.f;
      if (n >= r0 && n < r0 + nr) {   // this workgroup's rows
        const long o = (static_cast<long>(b0 + bb) * a.K + k) * r + n;
        a.Sf[o] = acc;
        if (a.tap) a.tap[o] = acc;
        if (kBf16 && sw) {
          if ((n & 1) == 0) {
            const uint32_t lo = f32_to_bf16(acc);
            const uint32_t hi = f32_to_bf16(acc_pair);
            __hip_atomic_store(sw + o / 2, (static_cast<uint64_t>(tag) << 32) | (hi << 16) | lo,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          static_cast<T*>(a.Sb)[o] = Elem<T>::from_f32(acc);
        }
      }
    }
    __syncthreads();
  }
}

inline size_t scan_smem(int r, int rpt, int K) {
  return (static_cast<size_t>(rpt) * r + rpt * 64 + static_cast<size_t>(rpt) * K * 64 + 8 * rpt * 64) * 4 +
         (static_cast<size_t>(rpt) * r + rpt * 64) * 2;
}

// Team LDS with the weight staging area behind the scan's own regions when
// it fits (bf16 weights, 16-byte row slices, one pass of P values).
constexpr size_t kTeamLdsMax = 152 * 1024;
inline size_t team_lds(int r, int team, int rpt, int K, bool bf16, int* stage) {
  const size_t base = (scan_smem(r, rpt, K) + 255) / 256 * 256;
  const int nr = r / team;
  const size_t st = (static_cast<size_t>(r) * 8 + static_cast<size_t>(nr) * (r / 8)) * 16;   // [r][8] + [nr][r/8] chunks
  const bool ok = bf16 && nr % 8 == 0 && static_cast<long>(rpt) * K * nr <= 8 * kThreads &&
                  base + st <= kTeamLdsMax;
  *stage = ok ? static_cast<int>(base) : 0;
  return ok ? base + st : scan_smem(r, rpt, K);
}

// Requests per team: enough to cover B with one launch of the most teams a
// launch holds, at most kReq.
inline int pick_rpt(int B, int r) {
  const int tpl = teams_per_launch(r, B);
  int rpt = (B + tpl - 1) / tpl;
  return rpt < kReq ? rpt : kReq;
}

}  // namespace scan_detail

}  // namespace dlite
