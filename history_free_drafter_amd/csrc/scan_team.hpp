// Sequential head: K dependent steps of a rank-r recurrent state.  The team
// routine here is shared by the stand-alone scan kernel and the fused
// scan + vocabulary kernel.
//
//   s_0 = 0,  s_k = s_{k-1} + W_up silu(P_k + W_s s_{k-1}),
//   P_k = W_down[:, :D] h_k (one batched GEMM before this kernel),
//   W_s = W_down[:, D:].
//
// Both r x r matrices are re-applied at every step, so one workgroup would
// re-read them from L2 K times.  Instead a team of kTeam workgroups splits the
// state index: workgroup j keeps rows [r0, r1) of W_s and the same columns of
// W_up in registers (fp32) for the whole kernel.  Per step it forms its slice
// of the gate input t = P_k + W_s s (wave w multiplies its 1/8 of the columns,
// lane = row; the eight partial sums are added through LDS in wave order),
// then its full-length contribution W_up[:, r0:r1] silu(t[r0:r1]) (thread =
// output row); after one team barrier every workgroup adds all kTeam
// contributions in the same fixed order, so each holds the identical new state
// without a second exchange.  Requests are split into teams of up to kReq
// requests; teams run independently.
//
// Latency matters more than bandwidth here: the weight slices and every
// step's P values are requested at once at the start (W_s last: the first
// step multiplies a zero state and does not need it), the state is read from
// LDS as broadcasts, and the partial contributions are read back with one
// 16-byte load per team member.
//
// The members of a team run on one XCD (workgroup i runs on XCD i % 8, so
// member j of team t gets workgroup ((t / 8) kTeam + j) 8 + t % 8) and
// exchange their contributions through that XCD's L2: device-coherent
// stores and loads that skip the per-CU L1, a wait for the stores, and a
// relaxed arrival counter, with no L2 write-back or invalidate per step.
// Every member checks its XCD id once; unless all members confirm the
// placement, the team uses release/acquire barriers instead (L2 write-back
// and invalidate around every exchange).
//
// All workgroups of a launch are resident at once (at most 256 workgroups,
// one per CU), and every wait is bounded: a barrier that does not complete
// within its spin budget is flagged in the status word and released, so the
// kernel always drains.
#pragma once

#include "kernels.hpp"

namespace dlite {

namespace scan_detail {

constexpr int kThreads = 512;
constexpr int kTeam = 8;
constexpr int kReq = 8;
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kPolicySc1 = 16;            // buffer-load cache policy: device scope
constexpr int kRsrcWord3 = 0x00020000;    // raw 32-bit buffer resource
// Requests per launch: at most 256 workgroups (one per CU, so that every team
// is resident at once).
constexpr int kTeamsPerLaunch = 256 / kTeam;

// Team barrier.  safe: release arrival and acquire after the wait (formal
// device-scope ordering).  Otherwise (all members on one XCD): every thread
// waits for its own device-coherent stores, and the arrival and the polling
// are relaxed atomics.
__device__ __forceinline__ void team_sync(unsigned* cnt, unsigned target, unsigned* status, bool safe) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    if (safe) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    else __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
        break;
      }
    }
    if (safe) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Device-coherent 32-bit accesses (served by L2, never by a stale L1 line).
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at float index i of a buffer, device-coherent (policy bit sc1);
// indices past the buffer read zeros.
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t rs, int i) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 4, 0, kPolicySc1);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Up to 64 consecutive elements (count of them, a multiple of 4) into fp32
// registers; the rest are zero.  vec: 16-byte aligned rows.
template <typename T>
__device__ __forceinline__ void load_row64(const T* p, int count, bool vec, float (&out)[64]) {
  constexpr int PER = Elem<T>::kPerLane;
  if (vec) {
#pragma unroll
    for (int e = 0; e < 64; e += PER) {
      const bool ok = e < count;
      float v[PER];
      load16_f32(p + (ok ? e : 0), v);
#pragma unroll
      for (int q = 0; q < PER; ++q) out[e + q] = ok ? v[q] : 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const bool ok = e < count;
      const float v = Elem<T>::to_f32(p[ok ? e : 0]);
      out[e] = ok ? v : 0.f;
    }
  }
}

// LDS layout (fp32):
//   s   [rpt][r]        state (identical in every team member)
//   u   [rpt][64]       silu(t) of this workgroup's rows
//   pk  [rpt][K][64]    P values of this workgroup's rows
//   red [8][rpt][64]    per-wave partial sums of t
// One team member: workgroup j of team `team` (requests team * rpt ...).
// done: when given (bf16 states), the bf16 states are stored with
// device-scope stores and the member counts itself in there once they are
// complete, for readers in other workgroups (device-scope loads).
template <typename T>
__device__ __forceinline__ void scan_team(const ScanArgs& a, float* sm, int team, int j, unsigned* done) {
  const int r = a.r;
  const int rpt = a.rpt;                      // requests per team
  const int b0 = team * rpt;
  if (b0 >= a.B) return;   // placeholder workgroup of a partly used XCD slot
  const int nb = (a.B - b0) < rpt ? (a.B - b0) : rpt;
  const int nr = r / kTeam, r0 = j * nr;     // this workgroup's rows; also columns per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  float* s = sm;
  float* u = s + rpt * r;
  float* pk = u + rpt * 64;
  float* red = pk + rpt * a.K * 64;

  const T* Wd = static_cast<const T*>(a.w_down);
  const T* Wu = static_cast<const T*>(a.w_up);
  const long ldd = static_cast<long>(a.D) + r;
  const bool vec = Elem<T>::kPerLane == 4 || (nr % 8) == 0;   // 16-byte aligned slices

  // ---- one-shot preload: W_up columns (phase 2, thread = output row n),
  //      the P values, then W_s rows (phase 1 from the second step on)
  float wu_reg[64], ws_reg[64];
  {
    const int n = threadIdx.x < r ? threadIdx.x : 0;
    load_row64(Wu + static_cast<long>(n) * r + r0, nr, vec, wu_reg);
  }
  {
    constexpr int kPMax = 8;                  // values per thread and pass
    const int np = nb * a.K * nr;
    for (int base = threadIdx.x; base < np; base += kPMax * kThreads) {
      float pv[kPMax];
#pragma unroll
      for (int q = 0; q < kPMax; ++q) {
        int idx = base + q * kThreads;
        idx = idx < np ? idx : np - 1;   // clamped: unconditional loads
        const int bb = idx / (a.K * nr), k = (idx / nr) % a.K, i = idx % nr;
        pv[q] = a.P[(static_cast<long>(b0 + bb) * a.K + k) * r + r0 + i];
      }
#pragma unroll
      for (int q = 0; q < kPMax; ++q) {
        const int idx = base + q * kThreads;
        if (idx < np) {
          const int bb = idx / (a.K * nr), k = (idx / nr) % a.K, i = idx % nr;
          pk[(bb * a.K + k) * 64 + i] = pv[q];
        }
      }
    }
  }
  {
    const int row = lane < nr ? lane : 0;
    load_row64(Wd + (r0 + row) * ldd + a.D + wave * nr, nr, vec, ws_reg);
  }

  unsigned* cnt = a.counters + CNT_TEAM0 + team;
  unsigned* place = a.counters + CNT_TEAM0 + kTeamsPerLaunch + team;
  unsigned* status = a.counters + CNT_STATUS;
  __shared__ int safe_sh;
  // placement check, settled before the first step while the W_s loads are in
  // flight: every member adds 1 to the team's placement word if XCC_ID
  // (hardware register 20, 4 bits) matches the assumed workgroup -> XCD
  // assignment, 1 << 16 if not; once all members have counted in, any high
  // bit selects the release/acquire barriers.  One device-scope atomic word
  // carries both, so no other ordering is needed.
  if (threadIdx.x == 0) {
    const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15;
    const unsigned mine = xcc == static_cast<int>(blockIdx.x & 7) ? 1u : (1u << 16);
    unsigned v = __hip_atomic_fetch_add(place, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + mine;
    const unsigned target = (a.cnt_base / static_cast<unsigned>(a.K * kTeam) + 1) * kTeam;
    unsigned spins = 0;
    while ((v & 0xffffu) < target) {
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(place, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (++spins > kSpinLimit) {
        atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
        v |= 1u << 16;
        break;
      }
    }
    safe_sh = (v >> 16) != 0;
  }
  for (int idx = threadIdx.x; idx < rpt * r; idx += kThreads) s[idx] = 0.f;
  // u past the workgroup's rows stays zero (read by the 8-wide chunks)
  for (int idx = threadIdx.x; idx < rpt * 64; idx += kThreads) u[idx] = 0.f;
  __syncthreads();
  const bool safe = safe_sh != 0;
  const __amdgpu_buffer_rsrc_t urs = __builtin_amdgcn_make_buffer_rsrc(
      a.U, 0, 2 * a.B * kTeam * r * static_cast<int>(sizeof(float)), kRsrcWord3);

  for (int k = 0; k < a.K; ++k) {
    // (1) t = P_k + W_s s: wave w multiplies columns [w nr, (w+1) nr) for
    //     row r0 + lane; the state is zero at the first step
    if (k > 0) {
      for (int bb = 0; bb < nb; ++bb) {
        const float* sv = s + bb * r + wave * nr;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int e = 0; e < 64; e += 8) {
          if (e < nr) {   // uniform
            const float4 x0 = *reinterpret_cast<const float4*>(sv + e);
            const float4 x1 = *reinterpret_cast<const float4*>(sv + e + 4);
            acc0 += (ws_reg[e] * x0.x + ws_reg[e + 1] * x0.y) + (ws_reg[e + 2] * x0.z + ws_reg[e + 3] * x0.w);
            acc1 += (ws_reg[e + 4] * x1.x + ws_reg[e + 5] * x1.y) + (ws_reg[e + 6] * x1.z + ws_reg[e + 7] * x1.w);
          }
        }
        red[(wave * rpt + bb) * 64 + lane] = acc0 + acc1;
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
        u[bb * 64 + lane] = t / (1.0f + expf(-t));
      }
    }
    __syncthreads();
    // (2) this workgroup's contribution c_n = sum_i W_up[n, r0 + i] u_i,
    //     thread = output row n
    float* part_out = a.U + ((static_cast<long>(k & 1) * a.B + b0) * kTeam + j) * r;
    if (static_cast<int>(threadIdx.x) < r) {
      for (int bb = 0; bb < nb; ++bb) {
        const float* uv = u + bb * 64;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int e = 0; e < 64; e += 8) {
          if (e < nr) {   // uniform
            const float4 x0 = *reinterpret_cast<const float4*>(uv + e);
            const float4 x1 = *reinterpret_cast<const float4*>(uv + e + 4);
            acc0 += (wu_reg[e] * x0.x + wu_reg[e + 1] * x0.y) + (wu_reg[e + 2] * x0.z + wu_reg[e + 3] * x0.w);
            acc1 += (wu_reg[e + 4] * x1.x + wu_reg[e + 5] * x1.y) + (wu_reg[e + 6] * x1.z + wu_reg[e + 7] * x1.w);
          }
        }
        st_dev(part_out + static_cast<long>(bb) * kTeam * r + threadIdx.x, acc0 + acc1);
      }
    }
    team_sync(cnt, a.cnt_base + static_cast<unsigned>((k + 1) * kTeam), status, safe);
    // (3) s += sum over the team's contributions, in workgroup order
    const float* pkk = a.U + (static_cast<long>(k & 1) * a.B + b0) * kTeam * r;
    for (int q = threadIdx.x; q < nb * (r / 4); q += kThreads) {
      const int bb = q / (r / 4), n = (q % (r / 4)) * 4;
      float4 v[kTeam];
#pragma unroll
      for (int w = 0; w < kTeam; ++w)
        v[w] = ld_dev4(urs, static_cast<int>((pkk - a.U) + (static_cast<long>(bb) * kTeam + w) * r + n));
      float4 acc = *reinterpret_cast<const float4*>(s + bb * r + n);
#pragma unroll
      for (int w = 0; w < kTeam; ++w) {
        acc.x += v[w].x; acc.y += v[w].y; acc.z += v[w].z; acc.w += v[w].w;
      }
      *reinterpret_cast<float4*>(s + bb * r + n) = acc;
      if (n >= r0 && n < r0 + nr) {   // this workgroup's rows (n, r0, nr are multiples of 4)
        const long o = (static_cast<long>(b0 + bb) * a.K + k) * r + n;
        *reinterpret_cast<float4*>(a.Sf + o) = acc;
        if (a.tap) *reinterpret_cast<float4*>(a.tap + o) = acc;
        const float av[4] = {acc.x, acc.y, acc.z, acc.w};
        if (sizeof(T) == 2 && done) {
          // read by other workgroups in this launch: one device-scope store
          uint64_t pk4 = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk4 |= static_cast<uint64_t>(Elem<T>::from_f32(av[e])) << (16 * e);
          __hip_atomic_store(reinterpret_cast<uint64_t*>(static_cast<T*>(a.Sb) + o), pk4, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) static_cast<T*>(a.Sb)[o + e] = Elem<T>::from_f32(av[e]);
        }
      }
    }
    __syncthreads();
  }
  if (done) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's state stores are done
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

inline size_t scan_smem(int r, int rpt, int K) {
  return (static_cast<size_t>(rpt) * r + rpt * 64 + static_cast<size_t>(rpt) * K * 64 + 8 * rpt * 64) * 4;
}

// Requests per team: enough to cover B with one launch of kTeamsPerLaunch
// teams, at most kReq.
inline int pick_rpt(int B) {
  int rpt = (B + kTeamsPerLaunch - 1) / kTeamsPerLaunch;
  return rpt < kReq ? rpt : kReq;
}

}  // namespace scan_detail

}  // namespace dlite
