// Sequential head: K dependent steps of a rank-r recurrent state.
//
//   s_0 = 0,  s_k = s_{k-1} + W_up silu(P_k + W_s s_{k-1}),
//   P_k = W_down[:, :D] h_k (one batched GEMM before this kernel),
//   W_s = W_down[:, D:].
//
// Both r x r matrices are re-applied at every step, so one workgroup would
// re-read them from L2 K times.  Instead a team of kTeam workgroups splits the
// state index: workgroup j keeps rows [r0, r1) of W_s and the same columns of
// W_up in LDS for the whole kernel.  Per step it forms its slice of the gate
// input t = P_k + W_s s, then its full-length contribution W_up[:, r0:r1]
// silu(t[r0:r1]) to the state update; after one team barrier every workgroup
// adds all kTeam contributions in the same fixed order, so each holds the
// identical new state without a second exchange.  Requests are split into
// teams of up to kReq requests; teams run independently.
//
// Latency matters more than bandwidth here: the weight slices and every
// step's P values are requested at once at the start, and the partial
// contributions are read back with one vector load per team member.
//
// All workgroups of a launch are resident at once (at most 256 workgroups,
// one per CU), and every wait is bounded: a barrier that does not complete
// within its spin budget is flagged in the status word and released, so the
// kernel always drains.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kThreads = 512;
constexpr int kTeam = 8;
constexpr int kReq = 4;
constexpr unsigned kSpinLimit = 1u << 22;

__device__ __forceinline__ void team_sync(unsigned* cnt, unsigned target, unsigned* status) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(cnt, 1u);
    unsigned spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
}

// 8-element dot product chunk: w (storage type, 16-byte aligned) . x (fp32)
template <typename T>
__device__ __forceinline__ float dot8(const T* w, const float* x) {
  float wv[8];
  load16_f32(w, wv);
  if constexpr (Elem<T>::kPerLane == 4) load16_f32(w + 4, wv + 4);
  const float4 x0 = *reinterpret_cast<const float4*>(x);
  const float4 x1 = *reinterpret_cast<const float4*>(x + 4);
  return (wv[0] * x0.x + wv[1] * x0.y) + (wv[2] * x0.z + wv[3] * x0.w) +
         (wv[4] * x1.x + wv[5] * x1.y) + (wv[6] * x1.z + wv[7] * x1.w);
}

// LDS layout:
//   ws [nrmax][r + 8]   W_s rows r0..r1 (storage type; padded rows stay 16-byte aligned)
//   wu [r][nrmax + 8]   W_up[:, r0..r1] in its natural row-major layout
//   s  [rpt][r]         fp32 state (identical in every team member)
//   u  [rpt][nrmax]     fp32 silu(t) of this workgroup's rows
//   pk [rpt][K][nrmax]  fp32 P values of this workgroup's rows
template <typename T>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int PER = Elem<T>::kPerLane;
  const int r = a.r;
  const int rpt = a.rpt;                      // requests per team
  const int team = blockIdx.x / kTeam, j = blockIdx.x % kTeam;
  const int b0 = team * rpt;
  const int nb = (a.B - b0) < rpt ? (a.B - b0) : rpt;
  const int r0 = (j * r) / kTeam, r1 = ((j + 1) * r) / kTeam, nr = r1 - r0;
  const int nrmax = (r + kTeam - 1) / kTeam;
  const int lds = r + 8, ldu = nrmax + 8;

  T* ws = reinterpret_cast<T*>(smem);
  T* wu = ws + static_cast<size_t>(nrmax) * lds;
  float* s = reinterpret_cast<float*>(wu + static_cast<size_t>(r) * ldu);
  float* u = s + rpt * r;
  float* pk = u + rpt * nrmax;

  const T* Wd = static_cast<const T*>(a.w_down);
  const T* Wu = static_cast<const T*>(a.w_up);
  const long ldd = static_cast<long>(a.D) + r;

  // ---- one-shot preload: the P values of every step (registers), both
  //      weight slices (16-byte loads), all requested before any is used
  {
    constexpr int kPMax = 8;                  // rpt * K * nr <= 4 * 16 * 64 values / 512 threads
    float pv[kPMax];
    const int np = nb * a.K * nr;
#pragma unroll
    for (int q = 0; q < kPMax; ++q) {
      int idx = threadIdx.x + q * kThreads;
      idx = idx < np ? idx : np - 1;   // clamped: unconditional loads
      const int bb = idx / (a.K * nr), k = (idx / nr) % a.K, i = idx % nr;
      pv[q] = a.P[(static_cast<long>(b0 + bb) * a.K + k) * r + r0 + i];
    }
    const bool vec = (r % (PER * kTeam)) == 0;   // 16-byte aligned slices
    if (vec) {
      const int vr = r / PER, vn = nr / PER;
      const int nv_s = nr * vr, nv = nv_s + r * vn;
      constexpr int kBatch = 16;
      for (int base = threadIdx.x; base < nv; base += kBatch * kThreads) {
        uint4 v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          int idx = base + q * kThreads;
          idx = idx < nv ? idx : nv - 1;   // clamped: every load is issued unconditionally
          const T* src;
          if (idx < nv_s) {
            src = Wd + (r0 + idx / vr) * ldd + a.D + (idx % vr) * PER;
          } else {
            const int t = idx - nv_s;
            src = Wu + static_cast<long>(t / vn) * r + r0 + (t % vn) * PER;
          }
          v[q] = *reinterpret_cast<const uint4*>(src);
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const int idx = base + q * kThreads;
          if (idx < nv_s) {
            *reinterpret_cast<uint4*>(ws + (idx / vr) * lds + (idx % vr) * PER) = v[q];
          } else if (idx < nv) {
            const int t = idx - nv_s;
            *reinterpret_cast<uint4*>(wu + (t / vn) * ldu + (t % vn) * PER) = v[q];
          }
        }
      }
    } else {
      for (int idx = threadIdx.x; idx < nr * r; idx += kThreads) {
        const int i = idx / r, c = idx % r;
        ws[i * lds + c] = Wd[(r0 + i) * ldd + a.D + c];
      }
      for (int idx = threadIdx.x; idx < nr * r; idx += kThreads) {
        const int n = idx / nr, i = idx % nr;
        wu[n * ldu + i] = Wu[static_cast<long>(n) * r + r0 + i];
      }
    }
    // zero the row tails so that 8-wide chunks past nr add nothing
    for (int idx = threadIdx.x; idx < r * 8; idx += kThreads)
      wu[(idx / 8) * ldu + nr + idx % 8] = Elem<T>::from_f32(0.f);
#pragma unroll
    for (int q = 0; q < kPMax; ++q) {
      const int idx = threadIdx.x + q * kThreads;
      if (idx < np) {
        const int bb = idx / (a.K * nr), k = (idx / nr) % a.K, i = idx % nr;
        pk[(bb * a.K + k) * nrmax + i] = pv[q];
      }
    }
    for (int idx = threadIdx.x; idx < rpt * r; idx += kThreads) s[idx] = 0.f;
    for (int idx = threadIdx.x; idx < rpt * nrmax; idx += kThreads) u[idx] = 0.f;
  }
  __syncthreads();

  unsigned* cnt = a.counters + CNT_TEAM0 + team;
  unsigned* status = a.counters + CNT_STATUS;
  // phase 1: thread -> (row i, one of 8 column parts); part p takes the
  // 8-column chunks p, p + 8, ... so that neighbouring lanes read neighbouring
  // 16-byte chunks (no bank conflicts); parts sit in consecutive lanes and are
  // combined by shuffles
  const int part = threadIdx.x & 7, i1 = threadIdx.x >> 3;

  for (int k = 0; k < a.K; ++k) {
    // (1) t_i = P_k[i] + sum_c W_s[i, c] s[c]
    for (int bb = 0; bb < nb; ++bb) {
      for (int i = i1; i < ((nrmax + 63) / 64) * 64; i += kThreads / 8) {
        float acc = 0.f;
        if (i < nr) {
          const T* wrow = ws + i * lds;
          const float* sv = s + bb * r;
          float a0 = 0.f, a1 = 0.f;
          int c = part * 8;
          for (; c + 64 < r; c += 128) {
            a0 += dot8(wrow + c, sv + c);
            a1 += dot8(wrow + c + 64, sv + c + 64);
          }
          if (c < r) a0 += dot8(wrow + c, sv + c);
          acc = a0 + a1;
        }
        acc += __shfl_xor(acc, 1, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        acc += __shfl_xor(acc, 4, kWave);
        if (i < nr && part == 0) {
          const float t = pk[(bb * a.K + k) * nrmax + i] + acc;
          u[bb * nrmax + i] = t / (1.0f + expf(-t));
        }
      }
    }
    __syncthreads();
    // (2) this workgroup's contribution c_n = sum_i W_up[n, r0 + i] u_i
    float* part_out = a.U + ((static_cast<long>(k & 1) * a.B + b0) * kTeam + j) * r;
    for (int q = threadIdx.x; q < nb * r; q += kThreads) {
      const int bb = q / r, n = q % r;
      const T* wrow = wu + n * ldu;
      const float* uv = u + bb * nrmax;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      int i = 0;
      for (; i + 32 <= nr; i += 32) {
        a0 += dot8(wrow + i, uv + i);
        a1 += dot8(wrow + i + 8, uv + i + 8);
        a2 += dot8(wrow + i + 16, uv + i + 16);
        a3 += dot8(wrow + i + 24, uv + i + 24);
      }
      for (; i < nr; i += 8) a0 += dot8(wrow + i, uv + i);   // tail: zero-padded
      part_out[static_cast<long>(bb) * kTeam * r + n] = (a0 + a1) + (a2 + a3);
    }
    team_sync(cnt, a.cnt_base + static_cast<unsigned>((k + 1) * kTeam), status);
    // (3) s += sum over the team's contributions, in workgroup order
    const float* pkk = a.U + (static_cast<long>(k & 1) * a.B + b0) * kTeam * r;
    for (int q = threadIdx.x; q < nb * (r / 4); q += kThreads) {
      const int bb = q / (r / 4), n = (q % (r / 4)) * 4;
      float4 v[kTeam];
#pragma unroll
      for (int w = 0; w < kTeam; ++w)
        v[w] = *reinterpret_cast<const float4*>(pkk + (static_cast<long>(bb) * kTeam + w) * r + n);
      float4 acc = *reinterpret_cast<const float4*>(s + bb * r + n);
#pragma unroll
      for (int w = 0; w < kTeam; ++w) {
        acc.x += v[w].x; acc.y += v[w].y; acc.z += v[w].z; acc.w += v[w].w;
      }
      *reinterpret_cast<float4*>(s + bb * r + n) = acc;
      const float av[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e >= r0 && n + e < r1) {
          const long o = (static_cast<long>(b0 + bb) * a.K + k) * r + n + e;
          a.Sf[o] = av[e];
          static_cast<T*>(a.Sb)[o] = Elem<T>::from_f32(av[e]);
          if (a.tap) a.tap[o] = av[e];
        }
      }
    }
    __syncthreads();
  }
}

size_t scan_smem(int r, bool bf16, int rpt, int K) {
  const int nr = (r + kTeam - 1) / kTeam;
  const size_t es = bf16 ? 2 : 4;
  size_t bytes = (static_cast<size_t>(nr) * (r + 8) + static_cast<size_t>(r) * (nr + 8)) * es;
  bytes = (bytes + 15) & ~static_cast<size_t>(15);
  return bytes + (static_cast<size_t>(rpt) * r + rpt * nr + static_cast<size_t>(rpt) * K * nr) * 4;
}

// Requests per team: as many as fit in LDS (at most kReq).
int pick_rpt(int r, bool bf16, int K) {
  for (int rpt = kReq; rpt > 1; rpt /= 2)
    if (scan_smem(r, bf16, rpt, K) <= 160 * 1024) return rpt;
  return 1;
}

// Requests per launch: at most 256 workgroups (one per CU, so that every team
// is resident at once).
constexpr int kTeamsPerLaunch = 256 / kTeam;

}  // namespace

size_t scan_scratch_floats(int B, int r) {
  const int b = B < kTeamsPerLaunch * kReq ? B : kTeamsPerLaunch * kReq;
  return 2 * static_cast<size_t>(b) * kTeam * r;
}
int scan_counters() { return kTeamsPerLaunch; }
size_t scan_lds_bytes(int r, bool bf16, int K) { return scan_smem(r, bf16, pick_rpt(r, bf16, K), K); }

hipError_t launch_scan(const ScanArgs& a0, bool bf16, hipStream_t st) {
  const int rpt = pick_rpt(a0.r, bf16, a0.K);
  const size_t sm = scan_smem(a0.r, bf16, rpt, a0.K);
  const int per_launch = kTeamsPerLaunch * rpt;
  const void* fn = bf16 ? reinterpret_cast<const void*>(&scan_kernel<uint16_t>)
                        : reinterpret_cast<const void*>(&scan_kernel<float>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(sm));
  if (e != hipSuccess) return e;
  int chunk = 0;
  for (int b = 0; b < a0.B; b += per_launch, ++chunk) {
    ScanArgs a = a0;
    a.rpt = rpt;
    a.B = (a0.B - b) < per_launch ? (a0.B - b) : per_launch;
    const long off = static_cast<long>(b) * a0.K * a0.r;
    a.P = a0.P + off;
    a.Sf = a0.Sf + off;
    a.Sb = static_cast<char*>(a0.Sb) + off * (bf16 ? 2 : 4);
    a.tap = a0.tap ? a0.tap + off : nullptr;
    a.cnt_base = static_cast<unsigned>(chunk * a0.K * kTeam);
    const dim3 grid(((a.B + rpt - 1) / rpt) * kTeam), block(kThreads);
    if (bf16)
      hipLaunchKernelGGL(scan_kernel<uint16_t>, grid, block, sm, st, a);
    else
      hipLaunchKernelGGL(scan_kernel<float>, grid, block, sm, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dlite
