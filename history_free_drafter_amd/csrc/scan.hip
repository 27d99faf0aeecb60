// Sequential head: K dependent steps of a rank-r recurrent state.
//
//   s_0 = 0,  s_k = s_{k-1} + W_up silu(P_k + W_s s_{k-1}),
//   P_k = W_down[:, :D] h_k (one batched GEMM before this kernel),
//   W_s = W_down[:, D:].
//
// The state is narrow (r <= 1024) but its two r x r matrices are re-applied at
// every step, so a single workgroup would re-read them from L2 K times.  The
// rows are spread over NWG workgroups instead: each owns a slice of rows of
// W_s and W_up for all requests, and the workgroups meet at a device-scope
// barrier after each half step (state -> gate input, gate -> state).  All
// workgroups are resident at once (NWG <= 128 small groups), and every wait is
// bounded: a barrier that does not complete within its spin budget is marked in
// the status word and released, so the kernel always drains.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 22;

__device__ __forceinline__ void grid_sync(unsigned* cnt, unsigned target, unsigned* status) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(cnt, 1u);
    unsigned spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        atomicOr(status, static_cast<unsigned>(STATUS_BARRIER_TIMEOUT));
        break;
      }
    }
  }
  __syncthreads();
  __threadfence();
}

template <typename T>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  const int NWG = gridDim.x, g = blockIdx.x;
  const int r = a.r;
  const int r0 = (g * r) / NWG, r1 = ((g + 1) * r) / NWG;
  const int nrows = r1 - r0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const T* Wd = static_cast<const T*>(a.w_down);
  const T* Wu = static_cast<const T*>(a.w_up);
  const long ldd = static_cast<long>(a.D) + r;
  const int pairs = a.B * nrows;
  unsigned* cnt = a.counters + CNT_SCAN_BAR;
  unsigned* status = a.counters + CNT_STATUS;
  unsigned bar = 0;

  for (int k = 0; k < a.K; ++k) {
    // gate input of my rows: P_k + W_s s_{k-1}
    for (int p = wave; p < pairs; p += nw) {
      const int b = p / nrows, row = r0 + p % nrows;
      float acc = 0.f;
      if (k > 0) {
        const float* sp = a.Sf + (static_cast<long>(b) * a.K + k - 1) * r;
        const T* wr = Wd + row * ldd + a.D;
        for (int j = lane; j < r; j += 64) acc += Elem<T>::to_f32(wr[j]) * sp[j];
      }
      acc = wave_sum(acc);
      if (lane == 0) {
        const float t = a.P[(static_cast<long>(b) * a.K + k) * r + row] + acc;
        a.U[static_cast<long>(b) * r + row] = t / (1.0f + expf(-t));
      }
    }
    grid_sync(cnt, ++bar * NWG, status);
    // state of my rows: s_{k-1} + W_up silu(.)
    for (int p = wave; p < pairs; p += nw) {
      const int b = p / nrows, row = r0 + p % nrows;
      const float* up = a.U + static_cast<long>(b) * r;
      const T* wr = Wu + static_cast<long>(row) * r;
      float acc = 0.f;
      for (int j = lane; j < r; j += 64) acc += Elem<T>::to_f32(wr[j]) * up[j];
      acc = wave_sum(acc);
      if (lane == 0) {
        const long o = (static_cast<long>(b) * a.K + k) * r + row;
        const float prev = k > 0 ? a.Sf[o - r] : 0.f;
        const float s = prev + acc;
        a.Sf[o] = s;
        static_cast<T*>(a.Sb)[o] = Elem<T>::from_f32(s);
        if (a.tap) a.tap[o] = s;
      }
    }
    if (k + 1 < a.K) grid_sync(cnt, ++bar * NWG, status);
  }
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, bool bf16, hipStream_t st) {
  const int nwg = a.r < 128 ? a.r : 128;
  const dim3 grid(nwg), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL(scan_kernel<uint16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(scan_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dlite
