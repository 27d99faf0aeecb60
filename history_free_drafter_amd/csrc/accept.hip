// Greedy prefix accept: one lane per request.
//
// A = number of leading positions where the draft equals the target's greedy
// token (DLite walkthrough, section "一次因果前向评估整条候选": only the first
// unbroken run of matches is committed); the next anchor is the target token at
// verify index A ("一轮执行后，缓存、锚点与隐藏状态怎样对齐").  Integer only.
#include "kernels.hpp"

namespace dlite {

namespace {

// K positions compared; candidate rows ldc apart, target rows ldt apart (a
// verify window shorter than the drafted block compares only its first
// candidates).
__global__ __launch_bounds__(256) void accept_kernel(const int32_t* __restrict__ cand,
                                                     const int32_t* __restrict__ tgt,
                                                     int B, int K, int ldc, int ldt,
                                                     int32_t* __restrict__ A,
                                                     int32_t* __restrict__ next) {
  constexpr int kChunk = 16;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* c = cand + static_cast<long>(b) * ldc;
  const int32_t* t = tgt + static_cast<long>(b) * ldt;
  // positions are compared kChunk at a time: all loads of a chunk are issued
  // before any comparison, so a block costs one memory round trip, not K
  const int bonus = t[K];
  int n = 0, nv = bonus;
  for (int k0 = 0; k0 < K; k0 += kChunk) {
    int cv[kChunk], tv[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int k = k0 + i < K ? k0 + i : K - 1;
      cv[i] = c[k];
      tv[i] = t[k];
    }
    int run = 0;
    bool broken = false;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      broken = broken || k0 + i >= K || cv[i] != tv[i];
      run += broken ? 0 : 1;
    }
    n += run;
    if (run < kChunk) {
      // the first failing position lies in this chunk (or is the bonus slot)
#pragma unroll
      for (int i = 0; i < kChunk; ++i) nv = (i == run && k0 + i < K) ? tv[i] : nv;
      break;
    }
  }
  A[b] = n;
  if (next) next[b] = nv;
}

// One lane: the status word of the last draft step that used the workspace.
__global__ __launch_bounds__(64) void status_copy_kernel(const unsigned* __restrict__ word,
                                                         uint32_t* __restrict__ out) {
  if (threadIdx.x == 0) out[0] = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_status_copy(const unsigned* word, uint32_t* out, hipStream_t st) {
  launch_k(status_copy_kernel, dim3(1), dim3(64), 0, st, word, out);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* cand, const int32_t* tgt, int B, int K,
                         int32_t* A, int32_t* next, hipStream_t st) {
  return launch_accept_window(cand, K, tgt, B, K + 1, A, next, st);
}

hipError_t launch_accept_window(const int32_t* cand, int K, const int32_t* tgt, int B, int W,
                                int32_t* A, int32_t* next, hipStream_t st) {
  const dim3 block(256), grid((B + 255) / 256);
  launch_k(accept_kernel, grid, block, 0, st, cand, tgt, B, W - 1, K, W, A, next);
  return hipGetLastError();
}

}  // namespace dlite
