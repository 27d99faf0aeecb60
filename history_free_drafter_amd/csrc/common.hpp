// Device helpers shared by the DLite kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlite {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte load of data read exactly once (weights): non-temporal hint.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at l + 16 i (l is the same for the whole wave; inactive lanes write nothing).
__device__ __forceinline__ void load_lds16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(l), 16, 0, 0);
}
// The same with the non-temporal hint (data read once from HBM).
__device__ __forceinline__ void load_lds16_nt(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(l), 16, 0, 2);
}

// ------------------------------------------------------------ bf16 <-> f32 --

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Storage-type traits: 16 bytes per lane per k-step of one MFMA group.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {        // bf16 storage
  static constexpr int kPerLane = 8;       // elements in 16 bytes
  __device__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static constexpr int kPerLane = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};

// Load 16 bytes holding kPerLane elements as floats.
__device__ __forceinline__ void load16_f32(const uint16_t* p, float* out) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load16_f32(const float* p, float* out) {
  float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

// One k-step of a 16x16 MFMA tile: acc[16 x 16] += A[16 x k] * B[k x 16].
// Each lane supplies 16 bytes of A (row lane%16) and of B (column lane%16);
// the lane group lane/16 selects which k elements; A and B use the same
// lane -> k assignment, so any consistent assignment gives the exact sum.
__device__ __forceinline__ floatx4 mma_step(uint4 a, uint4 b, floatx4 acc, uint16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_step(uint4 a, uint4 b, floatx4 acc, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  return acc;
}

// Pack kPerLane floats into the 16-byte storage form.
__device__ __forceinline__ uint4 pack16(const float* v, uint16_t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 pack16(const float* v, float) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                    __float_as_uint(v[2]), __float_as_uint(v[3]));
}

// ------------------------------------------------------------- reductions --

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// (value, index) max with ties to the lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Physical row of logical token row r under a (group, stride, offset) map:
// tokens come in groups of g consecutive rows starting at `off` inside blocks
// of `stride` rows.
struct RowMap {
  int g = 1, stride = 1, off = 0;   // default: the identity
  __device__ __forceinline__ long row(int r) const {
    return static_cast<long>(r / g) * stride + off + (r % g);
  }
};

// Local token group of one request (DLite walkthrough, section "局部位置编码
// 切断草稿端的全局位置增长": the position builder may take a fixed-length group
// of local tokens and puts the origin at the start of its valid part).  The
// group is the G - 1 tokens before the anchor (oldest first, ids[0 .. G-2])
// and the anchor; leading negative ids are padding (fewer tokens exist).
// Returns the number of padding slots, 0 .. G - 1 (the anchor always counts).
__device__ __forceinline__ int group_pad(const int32_t* ids, int G) {
  int pad = 0;
  while (pad < G - 1 && ids[pad] < 0) ++pad;
  return pad;
}

// Local position of slot s of a request with m feature slots, a group of G
// slots (pad of them padding) and placeholders after it: the first real group
// token at 0, the anchor at n - 1 (n = G - pad real tokens), the feature slots
// with the anchor, placeholder k (slot m + G - 1 + k) at n - 1 + k.  Padding
// slots are no keys; their position is 0.  G = 1 is the Figure 3 layout.
__device__ __forceinline__ int group_position(int s, int m, int G, int pad) {
  const int n = G - pad;
  if (s < m) return n - 1;
  if (s < m + G) return s - m >= pad ? s - m - pad : 0;
  return n - 1 + (s - m - G + 1);
}

}  // namespace dlite
