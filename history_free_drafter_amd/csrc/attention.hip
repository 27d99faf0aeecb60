// Non-causal block attention over the m + G + K slots of one request.
//
// One workgroup per (request, group of HPW query heads of one key/value head):
// the block is tiny (at most 96 keys and 32 query rows), so with few requests
// the work is latency-bound and HPW = 1 spreads it over n_q * B workgroups;
// with many requests HPW grows so that the heads sharing a key/value head
// load and rotate it once.  A workgroup loads its key/value head and its query
// rows once (all global loads issued up front), builds the rotation table for
// local positions 0..G+K-1 meanwhile, rotates keys and queries into LDS, then
// each wave takes whole (head, query row) pairs: scores with one lane per key,
// the softmax in registers (wave max and sum), and the weighted sum with one
// lane per output element.  Local RoPE positions (DLite walkthrough, Figure 3
// layout and "局部位置编码切断草稿端的全局位置增长"): the first real token of
// the local group at 0, the anchor at n - 1 with every context slot, and
// placeholder k at n - 1 + k (G = 1: all at 0 but placeholder k at k); group
// padding slots are no keys.  Nothing is kept after the call.
#include "kernels.hpp"

namespace dlite {

namespace {

constexpr int kThreads = 512;
constexpr int kMaxD = 128;
constexpr int kLd = kMaxD + 4;   // padded LDS row: 16-byte aligned, banks spread
constexpr int kMaxS = 96;        // m <= 64, G <= 16, K <= 16
constexpr int kLoads = 4;        // 16-byte global loads per thread and pass

template <typename T, int DH>   // DH: head width (64 or 128), fixed so the dot products unroll
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnArgs a) {
  extern __shared__ __align__(16) float sm[];
  const int hpw = a.n_q / gridDim.x;          // query heads of this workgroup
  const int h0 = blockIdx.x * hpw, b = blockIdx.y;
  const int qpk = a.n_q / a.n_kv, kvh = h0 / qpk;   // query heads per key/value head
  constexpr int d = DH, half = d / 2, hq = half / 4;   // float4 groups per half row
  const int S = a.m + a.G + a.K, L = a.G + a.K;
  const int Hq = a.n_q * d, Hkv = a.n_kv * d;
  // group padding: slots m .. m + pad - 1 are no keys
  const int pad = a.G > 1 ? group_pad(a.gids + static_cast<long>(b) * (a.G - 1), a.G) : 0;
  const int nokey0 = a.m, nokey1 = a.m + pad;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int nw = kThreads / 64;

  float* Ks = sm;                    // [S][kLd] rotated keys
  float* Vs = Ks + S * kLd;          // [S][kLd]
  float* Qs = Vs + S * kLd;          // [hpw][L][kLd] rotated queries
  float* Ps = Qs + hpw * L * kLd;    // [hpw][L][S + 1] probabilities
  float* rc = Ps + hpw * L * (S + 1);   // [L][half] cos
  float* rs = rc + L * half;         // [L][half] sin

  // ---- work items: (key row, pair group) | (query row, pair group) |
  //      (value row, float4); every load issued before any is used
  const int nk = S * hq, nq = hpw * L * hq, nv = S * (d / 4);
  const int ntot = nk + nq + nv;
  const float* Kg = a.KV + static_cast<long>(b) * S * 2 * Hkv + kvh * d;
  const float* Vg = Kg + Hkv;
  const float* Qg = a.Q + static_cast<long>(b) * L * Hq + h0 * d;
  const int npass = (ntot + kLoads * kThreads - 1) / (kLoads * kThreads);   // same for all threads
  for (int ps = 0; ps < npass; ++ps) {
    const int base = ps * kLoads * kThreads + threadIdx.x;
    float4 lo[kLoads], hi[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      int it = base + q * kThreads;
      it = it < ntot ? it : ntot - 1;   // clamped: unconditional loads
      const float* p;
      int off2 = 0;
      if (it < nk) {
        p = Kg + static_cast<long>(it / hq) * 2 * Hkv + (it % hq) * 4;
        off2 = half;
      } else if (it < nk + nq) {
        const int t = it - nk, qrow = t / hq;   // qrow = head * L + row
        p = Qg + static_cast<long>(qrow % L) * Hq + (qrow / L) * d + (t % hq) * 4;
        off2 = half;
      } else {
        const int t = it - nk - nq;
        p = Vg + static_cast<long>(t / (d / 4)) * 2 * Hkv + (t % (d / 4)) * 4;
      }
      lo[q] = *reinterpret_cast<const float4*>(p);
      hi[q] = *reinterpret_cast<const float4*>(p + off2);
    }
    if (ps == 0) {
      // rotation table for local positions 0..L-1 while the loads are in flight:
      // frequency i is theta^(-2 i / d)
      const float l2t = log2f(a.theta);
      for (int idx = threadIdx.x; idx < L * half; idx += kThreads) {
        const int p = idx / half, i = idx % half;
        const float f = exp2f(-2.0f * static_cast<float>(i) / static_cast<float>(d) * l2t);
        float sn, cs;
        sincosf(static_cast<float>(p) * f, &sn, &cs);
        rc[idx] = cs;
        rs[idx] = sn;
      }
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int it = base + q * kThreads;
      if (it >= ntot) continue;
      if (it < nk + nq) {
        // rotate pairs (i, i + half), i = 4 g .. 4 g + 3
        const bool key = it < nk;
        const int row = key ? it / hq : (it - nk) / hq, g = key ? it % hq : (it - nk) % hq;
        const int pos = group_position(key ? row : a.m + row % L, a.m, a.G, pad);
        const float* c = rc + pos * half + 4 * g;
        const float* sn = rs + pos * half + 4 * g;
        float* dst = (key ? Ks : Qs) + row * kLd + 4 * g;
        const float x1[4] = {lo[q].x, lo[q].y, lo[q].z, lo[q].w};
        const float x2[4] = {hi[q].x, hi[q].y, hi[q].z, hi[q].w};
        float y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y1[e] = x1[e] * c[e] - x2[e] * sn[e];
          y2[e] = x1[e] * sn[e] + x2[e] * c[e];
        }
        *reinterpret_cast<float4*>(dst) = make_float4(y1[0], y1[1], y1[2], y1[3]);
        *reinterpret_cast<float4*>(dst + half) = make_float4(y2[0], y2[1], y2[2], y2[3]);
      } else {
        const int t = it - nk - nq, row = t / (d / 4);
        const bool key = row < nokey0 || row >= nokey1;   // padding values read as 0
        *reinterpret_cast<float4*>(Vs + row * kLd + (t % (d / 4)) * 4) =
            key ? lo[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  __syncthreads();

  const float scale = 1.0f / sqrtf(static_cast<float>(d));
  // ---- scores and softmax: wave w takes (head, row) pairs w, w + nw, ...
  const int lr = L - a.q0;
  for (int t = wave; t < hpw * lr; t += nw) {
    const int hh = t / lr, j = a.q0 + t % lr;
    const float* qr = Qs + (hh * L + j) * kLd;
    float sc[2];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int s = lane + 64 * ps;
      const bool ok = s < S && (s < nokey0 || s >= nokey1);
      const float* kr = Ks + (ok ? s : 0) * kLd;
      float a0 = 0.f, a1 = 0.f;
      // a partial unroll: unrolled fully, the 128-wide product's LDS reads
      // are all hoisted and the registers spill
#pragma unroll 4
      for (int e = 0; e < d; e += 8) {
        const float4 k0 = *reinterpret_cast<const float4*>(kr + e);
        const float4 k1 = *reinterpret_cast<const float4*>(kr + e + 4);
        const float4 q0 = *reinterpret_cast<const float4*>(qr + e);
        const float4 q1 = *reinterpret_cast<const float4*>(qr + e + 4);
        a0 += (q0.x * k0.x + q0.y * k0.y) + (q0.z * k0.z + q0.w * k0.w);
        a1 += (q1.x * k1.x + q1.y * k1.y) + (q1.z * k1.z + q1.w * k1.w);
      }
      sc[ps] = ok ? (a0 + a1) * scale : -INFINITY;
      if (S <= 64) break;   // uniform
    }
    if (S <= 64) sc[1] = -INFINITY;
    const float mx = wave_max(fmaxf(sc[0], sc[1]));
    const float p0 = lane < S ? expf(sc[0] - mx) : 0.f;
    const float p1 = lane + 64 < S ? expf(sc[1] - mx) : 0.f;
    const float inv = 1.0f / wave_sum(p0 + p1);
    float* pr = Ps + (hh * L + j) * (S + 1);
    if (lane < S) pr[lane] = p0 * inv;
    if (lane + 64 < S) pr[lane + 64] = p1 * inv;
  }
  __syncthreads();

  // ---- outputs: wave w takes pairs as above; lane = output element(s)
  for (int t = wave; t < hpw * lr; t += nw) {
    const int hh = t / lr, j = a.q0 + t % lr;
    const float* pr = Ps + (hh * L + j) * (S + 1);
    T* out = static_cast<T*>(a.out) + (static_cast<long>(b) * L + j) * Hq + (h0 + hh) * d;
    // lane owns elements lane + 64 c; keys in groups of four, all reads of a
    // group issued together
    constexpr int NE = d / 64;
    float acc[NE][2];
#pragma unroll
    for (int c = 0; c < NE; ++c) acc[c][0] = acc[c][1] = 0.f;
    int s = 0;
    for (; s + 3 < S; s += 4) {
      float pv[4], vv[4][NE];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pv[u] = pr[s + u];
#pragma unroll
        for (int c = 0; c < NE; ++c) vv[u][c] = Vs[(s + u) * kLd + lane + 64 * c];
      }
#pragma unroll
      for (int c = 0; c < NE; ++c) {
        acc[c][0] += pv[0] * vv[0][c] + pv[1] * vv[1][c];
        acc[c][1] += pv[2] * vv[2][c] + pv[3] * vv[3][c];
      }
    }
    for (; s < S; ++s) {
      const float p = pr[s];
#pragma unroll
      for (int c = 0; c < NE; ++c) acc[c][0] += p * Vs[s * kLd + lane + 64 * c];
    }
#pragma unroll
    for (int c = 0; c < NE; ++c) out[lane + 64 * c] = Elem<T>::from_f32(acc[c][0] + acc[c][1]);
  }
}

size_t smem_hpw(const AttnArgs& a, int hpw) {
  const int S = a.m + a.G + a.K, L = a.G + a.K;
  return (static_cast<size_t>(2 * S * kLd) + hpw * L * kLd + hpw * L * (S + 1) + L * a.d_h) * 4;
}

// Query heads per workgroup: 1 while requests x key/value heads leave CUs
// idle, else the largest divisor of the group size whose LDS fits.
int pick_hpw(const AttnArgs& a) {
  const int qpk = a.n_q / a.n_kv;
  if (static_cast<long>(a.B) * a.n_kv < 256) return 1;
  for (int h = qpk; h > 1; --h)
    if (qpk % h == 0 && smem_hpw(a, h) <= 160 * 1024) return h;
  return 1;
}

}  // namespace

size_t attention_smem(const AttnArgs& a) { return smem_hpw(a, pick_hpw(a)); }

hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t st) {
  if (a.G < 1 || a.m + a.G + a.K > kMaxS || a.d_h > kMaxD || (a.G > 1 && !a.gids))
    return hipErrorInvalidValue;
  const dim3 grid(a.n_q / pick_hpw(a), a.B), block(kThreads);
  const size_t sm = attention_smem(a);
  if (a.d_h != 64 && a.d_h != 128) return hipErrorInvalidValue;
  const void* fn;
  if (bf16) fn = a.d_h == 128 ? reinterpret_cast<const void*>(&attention_kernel<uint16_t, 128>)
                              : reinterpret_cast<const void*>(&attention_kernel<uint16_t, 64>);
  else fn = a.d_h == 128 ? reinterpret_cast<const void*>(&attention_kernel<float, 128>)
                         : reinterpret_cast<const void*>(&attention_kernel<float, 64>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(sm));
  if (e != hipSuccess) return e;
  if (bf16) {
    if (a.d_h == 128) launch_k((attention_kernel<uint16_t, 128>), grid, block, sm, st, a);
    else launch_k((attention_kernel<uint16_t, 64>), grid, block, sm, st, a);
  } else {
    if (a.d_h == 128) launch_k((attention_kernel<float, 128>), grid, block, sm, st, a);
    else launch_k((attention_kernel<float, 64>), grid, block, sm, st, a);
  }
  return hipGetLastError();
}

}  // namespace dlite
