// Sequential head: K dependent steps of a rank-r recurrent state (the team
// routine lives in scan_team.hpp); this file holds the stand-alone launch.
#include "scan_team.hpp"

namespace dlite {

using namespace scan_detail;

namespace {

template <typename T>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) float sm[];
  scan_team<T>(a, sm, blockIdx.x / kTeam, blockIdx.x % kTeam, nullptr);
}

}  // namespace

size_t scan_scratch_floats(int B, int r) {
  const int b = B < kTeamsPerLaunch * kReq ? B : kTeamsPerLaunch * kReq;
  return 4 * static_cast<size_t>(b) * kTeam * r;   // [2][b][kTeam][r] tagged 64-bit words
}

hipError_t launch_scan(const ScanArgs& a0, bool bf16, hipStream_t st) {
  const int rpt = pick_rpt(a0.B);
  int stage = 0;
  const size_t sm = team_lds(a0.r, rpt, a0.K, bf16, &stage);
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
    a.stage = stage;
    a.B = (a0.B - b) < per_launch ? (a0.B - b) : per_launch;
    const long off = static_cast<long>(b) * a0.K * a0.r;
    a.P = a0.P + off;
    a.Sf = a0.Sf + off;
    a.Sb = static_cast<char*>(a0.Sb) + off * (bf16 ? 2 : 4);
    a.tap = a0.tap ? a0.tap + off : nullptr;
    a.tag0 = static_cast<unsigned>(chunk * a0.K);
    const int nteam = (a.B + rpt - 1) / rpt;
    const dim3 grid(nteam * kTeam), block(kThreads);
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
