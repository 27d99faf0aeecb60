// Sequential head: K dependent steps of a rank-r recurrent state (the team
// routine lives in scan_team.hpp); this file holds the stand-alone launch.
#include "scan_team.hpp"

namespace dlite {

using namespace scan_detail;

namespace {

template <typename T, int TEAM>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) float sm[];
  scan_team<T, TEAM>(a, sm, blockIdx.x / TEAM, blockIdx.x % TEAM, nullptr);
}

template <typename T, int TEAM>
hipError_t launch_team(const ScanArgs& a, size_t sm, hipStream_t st) {
  const int nteam = (a.B + a.rpt - 1) / a.rpt;
  launch_k((scan_kernel<T, TEAM>), dim3(nteam * TEAM), dim3(kThreads), sm, st, a);
  return hipGetLastError();
}

}  // namespace

size_t scan_scratch_floats(int B, int r) {
  const int per = teams_per_launch(r, B) * kReq;
  const int b = B < per ? B : per;
  return 4 * static_cast<size_t>(b) * team_size(r, B) * r;   // [2][b][team][r] tagged 64-bit words
}

hipError_t launch_scan(const ScanArgs& a0, bool bf16, hipStream_t st) {
  const int team = team_size(a0.r, a0.B);
  const int rpt = pick_rpt(a0.B, a0.r);
  int stage = 0;
  const size_t sm = team_lds(a0.r, team, rpt, a0.K, bf16, &stage);
  const int per_launch = teams_per_launch(a0.r, a0.B) * rpt;
  const void* fn = bf16 ? (team == 16 ? reinterpret_cast<const void*>(&scan_kernel<uint16_t, 16>)
                                      : reinterpret_cast<const void*>(&scan_kernel<uint16_t, 8>))
                        : (team == 16 ? reinterpret_cast<const void*>(&scan_kernel<float, 16>)
                                      : reinterpret_cast<const void*>(&scan_kernel<float, 8>));
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
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
    if (bf16) e = team == 16 ? launch_team<uint16_t, 16>(a, sm, st) : launch_team<uint16_t, 8>(a, sm, st);
    else e = team == 16 ? launch_team<float, 16>(a, sm, st) : launch_team<float, 8>(a, sm, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dlite
