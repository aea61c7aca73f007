// ue8m0.hip -- the dense GEMM with power-of-two (UE8M0) factors, in a
// translation unit of its own so that it is compiled without the VGPR-form
// MFMA option (see ue8m0_launch.hpp).  The kernel is gemm_fp8_ue8m0_kernel in
// gemm_kernel.hpp; the C entry point and its checks are in fp8gemm.hip.

#include "ue8m0_launch.hpp"

namespace fg {
namespace {

template <class C>
int occupancy() {
  int o = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, gemm_fp8_ue8m0_kernel<C>, C::THREADS, 0);
  return (e == hipSuccess && o >= 1) ? o : 1;
}

template <class C>
hipError_t launch(const GemmParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp8_ue8m0_kernel<C>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int ue8m0_occupancy(int tile) {
  switch (tile) {
    case kUe8m0Tile256x160: return occupancy<BigCfg<256, 160, 4, 2>>();
    case kUe8m0Tile128x256: return occupancy<BigCfg<128, 256, 2, 4>>();
    default: return occupancy<BigCfg<256, 224, 4, 2>>();
  }
}

hipError_t ue8m0_launch(const GemmParams& p, int tile, int64_t grid, hipStream_t stream) {
  switch (tile) {
    case kUe8m0Tile256x160: return launch<BigCfg<256, 160, 4, 2>>(p, grid, stream);
    case kUe8m0Tile128x256: return launch<BigCfg<128, 256, 2, 4>>(p, grid, stream);
    default: return launch<BigCfg<256, 224, 4, 2>>(p, grid, stream);
  }
}

}  // namespace fg
