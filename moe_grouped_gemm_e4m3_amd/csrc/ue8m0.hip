// ue8m0.hip -- the dense and grouped GEMMs with power-of-two (UE8M0)
// factors, in a translation unit of its own so that it is compiled without the VGPR-form
// MFMA option (see ue8m0_launch.hpp).  The kernel is gemm_fp8_ue8m0_kernel in
// gemm_kernel.hpp; the C entry point and its checks are in fp8gemm.hip.

#include "ue8m0_launch.hpp"

namespace fg {
namespace {

template <class C, int L>
int occupancy() {
  int o = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, gemm_fp8_ue8m0_kernel<C, L>, C::THREADS, 0);
  return (e == hipSuccess && o >= 1) ? o : 1;
}

template <class C, int L>
hipError_t launch(const GemmParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp8_ue8m0_kernel<C, L>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int L>
int occupancy_of(int tile) {
  switch (tile) {
    case kUe8m0Tile256x160: return occupancy<BigCfg<256, 160, 4, 2>, L>();
    case kUe8m0Tile128x256: return occupancy<BigCfg<128, 256, 2, 4>, L>();
    default: return occupancy<BigCfg<256, 224, 4, 2>, L>();
  }
}

template <int L>
hipError_t launch_of(const GemmParams& p, int tile, int64_t grid, hipStream_t stream) {
  switch (tile) {
    case kUe8m0Tile256x160: return launch<BigCfg<256, 160, 4, 2>, L>(p, grid, stream);
    case kUe8m0Tile128x256: return launch<BigCfg<128, 256, 2, 4>, L>(p, grid, stream);
    default: return launch<BigCfg<256, 224, 4, 2>, L>(p, grid, stream);
  }
}

}  // namespace

int ue8m0_occupancy(int tile, int layout) {
  switch (layout) {
    case kMasked: return occupancy_of<kMasked>(tile);
    case kContiguous: return occupancy_of<kContiguous>(tile);
    default: return occupancy_of<kDense>(tile);
  }
}

hipError_t ue8m0_launch(const GemmParams& p, int tile, int layout, int64_t grid, hipStream_t stream) {
  switch (layout) {
    case kMasked: return launch_of<kMasked>(p, tile, grid, stream);
    case kContiguous: return launch_of<kContiguous>(p, tile, grid, stream);
    default: return launch_of<kDense>(p, tile, grid, stream);
  }
}

}  // namespace fg
