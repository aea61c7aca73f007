// ue8m0.hip -- the dense and grouped GEMMs with power-of-two (UE8M0)
// factors, in a translation unit of its own so that it is compiled without the VGPR-form
// MFMA option (see ue8m0_launch.hpp).  The kernel is gemm_fp8_ue8m0_kernel in
// gemm_kernel.hpp; the C entry point and its checks are in fp8gemm.hip.

#include "ue8m0_launch.hpp"

namespace fg {
namespace {

template <class C, int L, bool KTAIL>
int occupancy() {
  int o = 0;
  const hipError_t e =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, gemm_fp8_ue8m0_kernel<C, L, KTAIL>, C::THREADS, 0);
  return (e == hipSuccess && o >= 1) ? o : 1;
}

template <class C, int L, bool KTAIL>
hipError_t launch(const GemmParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp8_ue8m0_kernel<C, L, KTAIL>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int L, bool KTAIL>
int occupancy_of(int tile) {
  switch (tile) {
    case kUe8m0Tile256x160: return occupancy<BigCfg<256, 160, 4, 2>, L, KTAIL>();
    case kUe8m0Tile128x256: return occupancy<BigCfg<128, 256, 2, 4>, L, KTAIL>();
    default: return occupancy<BigCfg<256, 224, 4, 2>, L, KTAIL>();
  }
}

template <int L, bool KTAIL>
hipError_t launch_of(const GemmParams& p, int tile, int64_t grid, hipStream_t stream) {
  switch (tile) {
    case kUe8m0Tile256x160: return launch<BigCfg<256, 160, 4, 2>, L, KTAIL>(p, grid, stream);
    case kUe8m0Tile128x256: return launch<BigCfg<128, 256, 2, 4>, L, KTAIL>(p, grid, stream);
    default: return launch<BigCfg<256, 224, 4, 2>, L, KTAIL>(p, grid, stream);
  }
}

template <bool KTAIL>
int occupancy_k(int tile, int layout) {
  switch (layout) {
    case kMasked: return occupancy_of<kMasked, KTAIL>(tile);
    case kContiguous: return occupancy_of<kContiguous, KTAIL>(tile);
    default: return occupancy_of<kDense, KTAIL>(tile);
  }
}

template <bool KTAIL>
hipError_t launch_k(const GemmParams& p, int tile, int layout, int64_t grid, hipStream_t stream) {
  switch (layout) {
    case kMasked: return launch_of<kMasked, KTAIL>(p, tile, grid, stream);
    case kContiguous: return launch_of<kContiguous, KTAIL>(p, tile, grid, stream);
    default: return launch_of<kDense, KTAIL>(p, tile, grid, stream);
  }
}

}  // namespace

int ue8m0_occupancy(int tile, int layout, bool ktail) {
  return ktail ? occupancy_k<true>(tile, layout) : occupancy_k<false>(tile, layout);
}

hipError_t ue8m0_launch(const GemmParams& p, int tile, int layout, int64_t grid, hipStream_t stream) {
  return (p.K & 127) ? launch_k<true>(p, tile, layout, grid, stream) : launch_k<false>(p, tile, layout, grid, stream);
}

}  // namespace fg
