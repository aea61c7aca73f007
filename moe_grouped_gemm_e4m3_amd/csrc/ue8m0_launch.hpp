// ue8m0_launch.hpp -- launch hooks of the power-of-two-factor GEMM kernel.
//
// The kernel lives in ue8m0.hip, a translation unit compiled without the
// option that keeps MFMA results in VGPRs: it accumulates in the matrix core
// (no VALU promotion reads the results), so its 128 accumulators go to the
// accumulation registers and the operand fragments keep the VGPRs.  The rest
// of the library calls it through these two functions (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace fg {

// Tile shapes the kernel is built for (rows x columns).
enum { kUe8m0Tile256x224 = 0, kUe8m0Tile256x160 = 1, kUe8m0Tile128x256 = 2 };
constexpr int ue8m0_tile_bm(int tile) { return tile == kUe8m0Tile128x256 ? 128 : 256; }
constexpr int ue8m0_tile_bn(int tile) { return tile == kUe8m0Tile256x160 ? 160 : tile == kUe8m0Tile128x256 ? 256 : 224; }

// Workgroups per CU of the kernel for a tile shape, layout (kDense,
// kContiguous or kMasked) and K (ktail: K % 128 != 0).
__attribute__((visibility("hidden"))) int ue8m0_occupancy(int tile, int layout, bool ktail);

// Launch on `grid` workgroups; p.tiles_m, tiles_n, num_tiles and group_m set
// (grouped layouts: p.kb_factor = ceil(Kb/4); masked: num_tiles covers all
// groups).  K % 128 != 0 takes the build that clips the last slice at K.
__attribute__((visibility("hidden"))) hipError_t ue8m0_launch(const GemmParams& p, int tile, int layout,
                                                              int64_t grid, hipStream_t stream);

}  // namespace fg
