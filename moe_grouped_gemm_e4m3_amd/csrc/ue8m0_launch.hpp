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

// Workgroups per CU of the kernel for tile width bn (224 or 160).
__attribute__((visibility("hidden"))) int ue8m0_occupancy(int bn);

// Launch on `grid` workgroups; p.tiles_m, tiles_n, num_tiles and group_m set.
__attribute__((visibility("hidden"))) hipError_t ue8m0_launch(const GemmParams& p, int bn, int64_t grid,
                                                              hipStream_t stream);

}  // namespace fg
