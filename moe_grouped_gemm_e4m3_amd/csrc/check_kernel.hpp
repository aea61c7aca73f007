// check_kernel.hpp -- opt-in validation of the grouped GEMMs' device metadata.
//
// The grouped forms read their row mapping from device memory that the host
// never sees (DeepGEMM digest, GeekNews topic 19459, "Dense ve Grouped GEMM":
// the contiguous layout's per-row expert index and the masked layout's
// per-group counts live on the GPU).  The GEMM kernels trust them.  These
// kernels check them before a GEMM when the library runs in its debug mode,
// and record the first offending position in a two-int result word:
//   word[0]  lowest offending row (contiguous) or group (masked), INT_MAX if none
//   word[1]  unused by the kernels (the host reads the offending value itself)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

constexpr int kCheckNone = 0x7fffffff;

__global__ void check_reset_kernel(int* word) {
  if (threadIdx.x == 0) {
    word[0] = kCheckNone;
    word[1] = 0;
  }
}

// One workgroup of 128 threads per aligned 128-row block.  A row is bad when
// its index is outside [-1, G) or when it is an index in [0, G) that differs
// from the block's largest such index (a block holds one expert; the GEMM
// computes the block against its largest index).
__global__ __launch_bounds__(128) void check_m_indices_kernel(const int32_t* idx, int M_total, int G, int* word) {
  __shared__ int smax[2];
  const int m = blockIdx.x * 128 + threadIdx.x;
  const int e = m < M_total ? idx[m] : -1;
  int v = (e >= 0 && e < G) ? e : -1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = v;
  __syncthreads();
  const int block_max = max(smax[0], smax[1]);
  const bool bad = m < M_total && (e < -1 || e >= G || (e >= 0 && e != block_max));
  if (bad) atomicMin(word, m);
}

// Counts outside [0, M_cap] (which the GEMM would clamp) are reported.
__global__ __launch_bounds__(256) void check_masked_m_kernel(const int32_t* mask, int G, int M_cap, int* word) {
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int c = mask[g];
    if (c < 0 || c > M_cap) atomicMin(word, g);
  }
}

}  // namespace fg
