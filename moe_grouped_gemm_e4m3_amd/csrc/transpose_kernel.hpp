// transpose_kernel.hpp -- byte transpose of an e4m3 operand stored MN-major.
//
// The NN, TN and TT storage layouts of the digest's fp8_gemm_{nn,tn,tt}
// (GeekNews topic 19459, "Dense ve Grouped GEMM") hold A as [K, M] and/or B
// as [K, N].  The matrix-core operands of the NT kernels are K-contiguous per
// lane, so such an operand is first rewritten K-major: out[c][r] = in[r][c].
// This is pure data movement, bound by HBM: 128 x 128-byte tiles go through
// LDS so that both the global reads and the global writes are whole 128-byte
// row segments.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

constexpr int kTrTile = 128;

// One 128 x 128 tile per workgroup of 256 threads; grid (ceil(C/128),
// ceil(R/128)).  in: [R, C] bytes, row stride ld_in; out: [C, R] bytes, row
// stride ld_out.  Elements outside [R, C] are neither read nor written.
__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ in, int64_t ld_in,
                                                           uint8_t* __restrict__ out, int64_t ld_out, int R,
                                                           int C) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  // Row r of the tile keeps its 16-byte chunk q at chunk position q ^ (r/16 % 8):
  // the gather below reads one column from rows 16 apart in eight lanes at
  // once, and the swizzle puts those reads in different banks.
  __shared__ __attribute__((aligned(16))) uint8_t t[kTrTile * kTrTile];
  const int r0 = blockIdx.y * kTrTile, c0 = blockIdx.x * kTrTile;
  const int tid = threadIdx.x;
  const bool in_vec = ((ld_in & 15) == 0) && (((uintptr_t)in & 15) == 0);
  const bool out_vec = ((ld_out & 15) == 0) && (((uintptr_t)out & 15) == 0);

  // tile rows: 128 rows x 8 chunks, 4 chunks per thread, 8 lanes per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int r = q >> 3, ch = q & 7;
    const int gr = r0 + r, gc = c0 + 16 * ch;
    v4i v = {0, 0, 0, 0};
    if (gr < R && gc < C) {
      const uint8_t* src = in + (int64_t)gr * ld_in + gc;
      if (in_vec && gc + 16 <= C) {
        v = *(const v4i*)src;
      } else {
        uint8_t b[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) b[j] = gc + j < C ? src[j] : 0;
        __builtin_memcpy(&v, b, 16);
      }
    }
    *(v4i*)(t + r * kTrTile + ((ch ^ ((r >> 4) & 7)) << 4)) = v;
  }
  __syncthreads();

  // output rows (tile columns): 128 x 8 chunks of 16 input rows, 8 lanes per
  // output row so that each row segment is written whole
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int ch = q & 7, c = q >> 3;
    const int gc = c0 + c, gr = r0 + 16 * ch;
    // rows 16ch .. 16ch+15 share the swizzle ch, so one base address serves all 16
    const uint8_t* col = t + (16 * ch) * kTrTile + ((((c >> 4) ^ ch)) << 4) + (c & 15);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      w[d] = (uint32_t)col[(4 * d) * kTrTile] | ((uint32_t)col[(4 * d + 1) * kTrTile] << 8) |
             ((uint32_t)col[(4 * d + 2) * kTrTile] << 16) | ((uint32_t)col[(4 * d + 3) * kTrTile] << 24);
    }
    if (gc < C && gr < R) {
      uint8_t* dst = out + (int64_t)gc * ld_out + gr;
      if (out_vec && gr + 16 <= R) {
        const v4i v = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        *(v4i*)dst = v;
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (gr + j < R) dst[j] = (uint8_t)(w[j >> 2] >> ((j & 3) * 8));
      }
    }
  }
}

}  // namespace fg
