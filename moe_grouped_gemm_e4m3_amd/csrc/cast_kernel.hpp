// cast_kernel.hpp -- fine-grained FP8 e4m3 casts (1x128 per token, 128x128 per block).
//
// The digest leaves FP8 casting to the user ("GEMM arayuzu ve yerlesim
// kisitlari", DeepGEMM digest, GeekNews topic 19459) and fixes the factors as
// fp32; the granularity (1x128 activations, 128x128 weights) is the
// DeepSeek-V3 fine-grained scheme the release summary names.  Per group:
//     amax = max |x|,  s = max(amax, 1e-4f) / 448,  q = e4m3_RNE(x / s)
// with an IEEE fp32 division (hipcc's default float division is correctly
// rounded) and a bit-exact round-to-nearest-even encoder.  Both kernels are
// HBM-bound streams: 16-byte loads, one pass over the input.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

// fp32 -> e4m3fn code, round to nearest even, for |v| < 464 (the caller's
// division by s = amax/448 guarantees |v| <= 448 * (1 + 2^-23)).
//  * |v| >= 2^-6 (normal e4m3): round the fp32 significand to 3 bits with a
//    nearest-even bias (carries move into the exponent), then re-bias the
//    exponent from 127 to 7.
//  * |v| <  2^-6 (subnormal e4m3, step 2^-9): code = rint(|v| * 512), where
//    rint rounds half to even; 8 lands exactly on the smallest normal code.
// The sign bit is copied, so -0 and tiny negatives give 0x80.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3c800000u) {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return code | sign;
}

__device__ __forceinline__ float scale_of(float amax) { return fmaxf(amax, 1e-4f) / 448.0f; }

// Power-of-two (UE8M0) factors, the digest's packed format for the newer
// architecture (same section): the fp32 factor rounded up to a power of two
// so that no code saturates, stored as its biased exponent (value
// 2^(e - 127)).  s is a positive normal fp32 here, so the exponent field is
// the floor of log2(s) and any set significand bit rounds it up.
__device__ __forceinline__ uint32_t ue8m0_of(float s) {
  const uint32_t u = __float_as_uint(s);
  return ((u >> 23) & 0xffu) + ((u & 0x7fffffu) != 0u ? 1u : 0u);
}
__device__ __forceinline__ float ue8m0_value(uint32_t e) { return __uint_as_float(e << 23); }

__device__ __forceinline__ float absmax4(float4 v, float m) {
  return fmaxf(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))), m);
}

__device__ __forceinline__ uint32_t encode4(float4 v, float s) {
  return e4m3_rne(v.x / s) | (e4m3_rne(v.y / s) << 8) | (e4m3_rne(v.z / s) << 16) | (e4m3_rne(v.w / s) << 24);
}

// Inputs: fp32, or bf16 (raw bits, uint16_t) widened exactly to fp32 first
// (the digest names BF16-input helpers beside the fp32 ones, "GEMM arayuzu
// ve yerlesim kisitlari"), so a bf16 input quantises as its fp32 value does.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// 8 consecutive inputs (16-byte aligned) as two float4.
__device__ __forceinline__ void load8(const float* src, float4& v0, float4& v1) {
  v0 = *(const float4*)src;
  v1 = *(const float4*)(src + 4);
}
__device__ __forceinline__ void load8(const uint16_t* src, float4& v0, float4& v1) {
  const uint4 u = *(const uint4*)src;
  v0 = make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffffu),
                   bf16_to_f32(u.y >> 16));
  v1 = make_float4(bf16_to_f32(u.z & 0xffffu), bf16_to_f32(u.z >> 16), bf16_to_f32(u.w & 0xffffu),
                   bf16_to_f32(u.w >> 16));
}
// 4 consecutive inputs (16-byte aligned for fp32, 8-byte for bf16).
__device__ __forceinline__ float4 load4(const float* src) { return *(const float4*)src; }
__device__ __forceinline__ float4 load4(const uint16_t* src) {
  const uint2 u = *(const uint2*)src;
  return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffffu),
                     bf16_to_f32(u.y >> 16));
}

// LPG lanes per (row, 128-column group); each lane makes CH loads of 16 bytes
// (4 fp32 or 8 bf16 inputs), strided by LPG * 16 bytes, so every load
// instruction reads whole groups' 16*LPG-byte runs back to back and a lane
// keeps CH loads in flight.  The factor is the max over the LPG lanes.
// UE8M0: sa is int32 [ceil(Kb/4)][ld_sa], the factor of K group kb of row m in
// byte kb % 4 of element [kb / 4][m] (one byte store per group).
// K tails (K % 128 != 0, K % 16 == 0): the last group holds K % 128 columns;
// loads past K are skipped (a load's 4 or 8 columns are all in or all out),
// add nothing to the amax and store nothing.
template <bool UE8M0, typename T, int LPG>
__global__ __launch_bounds__(256) void cast_per_token_kernel(const T* __restrict__ x, int64_t ldx,
                                                             uint8_t* __restrict__ q, void* __restrict__ sa,
                                                             int64_t ld_sa, int M, int K, int64_t total_lanes) {
  constexpr int VE = 16 / sizeof(T);    // inputs per 16-byte load
  constexpr int CH = 128 / (LPG * VE);  // loads per lane
  static_assert(CH >= 1 && CH * LPG * VE == 128, "LPG must split a group into whole 16-byte loads");
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total_lanes) return;  // total_lanes % LPG == 0: a group is all in or all out
  const int Kb = (K + 127) >> 7;
  const int64_t grp = gid / LPG;
  const int sub = (int)(gid & (LPG - 1));
  const int m = (int)(grp / Kb);
  const int kb = (int)(grp - (int64_t)m * Kb);
  const T* src = x + (int64_t)m * ldx;
  float4 v[CH][VE / 4];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int col = kb * 128 + j * LPG * VE + sub * VE;
#pragma unroll
    for (int t = 0; t < VE / 4; ++t) v[j][t] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < K) {
      if constexpr (VE == 8)
        load8(src + col, v[j][0], v[j][VE / 4 - 1]);
      else
        v[j][0] = load4(src + col);
    }
#pragma unroll
    for (int t = 0; t < VE / 4; ++t) amax = absmax4(v[j][t], amax);
  }
#pragma unroll
  for (int o = LPG / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, LPG));
  const float s32 = scale_of(amax);
  const uint32_t e = UE8M0 ? ue8m0_of(s32) : 0u;
  const float s = UE8M0 ? ue8m0_value(e) : s32;
  uint8_t* dst = q + (int64_t)m * K;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int col = kb * 128 + j * LPG * VE + sub * VE;
    if (col < K) {
      if constexpr (VE == 8) {
        uint2 out;
        out.x = encode4(v[j][0], s);
        out.y = encode4(v[j][VE / 4 - 1], s);
        *(uint2*)(dst + col) = out;
      } else {
        *(uint32_t*)(dst + col) = encode4(v[j][0], s);
      }
    }
  }
  if (sub == 0) {
    if (UE8M0)
      ((uint8_t*)sa)[((int64_t)(kb >> 2) * ld_sa + m) * 4 + (kb & 3)] = (uint8_t)e;
    else
      ((float*)sa)[(int64_t)kb * ld_sa + m] = s;
  }
}

// One workgroup per 128x128 block: 32 lanes cover a 128-float row, 8 rows per
// pass, 16 passes; the block is kept in registers between the amax reduction
// and the encode.  UE8M0: sb is int32 [Nb][ceil(Kb/4)], the factor of block
// (nb, kb) in byte kb % 4 of element [nb][kb / 4].  The last row block may
// hold fewer than 128 rows (N % 128) and the last column block fewer than
// 128 columns (K % 128, a multiple of 16); lanes outside take no part.
template <bool UE8M0, typename T>
__global__ __launch_bounds__(256) void cast_per_block_kernel(const T* __restrict__ w, int64_t ldw,
                                                             uint8_t* __restrict__ q, void* __restrict__ sb,
                                                             int N, int K) {
  __shared__ float red[4];
  const int Kb = (K + 127) >> 7;
  const int nb = blockIdx.x / Kb;
  const int kb = blockIdx.x - nb * Kb;
  const int tid = threadIdx.x;
  const int c = tid & 31;
  const int r0 = tid >> 5;
  // rows of the block this lane reads: none when its 4 columns lie past K
  const int rows = kb * 128 + c * 4 < K ? min(128, N - nb * 128) : 0;
  const T* base = w + (int64_t)nb * 128 * ldw + kb * 128 + c * 4;
  float4 v[16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + 8 * i;
    if (r < rows) {
      v[i] = load4(base + (int64_t)r * ldw);
      amax = absmax4(v[i], amax);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s32 = scale_of(amax);
  const uint32_t e = UE8M0 ? ue8m0_of(s32) : 0u;
  const float s = UE8M0 ? ue8m0_value(e) : s32;
  uint8_t* qb = q + (int64_t)nb * 128 * K + kb * 128 + c * 4;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + 8 * i;
    if (r < rows) *(uint32_t*)(qb + (int64_t)r * K) = encode4(v[i], s);
  }
  if (tid == 0) {
    if (UE8M0)
      ((uint8_t*)sb)[((int64_t)nb * ((Kb + 3) >> 2) + (kb >> 2)) * 4 + (kb & 3)] = (uint8_t)e;
    else
      ((float*)sb)[(int64_t)nb * Kb + kb] = s;
  }
}

}  // namespace fg
