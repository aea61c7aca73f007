// skinny_kernel.hpp -- dense FP8 GEMM for few activation rows (decode, M <= 128).
//
// Same operation as gemm_kernel.hpp (per-128-K-slice fp32 partials promoted
// with sa[kb][m] * sb[n/128][kb]; DeepGEMM digest, GeekNews topic 19459,
// "GEMM arayuzu ve yerlesim kisitlari"), for the memory-bound case in which
// the weights are read once and every activation row is reused across all of
// them.  The work is the weight stream, so the kernel is built around it:
//
//  * No LDS staging and no barriers in the main loop.  Every wave loads its
//    own operand fragments straight from memory into registers, already in
//    MFMA operand layout, one K slice ahead of the slice it multiplies; the
//    waves of a CU run independently and keep the memory pipe busy.
//  * Inside a K slice both operands are read with the same byte permutation
//    (lane group q holds bytes [16q, 16q+16) and [64+16q, 64+16q+16) of its
//    row, where the MFMA expects [32q, 32q+32)); a dot product over the slice
//    does not depend on the order of its terms' pairing, and each load
//    instruction then covers 64 contiguous bytes of 16 rows.
//  * A workgroup is four waves on one column tile (16 * CF weight rows) and
//    one row part (16 * MF activation rows; more rows go to further parts),
//    each wave on a quarter of the workgroup's K range.  The four fp32
//    partials are added in LDS in wave order.
//  * When the tiles alone cannot occupy the device, the K range is also
//    split over `splits` workgroups.  Their partials go to a workspace with
//    system-coherent stores; the last workgroup to arrive at a (tile, part)
//    unit (an arrival counter) adds them in split order and stores bf16.
//    Both additions have a fixed order, so results are reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace fg {

#ifndef FG_SKINNY_DEPTH
#define FG_SKINNY_DEPTH 2
#endif
constexpr int kSkinnyDepth = FG_SKINNY_DEPTH;

// Workgroups per CU the registers allow: a wave holds DEPTH slices of
// fragments and scales, the slice partials and the accumulators; two
// workgroups per CU (two waves per SIMD) leave it 256 registers.
constexpr __host__ __device__ int skinny_occupancy(int mf, int cf) {
  return kSkinnyDepth * (8 * mf + 8 * cf + mf) + 8 * mf * cf <= 240 ? 2 : 1;
}

template <int MF_, int CF_>
struct SkinnyCfg {
  static constexpr int MF = MF_;  // 16-row activation fragments (rows = 16 MF)
  static constexpr int CF = CF_;  // 16-column weight fragments per wave
  static constexpr int WAVES = 4, THREADS = 256;
  static constexpr int ROWS = 16 * MF, COLS = 16 * CF;
  static constexpr int GROUPS = MF * CF;  // 16x16 output blocks of the tile
  static constexpr int GPW = GROUPS / WAVES;
  static constexpr int DEPTH = kSkinnyDepth;  // slices of fragments per wave in the ring
  static constexpr int OCC = skinny_occupancy(MF, CF);
  static constexpr int LDS = WAVES * GROUPS * 64 * 16 + 16;  // wave partials + flag
  static_assert(GROUPS % WAVES == 0, "output blocks split over the waves");
  static_assert(128 % COLS == 0, "a column tile lies in one weight-scale block");
};

// Fragments and scales of one K slice, as this wave needs them.
template <class C>
struct SkinnySlice {
  i32x8 a[C::MF];
  i32x8 b[C::CF];
  float sa[C::MF];
  float sb;
};

// Per-lane load geometry of a wave (constant over the K loop).
struct SkinnyLanes {
  __amdgpu_buffer_rsrc_t ra, rb, rsa;
  int a_voff, b_voff;  // this lane's row (16 apart per fragment) and 16-byte column
  int a_step, b_step;  // bytes between fragments (16 rows)
  int sa_voff;         // this lane's activation row, bytes
  int sa_kstep;        // bytes between K slices of sa
  const float* sb;     // sb[nb][.] of the tile's weight-scale block
  int kq16;            // first column of this lane's 16-byte chunk inside a slice (16 * lane group)
  int K;
};

template <class C>
__device__ __forceinline__ void skinny_load(SkinnySlice<C>& f, const SkinnyLanes& g, int kb) {
  const int k0 = kb * 128;
  // K tail: chunks at or past column K read as zeros (k_clip).  Always true
  // for whole slices; the selects cost a few VALU ops in a kernel that waits
  // on memory.
  const bool lo_in = k0 + g.kq16 < g.K, hi_in = k0 + 64 + g.kq16 < g.K;
#pragma unroll
  for (int i = 0; i < C::MF; ++i) {
    const int v = g.a_voff + i * g.a_step;
    const i32x4 lo =
        __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(g.ra, lo_in ? v : kOobOffset, k0, 0));
    const i32x4 hi =
        __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(g.ra, hi_in ? v : kOobOffset, k0 + 64, 0));
    f.a[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
#pragma unroll
  for (int j = 0; j < C::CF; ++j) {
    const int v = g.b_voff + j * g.b_step;
    const i32x4 lo =
        __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(g.rb, lo_in ? v : kOobOffset, k0, 0));
    const i32x4 hi =
        __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(g.rb, hi_in ? v : kOobOffset, k0 + 64, 0));
    f.b[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
#pragma unroll
  for (int i = 0; i < C::MF; ++i)
    f.sa[i] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(g.rsa, g.sa_voff + kb * g.sa_kstep + i * 64, 0, 0));
  f.sb = *(const __attribute__((address_space(4))) float*)(g.sb + kb);
}

// acc += P_kb * (sa * sb) for every output block of the wave.
template <class C>
__device__ __forceinline__ void skinny_compute(const SkinnySlice<C>& f, float (&acc)[C::GROUPS][4]) {
  f32x4 P[C::MF][C::CF];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < C::MF; ++i)
#pragma unroll
    for (int j = 0; j < C::CF; ++j)
      P[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[j], f.a[i], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < C::MF; ++i) {
    const float s = f.sa[i] * f.sb;
#pragma unroll
    for (int j = 0; j < C::CF; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i * C::CF + j][r] = __builtin_fmaf(P[i][j][r], s, acc[i * C::CF + j][r]);
  }
}

// Store 16x16 block g (lane: row 16i + l%16, columns 16j + 4(l/16) .. +3) as bf16.
// With ADD_C the fp32 addend C is added first (D = C + A B^T).
template <class C, bool ADD_C>
__device__ __forceinline__ void skinny_store(const GemmParams& p, int r0, int n_tile0, int g, const float (&acc)[4],
                                             int lane) {
  const int i = g / C::CF, j = g % C::CF;
  const int m = r0 + 16 * i + (lane & 15);
  const int n = n_tile0 + 16 * j + 4 * (lane >> 4);
  if (m >= p.rows || n >= p.N) return;
  float v[4] = {acc[0], acc[1], acc[2], acc[3]};
  if (ADD_C) add_addend4(p, m, n, v);
  uint16_t* dst = p.D + (int64_t)m * p.ldd + n;
  if (n + 4 <= p.N && (p.ldd & 3) == 0 && ((uintptr_t)p.D & 7) == 0) {
    *(uint2*)dst = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < p.N) dst[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xffff);
  }
}

// Grid: (column tiles) x parts x splits workgroups.  Workgroup b works on K
// split b % splits of unit u = b / splits: column tile u / parts and rows
// [16 MF (u % parts), 16 MF (u % parts + 1)) -- activation rows beyond one
// tile's 16 MF are spread over `parts` workgroups (the two row halves of a
// column tile run side by side and share its weights in L2).
template <class C, bool ADD_C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void gemm_fp8_skinny_kernel(GemmParams p, int splits, int parts) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x / splits;
  const int split = blockIdx.x - unit * splits;
  const int tile = unit / parts;
  const int r0 = (unit - tile * parts) * C::ROWS;  // first activation row of this workgroup
  const int n0 = tile * C::COLS;

  // this workgroup's K slices, and this wave's quarter of them
  const int kb0 = p.Kb * split / splits, kb1 = p.Kb * (split + 1) / splits;
  const int kw0 = kb0 + (kb1 - kb0) * wave / C::WAVES, kw1 = kb0 + (kb1 - kb0) * (wave + 1) / C::WAVES;

  SkinnyLanes g;
  const int l16 = lane & 15, q = lane >> 4;
  g.ra = make_rsrc(p.A + (int64_t)r0 * p.lda, (int64_t)(p.rows - r0 - 1) * p.lda + p.K);
  g.a_voff = l16 * (int)p.lda + 16 * q;
  g.a_step = 16 * (int)p.lda;
  g.rb = make_rsrc(p.B + (int64_t)n0 * p.ldb, (int64_t)(p.N - n0 - 1) * p.ldb + p.K);
  g.b_voff = l16 * (int)p.ldb + 16 * q;
  g.b_step = 16 * (int)p.ldb;
  g.rsa = make_rsrc(p.sa + r0, ((int64_t)(p.Kb - 1) * p.ld_sa + p.rows - r0) * 4);
  g.sa_voff = l16 * 4;
  g.sa_kstep = (int)p.ld_sa * 4;
  g.sb = p.sb + (int64_t)(n0 >> 7) * p.ld_sb;
  g.kq16 = 16 * q;
  g.K = p.K;

  float acc[C::GROUPS][4];
#pragma unroll
  for (int x = 0; x < C::GROUPS; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[x][r] = 0.f;

  {
    // The wave visits its slices in a rotated order that depends on the
    // workgroup: workgroups running side by side then read different K slices
    // of the (shared, few-row) activations instead of all requesting the
    // same L2 lines at once.  The order is a fixed function of the workgroup
    // and wave, so the fp32 sum is reproducible.
    const int n = kw1 - kw0;
    const int rot = n > 0 ? (int)((blockIdx.x * 5u + (unsigned)wave * 3u) % (unsigned)n) : 0;
    auto kat = [&](int i) {
      const int j = i + rot;
      return kw0 + (j >= n ? j - n : j);
    };
    // A ring of DEPTH register slices: the loads of the next DEPTH - 1
    // slices are in flight while one slice's MFMAs run.  The n % DEPTH
    // leading slices go first on their own, so the pipelined loop has no
    // conditional work (the compiler would otherwise sink a conditionally
    // used load down to its use); its last iterations fetch the final slice
    // again, unused.  The scheduling barriers keep each batch of loads ahead
    // of the MFMAs that do not need it.
    constexpr int DEPTH = C::DEPTH;
    SkinnySlice<C> f[DEPTH];
    int i = 0;
    for (const int lead = n % DEPTH; i < lead; ++i) {
      skinny_load<C>(f[0], g, kat(i));
      skinny_compute<C>(f[0], acc);
    }
    if (i < n) {
#pragma unroll
      for (int d = 0; d + 1 < DEPTH; ++d) skinny_load<C>(f[d], g, kat(min(i + d, n - 1)));
      for (; i < n; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          __builtin_amdgcn_sched_barrier(0);
          skinny_load<C>(f[(d + DEPTH - 1) % DEPTH], g, kat(min(i + d + DEPTH - 1, n - 1)));
          __builtin_amdgcn_sched_barrier(0);
          skinny_compute<C>(f[d], acc);
        }
      }
    }
  }

  // ---- add the four wave partials in wave order; wave w keeps blocks
  // [w GPW, (w+1) GPW) ----
  float4* red = (float4*)lds;
#pragma unroll
  for (int x = 0; x < C::GROUPS; ++x) red[(wave * C::GROUPS + x) * 64 + lane] = make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
  __syncthreads();
  float sum[C::GPW][4];
#pragma unroll
  for (int y = 0; y < C::GPW; ++y) {
    const int x = wave * C::GPW + y;
    float4 t = red[x * 64 + lane];
#pragma unroll
    for (int w = 1; w < C::WAVES; ++w) {
      const float4 u = red[(w * C::GROUPS + x) * 64 + lane];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    sum[y][0] = t.x;
    sum[y][1] = t.y;
    sum[y][2] = t.z;
    sum[y][3] = t.w;
  }

  if (splits == 1) {
#pragma unroll
    for (int y = 0; y < C::GPW; ++y) skinny_store<C, ADD_C>(p, r0, n0, wave * C::GPW + y, sum[y], lane);
    return;
  }

  // ---- split K: publish this split's partial, the last arrival adds them ----
  // partial of (unit, split): [GROUPS][64 lanes] float4, 1 KiB per block
  const int64_t slot_floats = (int64_t)C::GROUPS * 64 * 4;
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(p.ws_partials + (int64_t)unit * splits * slot_floats,
                (int64_t)splits * slot_floats * (int64_t)sizeof(float));
#pragma unroll
  for (int y = 0; y < C::GPW; ++y) {
    const int x = wave * C::GPW + y;
    const int off = ((split * C::GROUPS + x) * 64 + lane) * 16;
    const f32x4 v = {sum[y][0], sum[y][1], sum[y][2], sum[y][3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), prs, off, 0, kSysCoherent);
  }
  // the stores are acknowledged at the point of coherence before counting in
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* last_flag = (int*)(lds + C::LDS - 16);
  if (tid == 0) {
    const int before = __hip_atomic_fetch_add(p.ws_counters + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *last_flag = before == splits - 1;
  }
  __syncthreads();
  if (!*last_flag) return;

  // The partials are added in split order.  Their loads are issued in
  // batches of up to kBatch splits for all of the wave's blocks before any
  // is used, so a batch costs one memory round trip instead of one per
  // split and block.
  constexpr int kBatch = 4;
  float t[C::GPW][4];
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    i32x4 u[kBatch][C::GPW];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j;
#pragma unroll
      for (int y = 0; y < C::GPW; ++y) {
        const int x = wave * C::GPW + y;
        if (s < splits && s != split)
          u[j][y] = __builtin_amdgcn_raw_buffer_load_b128(prs, ((s * C::GROUPS + x) * 64 + lane) * 16, 0,
                                                          kSysCoherent);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j;
      if (s >= splits) break;
#pragma unroll
      for (int y = 0; y < C::GPW; ++y) {
        const f32x4 v = s == split ? f32x4{sum[y][0], sum[y][1], sum[y][2], sum[y][3]}
                                   : __builtin_bit_cast(f32x4, u[j][y]);
#pragma unroll
        for (int r = 0; r < 4; ++r) t[y][r] = s == 0 ? v[r] : t[y][r] + v[r];
      }
    }
  }
#pragma unroll
  for (int y = 0; y < C::GPW; ++y) skinny_store<C, ADD_C>(p, r0, n0, wave * C::GPW + y, t[y], lane);
  // every workgroup of the unit has counted in: reset for the next launch
  if (tid == 0) __hip_atomic_store(p.ws_counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Zero n ints (the split-K arrival counters of a shared scratch), without a
// memset node, so that the launch can be captured into a graph.
__global__ __launch_bounds__(256) void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace fg
