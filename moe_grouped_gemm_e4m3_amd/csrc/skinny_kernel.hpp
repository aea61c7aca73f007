// skinny_kernel.hpp -- dense FP8 GEMM for few activation rows (decode, M <= 128).
//
// Same operation as gemm_kernel.hpp (per-128-K-slice fp32 partials promoted
// with sa[kb][m] * sb[n/128][kb]; DeepGEMM digest, GeekNews topic 19459,
// "GEMM arayuzu ve yerlesim kisitlari"), for the memory-bound case in which
// the weights are read once and every activation row is reused across all of
// them.  The work is the weight stream, so the kernel is built around it:
//
//  * No barriers in the main loop.  Every wave streams its own K slices
//    through a two-slot LDS ring of its own, one slice ahead of the slice it
//    multiplies; the waves of a CU run independently and keep the memory
//    pipe busy.
//  * Both operands reach the ring by direct-to-LDS loads of whole 128-byte
//    rows (8 rows per instruction), and the MFMA fragments are read from
//    there.  The fragment layout (16 rows per instruction, 32 bytes per lane)
//    would make a register load touch 16 rows at 64 bytes each, and such
//    half-row loads move 2-3x fewer bytes per unit of time than whole-row
//    loads when they hit in the cache (as the activations do: every column
//    tile reads them) and about 10 % fewer from HBM.
//  * Both operands' fragments take, in lane group q, the 16-byte chunks q
//    and 4 + q of their row (the MFMA expects chunks 2q and 2q + 1): one
//    permutation of K applied to both sides of every dot product leaves the
//    product unchanged.
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

// Workgroups per CU the registers allow: a wave holds one slice of
// fragments, the slice partials of one fragment row and the accumulators;
// two workgroups per CU (two waves per SIMD) leave it 256 registers.
constexpr __host__ __device__ int skinny_occupancy(int mf, int cf) {
  return 8 * mf + 8 * cf + 4 * cf + 4 * mf * cf <= 200 ? 2 : 1;
}

template <int MF_, int CF_>
struct SkinnyCfg {
  static constexpr int MF = MF_;  // 16-row activation fragments (rows = 16 MF)
  static constexpr int CF = CF_;  // 16-column weight fragments per wave
  static constexpr int WAVES = 4, THREADS = 256;
  static constexpr int ROWS = 16 * MF, COLS = 16 * CF;
  static constexpr int GROUPS = MF * CF;  // 16x16 output blocks of the tile
  static constexpr int GPW = GROUPS / WAVES;
  static constexpr int DEPTH = kSkinnyDepth;  // slices in flight per wave
  // a wave's LDS ring slot: the slice's activation rows and weight rows
  // (128 B each), then the activation scales (4 B each)
  static constexpr int SLOT = ROWS * 128 + COLS * 128 + ROWS * 4;
  static constexpr int B_OFF = ROWS * 128;
  static constexpr int SA_OFF = (ROWS + COLS) * 128;
  static constexpr int RING = DEPTH * SLOT;
  // direct-to-LDS loads per slice: 8 activation or weight rows each, 64 scales each
  static constexpr int A_LOADS = ROWS / 8, B_LOADS = COLS / 8, SA_LOADS = (ROWS + 63) / 64;
  static constexpr int NLOADS = A_LOADS + B_LOADS + SA_LOADS;
  static constexpr int LDS = WAVES * RING + 16;  // rings (then wave partials) + flag
  static constexpr int OCC = skinny_occupancy(MF, CF) == 2 && 2 * LDS <= 160 * 1024 ? 2 : 1;
  static_assert(GROUPS % WAVES == 0, "output blocks split over the waves");
  static_assert(128 % COLS == 0, "a column tile lies in one weight-scale block");
  static_assert(GROUPS * 64 * 16 <= RING, "a wave's partials fit in its ring");
  static_assert(DEPTH == 2, "the LDS waits count one slice of loads in flight");
};

// The weight scale of one K slice (its operands are in the wave's ring slot).
template <class C>
struct SkinnySlice {
  float sb;
};

// Per-lane load geometry of a wave (constant over the K loop).
struct SkinnyLanes {
  __amdgpu_buffer_rsrc_t ra, rb, rsa;
  // 8-row load j puts lane l's 16 bytes at LDS place l % 8 of row 8 j + l / 8;
  // the place holds logical chunk (l % 8) ^ swz16(row), and swz16(8 j + r) =
  // r ^ (j & 1), so even and odd loads differ by one chunk
  int a_voff[2];       // activation lane offsets of even / odd loads (the odd ones carry their extra 8 rows)
  int b_voff[2];       // the same for the weights
  int a_col[2];        // first column of the lane's chunk in even / odd loads
  int a_step8, b_step8;  // bytes between 8-row loads
  int sa_voff;         // this lane's activation scale (row `lane` of the part), bytes
  int sa_kstep;        // bytes between K slices of sa
  const float* sb;     // sb[nb][.] of the tile's weight-scale block
  int K;
};

// Wait until at most N vector memory operations of this wave are outstanding
// (they complete in issue order); direct-to-LDS loads count, and the
// compiler does not track their LDS writes.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Issue the loads of slice kb into ring slot `slot`: activation rows, weight
// rows and activation scales (NLOADS direct-to-LDS loads), then the weight
// scale (a scalar load) into f.
template <class C>
__device__ __forceinline__ void skinny_load(SkinnySlice<C>& f, uint8_t* slot, const SkinnyLanes& g, int kb,
                                            int lane) {
  const int k0 = kb * 128;
  // K tail: chunks at or past column K read as zeros (k_clip).  Always in
  // range for whole slices; the selects cost a few VALU ops in a kernel that
  // waits on memory.
  const bool a_in[2] = {k0 + g.a_col[0] < g.K, k0 + g.a_col[1] < g.K};
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int v = a_in[j & 1] ? g.a_voff[j & 1] + (j >> 1) * 2 * g.a_step8 : kOobOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(g.ra, (__attribute__((address_space(3))) void*)(slot + j * 1024), 16, v,
                                             k0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < C::SA_LOADS; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rsa, (__attribute__((address_space(3))) void*)(slot + C::SA_OFF + j * 256),
                                             4, g.sa_voff + j * 256, kb * g.sa_kstep, 0, 0);
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int v = a_in[j & 1] ? g.b_voff[j & 1] + (j >> 1) * 2 * g.b_step8 : kOobOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rb, (__attribute__((address_space(3))) void*)(slot + C::B_OFF + j * 1024),
                                             16, v, k0, 0, 0);
  }
  f.sb = *(const __attribute__((address_space(4))) float*)(g.sb + kb);
}

// acc += P_kb * (sa * sb) for every output block of the wave, with the
// slice's operands read from ring slot `slot`.  WAIT: the loads issued after
// this slice's that may stay outstanding (those of the next slice, or none).
template <class C, int WAIT>
__device__ __forceinline__ void skinny_compute(const SkinnySlice<C>& f, const uint8_t* slot, int lane,
                                               float (&acc)[C::GROUPS][4]) {
  wait_vm<WAIT>();  // this slice's loads have landed in the ring
  const int l16 = lane & 15, q = lane >> 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < C::MF; ++i) {
    // row 16 i + l16, logical chunks q and 4 + q,
    // at their swizzled places
    const int r = 16 * i + l16;
    const i32x8 a = lds_frag(slot, r * 128 + ((q ^ swz16(r)) << 4), r * 128 + (((4 + q) ^ swz16(r)) << 4));
    const float s = *(const float*)(slot + C::SA_OFF + r * 4) * f.sb;
    f32x4 P[C::CF];
#pragma unroll
    for (int j = 0; j < C::CF; ++j) {
      const int rb = 16 * j + l16;
      const i32x8 b = lds_frag(slot + C::B_OFF, rb * 128 + ((q ^ swz16(rb)) << 4), rb * 128 + (((4 + q) ^ swz16(rb)) << 4));
      P[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, zero, 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::CF; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) acc[i * C::CF + j][r4] = __builtin_fmaf(P[j][r4], s, acc[i * C::CF + j][r4]);
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
  g.ra = make_rsrc(p.A + (int64_t)r0 * p.lda, (int64_t)(p.rows - r0 - 1) * p.lda + p.K);
  {
    const int r8 = lane >> 3, c_even = (lane & 7) ^ r8, c_odd = c_even ^ 1;
    g.a_voff[0] = r8 * (int)p.lda + 16 * c_even;
    g.a_voff[1] = (8 + r8) * (int)p.lda + 16 * c_odd;
    g.a_col[0] = 16 * c_even;
    g.a_col[1] = 16 * c_odd;
    g.a_step8 = 8 * (int)p.lda;
    g.b_voff[0] = r8 * (int)p.ldb + 16 * c_even;
    g.b_voff[1] = (8 + r8) * (int)p.ldb + 16 * c_odd;
    g.b_step8 = 8 * (int)p.ldb;
  }
  g.rb = make_rsrc(p.B + (int64_t)n0 * p.ldb, (int64_t)(p.N - n0 - 1) * p.ldb + p.K);
  g.rsa = make_rsrc(p.sa + r0, ((int64_t)(p.Kb - 1) * p.ld_sa + p.rows - r0) * 4);
  g.sa_voff = lane * 4;
  g.sa_kstep = (int)p.ld_sa * 4;
  g.sb = p.sb + (int64_t)(n0 >> 7) * p.ld_sb;
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
    // A ring of DEPTH slices (weights in registers, activations in the
    // wave's LDS slots): the loads of the next slice are in flight while one
    // slice's MFMAs run.  The n % DEPTH leading slices go first on their
    // own, so the pipelined loop has no conditional work (the compiler would
    // otherwise sink a conditionally used load down to its use); its last
    // iterations fetch the final slice again, unused.  The scheduling
    // barriers keep each batch of loads ahead of the MFMAs that do not need
    // it.
    constexpr int DEPTH = C::DEPTH;
    constexpr int NA = C::NLOADS;
    uint8_t* ring = lds + wave * C::RING;
    SkinnySlice<C> f[DEPTH];
    int i = 0;
    for (const int lead = n % DEPTH; i < lead; ++i) {
      skinny_load<C>(f[0], ring, g, kat(i), lane);
      skinny_compute<C, 0>(f[0], ring, lane, acc);
    }
    if (i < n) {
#pragma unroll
      for (int d = 0; d + 1 < DEPTH; ++d) skinny_load<C>(f[d], ring + d * C::SLOT, g, kat(min(i + d, n - 1)), lane);
      for (; i < n; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          __builtin_amdgcn_sched_barrier(0);
          skinny_load<C>(f[(d + DEPTH - 1) % DEPTH], ring + ((d + DEPTH - 1) % DEPTH) * C::SLOT, g,
                         kat(min(i + d + DEPTH - 1, n - 1)), lane);
          __builtin_amdgcn_sched_barrier(0);
          skinny_compute<C, NA>(f[d], ring + d * C::SLOT, lane, acc);
        }
      }
    }
    // no direct-to-LDS load may still be writing the ring (the partials go there)
    wait_vm<0>();
  }

  // ---- add the four wave partials in wave order; wave w keeps blocks
  // [w GPW, (w+1) GPW) ----
  // (each wave's partials in its own ring, which no other wave uses)
  auto red = [&](int w) { return (float4*)(lds + w * C::RING); };
#pragma unroll
  for (int x = 0; x < C::GROUPS; ++x) red(wave)[x * 64 + lane] = make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
  __syncthreads();
  float sum[C::GPW][4];
#pragma unroll
  for (int y = 0; y < C::GPW; ++y) {
    const int x = wave * C::GPW + y;
    float4 t = red(0)[x * 64 + lane];
#pragma unroll
    for (int w = 1; w < C::WAVES; ++w) {
      const float4 u = red(w)[x * 64 + lane];
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
