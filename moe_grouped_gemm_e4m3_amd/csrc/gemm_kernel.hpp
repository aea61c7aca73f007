// gemm_kernel.hpp -- gfx950 FP8 e4m3 GEMM with per-128-K-slice fp32 promotion.
//
// Computes D = bf16( sum_kb P_kb * sa[kb][m] * sb[n/128][kb] ) where P_kb is the
// fp32 matrix-core partial of one 128-wide K slice (DeepGEMM digest, GeekNews
// topic 19459, "GEMM arayuzu ve yerlesim kisitlari" for the NT operation;
// GeekNews topic 19444 opening bullets and 7minutos.es "Detalles y beneficios
// tecnicos" for the two-level accumulation).  One kernel body serves the
// dense, contiguous-grouped and masked-grouped forms ("Dense ve Grouped GEMM"
// of the same digest); they differ only in how a tile id becomes a problem
// tile and which output rows may be stored.
//
// Mapping to CDNA4:
//  * v_mfma_f32_16x16x128_f8f6f4 computes one 16x16 output block over a whole
//    128-deep K slice, so each MFMA result *is* a slice partial P (C input 0),
//    and the promotion is one v_fma_f32 per element per slice.
//  * The MFMA's first operand is the B (weight) fragment and its second the A
//    fragment, so the result block is transposed: lane l holds activation row
//    m = l%16 and 4 weight rows.  The activation scale is then a per-lane
//    register and the weight scale a per-wave scalar: s = sa[m] * sb.
//  * Weight rows are permuted inside each wave's N range so that after the
//    slices each lane owns WN/4 consecutive output columns (vector stores).
//  * Operands are staged through double-buffered LDS with 16-byte chunks
//    XOR-swizzled per row (conflict-free 128-bit fragment reads); the next
//    slice's global loads are in flight during the current slice's MFMAs.
//  * A persistent grid walks tiles in a grouped-M raster; consecutive tiles of
//    one raster window land on one XCD (workgroups are dealt to the 8 XCDs
//    round-robin) so they share that XCD's L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// kDenseC is the dense GEMM with an fp32 addend, D = C + A B^T: it runs
// exactly as kDense except that the epilogue adds C before the BF16 rounding.
// kKGrouped is the K-grouped GEMM of weight gradients, D[g] = C[g] + A_g^T B_g,
// on its operands as stored ([K, M] / [K, N]) or on K-major copies (see KGroups).
enum LayoutKind { kDense = 0, kContiguous = 1, kMasked = 2, kDenseC = 3, kKGrouped = 4 };

// The K-grouped GEMM's groups with work, in order: the output index of each
// and its first 128-deep K slice (kb0[n] is the end), and how far one slice
// moves each operand (128 rows of an MN-major operand, 128 bytes of a
// K-major one).  A kernel argument.
constexpr int kMaxKGroups = 256;
struct KGroups {
  int n;
  int g[kMaxKGroups];
  int kb0[kMaxKGroups + 1];
  int64_t a_step, b_step;
};

struct GemmParams {
  const uint8_t* A;  // dense/contiguous: [rows, K] (lda); masked: [G, M_cap, K] packed
  int64_t lda;       // bytes
  const float* sa;   // [Kb][ld_sa] (masked: per group)
  int64_t ld_sa;     // floats
  const uint8_t* B;  // [N, K] (ldb) or [G, N, K] packed
  int64_t ldb;       // bytes
  const float* sb;   // [Nb][Kb] or [G][Nb][Kb]
  uint16_t* D;       // [rows, N] (ldd) or [G, M_cap, N]
  int64_t ldd;       // elements
  const float* Cin;  // kDenseC: fp32 addend [rows, N] (ldc floats)
  int64_t ldc;
  const int32_t* m_indices;  // contiguous
  const int32_t* masked_m;   // masked
  int rows;     // dense: M; contiguous: M_total; masked: M_cap
  int N, K, G;
  int Kb, Nb;
  int ld_sb;             // row stride of sb in floats: Kb, or more when the K range is part of a wider sb
  int tiles_m, tiles_n;  // per group
  int num_tiles;         // tile slots walked by the persistent grid
  int group_m;           // raster band height in tiles
  int kb_factor;         // K extent of one group's factor arrays: 0 = Kb (fp32 factors), ceil(Kb/4) (packed UE8M0)
  // few-row split-K: fp32 partial slots and one arrival counter per output
  // unit, in the caller's workspace (counters zero between launches)
  float* ws_partials;
  int* ws_counters;
};

// Group stride, in K groups (fp32 factors) or packed words (UE8M0), of the
// masked layout's sa and of the grouped layouts' sb.
__device__ __forceinline__ int64_t factor_kb(const GemmParams& p) { return p.kb_factor > 0 ? p.kb_factor : p.Kb; }

// A value that no kernel writes while this one runs (the masked counts),
// read through the scalar cache: a vector load would make the wave wait for
// its whole queue of outstanding operand loads before using it.
__device__ __forceinline__ int load_invariant(const int* p) {
  return *(const __attribute__((address_space(4))) int*)p;
}

// Position of a workgroup in the persistent walk such that the workgroups of
// one XCD take consecutive work ids.
__device__ __forceinline__ int xcd_local_id(int b, int grid) {
  if (grid & 7) return b;
  return (b & 7) * (grid >> 3) + (b >> 3);
}

// Grouped-M raster: bands of group_m tile rows, walked column by column.
__device__ __forceinline__ void raster(int w, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int band_size = group_m * tiles_n;
  const int band = w / band_size;
  const int first = band * group_m;
  const int rows = min(group_m, tiles_m - first);
  const int idx = w - band * band_size;
  tm = first + idx % rows;
  tn = idx / rows;
}

// D = C + A B^T: the fp32 addend at row m, columns n .. n+3 (zeros where
// !valid and at columns >= N), added to the accumulator before the single BF16
// rounding.  Callers issue every load of an epilogue pass before the first
// use, so the pass waits for memory once.
__device__ __forceinline__ f32x4 load_addend4(const float* cbase, int64_t ldc, int N, int m, int n, bool valid) {
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float* c = cbase + (int64_t)m * ldc + n;
    if (n + 4 <= N && (ldc & 3) == 0 && ((uintptr_t)cbase & 15) == 0) {
      x = *(const f32x4*)c;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) x[r] = c[r];
    }
  }
  return x;
}

__device__ __forceinline__ f32x4 load_addend4(const GemmParams& p, int m, int n, bool valid) {
  return load_addend4(p.Cin, p.ldc, p.N, m, n, valid);
}

__device__ __forceinline__ void add_addend4(const GemmParams& p, int m, int n, float (&v)[4]) {
  const f32x4 x = load_addend4(p, m, n, true);
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] += x[r];
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// XOR swizzles of the 16-byte chunk index inside a 128-byte LDS row.
// A rows are read 16 consecutive rows at a time.
__device__ __forceinline__ int swz_a(int row) { return row & 7; }
// B rows are read in the permuted order n = Q*(i/4) + 4t + i%4 (Q = WN/4), so
// the 8 rows of one lane octet are {4t+j, Q+4t+j}: mix bit log2(Q) in.
template <int Q>
__device__ __forceinline__ int swz_b(int row) {
  return (row & 3) | (((row / Q) & 1) << 2);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int THREADS = WAVES_M * WAVES_N * 64;
  static constexpr int SM = WM / 16, SN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int CA = BM * 8 / THREADS;  // 16-byte chunks per thread per slice
  static constexpr int CB = BN * 8 / THREADS;
  static_assert(BM % WM == 0 && BN % WN == 0, "tile");
  static_assert(WM % 16 == 0 && WN % 32 == 0 && WN <= 128 && 128 % WN == 0, "wave tile");
  static_assert((BM * 8) % THREADS == 0 && (BN * 8) % THREADS == 0, "loader");
};

// Everything a workgroup needs to know about the tile it computes.
struct Tile {
  const uint8_t* A;   // row 0 of the (group's) A
  const float* sa;    // (group's) activation scales
  const uint8_t* B;   // row 0 of the (group's / expert's) B
  const float* sb;    // (group's / expert's) weight scales
  uint16_t* D;        // row 0 of the (group's) D
  int m0, n0;
  int rows_alloc;     // rows addressable in A / sa (reads clamp to it)
  int rows_valid;     // dense/masked: rows < rows_valid are stored
  int expert;         // contiguous: rows whose index equals it are stored
};

template <int L>
__device__ __forceinline__ bool resolve_tile(const GemmParams& p, int w, int BM, int BN, Tile& t) {
  int tm, tn;
  if (L == kMasked) {
    const int per_group = p.tiles_m * p.tiles_n;
    const int g = w / per_group;
    raster(w - g * per_group, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int valid = min(max(load_invariant(p.masked_m + g), 0), p.rows);
    if (tm * BM >= valid) return false;
    const int64_t Kb = p.Kb;
    t.A = p.A + (int64_t)g * p.rows * p.K;
    t.sa = p.sa + (int64_t)g * Kb * p.ld_sa;
    t.B = p.B + (int64_t)g * p.N * p.K;
    t.sb = p.sb + (int64_t)g * p.Nb * Kb;
    t.D = p.D + (int64_t)g * p.rows * p.N;
    t.rows_valid = valid;
    t.expert = 0;
  } else {
    raster(w, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    t.A = p.A;
    t.sa = p.sa;
    t.D = p.D;
    t.rows_valid = p.rows;
    if (L == kContiguous) {
      // expert of this 128-aligned row block: the largest index in it
      const int lane = threadIdx.x & 63;
      int e = -1;
      for (int r = lane; r < BM; r += 64) {
        const int m = min(tm * BM + r, p.rows - 1);
        const int v = p.m_indices[m];
        if (v < p.G) e = max(e, v);  // an index past the experts is padding
      }
      e = wave_max(e);
      e = __builtin_amdgcn_readfirstlane(e);
      if (e < 0) return false;  // padding only
      t.expert = e;
      t.B = p.B + (int64_t)e * p.N * p.K;
      t.sb = p.sb + (int64_t)e * p.Nb * p.Kb;
    } else {
      t.expert = 0;
      t.B = p.B;
      t.sb = p.sb;
    }
  }
  t.m0 = tm * BM;
  t.n0 = tn * BN;
  // masked: rows past the group's count are never read (they load as zeros)
  t.rows_alloc = L == kMasked ? t.rows_valid : p.rows;
  return true;
}

// Raw buffer resource over [base, base + bytes): loads at or past the end
// return zeros, which is how rows beyond M or N are fed to the MFMAs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// A lane offset at or past the end of every range make_rsrc builds (they
// hold at most 2^31 - 1 bytes), read as signed or unsigned, with or without
// the instruction's scalar offset (at most a 4 MiB row) added, and without
// 32-bit wrap-around: such a load returns zeros and touches no memory.
constexpr int kOobOffset = 0x7fffffff;

// Cache policy bits of a buffer access (sc0 | sc1): system-coherent, so the
// data neither stays in nor is served from a non-coherent cache.  Used for
// the fp32 partials that workgroups exchange.
constexpr int kSysCoherent = 1 | 16;

// K tails (K % 128 != 0, K % 16 == 0): the last slice holds K % 128 columns.
// A 16-byte chunk that starts at or past column K of its row is read as
// zeros (the bytes there belong to the next row or to padding), so both
// operands contribute 0 * 0 past K.  `kcol` is the chunk's first column.
__device__ __forceinline__ int k_clip(int voff, int kcol, int K) { return kcol < K ? voff : kOobOffset; }

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <class C, int L>
__global__ __launch_bounds__(C::THREADS, 2) void gemm_fp8_kernel(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  constexpr int SM = C::SM, SN = C::SN, CA = C::CA, CB = C::CB;
  constexpr int NT = C::THREADS;
  constexpr int Q = WN / 4;
  constexpr int ROWS_PER_PASS = NT / 8;  // loader rows covered by one pass of the workgroup

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int l16 = lane & 15;
  const int kq = lane >> 4;  // which 32-byte quarter of the slice this lane feeds

  // loader: thread -> (row, chunk); passes add ROWS_PER_PASS rows
  const int ld_row = tid >> 3, ld_c = tid & 7;
  // swizzles depend on row & 7 (A) and row bits 0,1,log2(Q) (B); ROWS_PER_PASS
  // is a multiple of 8 and of 2Q, so they are the same on every pass.
  static_assert(ROWS_PER_PASS % 8 == 0 && ROWS_PER_PASS % (2 * Q) == 0, "loader swizzle invariance");
  const int a_dst0 = ld_row * 128 + ((ld_c ^ swz_a(ld_row)) << 4);
  const int b_dst0 = C::A_BYTES + ld_row * 128 + ((ld_c ^ swz_b<Q>(ld_row)) << 4);

  // fragment reads: the swizzle of a fragment row does not depend on the
  // subtile index, so one base offset per half suffices.
  const int a_row0 = wm * WM + l16;
  const int b_row0 = wn * WN + Q * (l16 >> 2) + (lane & 3);
  int a_frag0[2], b_frag0[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    a_frag0[h] = a_row0 * 128 + (((2 * kq + h) ^ swz_a(a_row0)) << 4);
    b_frag0[h] = C::A_BYTES + b_row0 * 128 + (((2 * kq + h) ^ swz_b<Q>(b_row0)) << 4);
  }

  const int grid = gridDim.x;
  const int local = xcd_local_id(blockIdx.x, grid);

  for (int it = 0;; ++it) {
    const int w = it * grid + local;
    if (w >= p.num_tiles) break;
    Tile t;
    if (!resolve_tile<L>(p, w, BM, BN, t)) continue;

    __syncthreads();  // the previous tile's last LDS stage is no longer read

    // A rows [m0, rows_alloc) and B rows [n0, N) as buffer ranges
    const uint8_t* a_base = t.A + (int64_t)t.m0 * p.lda;
    const uint8_t* b_base = t.B + (int64_t)t.n0 * p.ldb;
    const int64_t a_bytes = (int64_t)(t.rows_alloc - t.m0 - 1) * p.lda + p.K;
    const int64_t b_bytes = (int64_t)(p.N - t.n0 - 1) * p.ldb + p.K;
    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(a_base, a_bytes);
    const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(b_base, b_bytes);
    const int a_voff = ld_row * (int)p.lda + ld_c * 16;
    const int b_voff = ld_row * (int)p.ldb + ld_c * 16;
    const int a_pass = ROWS_PER_PASS * (int)p.lda;
    const int b_pass = ROWS_PER_PASS * (int)p.ldb;

    // this lane's activation rows for the scales (clamped: scales of rows
    // past the end only multiply zeros)
    int sa_row[SM];
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) sa_row[ms] = min(t.m0 + a_row0 + ms * 16, t.rows_alloc - 1);
    const int nb_wave = min((t.n0 + wn * WN) >> 7, p.Nb - 1);
    const float* sb_wave = t.sb + (int64_t)nb_wave * p.ld_sb;

    float acc[SM][SN][4];
#pragma unroll
    for (int ms = 0; ms < SM; ++ms)
#pragma unroll
      for (int tt = 0; tt < SN; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ms][tt][r] = 0.f;

    const int Kb = p.Kb;
    i32x4 ra[CA], rb[CB];
    if (Kb > 0) {
#pragma unroll
      for (int i = 0; i < CA; ++i)
        ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, k_clip(a_voff + i * a_pass, ld_c * 16, p.K), 0, 0);
#pragma unroll
      for (int i = 0; i < CB; ++i)
        rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, k_clip(b_voff + i * b_pass, ld_c * 16, p.K), 0, 0);
#pragma unroll
      for (int i = 0; i < CA; ++i) *(i32x4*)(smem + a_dst0 + i * ROWS_PER_PASS * 128) = ra[i];
#pragma unroll
      for (int i = 0; i < CB; ++i) *(i32x4*)(smem + b_dst0 + i * ROWS_PER_PASS * 128) = rb[i];
      __syncthreads();
    }

    for (int kb = 0; kb < Kb; ++kb) {
      const bool more = kb + 1 < Kb;
      if (more) {
        const int ko = (kb + 1) * 128;
        const int kc = ko + ld_c * 16;
#pragma unroll
        for (int i = 0; i < CA; ++i)
          ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, k_clip(a_voff + i * a_pass, kc, p.K), ko, 0);
#pragma unroll
        for (int i = 0; i < CB; ++i)
          rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, k_clip(b_voff + i * b_pass, kc, p.K), ko, 0);
      }
      // slice scales: s = sa[kb][m] * sb[nb][kb]
      const float sbv = sb_wave[kb];
      const float* sa_k = t.sa + (int64_t)kb * p.ld_sa;
      float s[SM];
#pragma unroll
      for (int ms = 0; ms < SM; ++ms) s[ms] = sa_k[sa_row[ms]] * sbv;

      const uint8_t* st = smem + (kb & 1) * C::STAGE;
      i32x8 af[SM];
#pragma unroll
      for (int ms = 0; ms < SM; ++ms) {
        const i32x4 lo = *(const i32x4*)(st + a_frag0[0] + ms * 16 * 128);
        const i32x4 hi = *(const i32x4*)(st + a_frag0[1] + ms * 16 * 128);
        af[ms] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int tt = 0; tt < SN; ++tt) {
        const i32x4 lo = *(const i32x4*)(st + b_frag0[0] + tt * 4 * 128);
        const i32x4 hi = *(const i32x4*)(st + b_frag0[1] + tt * 4 * 128);
        const i32x8 bf = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int ms = 0; ms < SM; ++ms) {
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4 P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[ms], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ms][tt][r] = __builtin_fmaf(P[r], s[ms], acc[ms][tt][r]);
        }
      }
      if (more) {
        uint8_t* nx = smem + ((kb + 1) & 1) * C::STAGE;
#pragma unroll
        for (int i = 0; i < CA; ++i) *(i32x4*)(nx + a_dst0 + i * ROWS_PER_PASS * 128) = ra[i];
#pragma unroll
        for (int i = 0; i < CB; ++i) *(i32x4*)(nx + b_dst0 + i * ROWS_PER_PASS * 128) = rb[i];
      }
      __syncthreads();
    }

    // ---- epilogue: each lane owns Q consecutive columns of SM rows ----
    const int n_base = t.n0 + wn * WN + Q * kq;
    const bool vec = (p.ldd & 7) == 0 && ((uintptr_t)p.D & 15) == 0;
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
      const int m = t.m0 + a_row0 + ms * 16;
      bool ok;
      if (L == kContiguous) {
        ok = m < t.rows_alloc && p.m_indices[m] == t.expert;
      } else {
        ok = m < t.rows_valid;
      }
      if (!ok) continue;
      uint16_t* drow = t.D + (int64_t)m * p.ldd;
      f32x4 cv[SN];
#pragma unroll
      for (int tt = 0; tt < SN; ++tt)
        cv[tt] = L == kDenseC ? load_addend4(p, m, n_base + 4 * tt, n_base + 4 * tt < p.N) : f32x4{0.f, 0.f, 0.f, 0.f};
      uint32_t pk[Q / 2];
#pragma unroll
      for (int tt = 0; tt < SN; ++tt) {
        float v[4] = {acc[ms][tt][0], acc[ms][tt][1], acc[ms][tt][2], acc[ms][tt][3]};
        if (L == kDenseC)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += cv[tt][r];
        pk[2 * tt] = pack_bf16x2(v[0], v[1]);
        pk[2 * tt + 1] = pack_bf16x2(v[2], v[3]);
      }
      if (vec && n_base + Q <= p.N) {
#pragma unroll
        for (int v = 0; v < Q / 8; ++v) {
          const i32x4 o = {(int)pk[4 * v], (int)pk[4 * v + 1], (int)pk[4 * v + 2], (int)pk[4 * v + 3]};
          *(i32x4*)(drow + n_base + 8 * v) = o;
        }
      } else {
#pragma unroll
        for (int j = 0; j < Q; ++j) {
          if (n_base + j < p.N) drow[n_base + j] = (uint16_t)(pk[j >> 1] >> ((j & 1) * 16));
        }
      }
    }
  }
}


// ===========================================================================
// Large-tile kernel: BM x BN workgroup tile, WAVES_M x WAVES_N waves (two per
// SIMD), operands fetched straight into LDS by buffer loads (no VGPR staging),
// double-buffered stages.  The persistent loop is flattened over (tile,
// segment, K slice) so the first slice of the next tile is already in flight
// while the current tile finishes and stores.  A contiguous-layout tile whose
// two 128-row halves belong to different experts is computed as two segments
// (one per expert, the other half's waves idle); every other tile is one
// segment.
// ===========================================================================

// BROWS: the B rows a stage holds (BN; 256 for a B staged MN-major, whose
// slice takes 128 K rows of 256 bytes whatever the tile width).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BROWS_ = BN_>
struct BigCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, BROWS = BROWS_;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = NWAVES * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int SM = WM / 16, SN = WN / 16;
  static constexpr int STAGE = (BM + BROWS) * 128;
  // 1 KiB (8-row) loads per slice: each wave of the first half loads
  // LOADS_A consecutive A loads and LOADS_B consecutive B loads
  static constexpr int LOADS_A = BM / 8 / (NWAVES / 2), LOADS_B = BN / 8 / (NWAVES / 2);
  // LDS: two operand stages, then the activation scales of each stage (one
  // fp32 per tile row, 1 KiB per stage)
  static constexpr int SA_OFF = 2 * STAGE;
  static constexpr int LDS_BYTES = 2 * STAGE + 2 * 1024;
  // A wave's columns lie in one 128-wide weight-scale block when the tile
  // width is a multiple of 128 and the wave width divides 128; otherwise a
  // wave may straddle one block boundary and picks the scale per subtile.
  static constexpr bool SCALE_PER_WAVE = (BN % 128 == 0) && (128 % WN == 0);
  static_assert(NWAVES % 2 == 0 && BM % (4 * NWAVES) == 0 && BN % (4 * NWAVES) == 0, "loads");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && WN <= 128, "wave tile");
  static_assert(BN <= 256, "epilogue staging rows are 512 bytes");
  static_assert(BM <= 64 * (NWAVES / 2), "one 64-row activation-scale load per A wave");
  static_assert(BM % 128 == 0 || BM <= 128, "row halves");
};

// 16-byte chunk swizzle inside a 128-byte LDS row for the large kernel.
// A fragment read touches 16 consecutive rows at one logical chunk; the
// chunk index is XORed with the row's low 3 bits (8 consecutive rows land in
// 8 different 16-byte bank groups) and with bit 3 (rows r and r+8 of the same
// parity also differ, for 16-lane service over 256 bytes).
__device__ __forceinline__ int swz16(int row) { return (row & 7) ^ ((row >> 3) & 1); }

struct Work {
  const uint8_t* A;
  const float* sa;
  const uint8_t* B;
  const float* sb;
  uint16_t* D;
  int m0, n0;
  int rows_alloc, rows_valid;
  int seg, nseg;      // segment of the tile and how many it has
  int half_mask;      // contiguous: 128-row halves computed in this segment
  int e_lo, e_hi;     // contiguous: expert of each half (-1 = padding only)
  int w;              // tile id (< 0: no more work)
  int kbn;            // 128-deep K slices of the tile
  int krows;          // K rows readable from A / B (rows past them load as zeros)
  const float* C;     // K-grouped: the group's fp32 addend, or NULL
};

__device__ __forceinline__ int block_max_index(const int32_t* idx, int from, int count, int rows, int G) {
  const int lane = threadIdx.x & 63;
  int e = -1;
  for (int r = lane; r < count; r += 64) {
    const int m = from + r;
    if (m < rows) {
      const int v = idx[m];
      if (v < G) e = max(e, v);  // an index past the experts is padding: no weight is addressed with it
    }
  }
  e = wave_max(e);
  return __builtin_amdgcn_readfirstlane(e);
}

// Resolve tile id w into its first segment; false if the tile has no work.
template <int L, int BM, int BN>
__device__ __forceinline__ bool resolve_big(const GemmParams& p, int w, Work& t, const KGroups* kg = nullptr) {
  int tm, tn;
  t.w = w;
  t.seg = 0;
  t.nseg = 1;
  t.half_mask = 3;
  t.e_lo = t.e_hi = 0;
  t.kbn = p.Kb;
  t.krows = p.K;
  t.C = nullptr;
  if (L == kKGrouped) {
    // group idx owns the K range [128 kb0, 128 kb1) of A and B and writes
    // D[g] (packed [G, M, N])
    const int per = p.tiles_m * p.tiles_n;
    const int idx = w / per;
    raster(w - idx * per, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int g = kg->g[idx];
    const int kb0 = kg->kb0[idx];
    t.kbn = kg->kb0[idx + 1] - kb0;
    t.krows = t.kbn * 128;
    t.A = p.A + kb0 * kg->a_step;
    t.sa = p.sa + (int64_t)kb0 * p.ld_sa;
    t.B = p.B + kb0 * kg->b_step;
    t.sb = p.sb + kb0;
    t.D = p.D + (int64_t)g * p.rows * p.N;
    t.C = p.Cin ? p.Cin + (int64_t)g * p.rows * p.N : nullptr;
    t.rows_valid = p.rows;
  } else if (L == kMasked) {
    const int per_group = p.tiles_m * p.tiles_n;
    const int g = w / per_group;
    raster(w - g * per_group, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int valid = min(max(load_invariant(p.masked_m + g), 0), p.rows);
    if (tm * BM >= valid) return false;
    const int64_t Kb = factor_kb(p);
    t.A = p.A + (int64_t)g * p.rows * p.K;
    t.sa = p.sa + (int64_t)g * Kb * p.ld_sa;
    t.B = p.B + (int64_t)g * p.N * p.K;
    t.sb = p.sb + (int64_t)g * p.Nb * Kb;
    t.D = p.D + (int64_t)g * p.rows * p.ldd;
    t.rows_valid = valid;
  } else {
    raster(w, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    t.A = p.A;
    t.sa = p.sa;
    t.D = p.D;
    t.rows_valid = p.rows;
    t.B = p.B;
    t.sb = p.sb;
    if (L == kContiguous) {
      const int m0 = tm * BM;
      const int half = BM >= 256 ? BM / 2 : BM;
      const int lo = block_max_index(p.m_indices, m0, half, p.rows, p.G);
      const int hi = BM >= 256 ? block_max_index(p.m_indices, m0 + half, half, p.rows, p.G) : -1;
      if (lo < 0 && hi < 0) return false;
      t.e_lo = lo;
      t.e_hi = hi;
      if (lo >= 0 && hi >= 0 && lo != hi) {
        t.nseg = 2;
        t.half_mask = 1;
      } else {
        t.half_mask = (lo >= 0 ? 1 : 0) | (hi >= 0 ? 2 : 0);
      }
      const int e = lo >= 0 ? lo : hi;
      t.B = p.B + (int64_t)e * p.N * p.K;
      t.sb = p.sb + (int64_t)e * p.Nb * factor_kb(p);
    }
  }
  t.m0 = tm * BM;
  t.n0 = tn * BN;
  // masked: rows past the group's count are never read (they load as zeros)
  t.rows_alloc = L == kMasked ? t.rows_valid : p.rows;
  return true;
}

// Next segment of the same tile, or the next tile with work for this workgroup.
template <int L, int BM, int BN>
__device__ __forceinline__ void advance_big(const GemmParams& p, Work& t, int& it, int local, int grid,
                                            const KGroups* kg = nullptr) {
  if (L == kContiguous && t.seg + 1 < t.nseg) {
    t.seg += 1;
    t.half_mask = 2;
    t.B = p.B + (int64_t)t.e_hi * p.N * p.K;
    t.sb = p.sb + (int64_t)t.e_hi * p.Nb * factor_kb(p);
    return;
  }
  for (;;) {
    ++it;
    const int w = it * grid + local;
    if (w >= p.num_tiles) {
      t.w = -1;
      return;
    }
    if (resolve_big<L, BM, BN>(p, w, t, kg)) return;
  }
}

// sa_k: the row of the activation-factor array that holds slice kb's factors
// (kb itself for fp32 factors; kb / 4 for packed power-of-two factors).
// KTAIL: the kernel is built for K % 128 != 0 (launches with whole slices
// only use the build without it, whose loads carry no clipping code at all).
// n consecutive 8-row loads of one operand, starting at 8-row load q0 of the
// stage (A rows first, then B rows).
template <int N, bool CLIP>
__device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t rs, int64_t ld, int q0, int row0, uint8_t* stage,
                                           int lane, int kb, int kleft) {
  const int comb0 = q0 * 8 + (lane >> 3);  // combined (A|B) row of this lane in load 0
  const int p_chunk = lane & 7;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int comb = comb0 + 8 * j;
    const int r = row0 + 8 * j + (lane >> 3);
    const int c = p_chunk ^ swz16(comb);
    int voff = r * (int)ld + c * 16;
    if (CLIP) voff = k_clip(voff, c * 16, kleft);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + (q0 + j) * 1024),
                                             16, voff, kb * 128, 0, 0);
  }
}

// Operands stored MN-major ([K, M] or [K, N], the NN / TN / TT layouts and
// the K-grouped GEMM) are staged as they are stored: the slice's 128 K rows
// of the tile's 256 MN columns, K row r at byte 256 r of the operand's stage
// area.  The 16-byte chunk c of row r sits at chunk c ^ kmn_swz(r): the
// transposing fragment reads (lds_frag_mn) take 8 consecutive K rows at one
// chunk per 16 lanes, and this puts those rows, and the rows 32 apart that
// the neighbouring lanes take, in different banks.
__device__ __forceinline__ int kmn_swz(int r) { return (r & 7) | (((r >> 5) & 1) << 3); }

// This wave's N loads of 4 K rows (1 KiB) each into an MN-major stage area,
// from 1 KiB load q0; chunks at or past column `cols` of the tile (a
// multiple of 16) are not read and load as zeros.
template <int N>
__device__ __forceinline__ void issue_rows_mn(__amdgpu_buffer_rsrc_t rs, int64_t ld, int q0, uint8_t* area, int lane,
                                              int cols) {
  const int p_chunk = lane & 15;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int r = (q0 + j) * 4 + (lane >> 4);
    const int c = p_chunk ^ kmn_swz(r);
    const int voff = c * 16 < cols ? r * (int)ld + c * 16 : kOobOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(area + (q0 + j) * 1024), 16,
                                             voff, 0, 0, 0);
  }
}

// Buffer range over one slice of an MN-major operand of `ext` columns
// (ext % 16 == 0): its K rows from slice kb on, from column mn0 to the last
// K row's column ext.  K rows past `krows` read as zeros; columns past ext
// are never requested (issue_rows_mn's `cols`).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mn_slice_rsrc(const uint8_t* base, int64_t ld, int kb, int krows,
                                                                 int mn0, int ext) {
  return make_rsrc(base + (int64_t)kb * 128 * ld + mn0, (int64_t)(krows - kb * 128 - 1) * ld + (ext - mn0));
}

// KTAIL: the kernel is built for K % 128 != 0 (launches with whole slices
// only use the build without it, whose loads carry no clipping code at all).
// TA / TB: A / B stored MN-major.
template <class C, bool KTAIL = false, bool TA = false, bool TB = false>
__device__ __forceinline__ void issue_slice_loads(const GemmParams& p, const Work& t, int kb, uint8_t* stage,
                                                  uint8_t* sa_area, int wave, int lane, int sa_k = -1) {
  constexpr int BM = C::BM;
  constexpr int HALF = C::NWAVES / 2, LA = C::LOADS_A, LB = C::LOADS_B;
  static_assert(!(TA || TB) || (BM == 256 && HALF == 4), "MN-major operands: 256-row tiles, 4 loading waves");
  static_assert(!TB || C::BROWS >= 256, "an MN-major B needs 256-byte K rows in the stage");
  const bool is_a = wave < HALF;  // wave-uniform: one wave of each SIMD loads
  const int64_t bytes_a = (int64_t)(t.rows_alloc - t.m0 - 1) * p.lda + t.krows;
  const int64_t bytes_b = (int64_t)(p.N - t.n0 - 1) * p.ldb + t.krows;
  // A whole slice loads as is; only the partial last slice of a K tail
  // (wave-uniform branch) clips its chunks at column K.
  const int kleft = p.K - kb * 128;
  const bool clip = KTAIL && kleft < 128;
  // The first half of the waves (one per SIMD) loads both operands' rows and
  // the activation scales; the other half only multiplies, so each SIMD
  // always has a wave ready to issue MFMAs while its partner waits on the
  // memory pipe (measured: 1-4 % faster than splitting A and B loads over the
  // two halves).
  if (is_a) {
    const int qa = wave * LA, qb = BM / 8 + wave * LB;  // first 8-row load of each operand
    if (TA) {
      issue_rows_mn<8>(mn_slice_rsrc(t.A, p.lda, kb, t.krows, t.m0, t.rows_alloc), p.lda, wave * 8, stage, lane,
                       t.rows_alloc - t.m0);
    } else {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(t.A + (int64_t)t.m0 * p.lda, bytes_a);
      if (clip)
        issue_rows<LA, true>(ra, p.lda, qa, qa * 8, stage, lane, kb, kleft);
      else
        issue_rows<LA, false>(ra, p.lda, qa, qa * 8, stage, lane, kb, kleft);
    }
    if (TB) {
      issue_rows_mn<8>(mn_slice_rsrc(t.B, p.ldb, kb, t.krows, t.n0, p.N), p.ldb, wave * 8, stage + BM * 128, lane,
                       min(C::BN, p.N - t.n0));
    } else {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(t.B + (int64_t)t.n0 * p.ldb, bytes_b);
      if (clip)
        issue_rows<LB, true>(rb, p.ldb, qb, qb * 8 - BM, stage, lane, kb, kleft);
      else
        issue_rows<LB, false>(rb, p.ldb, qb, qb * 8 - BM, stage, lane, kb, kleft);
    }
    // sa[kb][m0 + 64 wave + lane] into the stage's scale area; rows past
    // rows_alloc read as 0 (their outputs are never stored)
    const float* sbase = t.sa + (int64_t)(sa_k < 0 ? kb : sa_k) * p.ld_sa + t.m0;
    const int sbytes = max(t.rows_alloc - t.m0, 0) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(sbase, sbytes),
                                             (__attribute__((address_space(3))) void*)(sa_area + wave * 256), 4,
                                             (wave * 64 + lane) * 4, 0, 0, 0);
  }
}

// Weight-block scales sb[nb][kb] of the (at most two) 128-column blocks the
// wave's columns touch, for one K slice.  They are wave-uniform and never
// written while a GEMM runs, so they are read through the scalar cache; the
// activation scales of the slice arrive in LDS with its operands.
// UE8M0 byte -> the fp32 power of two 2^(e - 127) (e = 0 is the subnormal
// 2^-127, e = 255 overflows to infinity).
__device__ __forceinline__ float ue8m0_factor(int e) {
  return __builtin_bit_cast(float, e == 0 ? 0x00400000 : e << 23);
}

// UE8: the factors are UE8M0 bytes packed four K groups to an int32 (sb rows
// of ceil(Kb / 4) words), decoded to fp32 here.
template <class C, bool UE8 = false>
__device__ __forceinline__ void load_sb(const GemmParams& p, const Work& t, int kb, int wn, float (&sb_r)[2]) {
  const int nw = t.n0 + wn * C::WN;
  const int nb0 = min(nw >> 7, p.Nb - 1);
  const int nb1 = C::SCALE_PER_WAVE ? nb0 : min(nb0 + 1, p.Nb - 1);
  if (UE8) {
    const int64_t kb4 = (p.Kb + 3) >> 2;
    const __attribute__((address_space(4))) int* sbk =
        (const __attribute__((address_space(4))) int*)((const int*)(const void*)t.sb + (kb >> 2));
    const int sh = 8 * (kb & 3);
    sb_r[0] = ue8m0_factor((sbk[(int64_t)nb0 * kb4] >> sh) & 0xff);
    sb_r[1] = C::SCALE_PER_WAVE ? sb_r[0] : ue8m0_factor((sbk[(int64_t)nb1 * kb4] >> sh) & 0xff);
  } else {
    const __attribute__((address_space(4))) float* sbk = (const __attribute__((address_space(4))) float*)(t.sb + kb);
    sb_r[0] = sbk[(int64_t)nb0 * p.ld_sb];
    sb_r[1] = C::SCALE_PER_WAVE ? sb_r[0] : sbk[(int64_t)nb1 * p.ld_sb];
  }
}

// s = sa * sb for this lane's SM rows, sa read from the stage's scale area
// (UE8: the packed word of the slice's four K groups; byte kb % 4 is the
// slice's).
template <class C, bool UE8 = false>
__device__ __forceinline__ void slice_scales(const uint8_t* sa_area, int wm, int l16, const float (&sb)[2],
                                             float (&s)[C::SM][2], int kb = 0) {
#pragma unroll
  for (int ms = 0; ms < C::SM; ++ms) {
    const int w = *(const int*)(sa_area + (wm * C::WM + ms * 16 + l16) * 4);
    const float a = UE8 ? ue8m0_factor((w >> (8 * (kb & 3))) & 0xff) : __builtin_bit_cast(float, w);
    s[ms][0] = a * sb[0];
    s[ms][1] = a * sb[1];
  }
}

// First weight subtile of the wave that lies in the second 128-column block
// (SN or more when the wave stays inside one block).
template <class C>
__device__ __forceinline__ int second_block_subtile(const Work& t, int wn) {
  if (C::SCALE_PER_WAVE) return C::SN;
  const int nw = t.n0 + wn * C::WN;
  return (128 - (nw & 127)) >> 4;
}

__device__ __forceinline__ i32x8 lds_frag(const uint8_t* st, int off0, int off1) {
  const i32x4 lo = *(const i32x4*)(st + off0);
  const i32x4 hi = *(const i32x4*)(st + off1);
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// Per-lane geometry of the MN-major fragment reads: within each 16-lane group
// q = lane / 16, lane 2j + h addresses K row 32q + j (and 8t further for read
// t) at byte 8h of the fragment's chunk; the transposing read then hands lane
// i of the group the 8 K bytes of MN row i.  Returns {row offset, swizzle}.
__device__ __forceinline__ void mn_frag_geom(int lane, int area, int (&g)[2]) {
  const int q = lane >> 4, i = lane & 15;
  const int r = 32 * q + (i >> 1);
  g[0] = area + r * 256 + 8 * (i & 1);
  g[1] = kmn_swz(r) << 4;  // the same for r + 8t (t < 4)
}

// The 16 x 128 fragment of MN rows [16 s, 16 s + 16) of an MN-major stage
// area, in MFMA operand layout (lane: row lane % 16, K bytes [32 (lane / 16),
// +32)), by four transposing 8-byte reads of 8 K rows each.
__device__ __forceinline__ i32x8 lds_frag_mn(const uint8_t* st, const int (&g)[2], int s) {
  const uint8_t* a = st + g[0] + ((s << 4) ^ g[1]);
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(a));
  const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(a + 2048));
  const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(a + 4096));
  const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(a + 6144));
  return (i32x8){r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

// One 128-deep K slice of the wave tile: SM x SN MFMAs, each a fresh partial
// P, promoted into acc with s = sa * sb.  Software-pipelined by weight subtile:
// step (tt, ms) issues the MFMA of (tt, ms) and the four promotion FMAs of
// (tt-1, ms), so an MFMA result is read SM MFMAs after it was issued (its
// latency and the MFMA->VALU hazard are hidden behind other MFMAs) and the
// matrix core never waits for the promotion.  Scheduling fences keep the
// compiler from pulling each MFMA down next to its consumers.  s[ms][0]
// applies to subtiles before `tb`, s[ms][1] from `tb` on (the wave's columns
// may cross one 128-column weight-scale block boundary).
// TA / TB: the operand is staged MN-major; its offsets are then mn_frag_geom's
// and a_s0 / b_s0 the chunk of the wave's first fragment row.
template <class C, bool TA = false, bool TB = false>
__device__ __forceinline__ void slice_mma(const uint8_t* st, const int (&a_off)[2], const int (&b_off)[2],
                                          const float (&s)[C::SM][2], int tb, float (&acc)[C::SM][C::SN][4],
                                          int a_s0 = 0, int b_s0 = 0) {
  constexpr int SM = C::SM, SN = C::SN;
  auto frag_a = [&](int ms) {
    return TA ? lds_frag_mn(st, a_off, a_s0 + ms) : lds_frag(st, a_off[0] + ms * 2048, a_off[1] + ms * 2048);
  };
  auto frag_b = [&](int tt) {
    return TB ? lds_frag_mn(st, b_off, b_s0 + tt) : lds_frag(st, b_off[0] + tt * 2048, b_off[1] + tt * 2048);
  };
  // the first weight fragment, then the activation fragments in the order
  // the first subtile's MFMAs use them: LDS reads return in order, so the
  // first MFMA waits for two fragments instead of all SM + 1
  i32x8 bf = frag_b(0);
  i32x8 af[SM];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms) af[ms] = frag_a(ms);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 prev[SM];
#pragma unroll
  for (int tt = 0; tt < SN; ++tt) {
    i32x8 bn = bf;
    if (tt + 1 < SN) bn = frag_b(tt + 1);
    f32x4 cur[SM];
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      cur[ms] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[ms], zero, 0, 0, 0, 0, 0, 0);
      if (tt > 0) {
        const float sc = C::SCALE_PER_WAVE ? s[ms][0] : (tt - 1 < tb ? s[ms][0] : s[ms][1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ms][tt - 1][r] = __builtin_fmaf(prev[ms][r], sc, acc[ms][tt - 1][r]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) prev[ms] = cur[ms];
    bf = bn;
  }
#pragma unroll
  for (int ms = 0; ms < SM; ++ms) {
    const float sc = C::SCALE_PER_WAVE ? s[ms][0] : (SN - 1 < tb ? s[ms][0] : s[ms][1]);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[ms][SN - 1][r] = __builtin_fmaf(prev[ms][r], sc, acc[ms][SN - 1][r]);
  }
}

// Workgroup barrier that waits only for this wave's LDS traffic (not for
// outstanding global stores or operand prefetches).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Epilogue: the finished tile is converted to bf16 and staged through the LDS
// stage that was just consumed, half a tile at a time, so that the global
// stores are whole 512-byte row segments (16 bytes per lane) instead of
// 32-byte pieces of 16 rows.  Staging rows are 512 bytes; the 16-byte chunk
// index is XORed with the row's low 4 bits, which keeps both the 8-byte
// fragment writes (16 rows at one chunk) and the row reads conflict-free.
template <class C>
struct StoreGeom {
  static constexpr int ROWB = 512;                 // staging row bytes (BN <= 256 bf16)
  static constexpr int CHUNKS = ROWB / 16;          // 16-byte chunks per staging row
  static constexpr int USED = C::BN / 8;            // chunks holding the tile's columns
  static constexpr int PASSES = (C::BM / 2) * ROWB <= C::STAGE ? 2 : 4;
  static constexpr int PASS_ROWS = C::BM / PASSES;
  static constexpr int MS_PER_PASS = C::SM / PASSES;
  static constexpr int ROWS_PER_READ = 64 / CHUNKS;
  static constexpr int READS = PASS_ROWS / (C::NWAVES * ROWS_PER_READ);
  static_assert(PASS_ROWS * ROWB <= C::STAGE && C::SM % PASSES == 0, "staging");
  static_assert(PASS_ROWS % (C::NWAVES * ROWS_PER_READ) == 0, "reads");
};

template <class C, int L>
__device__ __forceinline__ void store_tile(const GemmParams& p, const Work& t, const float (&acc)[C::SM][C::SN][4],
                                           uint8_t* stg, int wave, int lane) {
  using G = StoreGeom<C>;
  constexpr int BM = C::BM, WM = C::WM, WN = C::WN, SN = C::SN;
  constexpr int ROWB = G::ROWB, CHUNKS = G::CHUNKS, PASSES = G::PASSES;
  constexpr int WROWS = WM / PASSES;  // staging rows per wave-row per pass

  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int l16 = lane & 15, kq = lane >> 4;
  const bool vec = (p.ldd & 7) == 0 && ((uintptr_t)p.D & 15) == 0;
  // fp32 addend: C of the dense call, or the K-grouped tile's group slice
  constexpr bool ADDEND = L == kDenseC || L == kKGrouped;
  const float* cbase = L == kDenseC ? p.Cin : t.C;
  const int64_t ldc = L == kDenseC ? p.ldc : (int64_t)p.N;
  const bool add_c = ADDEND && cbase != nullptr;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    // the addend of this pass's fragments, all loads in flight together
    f32x4 cv[ADDEND ? G::MS_PER_PASS : 1][SN];
    if (add_c) {
#pragma unroll
      for (int j = 0; j < G::MS_PER_PASS; ++j) {
        const int m = t.m0 + wm * WM + (pass * G::MS_PER_PASS + j) * 16 + l16;
#pragma unroll
        for (int tt = 0; tt < SN; ++tt) {
          const int n = t.n0 + wn * WN + tt * 16 + 4 * kq;
          cv[j][tt] = load_addend4(cbase, ldc, p.N, m, n, m < t.rows_valid && n < p.N);
        }
      }
    }
    // write this wave's fragment rows of the pass
#pragma unroll
    for (int j = 0; j < G::MS_PER_PASS; ++j) {
      const int ms = pass * G::MS_PER_PASS + j;
      const int srow = wm * WROWS + j * 16 + l16;
#pragma unroll
      for (int tt = 0; tt < SN; ++tt) {
        const int byte = (wn * WN + tt * 16 + 4 * kq) * 2;
        const int c = byte >> 4;
        const int off = srow * ROWB + ((c ^ (srow & 15)) << 4) + (byte & 15);
        float v[4] = {acc[ms][tt][0], acc[ms][tt][1], acc[ms][tt][2], acc[ms][tt][3]};
        if (ADDEND && add_c)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += cv[j][tt][r];
        *(uint2*)(stg + off) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    lds_barrier();
    // read whole rows back and store them
#pragma unroll
    for (int rd = 0; rd < G::READS; ++rd) {
      const int srow = (wave * G::READS + rd) * G::ROWS_PER_READ + lane / CHUNKS;
      const int c = lane % CHUNKS;
      if (c < G::USED) {
        const i32x4 v = *(const i32x4*)(stg + srow * ROWB + ((c ^ (srow & 15)) << 4));
        // staging row -> tile row
        const int trow = (srow / WROWS) * WM + pass * WROWS + srow % WROWS;
        const int m = t.m0 + trow;
        bool ok;
        if (L == kContiguous) {
          const int e = trow < BM / 2 || BM < 256 ? t.e_lo : t.e_hi;
          ok = e >= 0 && m < t.rows_alloc && p.m_indices[m] == e;
        } else {
          ok = m < t.rows_valid;
        }
        const int n = t.n0 + c * 8;
        if (ok && n < p.N) {
          uint16_t* dst = t.D + (int64_t)m * p.ldd + n;
          if (vec && n + 8 <= p.N) {
            *(i32x4*)dst = v;
          } else {
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2)
              if (n + e2 < p.N) dst[e2] = (uint16_t)((uint32_t)v[e2 >> 1] >> ((e2 & 1) * 16));
          }
        }
      }
    }
    lds_barrier();  // staging free again (next pass, or the next tile's operand loads)
  }
}

// Epilogue of the fp32-factor large kernel, straight from registers: no LDS
// staging and no barrier, so each wave stores its 64 x WN block as soon as
// its last slice is done and goes on to the next tile.  Lane (l16, kq) holds
// columns [4 kq, 4 kq + 4) of row l16 of every 16 x 16 block; for each pair
// of neighbouring blocks, lanes kq and kq ^ 1 trade one block's half (a
// cross-lane permute), so that an even lane holds 8 consecutive columns of
// the first block and an odd lane 8 of the second: 16-byte stores that cover
// 64 contiguous bytes of 16 rows per instruction.  An odd block count leaves
// one block stored as 8 bytes per lane.  (Measured on MI355X against staging
// the tile through LDS into whole-row stores: 3 % faster on the contiguous
// MoE workload, 4 % on K = 1536, with identical bits.)
template <class C, int L>
__device__ __forceinline__ void store_direct(const GemmParams& p, const Work& t, const float (&acc)[C::SM][C::SN][4],
                                             int wave, int lane) {
  constexpr int SN = C::SN;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int l16 = lane & 15, kq = lane >> 4;
  const bool odd = (kq & 1) != 0;
  const bool vec16 = (p.ldd & 7) == 0 && ((uintptr_t)p.D & 15) == 0;
  const bool vec8 = (p.ldd & 3) == 0 && ((uintptr_t)p.D & 7) == 0;
  const int nw = t.n0 + wn * C::WN;  // the wave's first column
#pragma unroll
  for (int ms = 0; ms < C::SM; ++ms) {
    const int trow = wm * C::WM + ms * 16 + l16;
    const int m = t.m0 + trow;
    bool ok;
    if (L == kContiguous) {
      const int e = trow < C::BM / 2 || C::BM < 256 ? t.e_lo : t.e_hi;
      ok = e >= 0 && m < t.rows_alloc && p.m_indices[m] == e;
    } else {
      ok = m < t.rows_valid;
    }
    float v[SN][4];
#pragma unroll
    for (int tt = 0; tt < SN; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[tt][r] = acc[ms][tt][r];
    uint16_t* drow = t.D + (int64_t)m * p.ldd;
#pragma unroll
    for (int tp = 0; tp + 1 < SN; tp += 2) {
      const uint32_t a0 = pack_bf16x2(v[tp][0], v[tp][1]), a1 = pack_bf16x2(v[tp][2], v[tp][3]);
      const uint32_t b0 = pack_bf16x2(v[tp + 1][0], v[tp + 1][1]), b1 = pack_bf16x2(v[tp + 1][2], v[tp + 1][3]);
      // even lanes send their second block's half, odd lanes their first's
      const int r0 = __shfl_xor((int)(odd ? a0 : b0), 16), r1 = __shfl_xor((int)(odd ? a1 : b1), 16);
      const i32x4 w = odd ? i32x4{r0, r1, (int)b0, (int)b1} : i32x4{(int)a0, (int)a1, r0, r1};
      const int n = nw + tp * 16 + (odd ? 16 + 4 * (kq - 1) : 4 * kq);
      if (ok && n < p.N) {
        if (vec16 && n + 8 <= p.N) {
          *(i32x4*)(drow + n) = w;
        } else {
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2)
            if (n + e2 < p.N) drow[n + e2] = (uint16_t)((uint32_t)w[e2 >> 1] >> ((e2 & 1) * 16));
        }
      }
    }
    if (SN % 2 == 1) {
      const uint32_t a0 = pack_bf16x2(v[SN - 1][0], v[SN - 1][1]), a1 = pack_bf16x2(v[SN - 1][2], v[SN - 1][3]);
      const int n = nw + (SN - 1) * 16 + 4 * kq;
      if (ok && n < p.N) {
        if (vec8 && n + 4 <= p.N) {
          *(uint2*)(drow + n) = make_uint2(a0, a1);
        } else {
          const uint32_t w[2] = {a0, a1};
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            if (n + e2 < p.N) drow[n + e2] = (uint16_t)(w[e2 >> 1] >> ((e2 & 1) * 16));
        }
      }
    }
  }
}

// Accumulators at the start of a tile: zeros, or for D = C + A B^T the
// tile's fp32 addend (C of the dense call, or the K-grouped tile's group
// slice; t.w < 0, no tile, gives zeros), so that the epilogue adds nothing.
// The loads go out right after
// the previous tile's stores and nothing waits for them until the first
// promotion of the tile's first slice: the addend's read overlaps the stores
// and the first slice's loads and MFMAs instead of stalling the epilogue.
template <class C, int L>
__device__ __forceinline__ void init_acc(const GemmParams& p, const Work& t, float (&acc)[C::SM][C::SN][4],
                                         int wave, int lane) {
  constexpr bool ADDEND = L == kDenseC || L == kKGrouped;
  const float* cbase = L == kDenseC ? p.Cin : t.C;
  if (ADDEND && cbase != nullptr && t.w >= 0) {
    const int64_t ldc = L == kDenseC ? p.ldc : (int64_t)p.N;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int l16 = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ms = 0; ms < C::SM; ++ms) {
      const int m = t.m0 + wm * C::WM + ms * 16 + l16;
#pragma unroll
      for (int tt = 0; tt < C::SN; ++tt) {
        const int n = t.n0 + wn * C::WN + tt * 16 + 4 * kq;
        const f32x4 x = load_addend4(cbase, ldc, p.N, m, n, m < t.rows_valid && n < p.N);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ms][tt][r] = x[r];
      }
    }
    return;
  }
#pragma unroll
  for (int ms = 0; ms < C::SM; ++ms)
#pragma unroll
    for (int tt = 0; tt < C::SN; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[ms][tt][r] = 0.f;
}

// The large-tile kernel's body.  TA / TB: A / B stored MN-major (K rows of
// M / N bytes); kg: the K-grouped GEMM's groups (kKGrouped only).
template <class C, int L, bool KTAIL, bool TA, bool TB, bool UE8 = false>
__device__ __forceinline__ void big_kernel_body(const GemmParams& p, const KGroups* kg) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  constexpr int SM = C::SM, SN = C::SN;

  // two operand stages
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];
#define FG_STAGE(i) (lds + (i) * C::STAGE)
#define FG_SA(i) (lds + C::SA_OFF + (i) * 1024)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int l16 = lane & 15;
  const int kq = lane >> 4;
  const int half = (wm * WM) / 128;  // 128-row half of the tile this wave's rows lie in

  // fragment read offsets (the swizzle depends only on the row's low 4 bits);
  // MN-major operands: the transposing reads' geometry and the chunk of the
  // wave's first fragment row
  int a_off[2], b_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ra = wm * WM + l16;
    const int rb = BM + wn * WN + l16;
    a_off[h] = ra * 128 + (((2 * kq + h) ^ swz16(ra)) << 4);
    b_off[h] = rb * 128 + (((2 * kq + h) ^ swz16(rb)) << 4);
  }
  if (TA) mn_frag_geom(lane, 0, a_off);
  if (TB) mn_frag_geom(lane, BM * 128, b_off);
  const int a_s0 = (wm * WM) >> 4, b_s0 = (wn * WN) >> 4;

  const int grid = gridDim.x;
  const int local = xcd_local_id(blockIdx.x, grid);

  Work cur;
  int it = 0;
  cur.w = -1;
  if (!(local < p.num_tiles && resolve_big<L, BM, BN>(p, local, cur, kg)))
    advance_big<L, BM, BN>(p, cur, it, local, grid, kg);
  if (cur.w < 0) return;

  float sb_c[2];
  load_sb<C, UE8>(p, cur, 0, wn, sb_c);
  issue_slice_loads<C, KTAIL, TA, TB>(p, cur, 0, FG_STAGE(0), FG_SA(0), wave, lane, UE8 ? 0 : -1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // accumulators live across the segments of a tile; set up again after each store
  float acc[SM][SN][4];
  init_acc<C, L>(p, cur, acc, wave, lane);

  int stage = 0;
  while (cur.w >= 0) {
    Work nxt = cur;
    int it_n = it;
    advance_big<L, BM, BN>(p, nxt, it_n, local, grid, kg);
    const bool active = (L == kContiguous) ? (((cur.half_mask >> half) & 1) != 0)
                                           : (cur.m0 + wm * WM < cur.rows_valid);
    const int tb = second_block_subtile<C>(cur, wn);
    const int Kb = cur.kbn;

    for (int kb = 0; kb < Kb; ++kb) {
      // prefetch the following slice: this tile's next one, or the first of the next work item
      const bool last = kb + 1 == Kb;
      if (!last)
        issue_slice_loads<C, KTAIL, TA, TB>(p, cur, kb + 1, FG_STAGE(stage ^ 1), FG_SA(stage ^ 1), wave, lane,
                                            UE8 ? (kb + 1) >> 2 : -1);
      else if (nxt.w >= 0)
        issue_slice_loads<C, KTAIL, TA, TB>(p, nxt, 0, FG_STAGE(stage ^ 1), FG_SA(stage ^ 1), wave, lane,
                                            UE8 ? 0 : -1);

      if (active) {
        float s[SM][2];
        slice_scales<C, UE8>(FG_SA(stage), wm, l16, sb_c, s, kb);
        slice_mma<C, TA, TB>(FG_STAGE(stage), a_off, b_off, s, tb, acc, a_s0, b_s0);
      }

      // The next slice's weight scales are scalar loads, issued only now:
      // with one outstanding, every LDS wait inside the slice would have to
      // be a full lgkmcnt(0) (scalar loads return out of order), so the first
      // MFMAs could not start before all of the slice's fragment reads land.
      float sb_n[2] = {0.f, 0.f};
      if (!last)
        load_sb<C, UE8>(p, cur, kb + 1, wn, sb_n);
      else if (nxt.w >= 0)
        load_sb<C, UE8>(p, nxt, 0, wn, sb_n);

      // This wave's operand loads have landed in LDS; the barrier publishes
      // them to the other waves (and frees the stage just read).
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      stage ^= 1;
      sb_c[0] = sb_n[0];
      sb_c[1] = sb_n[1];
    }

    // ---- last segment of the tile: store its rows ----
    if (cur.seg == cur.nseg - 1) {
      store_direct<C, L>(p, cur, acc, wave, lane);
      if constexpr (L == kDenseC || L == kKGrouped || TA || TB) {
        init_acc<C, L>(p, nxt, acc, wave, lane);
      } else {
#pragma unroll
        for (int ms = 0; ms < SM; ++ms)
#pragma unroll
          for (int tt = 0; tt < SN; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[ms][tt][r] = 0.f;
      }
    }
    cur = nxt;
    it = it_n;
  }
  // no LDS-direct load may still be in flight when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);
#undef FG_STAGE
#undef FG_SA
}

template <class C, int L, bool KTAIL, bool TA = false, bool TB = false, bool UE8 = false>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_fp8_big_kernel(GemmParams p) {
  big_kernel_body<C, L, KTAIL, TA, TB, UE8>(p, nullptr);
}

// K-grouped GEMM, D[g] = C[g] + A_g^T B_g: one persistent launch over the
// tiles of every group with work.  MN: A [K, M] and B [K, N] as stored;
// otherwise K-major copies A^T [M, K] and B^T [N, K].
template <class C, bool MN>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_fp8_k_grouped_kernel(GemmParams p, KGroups kg) {
  big_kernel_body<C, kKGrouped, false, MN, MN>(p, &kg);
}

// D[g] = bf16(C[g]) or 0 for the K-grouped GEMM's groups without K rows:
// n elements from c (NULL: zeros) into d.
static __global__ __launch_bounds__(256) void fill_bf16_kernel(uint16_t* d, const float* c, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    d[i] = (uint16_t)(pack_bf16x2(c ? c[i] : 0.f, 0.f) & 0xffff);
}


// ===========================================================================
// Power-of-two (UE8M0) factors on the scaled MFMA (dense and grouped).  The digest's
// layout section gives the newer architecture's factors as UE8M0 bytes packed
// four to an int32.  gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes such a
// byte per lane for each operand (lane l: operand row l % 16, 32-wide K block
// l / 16) and applies 2^(e - 127) inside the matrix core, so with one factor
// per 128-deep slice every lane passes its row's byte and the MFMA can add
// each slice straight into the fp32 accumulator: the per-slice promotion
// (four VALU FMAs per MFMA with fp32 factors) disappears.  Tiles, loads and
// epilogue are the large kernel's; the activation factors of a slice arrive
// in the stage's scale area (the packed word of K groups 4i..4i+3 of each
// row), the weight factors through the scalar cache.
//
// Dense, contiguous and masked layouts (the grouped forms take each group's
// packed factors at a stride of ceil(Kb/4) words, kb_factor).  KTAIL: K % 128
// != 0, the partial last slice's chunks past column K load as zeros, as in
// the fp32-factor kernel.
// Built for 256x224, 256x160 and 128x256 tiles.  The accumulators are
// updated in place in VGPRs; with a 256x256 tile's 128 of them plus the
// operand fragments the register allocator falls back to copying every
// MFMA result and spills (two waves per SIMD leave 256 registers a wave).
// ===========================================================================

// Factor bytes of the (at most two) 128-column weight blocks the wave's
// columns touch, for slice kb: byte kb % 4 of element [nb][kb / 4].
template <class C>
__device__ __forceinline__ void load_sb_ue8m0(const GemmParams& p, const Work& t, int kb, int wn, int (&sb_r)[2]) {
  const int Kb4 = (p.Kb + 3) >> 2;
  const int nw = t.n0 + wn * C::WN;
  const int nb0 = min(nw >> 7, p.Nb - 1);
  const __attribute__((address_space(4))) int* sbk =
      (const __attribute__((address_space(4))) int*)((const int*)(const void*)t.sb + (kb >> 2));
  const int sh = 8 * (kb & 3);
  sb_r[0] = (sbk[(int64_t)nb0 * Kb4] >> sh) & 0xff;
  if (!C::SCALE_PER_WAVE) {
    const int nb1 = min(nb0 + 1, p.Nb - 1);
    sb_r[1] = (sbk[(int64_t)nb1 * Kb4] >> sh) & 0xff;
  } else {
    sb_r[1] = sb_r[0];
  }
}

// One slice: acc += 2^(sa - 127) * 2^(sb - 127) * (A_slice . B_slice^T) per
// 16x16 block, in the matrix core.  The weight fragment is the first operand
// (its rows are the block's weight rows, one factor for all of them), the
// activation fragment the second (lane l carries the factor of activation
// row l % 16).
template <class C>
__device__ __forceinline__ void slice_mma_ue8m0(const uint8_t* st, const int (&a_off)[2], const int (&b_off)[2],
                                                const uint8_t* sa_area, int wm, int l16, int kb, const int (&sb)[2],
                                                int tb, f32x4 (&acc)[C::SM][C::SN]) {
  constexpr int SM = C::SM, SN = C::SN;
  const int sh = 8 * (kb & 3);
  int sa[SM];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms) sa[ms] = (*(const int*)(sa_area + (wm * C::WM + ms * 16 + l16) * 4) >> sh) & 0xff;
  // fragments: all of A, B one subtile ahead; the fences keep the compiler
  // from reading further ahead (registers: the 128 accumulators are updated
  // in place only while the live fragments stay this few)
  i32x8 bf = lds_frag(st, b_off[0], b_off[1]);
  i32x8 af[SM];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms) af[ms] = lds_frag(st, a_off[0] + ms * 2048, a_off[1] + ms * 2048);
#pragma unroll
  for (int tt = 0; tt < SN; ++tt) {
    i32x8 bn = bf;
    if (tt + 1 < SN) bn = lds_frag(st, b_off[0] + (tt + 1) * 2048, b_off[1] + (tt + 1) * 2048);
    const int sbt = C::SCALE_PER_WAVE ? sb[0] : (tt < tb ? sb[0] : sb[1]);
#pragma unroll
    for (int ms = 0; ms < SM; ++ms)
      acc[ms][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[ms], acc[ms][tt], 0, 0, 0, sbt, 0, sa[ms]);
    __builtin_amdgcn_sched_barrier(0);
    bf = bn;
  }
}

template <class C, int L, bool KTAIL>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_fp8_ue8m0_kernel(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  constexpr int SM = C::SM, SN = C::SN;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];
#define FG_STAGE(i) (lds + (i) * C::STAGE)
#define FG_SA(i) (lds + C::SA_OFF + (i) * 1024)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int l16 = lane & 15;
  const int kq = lane >> 4;
  const int half = (wm * WM) / 128;  // 128-row half of the tile this wave's rows lie in

  int a_off[2], b_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ra = wm * WM + l16;
    const int rb = BM + wn * WN + l16;
    a_off[h] = ra * 128 + (((2 * kq + h) ^ swz16(ra)) << 4);
    b_off[h] = rb * 128 + (((2 * kq + h) ^ swz16(rb)) << 4);
  }

  const int grid = gridDim.x;
  const int local = xcd_local_id(blockIdx.x, grid);
  const int Kb = p.Kb;

  Work cur;
  int it = 0;
  cur.w = -1;
  if (!(local < p.num_tiles && resolve_big<L, BM, BN>(p, local, cur)))
    advance_big<L, BM, BN>(p, cur, it, local, grid);
  if (cur.w < 0) return;

  int sb_c[2];
  load_sb_ue8m0<C>(p, cur, 0, wn, sb_c);
  issue_slice_loads<C, KTAIL>(p, cur, 0, FG_STAGE(0), FG_SA(0), wave, lane, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[SM][SN];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms)
#pragma unroll
    for (int tt = 0; tt < SN; ++tt) acc[ms][tt] = zero;

  int stage = 0;
  while (cur.w >= 0) {
    Work nxt = cur;
    int it_n = it;
    advance_big<L, BM, BN>(p, nxt, it_n, local, grid);
    const bool active = (L == kContiguous) ? (((cur.half_mask >> half) & 1) != 0)
                                           : (cur.m0 + wm * WM < cur.rows_valid);
    const int tb = second_block_subtile<C>(cur, wn);

    for (int kb = 0; kb < Kb; ++kb) {
      const bool last = kb + 1 == Kb;
      if (!last)
        issue_slice_loads<C, KTAIL>(p, cur, kb + 1, FG_STAGE(stage ^ 1), FG_SA(stage ^ 1), wave, lane, (kb + 1) >> 2);
      else if (nxt.w >= 0)
        issue_slice_loads<C, KTAIL>(p, nxt, 0, FG_STAGE(stage ^ 1), FG_SA(stage ^ 1), wave, lane, 0);
      if (active) slice_mma_ue8m0<C>(FG_STAGE(stage), a_off, b_off, FG_SA(stage), wm, l16, kb, sb_c, tb, acc);
      // the next slice's weight factors (scalar loads) only after the MFMAs,
      // so that the slice's LDS waits can be partial
      int sb_n[2] = {127, 127};
      if (!last)
        load_sb_ue8m0<C>(p, cur, kb + 1, wn, sb_n);
      else if (nxt.w >= 0)
        load_sb_ue8m0<C>(p, nxt, 0, wn, sb_n);

      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      stage ^= 1;
      sb_c[0] = sb_n[0];
      sb_c[1] = sb_n[1];
    }

    // contiguous: a tile whose halves hold different experts runs as two
    // segments on the same accumulators (each half active in its own) and
    // is stored after the second
    if (cur.seg == cur.nseg - 1) {
      float accf[SM][SN][4];
#pragma unroll
      for (int ms = 0; ms < SM; ++ms)
#pragma unroll
        for (int tt = 0; tt < SN; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) accf[ms][tt][r] = acc[ms][tt][r];
      store_tile<C, L>(p, cur, accf, FG_STAGE(stage ^ 1), wave, lane);
#pragma unroll
      for (int ms = 0; ms < SM; ++ms)
#pragma unroll
        for (int tt = 0; tt < SN; ++tt) acc[ms][tt] = zero;
    }
    cur = nxt;
    it = it_n;
  }
  __builtin_amdgcn_s_waitcnt(0);
#undef FG_STAGE
#undef FG_SA
}

}  // namespace fg
