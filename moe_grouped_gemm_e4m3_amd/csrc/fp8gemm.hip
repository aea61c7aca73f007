// fp8gemm.hip -- C ABI of the gfx950 FP8 fine-grained-scaled GEMM library.
//
// Host side: argument validation (nothing is launched on a failed check),
// tile-configuration choice, persistent-grid sizing and asynchronous launch
// on the caller's stream.  The library allocates no device memory: the
// few-row split-K's exchange buffers come in a caller's workspace, and the
// only device data it owns is a result word of the opt-in metadata check.
// The API mirrors the operations of the DeepGEMM digest (GeekNews topic
// 19459): "GEMM arayuzu ve yerlesim kisitlari" (NT dense GEMM, fp32 scale
// factors with a transposed LHS layout), "Dense ve Grouped GEMM" (contiguous
// and masked M-grouped forms) and "Yardimci fonksiyonlar ve ortam
// degiskenleri" (CU cap, contiguous-layout alignment query).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <algorithm>
#include <string>

#include "fp8gemm.h"
#include "cast_kernel.hpp"
#include "gemm_kernel.hpp"
#include "ue8m0_launch.hpp"
#include "skinny_kernel.hpp"
#include "transpose_kernel.hpp"
#include "check_kernel.hpp"

#define FG_TRY(x)                    \
  do {                               \
    fg_status st__ = (x);            \
    if (st__ != FG_OK) return st__;  \
  } while (0)
#define FG_TRY_ST FG_TRY

namespace {

thread_local std::string g_err;
int g_num_cus_cap = 0;

fg_status fail(fg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ceil(x / 128) without int overflow near INT_MAX
int ceil128(int x) { return (int)(((int64_t)x + 127) / 128); }

// Result word of the opt-in metadata check (one copy per device).
__device__ int g_check_word[2];

// Per-device properties, looked up once per device.
struct DeviceInfo {
  int cus = 0;
  bool ok = false;
  int* check_word = nullptr;  // device address of this device's g_check_word
  void* scratch = nullptr;    // device address of this device's scratch array
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

fg_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FG_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FG_EHIP, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev[dev].ok) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(FG_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    g_dev[dev].cus = n;
    g_dev[dev].ok = true;
  }
  *cus = g_dev[dev].cus;
  return FG_OK;
}

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

bool stream_capturing(void* stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

// ---------------------------------------------------------------------------
// Debug mode (environment FG_CHECK_DEVICE=1): before a grouped GEMM is
// launched, a check kernel validates its device-resident row mapping and the
// host reads the result back, which synchronises the stream.  A bad value is
// reported as FG_EINVAL and the GEMM is not launched, so an out-of-range
// expert index never reaches the weight addressing.  Not allowed while the
// stream is being captured.

fg_status check_word_ptr(int** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FG_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FG_EHIP, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev[dev].check_word) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_check_word));
    if (e != hipSuccess) return fail(FG_EHIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_dev[dev].check_word = (int*)ptr;
  }
  *out = g_dev[dev].check_word;
  return FG_OK;
}

// Runs `check` (a launch on `stream` that records into the word) and returns
// the first offending position, or -1.
template <class F>
fg_status run_device_check(void* stream, const char* what, F check, int* bad) {
  *bad = -1;
  if (stream_capturing(stream))
    return fail(FG_EINVAL, "%s: FG_CHECK_DEVICE reads results back and cannot run while the stream is captured", what);
  int* word = nullptr;
  FG_TRY(check_word_ptr(&word));
  hipLaunchKernelGGL(fg::check_reset_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, word);
  check(word);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "%s check launch: %s", what, hipGetErrorString(e));
  int host[2] = {0, 0};
  e = hipMemcpyAsync(host, word, sizeof host, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(FG_EHIP, "%s check read-back: %s", what, hipGetErrorString(e));
  if (host[0] != fg::kCheckNone) *bad = host[0];
  return FG_OK;
}

int32_t read_device_int(const int32_t* p, void* stream) {
  int32_t v = 0;
  if (hipMemcpyAsync(&v, p, 4, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return 0;
  return v;
}

fg_status check_m_indices(const int32_t* idx, int M_total, int G, void* stream, const char* what) {
  if (!env_flag("FG_CHECK_DEVICE")) return FG_OK;
  int bad = -1;
  FG_TRY(run_device_check(stream, what, [&](int* word) {
    hipLaunchKernelGGL(fg::check_m_indices_kernel, dim3((unsigned)(M_total / 128)), dim3(128), 0, (hipStream_t)stream,
                       idx, M_total, G, word);
  }, &bad));
  if (bad >= 0)
    return fail(FG_EINVAL,
                "%s: m_indices[%d] = %d is outside [-1, %d) or differs from the other indices of its 128-row block",
                what, bad, read_device_int(idx + bad, stream), G);
  return FG_OK;
}

fg_status check_masked_m(const int32_t* mask, int G, int M_cap, void* stream, const char* what) {
  if (!env_flag("FG_CHECK_DEVICE")) return FG_OK;
  int bad = -1;
  FG_TRY(run_device_check(stream, what, [&](int* word) {
    hipLaunchKernelGGL(fg::check_masked_m_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, mask, G, M_cap, word);
  }, &bad));
  if (bad >= 0)
    return fail(FG_EINVAL, "%s: masked_m[%d] = %d is outside [0, %d]", what, bad, read_device_int(mask + bad, stream),
                M_cap);
  return FG_OK;
}

// ---------------------------------------------------------------------------
// GEMM configurations.

using CfgDefault = fg::TileCfg<128, 128, 64, 64>;
using CfgBig = fg::BigCfg<256, 256, 4, 2>;
using CfgBig224 = fg::BigCfg<256, 224, 4, 2>;
using CfgBig160 = fg::BigCfg<256, 160, 4, 2>;
// 160-wide tiles with a B staged MN-major (its K rows are 256 bytes)
using CfgBig160Mn = fg::BigCfg<256, 160, 4, 2, 256>;

template <class K>
int occupancy_of(K kernel, int threads, int* cache) {
  if (*cache == 0) {
    int o = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kernel, threads, 0);
    *cache = (e == hipSuccess && o >= 1) ? o : 1;
  }
  return *cache;
}

fg_status launch_grid(int occ, int64_t slots, int64_t* grid) {
  int cus = 0;
  fg_status st = device_cus(&cus);
  if (st != FG_OK) return st;
  if (g_num_cus_cap > 0 && g_num_cus_cap < cus) cus = g_num_cus_cap;
  int64_t g = (int64_t)cus * occ;
  if (g > slots) g = slots;
  if (g < 1) g = 1;
  *grid = g;
  return FG_OK;
}

void print_config(const char* what, const fg::GemmParams& p, int bm, int bn, int threads, int64_t grid, int occ) {
  if (env_flag("FG_PRINT_CONFIGS")) {
    fprintf(stderr, "[fp8gemm] %s M=%d N=%d K=%d G=%d tile=%dx%d threads=%d tiles=%d grid=%lld occ=%d\n", what, p.rows,
            p.N, p.K, p.G, bm, bn, threads, p.num_tiles, (long long)grid, occ);
  }
}

template <class C, int L>
fg_status launch_gemm(fg::GemmParams& p, hipStream_t stream, const char* what) {
  static int occ_cache = 0;
  const int occ = occupancy_of(fg::gemm_fp8_kernel<C, L>, C::THREADS, &occ_cache);
  p.group_m = 8;
  int64_t grid = 0;
  FG_TRY_ST(launch_grid(occ, p.num_tiles, &grid));
  print_config(what, p, C::BM, C::BN, C::THREADS, grid, occ);
  hipLaunchKernelGGL((fg::gemm_fp8_kernel<C, L>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return FG_OK;
}

// Raster band height (tile rows walked before the next tile column).  With
// long K a band's A and B stream through L2 for a long time, and a taller
// band reuses each B column block across more row blocks: measured on the
// M=4096 shapes, 16 rows is 3 % faster at K=16384 and 4-5 % slower at K=1536.
int raster_band(int K) {
  const char* f = getenv("FG_RASTER_BAND");  // tuning
  if (f && atoi(f) > 0) return atoi(f);
  return K >= 8192 ? 16 : 8;
}

// K % 128 != 0 runs a build of the kernel whose last slice clips its loads
// at column K; whole-slice problems keep the build without that code.
template <class C, int L, bool KTAIL, bool TA = false, bool TB = false, bool UE8 = false>
fg_status launch_big_k(fg::GemmParams& p, hipStream_t stream, const char* what) {
  static int occ_cache = 0;
  const int occ = occupancy_of(fg::gemm_fp8_big_kernel<C, L, KTAIL, TA, TB, UE8>, C::THREADS, &occ_cache);
  p.group_m = raster_band(p.K);
  int64_t grid = 0;
  FG_TRY_ST(launch_grid(occ, p.num_tiles, &grid));
  print_config(what, p, C::BM, C::BN, C::THREADS, grid, occ);
  hipLaunchKernelGGL((fg::gemm_fp8_big_kernel<C, L, KTAIL, TA, TB, UE8>), dim3((unsigned)grid), dim3(C::THREADS), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return FG_OK;
}

template <class C, int L, bool UE8 = false>
fg_status launch_big(fg::GemmParams& p, hipStream_t stream, const char* what) {
  return (p.K & 127) ? launch_big_k<C, L, true, false, false, UE8>(p, stream, what)
                     : launch_big_k<C, L, false, false, false, UE8>(p, stream, what);
}

// ---------------------------------------------------------------------------
// Split-K exchange buffers of the few-row kernel, in a workspace the caller
// owns: a fixed counter region (one int per output unit; it must be zero
// before a workspace is first used, and every launch leaves the counters it
// used at zero), then the fp32 partial slots.  The counter region has a fixed
// size so that calls of different shapes on one workspace never read old
// partials as counters.

constexpr int kSkinnyMaxUnits = 1 << 14;
constexpr int64_t kSplitCounterBytes = (int64_t)kSkinnyMaxUnits * 4;  // 64 KiB
constexpr int64_t kSplitPartialMax = (int64_t)8 << 20;                // 8 MiB

struct SplitWs {
  void* base = nullptr;  // counters, then partials
  int64_t bytes = 0;
  bool scratch = false;  // use this device's scratch array (base is looked up)
};

// Scratch of gemm_fp8_nt_noalloc: the split-K workspace of the largest plan
// (64 KiB of counters + 8 MiB of partials), one copy per device, for callers
// that cannot allocate.  Host code never uses the name itself (on the host it
// is a stand-in, not a device address): each device's address is looked up
// once with hipGetSymbolAddress and kept in g_dev.
constexpr int64_t kScratchBytes = kSplitCounterBytes + kSplitPartialMax;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

fg_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FG_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FG_EHIP, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev[dev].scratch) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(FG_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_dev[dev].scratch = ptr;
  }
  *out = g_dev[dev].scratch;
  return FG_OK;
}

// Width of the large kernel's 256-row tile.  The persistent grid runs whole
// tiles in rounds and a tile's time grows with its width, so the width with
// the least (rounds x width) finishes first: narrower tiles fill a last round
// that 256-wide tiles would leave mostly idle (N = 7168 on 16 row tiles:
// 448 tiles of 256 are 1.75 rounds of 256 CUs, 512 tiles of 224 are two
// full ones).  A fixed per-tile cost (prologue and epilogue), worth about 16
// columns, keeps near-ties on the wider tile.  FG_FORCE_BN=256|224|160
// overrides the choice (tuning and tests).
constexpr int kTileCostCols = 16;

int pick_bn(int64_t row_tiles, int N, bool allow_256 = true) {
  const char* f = getenv("FG_FORCE_BN");
  if (f && *f) {
    const int v = atoi(f);
    if (v == 224 || v == 160 || (v == 256 && allow_256)) return v;
  }
  int cus = 0;
  if (device_cus(&cus) != FG_OK) return allow_256 ? 256 : 224;
  if (g_num_cus_cap > 0 && g_num_cus_cap < cus) cus = g_num_cus_cap;
  static const int widths[] = {256, 224, 160};
  int best = 256;
  int64_t best_cost = -1;
  if (!allow_256) best = 224;
  for (int bn : widths) {
    if (bn == 256 && !allow_256) continue;
    const int64_t tiles = row_tiles * ((N + bn - 1) / bn);
    const int64_t rounds = (tiles + cus - 1) / cus;
    const int64_t cost = rounds * (bn + kTileCostCols);
    if (best_cost < 0 || cost < best_cost) {
      best = bn;
      best_cost = cost;
    }
  }
  return best;
}

// Large-kernel launch for `groups` independent [rows, N] outputs (1 for the
// dense and contiguous forms, G for the masked one) with tile width BN.
template <class C, int L, bool UE8 = false>
fg_status launch_big_tiled(fg::GemmParams& p, int64_t groups, hipStream_t stream, const char* what) {
  p.tiles_m = (p.rows + C::BM - 1) / C::BM;
  p.tiles_n = (p.N + C::BN - 1) / C::BN;
  const int64_t slots = groups * p.tiles_m * p.tiles_n;
  if (slots >= ((int64_t)1 << 30)) return fail(FG_EUNSUPPORTED, "too many tiles");
  p.num_tiles = (int)slots;
  return launch_big<C, L, UE8>(p, stream, what);
}

// Dense GEMM with power-of-two factors: the large kernel's tiles (widths as
// pick_bn chooses them) on the scaled MFMA; the kernel is in ue8m0.hip.
// Tile shape of the power-of-two-factor GEMM: the one with the least
// (rounds x tile time).  Tile times are relative, from measurement on the
// M=4096 shapes: 256x224 = 240, 256x160 = 176, 128x256 = 144 (a 128-row tile
// reuses each weight byte half as often, so it costs more than half a
// 256-row one).  FG_FORCE_BN=224|160 keeps the older width-only choice.
// Masked groups count as `groups` stacks of M rows; they take 256-row tiles
// only (rows256_only), so that a group's weights stream once (measured on the
// 16 x 256 decode shapes: the 128-row tile was 6-35 % slower than the best
// 256-row one).  FG_UE8M0_TILE=256x224|256x160|128x256 forces a shape (tuning
// and tests; 256x256 is the promotion kernel's tile, below).
int pick_ue8m0_tile(int M, int N, int64_t groups, bool rows256_only) {
  const char* ft = getenv("FG_UE8M0_TILE");
  if (ft && strcmp(ft, "128x256") == 0) return fg::kUe8m0Tile128x256;
  if (ft && strcmp(ft, "256x224") == 0) return fg::kUe8m0Tile256x224;
  if (ft && strcmp(ft, "256x160") == 0) return fg::kUe8m0Tile256x160;
  const char* f = getenv("FG_FORCE_BN");
  if (f && *f)
    return pick_bn(groups * ((M + 255) / 256), N, false) == 160 ? fg::kUe8m0Tile256x160 : fg::kUe8m0Tile256x224;
  int cus = 0;
  if (device_cus(&cus) != FG_OK) return fg::kUe8m0Tile256x224;
  if (g_num_cus_cap > 0 && g_num_cus_cap < cus) cus = g_num_cus_cap;
  static const int tiles[3] = {fg::kUe8m0Tile256x224, fg::kUe8m0Tile256x160, fg::kUe8m0Tile128x256};
  static const int cost[3] = {240, 176, 144};
  int best = tiles[0];
  int64_t best_cost = -1;
  for (int i = 0; i < (rows256_only ? 2 : 3); ++i) {
    const int bm = fg::ue8m0_tile_bm(tiles[i]), bn = fg::ue8m0_tile_bn(tiles[i]);
    const int64_t n = groups * ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t c = (n + cus - 1) / cus * cost[i];
    if (best_cost < 0 || c < best_cost) {
      best = tiles[i];
      best_cost = c;
    }
  }
  return best;
}

// layout: fg::kDense, kContiguous or kMasked.
// The 256x256 tile with power-of-two factors runs on the fp32-factor large
// kernel, each UE8M0 byte decoded to its fp32 power of two (the scaled-MFMA
// kernel has no 256-wide tile: its accumulators and fragments do not fit the
// registers of two waves per SIMD).  The two agree bit for bit except where
// a slice's dot product is not an fp32 number (more than 24 significant
// bits): the scaled MFMA adds it to the accumulator unrounded, the promotion
// FMA adds its fp32 rounding (1 element of 134 M, by 1 BF16 ulp, on the
// contiguous MoE workload).  The masked GEMM takes it where the
// plan's width is 256 (one weight stream per tile of 256 columns; measured at
// 16 x 256 rows, N = 4096, K = 7168: 130 against 161 us); the MFMA-bound forms
// keep the scaled MFMA, which needs no promotion (the promotion kernel was
// level at N = 4096 and slower elsewhere).  FG_UE8M0_TILE=256x256 forces it,
// another FG_UE8M0_TILE value forces the scaled-MFMA kernel.
bool ue8m0_on_promotion_kernel(bool by_default) {
  const char* ft = getenv("FG_UE8M0_TILE");
  if (ft && *ft) return strcmp(ft, "256x256") == 0;
  return by_default;
}

fg_status launch_ue8m0(fg::GemmParams& p, int tile, int64_t groups, int layout, hipStream_t stream,
                       const char* what) {
  static int occ_cache[2][4][3] = {};
  const bool ktail = (p.K & 127) != 0;
  int& occ = occ_cache[ktail ? 1 : 0][layout & 3][tile];
  if (occ == 0) occ = fg::ue8m0_occupancy(tile, layout, ktail);
  const int bm = fg::ue8m0_tile_bm(tile), bn = fg::ue8m0_tile_bn(tile);
  p.tiles_m = (p.rows + bm - 1) / bm;
  p.tiles_n = (p.N + bn - 1) / bn;
  const int64_t slots = groups * p.tiles_m * p.tiles_n;
  if (slots >= ((int64_t)1 << 30)) return fail(FG_EUNSUPPORTED, "too many tiles");
  p.num_tiles = (int)slots;
  p.group_m = raster_band(p.K);
  int64_t grid = 0;
  FG_TRY_ST(launch_grid(occ, p.num_tiles, &grid));
  print_config(what, p, bm, bn, 512, grid, occ);
  const hipError_t e = fg::ue8m0_launch(p, tile, layout, grid, stream);
  if (e != hipSuccess) return fail(FG_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return FG_OK;
}

template <int L, bool UE8 = false>
fg_status launch_big_width(fg::GemmParams& p, int64_t groups, hipStream_t stream, const char* what) {
  const int64_t row_tiles = groups * ((p.rows + CfgBig::BM - 1) / CfgBig::BM);
  switch (pick_bn(row_tiles, p.N)) {
    case 224: return launch_big_tiled<CfgBig224, L, UE8>(p, groups, stream, what);
    case 160: return launch_big_tiled<CfgBig160, L, UE8>(p, groups, stream, what);
    default: return launch_big_tiled<CfgBig, L, UE8>(p, groups, stream, what);
  }
}

// Tiles the large kernel would have; it is used when they cover at least
// half of the device, otherwise the 128x128 kernel spreads the work wider.
// FG_FORCE_CONFIG=big|small overrides the choice (tuning and tests).
bool prefer_big(int64_t big_tiles) {
  const char* f = getenv("FG_FORCE_CONFIG");
  if (f && strcmp(f, "big") == 0) return true;
  if (f && strcmp(f, "small") == 0) return false;
  int cus = 0;
  if (device_cus(&cus) != FG_OK) return true;
  return big_tiles * 2 >= cus;
}

// ---------------------------------------------------------------------------
// Skinny kernel (dense, M <= 128).  The plan picks the activation fragments
// per workgroup (64 rows; more rows go to a second row part), the column-tile
// width (16 CF weight rows per workgroup) and the K split.  Every CU reads
// the activations of its K range again, so wider tiles read fewer bytes per
// weight byte; a K split brings the workgroup count up to the CU count but
// adds an exchange of fp32 partials at the end, whose latency grows with the
// number of splits.  Measured on MI355X on the decode shapes (M = 64, 128;
// N = 2112, 4096, 7168; K = 7168, 2048), the best plans are: 32-column tiles
// split at most three ways while that fills three quarters of the CUs in
// one round, else 64-column tiles split at most three ways (when that gives
// more workgroups), one round where possible.
// The plan depends only on the shape, the device's CU count and whether the
// call brings split-K buffers (`split_ok`), never on earlier calls or on
// stream capture, so a call's summation order (and its bits) is fixed by its
// arguments.  FG_SKINNY="CF,SPLITS[,MF]" overrides the choice (tuning and
// tests; MF = 8 keeps 128 rows in one part, with CF = 1: the LDS ring of a
// wider tile would not fit).

struct SkinnyPlan {
  int mf = 0, cf = 0, splits = 1, parts = 1;
  int64_t units = 0;
  int64_t partial_bytes() const { return splits > 1 ? (int64_t)splits * units * mf * cf * 1024 : 0; }
};

bool plan_skinny(int M, int N, int K, int64_t lda, int64_t ld_sa, int cus, bool split_ok, SkinnyPlan* out) {
  if (M > 128 || K <= 0) return false;
  const int Kb = ceil128(K);
  SkinnyPlan pl;
  // 64-row activation fragments; more rows are spread over row parts
  pl.mf = 4;
  const char* f = getenv("FG_SKINNY");
  int cf_env = 0, sp_env = 0, mf_env = 0;
  const int nenv = (f && *f) ? sscanf(f, "%d,%d,%d", &cf_env, &sp_env, &mf_env) : 0;
  if (nenv == 3 && (mf_env == 4 || (mf_env == 8 && M > 64))) pl.mf = mf_env;
  pl.parts = (M + 16 * pl.mf - 1) / (16 * pl.mf);
  // 32-bit lane offsets
  if ((int64_t)16 * pl.mf * lda + K >= ((int64_t)1 << 31)) return false;
  if (((int64_t)(Kb - 1) * ld_sa + M) * 4 >= ((int64_t)1 << 31)) return false;
  auto units_of = [&](int cf) { return (int64_t)((N + 16 * cf - 1) / (16 * cf)) * pl.parts; };
  auto fits = [&](int cf, int sp) {
    const int64_t units = units_of(cf);
    return sp == 1 || (units <= kSkinnyMaxUnits && (int64_t)sp * units * pl.mf * cf * 1024 <= kSplitPartialMax);
  };
  if (nenv >= 2 && (cf_env == 1 || cf_env == 2 || cf_env == 4) && (pl.mf == 4 || cf_env == 1) && sp_env >= 1 &&
      (sp_env == 1 || split_ok)) {
    if (!fits(cf_env, sp_env)) return false;
    pl.cf = cf_env;
    pl.splits = sp_env;
    pl.units = units_of(pl.cf);
    *out = pl;
    return true;
  }
  // splits (up to three, with at least one K slice per wave) that keep the
  // launch in one round of the CUs
  const int smax = split_ok ? 3 : 1;
  auto splits_for = [&](int cf) {
    const int64_t u = units_of(cf);
    int sp = 1;
    while (sp < smax && u * (sp + 1) <= cus && Kb >= 4 * (sp + 1) && fits(cf, sp + 1)) ++sp;
    return sp;
  };
  const int64_t u2 = units_of(2), u4 = units_of(4);
  const int s2 = splits_for(2), s4 = splits_for(4);
  int sp;
  if (pl.mf == 8) {
    pl.cf = 1;  // 128-row fragments (FG_SKINNY only): the one width whose LDS ring fits
    sp = splits_for(1);
  } else if (u2 <= cus && (u2 * s2 * 4 >= (int64_t)cus * 3 || u4 * s4 <= u2 * s2)) {
    pl.cf = 2;
    sp = s2;
  } else {
    pl.cf = 4;
    sp = s4;
  }
  pl.units = units_of(pl.cf);
  pl.splits = sp;
  *out = pl;
  return pl.cf > 0;
}

template <int MF, int CF, bool ADD_C>
fg_status launch_skinny_cfg(fg::GemmParams& p, int splits, int parts, hipStream_t stream, const char* what) {
  using C = fg::SkinnyCfg<MF, CF>;
  const int64_t tiles = (p.N + C::COLS - 1) / C::COLS;
  const int64_t grid = tiles * parts * splits;
  if (grid >= ((int64_t)1 << 31)) return fail(FG_EUNSUPPORTED, "too many column tiles");
  p.num_tiles = (int)tiles;
  if (env_flag("FG_PRINT_CONFIGS"))
    fprintf(stderr, "[fp8gemm] %s M=%d N=%d K=%d skinny rows=%d parts=%d cols=%d splits=%d grid=%lld\n", what,
            p.rows, p.N, p.K, C::ROWS, parts, C::COLS, splits, (long long)grid);
  hipLaunchKernelGGL((fg::gemm_fp8_skinny_kernel<C, ADD_C>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, p, splits,
                     parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return FG_OK;
}

template <bool ADD_C>
fg_status launch_skinny(fg::GemmParams& p, const SkinnyPlan& pl, const SplitWs* ws, hipStream_t stream,
                        const char* what) {
  if (pl.splits > 1) {
    // the plan only splits when the call brought a workspace
    const int64_t need = kSplitCounterBytes + pl.partial_bytes();
    if (!ws || pl.units > kSkinnyMaxUnits) return fail(FG_EINVAL, "%s: the K split needs a workspace", what);
    void* base = ws->base;
    if (ws->scratch) {
      if (need > kScratchBytes)
        return fail(FG_EUNSUPPORTED, "%s: the plan needs %lld bytes of scratch, above the %lld this entry point has",
                    what, (long long)need, (long long)kScratchBytes);
      FG_TRY(scratch_ptr(&base));
    } else if (ws->bytes < need) {
      return fail(FG_EINVAL, "%s: workspace of %lld bytes is below the %lld this call needs", what,
                  (long long)ws->bytes, (long long)need);
    }
    p.ws_counters = (int*)base;
    p.ws_partials = (float*)((uint8_t*)base + kSplitCounterBytes);
    if (ws->scratch) {
      // a shared scratch keeps whatever an earlier call left: start from zero
      hipLaunchKernelGGL(fg::zero_ints_kernel, dim3((unsigned)((pl.units + 255) / 256)), dim3(256), 0, stream,
                         p.ws_counters, (int)pl.units);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(FG_EHIP, "%s counter clear launch: %s", what, hipGetErrorString(e));
    }
  }
#define FG_SKINNY_CASE(MF, CF) \
  if (pl.mf == MF && pl.cf == CF) return launch_skinny_cfg<MF, CF, ADD_C>(p, pl.splits, pl.parts, stream, what);
  FG_SKINNY_CASE(4, 1) FG_SKINNY_CASE(4, 2) FG_SKINNY_CASE(4, 4)
  FG_SKINNY_CASE(8, 1)
#undef FG_SKINNY_CASE
  return fail(FG_EUNSUPPORTED, "%s: no skinny configuration", what);
}

// Split-K partial bytes the few-row plan takes for (M, N, K) with
// buffers available; 0 when it does not split (or does not apply).
int64_t nt_split_partial_bytes(int M, int N, int K, int64_t lda, int64_t ld_sa) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const char* force = getenv("FG_FORCE_CONFIG");
  if (force && (strcmp(force, "big") == 0 || strcmp(force, "small") == 0)) return 0;
  int cus = 0;
  if (device_cus(&cus) != FG_OK) return -1;
  SkinnyPlan pl;
  if (!plan_skinny(M, N, K, lda, ld_sa, cus, true, &pl)) return 0;
  return pl.partial_bytes();
}

fg_status check_ld(int64_t ld, int64_t row, int64_t mult, const char* name) {
  if (ld < row) return fail(FG_EINVAL, "%s=%lld is smaller than the row length %lld", name, (long long)ld, (long long)row);
  if (ld % mult) return fail(FG_EALIGN, "%s=%lld is not a multiple of %lld", name, (long long)ld, (long long)mult);
  return FG_OK;
}


fg_status check_ptr(const void* p, uintptr_t align, const char* name) {
  if (!p) return fail(FG_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(FG_EALIGN, "%s is not %u-byte aligned", name, (unsigned)align);
  return FG_OK;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;
// Buffer offsets inside a tile are 32-bit: 256 rows of up to 4 MiB.
constexpr int64_t kMaxLd = (int64_t)1 << 22;

fg_status check_row_bytes(int64_t lda, int64_t ldb) {
  if (lda > kMaxLd || ldb > kMaxLd) return fail(FG_EUNSUPPORTED, "operand rows above 4 MiB");
  return FG_OK;
}


// Validation and dispatch shared by D = A B^T (kDense) and D = C + A B^T
// (kDenseC, C already checked and set in the parameters).
// `ws`: split-K buffers for the few-row kernel, or NULL (no K split).
template <int L>
fg_status dense_nt(fg::GemmParams& p, const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                   const uint8_t* B, int64_t ldb, const float* sb, uint16_t* D, int64_t ldd, int M, int N, int K,
                   const SplitWs* ws, void* stream, const char* what) {
  if (M < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || N == 0) return FG_OK;
  if (M > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M or N above 2^30");
  FG_TRY(check_ptr(D, 2, "D"));
  FG_TRY(check_ld(ldd, N, 1, "ldd"));
  if (K > 0) {
    FG_TRY(check_ptr(A, 16, "A"));
    FG_TRY(check_ptr(B, 16, "B"));
    FG_TRY(check_ptr(sa, 4, "sa"));
    FG_TRY(check_ptr(sb, 4, "sb"));
    FG_TRY(check_ld(lda, K, 16, "lda"));
    FG_TRY(check_ld(ldb, K, 16, "ldb"));
    FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
    FG_TRY(check_row_bytes(lda, ldb));
  }
  p.A = A; p.lda = lda; p.sa = sa; p.ld_sa = ld_sa; p.B = B; p.ldb = ldb; p.sb = sb; p.D = D; p.ldd = ldd;
  p.rows = M; p.N = N; p.K = K; p.G = 1; p.Kb = ceil128(K); p.Nb = ceil128(N);
  if (p.ld_sb == 0) p.ld_sb = p.Kb;
  if (K > 0) {
    // few activation rows: the weight-streaming kernel
    const char* force = getenv("FG_FORCE_CONFIG");
    if (!(force && (strcmp(force, "big") == 0 || strcmp(force, "small") == 0))) {
      int all_cus = 0;
      FG_TRY(device_cus(&all_cus));  // the plan (and so the summation order) does not depend on the CU cap
      SkinnyPlan pl;
      if (plan_skinny(M, N, K, lda, ld_sa, all_cus, ws != nullptr, &pl))
        return launch_skinny<L == fg::kDenseC>(p, pl, ws, (hipStream_t)stream, what);
    }
    using C = CfgBig;
    const int64_t tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
    if (prefer_big(tm * tn) && tm * tn < ((int64_t)1 << 30)) {
      p.tiles_m = (int)tm;
      p.tiles_n = (int)tn;
      p.num_tiles = (int)(tm * tn);
      return launch_big_width<L>(p, 1, (hipStream_t)stream, what);
    }
  }
  using C = CfgDefault;
  p.tiles_m = (M + C::BM - 1) / C::BM;
  p.tiles_n = (N + C::BN - 1) / C::BN;
  p.num_tiles = p.tiles_m * p.tiles_n;
  return launch_gemm<C, L>(p, (hipStream_t)stream, what);
}
// ---------------------------------------------------------------------------
// Storage layouts NN / TN / TT: an operand stored MN-major ([K, M] or [K, N])
// is transposed into the caller's workspace, K-major, and the NT kernels run
// on the copy.  Workspace: the copy of A (M*K bytes) then the copy of B
// (N*K bytes), each rounded up to 256 bytes.

int64_t ws_round(int64_t x) { return (x + 255) / 256 * 256; }

int64_t layout_ws_bytes(bool ta, bool tb, int M, int N, int K) {
  return (ta ? ws_round((int64_t)M * K) : 0) + (tb ? ws_round((int64_t)N * K) : 0);
}

// out [cols, rows] = in [rows, cols]^T, bytes.
fg_status launch_transpose(const uint8_t* in, int64_t ld_in, uint8_t* out, int64_t ld_out, int rows, int cols,
                           hipStream_t stream, const char* what) {
  if (rows == 0 || cols == 0) return FG_OK;
  const int64_t gx = (cols + fg::kTrTile - 1) / fg::kTrTile, gy = (rows + fg::kTrTile - 1) / fg::kTrTile;
  if (gy > 65535) return fail(FG_EUNSUPPORTED, "%s: %d rows to transpose is above %d", what, rows, 65535 * 128);
  if (env_flag("FG_PRINT_CONFIGS"))
    fprintf(stderr, "[fp8gemm] %s transpose %dx%d grid=%lldx%lld\n", what, rows, cols, (long long)gx, (long long)gy);
  hipLaunchKernelGGL(fg::transpose_u8_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, in, ld_in, out,
                     ld_out, rows, cols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "%s transpose launch: %s", what, hipGetErrorString(e));
  return FG_OK;
}

// An MN-major operand ([K, M] or [K, N]) of `ext` columns can be staged by
// the large kernel as stored when its rows start on 16-byte boundaries and
// end on one (the kernel reads whole 16-byte chunks up to column ext).
bool mn_direct(const void* x, int64_t ld, int ext) {
  return x && aligned(x, 16) && ld % 16 == 0 && ld <= kMaxLd && ext % 16 == 0;
}

// Given a workspace, whether to stage the MN-major operands as stored anyway
// (their alignment permitting): where the large kernel's 256x256 tiles keep
// the CUs at least three quarters busy over their rounds.  Measured on
// MI355X at M = 4096, N = 4096, 7168 and 24576: level with or 2-9 % faster
// than copying them first (the copies cost a pass over both operands); at
// N = 2112 (144 such tiles on 256 CUs; the copy-free path then runs the NT
// plan's 224 tiles of 256x160) the copies were still 2-7 % faster.
// FG_LAYOUT_COPY=1 keeps the copies, =0 skips them wherever the operands
// allow (tests and tuning).
bool layout_copy_free(int M, int N) {
  const char* f = getenv("FG_LAYOUT_COPY");
  if (f && *f) return strcmp(f, "0") == 0;
  int cus = 0;
  if (device_cus(&cus) != FG_OK) return false;
  if (g_num_cus_cap > 0 && g_num_cus_cap < cus) cus = g_num_cus_cap;
  const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  const int64_t rounds = (tiles + cus - 1) / cus;
  return tiles * 4 >= rounds * cus * 3;
}

// The large kernel on the operands as stored (TA / TB: MN-major).
template <class Cfg, bool TA, bool TB>
fg_status launch_layout_direct_w(fg::GemmParams& p, hipStream_t stream, const char* what) {
  p.tiles_m = (p.rows + Cfg::BM - 1) / Cfg::BM;
  p.tiles_n = (p.N + Cfg::BN - 1) / Cfg::BN;
  const int64_t slots = (int64_t)p.tiles_m * p.tiles_n;
  if (slots >= ((int64_t)1 << 30)) return fail(FG_EUNSUPPORTED, "too many tiles");
  p.num_tiles = (int)slots;
  // K tails matter only to a K-major operand (an MN-major one reads rows past K as zeros)
  const bool ktail = !(TA && TB) && (p.K & 127) != 0;
  if (p.Cin)
    return ktail ? launch_big_k<Cfg, fg::kDenseC, true, TA, TB>(p, stream, what)
                 : launch_big_k<Cfg, fg::kDenseC, false, TA, TB>(p, stream, what);
  return ktail ? launch_big_k<Cfg, fg::kDense, true, TA, TB>(p, stream, what)
               : launch_big_k<Cfg, fg::kDense, false, TA, TB>(p, stream, what);
}

// 256x256 tiles, or 256x160 where the NT plan takes those (the 256-wide
// tiles would leave many CUs idle).  Measured on MI355X at 4096 x 2112 x 7168,
// copy-free: NN 110 -> 100 us, TN 109 -> 96, TT 101 -> 86.  The 224-wide
// tiles the NT plan takes at N = 7168 were mixed here (NN 8 % slower at
// K = 16384, TT 2-4 % faster), so those shapes keep the 256-wide tiles.
// FG_LAYOUT_BN=256 keeps the 256-wide tiles everywhere (tuning).
template <bool TA, bool TB>
fg_status launch_layout_direct(fg::GemmParams& p, hipStream_t stream, const char* what) {
  const char* f = getenv("FG_LAYOUT_BN");
  const bool narrow = !(f && atoi(f) == 256) && pick_bn((p.rows + 255) / 256, p.N) == 160;
  if (narrow) {
    if constexpr (TB)
      return launch_layout_direct_w<CfgBig160Mn, TA, TB>(p, stream, what);
    else
      return launch_layout_direct_w<CfgBig160, TA, TB>(p, stream, what);
  }
  return launch_layout_direct_w<CfgBig, TA, TB>(p, stream, what);
}

template <bool TA, bool TB>
fg_status gemm_layout(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                      const float* sb, const float* C, int64_t ldc, uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream, const char* what) {
  g_err.clear();
  if (M < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || N == 0) return FG_OK;
  if (M > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M or N above 2^30");
  if (C) FG_TRY(check_ptr(C, 4, "C"));
  if (C) FG_TRY(check_ld(ldc, N, 1, "ldc"));
  const uint8_t* a = A;
  const uint8_t* b = B;
  // Without a workspace the large kernel stages the MN-major operands as
  // stored and the transposing LDS reads turn them into MFMA fragments; with
  // one it does so where the plan prefers it (the workspace, checked as for
  // the copies so that what a call accepts does not depend on the plan, is
  // then left untouched).
  bool direct = K > 0 && (TA || TB) && workspace_bytes == 0;
  if (K > 0 && (TA || TB) && workspace_bytes > 0 && K <= kMaxLd && (!TA || mn_direct(A, lda, M)) &&
      (!TB || mn_direct(B, ldb, N)) && layout_copy_free(M, N)) {
    const int64_t need = layout_ws_bytes(TA, TB, M, N, K);
    if (workspace_bytes < need)
      return fail(FG_EINVAL, "%s: workspace of %lld bytes is below the %lld this call needs", what,
                  (long long)workspace_bytes, (long long)need);
    FG_TRY(check_ptr(workspace, 16, "workspace"));
    direct = true;
  }
  if (direct) {
    if ((TA && !mn_direct(A, lda, M)) || (TB && !mn_direct(B, ldb, N)))
      return fail(FG_EALIGN,
                  "%s without a workspace: an MN-major operand needs 16-byte aligned rows, a row stride and a column "
                  "count that are multiples of 16",
                  what);
    if (TA) FG_TRY(check_ld(lda, M, 1, "lda"));
    if (TB) FG_TRY(check_ld(ldb, N, 1, "ldb"));
    if (K > kMaxLd) return fail(FG_EUNSUPPORTED, "K=%d above 4 Mi rows", K);
    FG_TRY(check_ptr(D, 2, "D"));
    FG_TRY(check_ld(ldd, N, 1, "ldd"));
    FG_TRY(check_ptr(sa, 4, "sa"));
    FG_TRY(check_ptr(sb, 4, "sb"));
    FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
    if (!TA) {
      FG_TRY(check_ptr(A, 16, "A"));
      FG_TRY(check_ld(lda, K, 16, "lda"));
    }
    if (!TB) {
      FG_TRY(check_ptr(B, 16, "B"));
      FG_TRY(check_ld(ldb, K, 16, "ldb"));
    }
    FG_TRY(check_row_bytes(lda, ldb));
    fg::GemmParams p{};
    p.A = A; p.lda = lda; p.sa = sa; p.ld_sa = ld_sa; p.B = B; p.ldb = ldb; p.sb = sb; p.D = D; p.ldd = ldd;
    p.Cin = C; p.ldc = ldc;
    p.rows = M; p.N = N; p.K = K; p.G = 1; p.Kb = ceil128(K); p.Nb = ceil128(N); p.ld_sb = p.Kb;
    return launch_layout_direct<TA, TB>(p, (hipStream_t)stream, what);
  }
  if (K > 0 && (TA || TB)) {
    if (TA) {
      FG_TRY(check_ptr(A, 1, "A"));
      FG_TRY(check_ld(lda, M, 1, "lda"));
    }
    if (TB) {
      FG_TRY(check_ptr(B, 1, "B"));
      FG_TRY(check_ld(ldb, N, 1, "ldb"));
    }
    if (K > kMaxLd) return fail(FG_EUNSUPPORTED, "K=%d: transposed rows above 4 MiB", K);
    const int64_t need = layout_ws_bytes(TA, TB, M, N, K);
    if (workspace_bytes < need)
      return fail(FG_EINVAL, "%s: workspace of %lld bytes is below the %lld this call needs", what,
                  (long long)workspace_bytes, (long long)need);
    FG_TRY(check_ptr(workspace, 16, "workspace"));
    uint8_t* ws = (uint8_t*)workspace;
    if (TA) {
      FG_TRY(launch_transpose(A, lda, ws, K, K, M, (hipStream_t)stream, what));
      a = ws;
      lda = K;
      ws += ws_round((int64_t)M * K);
    }
    if (TB) {
      FG_TRY(launch_transpose(B, ldb, ws, K, K, N, (hipStream_t)stream, what));
      b = ws;
      ldb = K;
    }
  }
  fg::GemmParams p{};
  if (C) {
    p.Cin = C;
    p.ldc = ldc;
    return dense_nt<fg::kDenseC>(p, a, lda, sa, ld_sa, b, ldb, sb, D, ldd, M, N, K, nullptr, stream, what);
  }
  return dense_nt<fg::kDense>(p, a, lda, sa, ld_sa, b, ldb, sb, D, ldd, M, N, K, nullptr, stream, what);
}
}  // namespace

// Lanes per 128-column group of the per-token cast: 8 (four fp32 or two bf16
// 16-byte loads per lane) when the cast has at least kCastWideGroups groups,
// else 16, which gives small casts twice the waves to hide load latency (at
// 256 x 7168 the 8-lane split was 10 % slower, from 4096 x 1536 up 5-16 %
// faster).
constexpr int64_t kCastWideGroups = 32768;

template <bool UE8M0, typename T>
static fg_status launch_cast_per_token(const T* x, int64_t ldx, uint8_t* q, void* sa, int64_t ld_sa, int M, int K,
                                       void* stream, const char* name) {
  const int64_t groups = (int64_t)M * (ceil128(K));
  const int lpg = groups >= kCastWideGroups ? 8 : 16;
  const int64_t lanes = groups * lpg;
  const int64_t blocks = (lanes + 255) / 256;
  if (blocks > 0x7fffffff) return fail(FG_EUNSUPPORTED, "input too large");
  if (lpg == 8)
    hipLaunchKernelGGL((fg::cast_per_token_kernel<UE8M0, T, 8>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, x, ldx, q, sa, ld_sa, M, K, lanes);
  else
    hipLaunchKernelGGL((fg::cast_per_token_kernel<UE8M0, T, 16>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, x, ldx, q, sa, ld_sa, M, K, lanes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "%s launch: %s", name, hipGetErrorString(e));
  return FG_OK;
}

extern "C" {

int64_t fg_layout_workspace_bytes(const char* layout, int M, int N, int K) {
  if (!layout || M < 0 || N < 0 || K < 0) return -1;
  if (M > kMaxDim || N > kMaxDim || K > kMaxLd) return -1;  // sizes the calls reject
  if (strcmp(layout, "nt") == 0) return 0;
  if (strcmp(layout, "nn") == 0) return layout_ws_bytes(false, true, M, N, K);
  if (strcmp(layout, "tn") == 0) return layout_ws_bytes(true, true, M, N, K);
  if (strcmp(layout, "tt") == 0) return layout_ws_bytes(true, false, M, N, K);
  return -1;
}

fg_status gemm_fp8_nn(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                      const float* sb, const float* C, int64_t ldc, uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_layout<false, true>(A, lda, sa, ld_sa, B, ldb, sb, C, ldc, D, ldd, M, N, K, workspace, workspace_bytes,
                                  stream, "gemm_fp8_nn");
}

fg_status gemm_fp8_tn(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                      const float* sb, const float* C, int64_t ldc, uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_layout<true, true>(A, lda, sa, ld_sa, B, ldb, sb, C, ldc, D, ldd, M, N, K, workspace, workspace_bytes,
                                 stream, "gemm_fp8_tn");
}

fg_status gemm_fp8_tt(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                      const float* sb, const float* C, int64_t ldc, uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_layout<true, false>(A, lda, sa, ld_sa, B, ldb, sb, C, ldc, D, ldd, M, N, K, workspace, workspace_bytes,
                                  stream, "gemm_fp8_tt");
}

int64_t fg_k_grouped_workspace_bytes(int M, int N, int64_t K_total) {
  if (M < 0 || N < 0 || K_total < 0) return -1;
  if (M > kMaxDim || N > kMaxDim || K_total > kMaxLd) return -1;  // sizes the call rejects
  return ws_round((int64_t)M * K_total) + ws_round((int64_t)N * K_total);
}

fg_status gemm_fp8_k_grouped_tn_contiguous(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                                           const uint8_t* B, int64_t ldb, const float* sb, const int* ks, int G,
                                           const float* C, uint16_t* D, int M, int N, void* workspace,
                                           int64_t workspace_bytes, void* stream) {
  const char* what = "gemm_fp8_k_grouped_tn_contiguous";
  g_err.clear();
  if (G <= 0) return fail(FG_EINVAL, "G=%d", G);
  if (M < 0 || N < 0) return fail(FG_EINVAL, "negative size M=%d N=%d", M, N);
  if (!ks) return fail(FG_EINVAL, "ks is NULL");
  int64_t K_total = 0;
  for (int g = 0; g < G; ++g) {
    if (ks[g] < 0) return fail(FG_EINVAL, "ks[%d]=%d is negative", g, ks[g]);
    if (ks[g] % 128) return fail(FG_EALIGN, "ks[%d]=%d is not a multiple of 128", g, ks[g]);
    K_total += ks[g];
  }
  if (M == 0 || N == 0) return FG_OK;
  if (M > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M or N above 2^30");
  if (K_total > kMaxLd) return fail(FG_EUNSUPPORTED, "K_total=%lld: transposed rows above 4 MiB", (long long)K_total);
  if ((int64_t)G * M * N >= ((int64_t)1 << 62) / 4) return fail(FG_EUNSUPPORTED, "output too large");
  FG_TRY(check_ptr(D, 2, "D"));
  if (C) FG_TRY(check_ptr(C, 4, "C"));
  const int Kbt = (int)(K_total / 128);
  hipStream_t st = (hipStream_t)stream;
  // With a workspace both operands are transposed K-major into it (the
  // faster path: the K-major staging streams at the NT kernel's rate);
  // without one the kernel stages them as stored.
  const bool mn = workspace_bytes == 0;
  if (K_total > 0) {
    FG_TRY(check_ptr(sa, 4, "sa"));
    FG_TRY(check_ptr(sb, 4, "sb"));
    FG_TRY(check_ld(lda, M, 1, "lda"));
    FG_TRY(check_ld(ldb, N, 1, "ldb"));
    FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
    if (mn) {
      if (!mn_direct(A, lda, M) || !mn_direct(B, ldb, N))
        return fail(FG_EALIGN,
                    "%s without a workspace: A and B need 16-byte aligned rows, row strides and M, N that are "
                    "multiples of 16",
                    what);
    } else {
      FG_TRY(check_ptr(A, 1, "A"));
      FG_TRY(check_ptr(B, 1, "B"));
      const int64_t need = fg_k_grouped_workspace_bytes(M, N, K_total);
      if (workspace_bytes < need)
        return fail(FG_EINVAL, "%s: workspace of %lld bytes is below the %lld this call needs", what,
                    (long long)workspace_bytes, (long long)need);
      FG_TRY(check_ptr(workspace, 16, "workspace"));
    }
  }
  // groups without K rows: D[g] = C[g] (or 0)
  for (int g = 0; g < G; ++g) {
    if (ks[g] > 0) continue;
    const int64_t n = (int64_t)M * N;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(fg::fill_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, D + (int64_t)g * M * N,
                       C ? C + (int64_t)g * M * N : nullptr, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FG_EHIP, "%s fill launch: %s", what, hipGetErrorString(e));
  }
  if (K_total == 0) return FG_OK;
  fg::GemmParams p{};
  fg::KGroups kg{};
  if (mn) {
    p.A = A; p.lda = lda; p.B = B; p.ldb = ldb;
    kg.a_step = 128 * lda;
    kg.b_step = 128 * ldb;
  } else {
    uint8_t* ws = (uint8_t*)workspace;
    FG_TRY(launch_transpose(A, lda, ws, K_total, (int)K_total, M, st, what));
    FG_TRY(launch_transpose(B, ldb, ws + ws_round((int64_t)M * K_total), K_total, (int)K_total, N, st, what));
    p.A = ws; p.lda = K_total; p.B = ws + ws_round((int64_t)M * K_total); p.ldb = K_total;
    kg.a_step = 128;
    kg.b_step = 128;
  }
  using Cfg = CfgBig;
  p.sa = sa; p.ld_sa = ld_sa; p.sb = sb; p.ld_sb = Kbt;
  p.D = D; p.ldd = N; p.Cin = C; p.ldc = N;
  p.rows = M; p.N = N; p.K = (int)K_total; p.G = G; p.Kb = Kbt; p.Nb = ceil128(N);
  p.tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
  p.tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
  static int occ_mn = 0, occ_k = 0;
  const int occ = mn ? occupancy_of(fg::gemm_fp8_k_grouped_kernel<Cfg, true>, Cfg::THREADS, &occ_mn)
                     : occupancy_of(fg::gemm_fp8_k_grouped_kernel<Cfg, false>, Cfg::THREADS, &occ_k);
  // one persistent launch per run of at most kMaxKGroups groups with K rows
  int64_t kb = 0;
  for (int g0 = 0; g0 < G;) {
    kg.n = 0;
    int g = g0;
    for (; g < G && kg.n < fg::kMaxKGroups; ++g) {
      if (ks[g] > 0) {
        kg.g[kg.n] = g;
        kg.kb0[kg.n] = (int)kb;
        ++kg.n;
      }
      kb += ks[g] / 128;
    }
    kg.kb0[kg.n] = (int)kb;
    g0 = g;
    if (kg.n == 0) continue;
    const int64_t slots = (int64_t)kg.n * p.tiles_m * p.tiles_n;
    if (slots >= ((int64_t)1 << 30)) return fail(FG_EUNSUPPORTED, "too many tiles");
    p.num_tiles = (int)slots;
    p.group_m = raster_band((int)((kg.kb0[kg.n] - kg.kb0[0]) * 128 / kg.n));
    int64_t grid = 0;
    FG_TRY(launch_grid(occ, p.num_tiles, &grid));
    print_config(what, p, Cfg::BM, Cfg::BN, Cfg::THREADS, grid, occ);
    if (mn)
      hipLaunchKernelGGL((fg::gemm_fp8_k_grouped_kernel<Cfg, true>), dim3((unsigned)grid), dim3(Cfg::THREADS), 0, st,
                         p, kg);
    else
      hipLaunchKernelGGL((fg::gemm_fp8_k_grouped_kernel<Cfg, false>), dim3((unsigned)grid), dim3(Cfg::THREADS), 0,
                         st, p, kg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FG_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  }
  return FG_OK;
}

fg_status gemm_fp8_nt(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                      const float* sb, uint16_t* D, int64_t ldd, int M, int N, int K, void* stream) {
  g_err.clear();
  fg::GemmParams p{};
  return dense_nt<fg::kDense>(p, A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, nullptr, stream, "gemm_fp8_nt");
}

int64_t fg_nt_workspace_max_bytes(void) { return kSplitCounterBytes + kSplitPartialMax; }

int64_t fg_nt_workspace_bytes(int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return -1;
  const int64_t part = nt_split_partial_bytes(M, N, K, ((int64_t)K + 15) / 16 * 16, ((int64_t)M + 3) / 4 * 4);
  if (part < 0) return -1;
  return part > 0 ? kSplitCounterBytes + part : 0;
}

fg_status gemm_fp8_nt_ws(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B,
                         int64_t ldb, const float* sb, uint16_t* D, int64_t ldd, int M, int N, int K, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  const char* what = "gemm_fp8_nt_ws";
  g_err.clear();
  if (workspace_bytes < 0) return fail(FG_EINVAL, "%s: workspace_bytes=%lld is negative", what, (long long)workspace_bytes);
  if (!workspace && workspace_bytes > 0) return fail(FG_EINVAL, "%s: workspace is NULL", what);
  if (workspace && !aligned(workspace, 256)) return fail(FG_EALIGN, "%s: workspace is not 256-byte aligned", what);
  SplitWs ws;
  ws.base = workspace;
  ws.bytes = workspace_bytes;
  fg::GemmParams p{};
  return dense_nt<fg::kDense>(p, A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, workspace ? &ws : nullptr, stream,
                              what);
}

fg_status gemm_fp8_nt_noalloc(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B,
                              int64_t ldb, const float* sb, uint16_t* D, int64_t ldd, int M, int N, int K,
                              void* stream) {
  const char* what = "gemm_fp8_nt_noalloc";
  g_err.clear();
  SplitWs ws;
  ws.scratch = true;
  fg::GemmParams p{};
  return dense_nt<fg::kDense>(p, A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, &ws, stream, what);
}

fg_status gemm_fp8_nt_c(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa, const uint8_t* B,
                        int64_t ldb, const float* sb, const float* C, int64_t ldc, uint16_t* D, int64_t ldd, int M,
                        int N, int K, void* stream) {
  g_err.clear();
  if (M > 0 && N > 0) {
    FG_TRY(check_ptr(C, 4, "C"));
    FG_TRY(check_ld(ldc, N, 1, "ldc"));
  }
  fg::GemmParams p{};
  p.Cin = C;
  p.ldc = ldc;
  return dense_nt<fg::kDenseC>(p, A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, nullptr, stream, "gemm_fp8_nt_c");
}

fg_status gemm_fp8_grouped_contiguous(const uint8_t* A, const float* sa, int64_t ld_sa, const uint8_t* B,
                                      const float* sb, const int32_t* m_indices, uint16_t* D, int M_total, int N,
                                      int K, int G, void* stream) {
  g_err.clear();
  if (M_total < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M_total=%d N=%d K=%d", M_total, N, K);
  if (G <= 0) return fail(FG_EINVAL, "G=%d must be positive", G);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M_total % 128) return fail(FG_EALIGN, "M_total=%d is not a multiple of 128", M_total);
  if (M_total == 0 || N == 0) return FG_OK;
  if (M_total > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M_total or N above 2^30");
  FG_TRY(check_ptr(D, 2, "D"));
  FG_TRY(check_ptr(m_indices, 4, "m_indices"));
  if (K > 0) {
    FG_TRY(check_ptr(A, 16, "A"));
    FG_TRY(check_ptr(B, 16, "B"));
    FG_TRY(check_ptr(sa, 4, "sa"));
    FG_TRY(check_ptr(sb, 4, "sb"));
    FG_TRY(check_ld(ld_sa, M_total, 1, "ld_sa"));
    FG_TRY(check_row_bytes(K, K));
  }
  FG_TRY(check_m_indices(m_indices, M_total, G, stream, "gemm_fp8_grouped_contiguous"));
  fg::GemmParams p{};
  p.A = A; p.lda = K; p.sa = sa; p.ld_sa = ld_sa; p.B = B; p.ldb = K; p.sb = sb; p.D = D; p.ldd = N;
  p.m_indices = m_indices;
  p.rows = M_total; p.N = N; p.K = K; p.G = G; p.Kb = ceil128(K); p.Nb = ceil128(N); p.ld_sb = p.Kb;
  if (K > 0) {
    // 256-row tiles: a tile whose halves hold different experts runs as two segments
    return launch_big_width<fg::kContiguous>(p, 1, (hipStream_t)stream, "gemm_fp8_grouped_contiguous");
  }
  using C = CfgDefault;
  static_assert(128 % C::BM == 0, "contiguous tiles must not straddle a 128-row expert block");
  p.tiles_m = M_total / C::BM;
  p.tiles_n = (N + C::BN - 1) / C::BN;
  p.num_tiles = p.tiles_m * p.tiles_n;
  return launch_gemm<C, fg::kContiguous>(p, (hipStream_t)stream, "gemm_fp8_grouped_contiguous");
}

fg_status gemm_fp8_grouped_masked(const uint8_t* A, const float* sa, int64_t ld_sa, const uint8_t* B, const float* sb,
                                  const int32_t* masked_m, uint16_t* D, int G, int M_cap, int N, int K,
                                  int expected_m, void* stream) {
  g_err.clear();
  (void)expected_m;
  if (M_cap < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M_cap=%d N=%d K=%d", M_cap, N, K);
  if (G <= 0) return fail(FG_EINVAL, "G=%d must be positive", G);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M_cap == 0 || N == 0) return FG_OK;
  if (M_cap > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M_cap or N above 2^30");
  FG_TRY(check_ptr(D, 2, "D"));
  FG_TRY(check_ptr(masked_m, 4, "masked_m"));
  if (K > 0) {
    FG_TRY(check_ptr(A, 16, "A"));
    FG_TRY(check_ptr(B, 16, "B"));
    FG_TRY(check_ptr(sa, 4, "sa"));
    FG_TRY(check_ptr(sb, 4, "sb"));
    FG_TRY(check_ld(ld_sa, M_cap, 1, "ld_sa"));
    FG_TRY(check_row_bytes(K, K));
  }
  FG_TRY(check_masked_m(masked_m, G, M_cap, stream, "gemm_fp8_grouped_masked"));
  fg::GemmParams p{};
  p.A = A; p.lda = K; p.sa = sa; p.ld_sa = ld_sa; p.B = B; p.ldb = K; p.sb = sb; p.D = D; p.ldd = N;
  p.masked_m = masked_m;
  p.rows = M_cap; p.N = N; p.K = K; p.G = G; p.Kb = ceil128(K); p.Nb = ceil128(N); p.ld_sb = p.Kb;
  if (K > 0) {
    return launch_big_width<fg::kMasked>(p, G, (hipStream_t)stream, "gemm_fp8_grouped_masked");
  }
  using C = CfgDefault;
  p.tiles_m = (M_cap + C::BM - 1) / C::BM;
  p.tiles_n = (N + C::BN - 1) / C::BN;
  const int64_t slots = (int64_t)G * p.tiles_m * p.tiles_n;
  if (slots > (int64_t)1 << 30) return fail(FG_EUNSUPPORTED, "too many tiles");
  p.num_tiles = (int)slots;
  return launch_gemm<C, fg::kMasked>(p, (hipStream_t)stream, "gemm_fp8_grouped_masked");
}

fg_status gemm_fp8_nt_ue8m0(const uint8_t* A, int64_t lda, const int32_t* sa, int64_t ld_sa, const uint8_t* B,
                            int64_t ldb, const int32_t* sb, uint16_t* D, int64_t ldd, int M, int N, int K,
                            void* stream) {
  g_err.clear();
  if (M < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || N == 0) return FG_OK;
  if (M > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M or N above 2^30");
  FG_TRY(check_ptr(D, 2, "D"));
  FG_TRY(check_ld(ldd, N, 1, "ldd"));
  fg::GemmParams p{};
  p.A = A; p.lda = lda; p.sa = (const float*)(const void*)sa; p.ld_sa = ld_sa; p.B = B; p.ldb = ldb;
  p.sb = (const float*)(const void*)sb; p.D = D; p.ldd = ldd;
  p.rows = M; p.N = N; p.K = K; p.G = 1; p.Kb = ceil128(K); p.Nb = ceil128(N); p.ld_sb = p.Kb;
  if (K == 0) {  // no factors are read: the plain kernel writes the zeros
    using C = CfgDefault;
    p.tiles_m = (M + C::BM - 1) / C::BM;
    p.tiles_n = (N + C::BN - 1) / C::BN;
    p.num_tiles = p.tiles_m * p.tiles_n;
    return launch_gemm<C, fg::kDense>(p, (hipStream_t)stream, "gemm_fp8_nt_ue8m0");
  }
  FG_TRY(check_ptr(A, 16, "A"));
  FG_TRY(check_ptr(B, 16, "B"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(lda, K, 16, "lda"));
  FG_TRY(check_ld(ldb, K, 16, "ldb"));
  FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
  FG_TRY(check_row_bytes(lda, ldb));
  if (ue8m0_on_promotion_kernel(false))
    return launch_big_tiled<CfgBig, fg::kDense, true>(p, 1, (hipStream_t)stream, "gemm_fp8_nt_ue8m0");
  return launch_ue8m0(p, pick_ue8m0_tile(M, N, 1, false), 1, fg::kDense, (hipStream_t)stream, "gemm_fp8_nt_ue8m0");
}

fg_status gemm_fp8_grouped_contiguous_ue8m0(const uint8_t* A, const int32_t* sa, int64_t ld_sa, const uint8_t* B,
                                            const int32_t* sb, const int32_t* m_indices, uint16_t* D, int M_total,
                                            int N, int K, int G, void* stream) {
  g_err.clear();
  if (M_total < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M_total=%d N=%d K=%d", M_total, N, K);
  if (G <= 0) return fail(FG_EINVAL, "G=%d must be positive", G);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M_total % 128) return fail(FG_EALIGN, "M_total=%d is not a multiple of 128", M_total);
  if (M_total == 0 || N == 0) return FG_OK;
  if (M_total > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M_total or N above 2^30");
  FG_TRY(check_ptr(D, 2, "D"));
  FG_TRY(check_ptr(m_indices, 4, "m_indices"));
  FG_TRY(check_m_indices(m_indices, M_total, G, stream, "gemm_fp8_grouped_contiguous_ue8m0"));
  fg::GemmParams p{};
  p.A = A; p.lda = K; p.sa = (const float*)(const void*)sa; p.ld_sa = ld_sa; p.B = B; p.ldb = K;
  p.sb = (const float*)(const void*)sb; p.D = D; p.ldd = N;
  p.m_indices = m_indices;
  p.rows = M_total; p.N = N; p.K = K; p.G = G; p.Kb = ceil128(K); p.Nb = ceil128(N); p.ld_sb = p.Kb;
  if (K == 0) {  // no factors are read: the plain kernel writes the zeros of the mapped rows
    using C = CfgDefault;
    p.tiles_m = M_total / C::BM;
    p.tiles_n = (N + C::BN - 1) / C::BN;
    p.num_tiles = p.tiles_m * p.tiles_n;
    return launch_gemm<C, fg::kContiguous>(p, (hipStream_t)stream, "gemm_fp8_grouped_contiguous_ue8m0");
  }
  FG_TRY(check_ptr(A, 16, "A"));
  FG_TRY(check_ptr(B, 16, "B"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(ld_sa, M_total, 1, "ld_sa"));
  FG_TRY(check_row_bytes(K, K));
  p.kb_factor = (p.Kb + 3) / 4;  // packed words per row of one expert's weight factors
  // 256-row tiles: a tile whose halves hold different experts runs as two
  // segments.  The widest tile: a prefill GEMM runs many rounds of tiles, so
  // per-tile reuse outweighs the rounding of the last round (measured at
  // 8 x 4096 rows, N=4096, K=7168: 256x224 849-968 us, 256x160 935-974,
  // 128x256 1116-1127).  FG_UE8M0_TILE still forces a shape.
  if (ue8m0_on_promotion_kernel(false))
    return launch_big_tiled<CfgBig, fg::kContiguous, true>(p, 1, (hipStream_t)stream,
                                                            "gemm_fp8_grouped_contiguous_ue8m0");
  const int tile = getenv("FG_UE8M0_TILE") ? pick_ue8m0_tile(M_total, N, 1, false) : fg::kUe8m0Tile256x224;
  return launch_ue8m0(p, tile, 1, fg::kContiguous, (hipStream_t)stream, "gemm_fp8_grouped_contiguous_ue8m0");
}

fg_status gemm_fp8_grouped_masked_ue8m0(const uint8_t* A, const int32_t* sa, int64_t ld_sa, const uint8_t* B,
                                        const int32_t* sb, const int32_t* masked_m, uint16_t* D, int G, int M_cap,
                                        int N, int K, int expected_m, void* stream) {
  g_err.clear();
  (void)expected_m;
  if (M_cap < 0 || N < 0 || K < 0) return fail(FG_EINVAL, "negative size M_cap=%d N=%d K=%d", M_cap, N, K);
  if (G <= 0) return fail(FG_EINVAL, "G=%d must be positive", G);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M_cap == 0 || N == 0) return FG_OK;
  if (M_cap > kMaxDim || N > kMaxDim) return fail(FG_EUNSUPPORTED, "M_cap or N above 2^30");
  FG_TRY(check_ptr(D, 2, "D"));
  FG_TRY(check_ptr(masked_m, 4, "masked_m"));
  FG_TRY(check_masked_m(masked_m, G, M_cap, stream, "gemm_fp8_grouped_masked_ue8m0"));
  fg::GemmParams p{};
  p.A = A; p.lda = K; p.sa = (const float*)(const void*)sa; p.ld_sa = ld_sa; p.B = B; p.ldb = K;
  p.sb = (const float*)(const void*)sb; p.D = D; p.ldd = N;
  p.masked_m = masked_m;
  p.rows = M_cap; p.N = N; p.K = K; p.G = G; p.Kb = ceil128(K); p.Nb = ceil128(N); p.ld_sb = p.Kb;
  if (K == 0) {  // no factors are read: the plain kernel writes the zeros of the valid rows
    using C = CfgDefault;
    p.tiles_m = (M_cap + C::BM - 1) / C::BM;
    p.tiles_n = (N + C::BN - 1) / C::BN;
    const int64_t slots = (int64_t)G * p.tiles_m * p.tiles_n;
    if (slots > (int64_t)1 << 30) return fail(FG_EUNSUPPORTED, "too many tiles");
    p.num_tiles = (int)slots;
    return launch_gemm<C, fg::kMasked>(p, (hipStream_t)stream, "gemm_fp8_grouped_masked_ue8m0");
  }
  FG_TRY(check_ptr(A, 16, "A"));
  FG_TRY(check_ptr(B, 16, "B"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(ld_sa, M_cap, 1, "ld_sa"));
  FG_TRY(check_row_bytes(K, K));
  p.kb_factor = (p.Kb + 3) / 4;  // packed words per row of one group's factor arrays
  if (ue8m0_on_promotion_kernel(pick_bn((int64_t)G * ((M_cap + 255) / 256), N) == 256))
    return launch_big_tiled<CfgBig, fg::kMasked, true>(p, G, (hipStream_t)stream, "gemm_fp8_grouped_masked_ue8m0");
  return launch_ue8m0(p, pick_ue8m0_tile(M_cap, N, G, true), G, fg::kMasked, (hipStream_t)stream,
                      "gemm_fp8_grouped_masked_ue8m0");
}

fg_status fp8_cast_per_token(const float* x, int64_t ldx, uint8_t* q, float* sa, int64_t ld_sa, int M, int K,
                             void* stream) {
  g_err.clear();
  if (M < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d K=%d", M, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(x, 16, "x"));
  FG_TRY(check_ptr(q, 8, "q"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ld(ldx, K, 4, "ldx"));
  FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
  return launch_cast_per_token<false>(x, ldx, q, (void*)sa, ld_sa, M, K, stream, "fp8_cast_per_token");
}

fg_status fp8_cast_per_token_ue8m0(const float* x, int64_t ldx, uint8_t* q, int32_t* sa, int64_t ld_sa, int M, int K,
                                   void* stream) {
  g_err.clear();
  if (M < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d K=%d", M, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(x, 16, "x"));
  FG_TRY(check_ptr(q, 8, "q"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ld(ldx, K, 4, "ldx"));
  FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
  return launch_cast_per_token<true>(x, ldx, q, (void*)sa, ld_sa, M, K, stream, "fp8_cast_per_token_ue8m0");
}

fg_status fp8_cast_per_block_ue8m0(const float* w, int64_t ldw, uint8_t* q, int32_t* sb, int N, int K,
                                   void* stream) {
  g_err.clear();
  if (N < 0 || K < 0) return fail(FG_EINVAL, "negative size N=%d K=%d", N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (N == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(w, 16, "w"));
  FG_TRY(check_ptr(q, 4, "q"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(ldw, K, 4, "ldw"));
  const int64_t blocks = (int64_t)(ceil128(N)) * (ceil128(K));
  if (blocks > 0x7fffffff) return fail(FG_EUNSUPPORTED, "input too large");
  hipLaunchKernelGGL((fg::cast_per_block_kernel<true, float>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w,
                     ldw, q, (void*)sb, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "fp8_cast_per_block_ue8m0 launch: %s", hipGetErrorString(e));
  return FG_OK;
}

fg_status fp8_cast_per_token_ue8m0_bf16(const uint16_t* x, int64_t ldx, uint8_t* q, int32_t* sa, int64_t ld_sa,
                                        int M, int K, void* stream) {
  g_err.clear();
  if (M < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d K=%d", M, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(x, 16, "x"));
  FG_TRY(check_ptr(q, 8, "q"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ld(ldx, K, 8, "ldx"));
  FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
  return launch_cast_per_token<true>(x, ldx, q, (void*)sa, ld_sa, M, K, stream, "fp8_cast_per_token_ue8m0_bf16");
}

fg_status fp8_cast_per_block_ue8m0_bf16(const uint16_t* w, int64_t ldw, uint8_t* q, int32_t* sb, int N, int K,
                                        void* stream) {
  g_err.clear();
  if (N < 0 || K < 0) return fail(FG_EINVAL, "negative size N=%d K=%d", N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (N == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(w, 16, "w"));
  FG_TRY(check_ptr(q, 4, "q"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(ldw, K, 4, "ldw"));
  const int64_t blocks = (int64_t)(ceil128(N)) * (ceil128(K));
  if (blocks > 0x7fffffff) return fail(FG_EUNSUPPORTED, "input too large");
  hipLaunchKernelGGL((fg::cast_per_block_kernel<true, uint16_t>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, w, ldw, q, (void*)sb, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "fp8_cast_per_block_ue8m0_bf16 launch: %s", hipGetErrorString(e));
  return FG_OK;
}

fg_status fp8_cast_per_token_bf16(const uint16_t* x, int64_t ldx, uint8_t* q, float* sa, int64_t ld_sa, int M, int K,
                                  void* stream) {
  g_err.clear();
  if (M < 0 || K < 0) return fail(FG_EINVAL, "negative size M=%d K=%d", M, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (M == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(x, 16, "x"));
  FG_TRY(check_ptr(q, 8, "q"));
  FG_TRY(check_ptr(sa, 4, "sa"));
  FG_TRY(check_ld(ldx, K, 8, "ldx"));
  FG_TRY(check_ld(ld_sa, M, 1, "ld_sa"));
  return launch_cast_per_token<false>(x, ldx, q, (void*)sa, ld_sa, M, K, stream, "fp8_cast_per_token_bf16");
}

fg_status fp8_cast_per_block_bf16(const uint16_t* w, int64_t ldw, uint8_t* q, float* sb, int N, int K,
                                  void* stream) {
  g_err.clear();
  if (N < 0 || K < 0) return fail(FG_EINVAL, "negative size N=%d K=%d", N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (N == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(w, 16, "w"));
  FG_TRY(check_ptr(q, 4, "q"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(ldw, K, 4, "ldw"));
  const int64_t blocks = (int64_t)(ceil128(N)) * (ceil128(K));
  if (blocks > 0x7fffffff) return fail(FG_EUNSUPPORTED, "input too large");
  hipLaunchKernelGGL((fg::cast_per_block_kernel<false, uint16_t>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, w, ldw, q, (void*)sb, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "fp8_cast_per_block_bf16 launch: %s", hipGetErrorString(e));
  return FG_OK;
}

fg_status fp8_cast_per_block(const float* w, int64_t ldw, uint8_t* q, float* sb, int N, int K, void* stream) {
  g_err.clear();
  if (N < 0 || K < 0) return fail(FG_EINVAL, "negative size N=%d K=%d", N, K);
  if (K % 16) return fail(FG_EALIGN, "K=%d is not a multiple of 16", K);
  if (N == 0 || K == 0) return FG_OK;
  FG_TRY(check_ptr(w, 16, "w"));
  FG_TRY(check_ptr(q, 4, "q"));
  FG_TRY(check_ptr(sb, 4, "sb"));
  FG_TRY(check_ld(ldw, K, 4, "ldw"));
  const int64_t blocks = (int64_t)(ceil128(N)) * (ceil128(K));
  if (blocks > 0x7fffffff) return fail(FG_EUNSUPPORTED, "input too large");
  hipLaunchKernelGGL((fg::cast_per_block_kernel<false, float>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, w, ldw, q,
                     sb, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_EHIP, "fp8_cast_per_block launch: %s", hipGetErrorString(e));
  return FG_OK;
}

int fg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

void fg_set_num_cus(int n) { g_num_cus_cap = n > 0 ? n : 0; }

int fg_get_num_cus(void) {
  if (g_num_cus_cap > 0) return g_num_cus_cap;
  int cus = 0;
  if (device_cus(&cus) != FG_OK) return 0;
  return cus;
}

const char* fg_last_error(void) { return g_err.c_str(); }

const char* fg_version(void) { return "fp8gemm-gfx950 0.1"; }

}  // extern "C"
