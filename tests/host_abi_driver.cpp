// host_abi_driver.cpp -- drives every C entry point of libfp8gemm through its
// host-side argument checks, for a build of the library's host code with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
//
// No GPU is needed: every call below either fails a host check before
// anything is launched, is an empty problem (no launch), or stops at the
// first device query (FG_EHIP without a device).  Pointers are fake device
// addresses that are never dereferenced.  Exit status 0 and "host abi ok"
// mean every status matched; a sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fp8gemm.h"

static int g_fail = 0;

#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const int st__ = (int)(call);                                                                       \
    const int w__ = (int)(want);                                                                        \
    if (st__ != w__ && !(w__ == -2 && (st__ == FG_OK || st__ == FG_EHIP))) {                            \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, st__, w__,     \
                   fg_last_error());                                                                    \
      ++g_fail;                                                                                         \
    }                                                                                                   \
  } while (0)

// -2: the call passed every host check; it stops at the device (FG_EHIP) or
// succeeds where a device exists.
static const int DEV = -2;

int main() {
  const uint8_t* A = reinterpret_cast<const uint8_t*>(0x10000);
  const uint8_t* A8 = reinterpret_cast<const uint8_t*>(0x10008);
  const float* S = reinterpret_cast<const float*>(0x10000);
  const int32_t* I = reinterpret_cast<const int32_t*>(0x10000);
  uint16_t* D = reinterpret_cast<uint16_t*>(0x10000);
  uint8_t* Q = reinterpret_cast<uint8_t*>(0x10000);
  float* SW = reinterpret_cast<float*>(0x10000);
  int32_t* IW = reinterpret_cast<int32_t*>(0x10000);
  const uint16_t* H = reinterpret_cast<const uint16_t*>(0x10000);
  void* WS = reinterpret_cast<void*>(0x10000);
  const int64_t big = (int64_t)1 << 40;

  // dense NT
  EXPECT(gemm_fp8_nt(A, 512, S, 64, A, 512, S, D, 256, -1, 256, 512, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 100, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_nt(nullptr, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt(A8, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_nt(A, 500, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt(A, big, S, 64, A, big, S, D, 256, 64, 256, 512, nullptr), FG_EUNSUPPORTED);
  EXPECT(gemm_fp8_nt(A, 512, S, big, A, 512, S, D, big, 0x7fffffff, 0x7fffffff, 512, nullptr), FG_EUNSUPPORTED);
  EXPECT(gemm_fp8_nt(nullptr, 0, nullptr, 0, nullptr, 0, nullptr, nullptr, 0, 0, 128, 256, nullptr), FG_OK);
  EXPECT(gemm_fp8_nt(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr), DEV);
  EXPECT(gemm_fp8_nt_c(A, 512, S, 64, A, 512, S, nullptr, 256, D, 256, 64, 256, 512, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt_c(A, 512, S, 64, A, 512, S, S, 100, D, 256, 64, 256, 512, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt_c(A, 512, S, 64, A, 512, S, S, 256, D, 256, 64, 256, 512, nullptr), DEV);

  // dense NT with a workspace
  EXPECT(gemm_fp8_nt_ws(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, WS, -1, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt_ws(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr, 4096, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_nt_ws(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, (void*)0x10010, 4096, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_nt_ws(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, WS, big, nullptr), DEV);
  EXPECT(gemm_fp8_nt_ws(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr, 0, nullptr), DEV);
  EXPECT(gemm_fp8_nt_noalloc(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 100, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_nt_noalloc(A, 512, S, 64, A, 512, S, D, 256, 64, 256, 512, nullptr), DEV);
  if (fg_nt_workspace_bytes(-1, 1, 1) != -1) ++g_fail;
  if (fg_nt_workspace_max_bytes() != (int64_t)(8 << 20) + (64 << 10)) ++g_fail;
  (void)fg_nt_workspace_bytes(64, 2112, 7168);  // -1 without a device
  (void)fg_nt_workspace_bytes(0x7fffffff, 0x7fffffff, 0x7ffffff0);

  // layouts
  const char* layouts[] = {"nt", "nn", "tn", "tt", "xx", nullptr};
  for (const char* l : layouts) (void)fg_layout_workspace_bytes(l, 0x7fffffff, 0x7fffffff, 0x7ffffff0);
  if (fg_layout_workspace_bytes("tn", 128, 256, 512) != 128 * 512 + 256 * 512) ++g_fail;
  EXPECT(gemm_fp8_nn(A, 512, S, 64, A, 256, S, nullptr, 0, D, 256, 64, 256, 512, WS, 1, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_tn(A, 64, S, 64, A, 256, S, nullptr, 0, D, 256, 64, 256, 512, nullptr, big, nullptr),
         FG_EINVAL);
  EXPECT(gemm_fp8_tt(A, 63, S, 64, A, 512, S, nullptr, 0, D, 256, 64, 256, 512, WS, big, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_tt(A, 64, S, 64, A, 512, S, nullptr, 0, D, 256, 64, 256, 100, WS, big, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_tn(A, 64, S, 64, A, 256, S, nullptr, 0, D, 256, 64, 256, (1 << 22) + 16, WS, big, nullptr),
         FG_EUNSUPPORTED);
  // no workspace: MN-major operands need 16-byte rows and M, N multiples of 16
  EXPECT(gemm_fp8_tn(A, 72, S, 64, A, 256, S, nullptr, 0, D, 256, 64, 256, 512, nullptr, 0, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_nn(A, 512, S, 64, A, 250, S, nullptr, 0, D, 250, 64, 250, 512, nullptr, 0, nullptr), FG_EALIGN);

  // K-grouped TN
  int ks[3] = {128, 0, 256};
  int ks_bad[2] = {128, 100};
  int ks_neg[2] = {128, -128};
  EXPECT(gemm_fp8_k_grouped_tn_contiguous(A, 64, S, 64, A, 256, S, ks, 0, nullptr, D, 64, 256, WS, big, nullptr),
         FG_EINVAL);
  EXPECT(gemm_fp8_k_grouped_tn_contiguous(A, 64, S, 64, A, 256, S, nullptr, 3, nullptr, D, 64, 256, WS, big,
                                          nullptr),
         FG_EINVAL);
  EXPECT(gemm_fp8_k_grouped_tn_contiguous(A, 64, S, 64, A, 256, S, ks_bad, 2, nullptr, D, 64, 256, WS, big, nullptr),
         FG_EALIGN);
  EXPECT(gemm_fp8_k_grouped_tn_contiguous(A, 64, S, 64, A, 256, S, ks_neg, 2, nullptr, D, 64, 256, WS, big, nullptr),
         FG_EINVAL);
  EXPECT(gemm_fp8_k_grouped_tn_contiguous(A, 72, S, 64, A, 256, S, ks, 3, nullptr, D, 64, 256, WS, 16, nullptr),
         FG_EINVAL);
  EXPECT(gemm_fp8_k_grouped_tn_contiguous(A, 64, S, 64, A, 256, S, ks, 3, nullptr, D, 60, 256, nullptr, 0, nullptr),
         FG_EALIGN);
  if (fg_k_grouped_workspace_bytes(-1, 1, 1) != -1) ++g_fail;
  (void)fg_k_grouped_workspace_bytes(0x7fffffff, 0x7fffffff, big);

  // grouped: contiguous and masked (fp32 and power-of-two factors)
  EXPECT(gemm_fp8_grouped_contiguous(A, S, 256, A, S, I, D, 256, 256, 512, 0, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_contiguous(A, S, 256, A, S, I, D, 200, 256, 512, 4, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_grouped_contiguous(A, S, 256, A, S, nullptr, D, 256, 256, 512, 4, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_contiguous(A, S, 128, A, S, I, D, 256, 256, 512, 4, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_contiguous(A, S, 256, A, S, I, D, 256, 256, 512, 4, nullptr), DEV);
  EXPECT(gemm_fp8_grouped_masked(A, S, 256, A, S, I, D, 0, 256, 256, 512, 0, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_masked(A, S, 256, A, S, nullptr, D, 4, 256, 256, 512, 0, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_masked(A, S, 100, A, S, I, D, 4, 256, 256, 512, 0, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_masked(A, S, 256, A, S, I, D, 4, 256, 256, 72, 0, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_grouped_masked(A, S, 256, A, S, I, D, 4, 256, 256, 512, 64, nullptr), DEV);
  EXPECT(gemm_fp8_grouped_masked(A, S, 256, A, S, I, D, 0x7fff, 0x7fffffff, 0x7fffffff, 512, 0, nullptr),
         FG_EUNSUPPORTED);
  EXPECT(gemm_fp8_nt_ue8m0(A, 512, I, 64, A, 512, I, D, 256, 64, 256, 100, nullptr), FG_EALIGN);
  EXPECT(gemm_fp8_nt_ue8m0(A, 512, I, 64, A, 512, I, D, 256, 64, 256, 512, nullptr), DEV);
  EXPECT(gemm_fp8_grouped_contiguous_ue8m0(A, I, 256, A, I, nullptr, D, 256, 256, 512, 2, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_contiguous_ue8m0(A, I, 256, A, I, I, D, 256, 256, 512, 2, nullptr), DEV);
  EXPECT(gemm_fp8_grouped_masked_ue8m0(A, I, 64, A, I, I, D, -1, 64, 256, 512, 0, nullptr), FG_EINVAL);
  EXPECT(gemm_fp8_grouped_masked_ue8m0(A, I, 64, A, I, I, D, 2, 64, 256, 512, 0, nullptr), DEV);

  // casts
  EXPECT(fp8_cast_per_token(S, 512, Q, SW, 64, 64, 500, nullptr), FG_EALIGN);
  EXPECT(fp8_cast_per_token(nullptr, 512, Q, SW, 64, 64, 512, nullptr), FG_EINVAL);
  EXPECT(fp8_cast_per_token(S, 512, Q, SW, 64, 64, 512, nullptr), DEV);
  EXPECT(fp8_cast_per_block(S, 255, Q, SW, 130, 256, nullptr), FG_EINVAL);
  EXPECT(fp8_cast_per_block(S, 256, Q, SW, 130, 256, nullptr), DEV);
  EXPECT(fp8_cast_per_token_bf16(H, 512, Q, SW, 64, 64, 512, nullptr), DEV);
  EXPECT(fp8_cast_per_block_bf16(H, 513, Q, SW, 130, 512, nullptr), FG_EALIGN);
  EXPECT(fp8_cast_per_token_ue8m0(S, 512, Q, IW, 63, 64, 512, nullptr), FG_EINVAL);
  EXPECT(fp8_cast_per_block_ue8m0(S, 256, Q, IW, 130, 256, nullptr), DEV);
  EXPECT(fp8_cast_per_token_ue8m0_bf16(H, 512, Q, IW, 64, 64, 512, nullptr), DEV);
  EXPECT(fp8_cast_per_block_ue8m0_bf16(H, 0x7ffffff0, Q, IW, 0x7fffffff, 0x7ffffff0, nullptr), FG_EUNSUPPORTED);

  // queries and settings
  if (fg_get_mk_alignment_for_contiguous_layout() != 128) ++g_fail;
  fg_set_num_cus(7);
  if (fg_get_num_cus() != 7) ++g_fail;
  fg_set_num_cus(-3);
  fg_set_num_cus(0);
  if (std::strncmp(fg_version(), "fp8gemm", 7) != 0) ++g_fail;
  (void)fg_last_error();

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host abi ok\n");
  return 0;
}
