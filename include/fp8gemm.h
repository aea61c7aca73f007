/*
 * fp8gemm.h -- C ABI of the MI355X (gfx950) FP8 e4m3 fine-grained-scaled GEMM library.
 *
 * Operation.  The NT GEMM D = A . B^T (DeepGEMM digest, GeekNews topic 19459,
 * section "GEMM arayuzu ve yerlesim kisitlari": the naming is D = C + A @ B
 * with NT meaning A row-major and B stored [N,K]; this library has no C
 * addend) with DeepSeek-V3 fine-grained scaling (GeekNews topic 19444,
 * opening bullets; 7minutos.es, "Detalles y beneficios tecnicos"):
 *
 *     D[m,n] = bf16( sum_kb  P_kb[m,n] * sa[kb][m] * sb[n/128][kb] )
 *     P_kb[m,n] = sum_{k in slice kb} e4m3(A[m,k]) * e4m3(B[n,k])
 *
 * Each 128-wide K slice is computed by the matrix cores into a fresh fp32
 * partial P_kb and then scaled and added ("promoted") into an fp32
 * accumulator; the accumulator is rounded once to BF16 (nearest-even).
 *
 * Types.  FP8 operands are e4m3fn bytes (OCP: bias 7, max 448, NaN 0x7F/0xFF)
 * passed as uint8_t.  Scales are IEEE fp32.  BF16 results are uint16_t bit
 * patterns.  Kb = ceil(K/128), Nb = ceil(N/128).
 *
 * K tails.  The digest leaves K % 128 != 0 open.  Reading taken here: K must
 * be a multiple of 16 (the 16-byte row granularity of the operand loads); the
 * last K group is then partial and holds the K % 128 remaining columns, with
 * its own factors (the casts take its amax over those columns alone).  This
 * holds for the power-of-two (UE8M0) calls too; the K-grouped GEMM keeps
 * K % 128 == 0.
 *
 * Scale layouts.  Activation scales are per (row, 128-wide K group) and are
 * stored K-group-major ("transposed", as the digest requires for the LHS
 * factors): sa[kb * ld_sa + m], ld_sa >= rows.  Weight scales
 * are per 128x128 block, row-major: sb[nb * Kb + kb].
 *
 * Ownership.  Every pointer named "device" is device memory owned by the
 * caller; the library never frees or retains caller pointers.  Each GEMM or
 * cast call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 * default stream) and returns: no call allocates device memory or
 * synchronises, so every call can be captured into a HIP graph (the masked
 * form, whose counts the host never learns, is made for that).  Scratch
 * memory, where a plan needs it, comes from the caller as a `workspace`
 * argument (gemm_fp8_nt_ws, the NN/TN/TT layouts, the K-grouped GEMM).  The
 * one exception is the opt-in debug check FG_CHECK_DEVICE (see the grouped
 * calls), which reads a result back.
 *
 * Errors.  Preconditions that the host can check are checked before anything
 * is launched; on failure the call returns the status, launches nothing, and
 * fg_last_error() describes the failure (thread-local, valid until the next
 * call on the same thread).  A call with no output elements (M == 0 or
 * N == 0, M_total == 0, M_cap == 0) returns FG_OK without launching.  A
 * launch failure returns FG_EHIP with the HIP error string.  Preconditions on
 * device-resident metadata (expert indices, masks) are documented per call
 * and are not checked by default (checking needs a host synchronisation);
 * the debug mode FG_CHECK_DEVICE=1 checks them (see the grouped calls).
 */
#ifndef FP8GEMM_H
#define FP8GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FG_OK = 0,
  FG_EINVAL = 1,      /* null pointer, negative size, G <= 0, leading dimension too small */
  FG_EALIGN = 2,      /* K % 16 != 0 (K % 128 != 0 where stated), M_total % 128 != 0, misaligned pointer or row stride */
  FG_EUNSUPPORTED = 3,/* sizes beyond what the kernels index (see per call) */
  FG_EHIP = 4         /* a HIP launch failed; see fg_last_error() */
} fg_status;

/*
 * Dense NT GEMM (the digest's fp8_gemm_nt without C).
 *   A   device [M, K] e4m3, row stride lda bytes   (lda >= K, lda % 16 == 0, A 16-byte aligned)
 *   sa  device fp32 [Kb][ld_sa]                    (ld_sa >= M, 4-byte aligned)
 *   B   device [N, K] e4m3, row stride ldb bytes   (ldb >= K, ldb % 16 == 0, B 16-byte aligned)
 *   sb  device fp32 [Nb][Kb]                       (4-byte aligned)
 *   D   device [M, N] bf16, row stride ldd elems   (ldd >= N, 2-byte aligned; rows that are 8- or
 *       16-byte aligned get vector stores); written
 * M, N >= 0 arbitrary; K % 16 == 0 (a partial last K group when K % 128 != 0).
 * K == 0 writes D = 0 (sa, sb may then be NULL).
 * Only D[0:M, 0:N] is written.  lda, ldb <= 4 MiB (FG_EUNSUPPORTED beyond).
 * Few rows (M <= 128) run a weight-streaming kernel; this call never splits
 * its K range over workgroups (gemm_fp8_nt_ws does, with a workspace).  The
 * kernel and plan depend only on the arguments and the device (not on the CU
 * cap, earlier calls or graph capture), so results are bit-for-bit
 * reproducible.  Allocates nothing.
 */
fg_status gemm_fp8_nt(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const uint8_t* B, int64_t ldb, const float* sb,
                      uint16_t* D, int64_t ldd, int M, int N, int K, void* stream);

/*
 * gemm_fp8_nt with a caller's workspace, which lets the few-row plan
 * (M <= 128) split the K range over several workgroups when the column tiles
 * alone cannot occupy the device (decode shapes); the fp32 partials of the
 * splits meet in the workspace and are added in a fixed split order, so the
 * result is reproducible and does not depend on the workspace's history.
 *   workspace        device, 256-byte aligned, or NULL (then the plan of gemm_fp8_nt)
 *   workspace_bytes  >= fg_nt_workspace_bytes(M, N, K) (FG_EINVAL otherwise); any
 *                    size works for a shape whose plan does not split (need 0)
 * Workspace contract: its first 64 KiB are arrival counters and must be zero
 * before the workspace is first used (e.g. allocate it zero-filled); every
 * call leaves them zero.  The rest holds partials and needs no
 * initialisation.  A workspace is in use until the call's work on `stream`
 * has finished; calls that may run at the same time (other streams, a graph
 * replayed on another stream) must use different workspaces.  Everything
 * else as gemm_fp8_nt; the output equals gemm_fp8_nt's within the stated
 * tolerance (bit for bit when the plan does not split).  Allocates nothing.
 */
fg_status gemm_fp8_nt_ws(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                         const uint8_t* B, int64_t ldb, const float* sb,
                         uint16_t* D, int64_t ldd, int M, int N, int K,
                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * gemm_fp8_nt_ws for callers that cannot allocate device memory at all (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same plan and the same results, bit for bit, as
 * gemm_fp8_nt_ws with a large enough workspace, with the split-K buffers in
 * a scratch array of the library instead: 8 MiB + 64 KiB per GPU, a static
 * device array that each GPU the library runs on holds until the process
 * ends.  Each split call clears the arrival counters it uses (a small fill
 * kernel, no memset) before its GEMM.  Every call on one GPU shares that
 * GPU's scratch, so calls that overlap in time on one GPU (other streams,
 * graphs replayed concurrently) race; serialise them.  The plan never needs
 * more scratch than the array holds (the split is bounded by it); a plan that
 * did would return FG_EUNSUPPORTED.  Nothing is allocated; everything else as
 * gemm_fp8_nt.
 */
fg_status gemm_fp8_nt_noalloc(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                              const uint8_t* B, int64_t ldb, const float* sb,
                              uint16_t* D, int64_t ldd, int M, int N, int K, void* stream);

/* Workspace bytes gemm_fp8_nt_ws needs for (M, N, K) on the current device:
 * 0 when its plan does not split K, else 64 KiB of counters plus the
 * partials.  -1 for a negative size or when the device cannot be queried. */
int64_t fg_nt_workspace_bytes(int M, int N, int K);

/* Upper bound of fg_nt_workspace_bytes over every shape (8 MiB + 64 KiB):
 * a workspace of this size serves every call. */
int64_t fg_nt_workspace_max_bytes(void);

/*
 * Dense NT GEMM with an addend, D = C + A . B^T (the digest, "GEMM arayuzu ve
 * yerlesim kisitlari": every GEMM kernel is named after D = C + A @ B, and
 * fp8_gemm_nt computes D = C + A @ B.T).
 *   C   device fp32 [M, N], row stride ldc elems   (ldc >= N, 4-byte aligned; rows that are
 *       16-byte aligned get vector loads); read only, may not overlap D
 *   every other argument as in gemm_fp8_nt.
 * C is added to the fp32 accumulator once, after the last K slice, and the sum
 * is rounded to BF16 once.  K == 0 writes D = bf16(C).  Same kernels and
 * plans as gemm_fp8_nt (no K split).  C == NULL is FG_EINVAL when M, N > 0.
 */
fg_status gemm_fp8_nt_c(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                        const uint8_t* B, int64_t ldb, const float* sb, const float* C, int64_t ldc,
                        uint16_t* D, int64_t ldd, int M, int N, int K, void* stream);

/*
 * The other storage layouts (the digest's fp8_gemm_{nn, tn, tt}, section
 * "Dense ve Grouped GEMM"; the same D = C + A @ B naming).  The first letter
 * says whether the stored A is used as is (n: A [M, K]) or transposed (t: A
 * stored [K, M]); the second the same for B, where t is the NT form's
 * B [N, K] and n stores B as [K, N]:
 *   gemm_fp8_nn   D = C + A . B      A [M, K] (lda bytes, as in gemm_fp8_nt), B [K, N] (ldb >= N bytes)
 *   gemm_fp8_tn   D = C + A^T . B    A [K, M] (lda >= M bytes),                B [K, N] (ldb >= N bytes)
 *   gemm_fp8_tt   D = C + A^T . B^T  A [K, M] (lda >= M bytes),                B [N, K] (as in gemm_fp8_nt)
 * The scale factors belong to the logical operands, in the NT layouts: sa
 * fp32 [Kb][ld_sa] (1x128 along K for each of the M rows), sb fp32 [Nb][Kb]
 * (128x128 blocks of the [N, K] operand).  C: fp32 [M, N] addend (row stride
 * ldc >= N) or NULL for none.  D: as in gemm_fp8_nt.  An operand stored MN-major
 * has no alignment requirement on the copying path.
 * Two paths serve the MN-major operands:
 *  - copies: each MN-major operand is first transposed, K-major, into the
 *    caller's device workspace (a byte copy bound by HBM), then the NT
 *    kernels run on the copy.  The stored [K, .] operands have at most
 *    65535*128 rows (FG_EUNSUPPORTED).
 *  - copy-free: the large-tile kernel stages each MN-major operand as
 *    stored.  Each such operand must be 16-byte aligned with a row stride
 *    and a column count (M for A, N for B) that are multiples of 16.
 * workspace_bytes > 0: workspace must be 16-byte aligned and hold at least
 *    fg_layout_workspace_bytes(layout, M, N, K) bytes (FG_EINVAL otherwise);
 *    it is in use until the call's work on `stream` has finished.  The call
 *    takes the copy-free path where the operands allow it and the large
 *    kernel's 256 x 256 tiles keep the device's CUs at least three quarters
 *    busy over their rounds (measured on MI355X at M = 4096: level with or
 *    2-9 % faster than the copies there, 2-7 % slower than them at
 *    N = 2112), and the copies otherwise.  Both paths give the same bits.
 * workspace_bytes == 0 (workspace ignored): the copy-free path; operands it
 *    cannot take give FG_EALIGN.  For callers without device memory to spare.
 * K <= 2^22 (FG_EUNSUPPORTED).  K % 16 == 0.  Nothing is allocated.
 */
fg_status gemm_fp8_nn(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const uint8_t* B, int64_t ldb, const float* sb, const float* C, int64_t ldc,
                      uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream);
fg_status gemm_fp8_tn(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const uint8_t* B, int64_t ldb, const float* sb, const float* C, int64_t ldc,
                      uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream);
fg_status gemm_fp8_tt(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                      const uint8_t* B, int64_t ldb, const float* sb, const float* C, int64_t ldc,
                      uint16_t* D, int64_t ldd, int M, int N, int K,
                      void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes the copying path of gemm_fp8_<layout> needs for (M, N, K)
 * (a workspace of 0 bytes selects the copy-free path instead); layout is one
 * of "nt" (0), "nn", "tn", "tt".  -1 for an unknown layout, a negative size
 * or sizes the call rejects. */
int64_t fg_layout_workspace_bytes(const char* layout, int M, int N, int K);

/*
 * K-grouped TN GEMM for MoE weight gradients (the digest's
 * k_grouped_fp8_gemm_tn_contiguous, section "Dense ve Grouped GEMM": grouped
 * along K, M and N fixed).  Group g owns the ks[g] consecutive K rows that
 * start at k_g = ks[0] + .. + ks[g-1] and computes
 *     D[g] = C[g] + A_g^T . B_g          (A_g = A[k_g : k_g + ks[g], :], B_g likewise)
 *   A   device [K_total, M] e4m3, row stride lda >= M bytes (K_total = sum of ks)
 *   sa  device fp32 [K_total/128][ld_sa], ld_sa >= M: 1x128 factors along K per column m of A
 *   B   device [K_total, N] e4m3, row stride ldb >= N bytes
 *   sb  device fp32 [Nb][K_total/128]: 128x128 blocks of the logical [N, K] operand
 *   ks  HOST int [G]; each a multiple of 128 (FG_EALIGN otherwise); 0 allowed (D[g] = C[g], or 0)
 *   C   device fp32 [G, M, N] addend, contiguous, or NULL
 *   D   device bf16 [G, M, N], contiguous; written
 * Group g uses the factors of its own K groups (columns k_g/128 .. of sa
 * and sb).  Groups with ks[g] = 0 get D[g] = C[g] (or 0) from a fill
 * kernel; the groups with K rows run as one persistent launch (one per run
 * of 256 such groups), all on `stream`.  The workspace selects how the
 * operands are read:
 *  - workspace_bytes > 0: both are transposed K-major into the caller's
 *    device workspace (16-byte aligned, at least
 *    fg_k_grouped_workspace_bytes(M, N, K_total) bytes; FG_EINVAL
 *    otherwise), which is in use until the call's work on `stream` has
 *    finished.  The faster path.
 *  - workspace_bytes == 0 (workspace ignored): no copy; the kernel stages A
 *    and B as stored.  They must be 16-byte aligned, with lda, ldb, M and N
 *    multiples of 16 (FG_EALIGN otherwise).
 * K_total <= 2^22 (FG_EUNSUPPORTED).  Nothing is allocated.
 */
fg_status gemm_fp8_k_grouped_tn_contiguous(const uint8_t* A, int64_t lda, const float* sa, int64_t ld_sa,
                                           const uint8_t* B, int64_t ldb, const float* sb,
                                           const int* ks, int G, const float* C, uint16_t* D, int M, int N,
                                           void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes the copying path of gemm_fp8_k_grouped_tn_contiguous needs
 * (0 bytes selects the copy-free path); -1 for a negative size or sizes the
 * call rejects. */
int64_t fg_k_grouped_workspace_bytes(int M, int N, int64_t K_total);

/*
 * M-grouped "contiguous" GEMM (digest, section "Dense ve Grouped GEMM": the
 * experts share N and K; every expert's rows are concatenated along M and each
 * expert segment is aligned to the GEMM M block, here 128 rows).
 *   A         device [M_total, K] e4m3, packed rows (row stride K)
 *   sa        device fp32 [Kb][ld_sa], ld_sa >= M_total
 *   B         device [G, N, K] e4m3, packed
 *   sb        device fp32 [G][Nb][Kb]
 *   m_indices device int32 [M_total]: expert of each row, or -1 for a padding row
 *   D         device [M_total, N] bf16, packed (row stride N)
 * M_total % 128 == 0, K % 16 == 0, G >= 1.
 * Device-side precondition (not checked): within each aligned 128-row block
 * every non-negative index is the same value e < G.  The block is computed
 * against B[e], where e is the largest index in the block below G; rows whose
 * index is not e (padding) are left untouched; a block of padding only is
 * skipped.  An index >= G counts as padding, so no weight outside B is ever
 * addressed.
 * Debug mode: with the environment variable FG_CHECK_DEVICE=1 a check kernel
 * validates m_indices first and the host reads its result back (this
 * synchronises the stream, and the call returns FG_EINVAL while the stream
 * is being captured); an index outside [-1, G), or one that differs from the
 * other non-negative indices of its 128-row block, returns FG_EINVAL naming
 * the row, and the GEMM is not launched.
 */
fg_status gemm_fp8_grouped_contiguous(const uint8_t* A, const float* sa, int64_t ld_sa,
                                      const uint8_t* B, const float* sb,
                                      const int32_t* m_indices,
                                      uint16_t* D, int M_total, int N, int K, int G, void* stream);

/*
 * M-grouped "masked" GEMM for decoding (digest, "Dense ve Grouped GEMM": the
 * per-expert token count lives on the device, the CPU does not know it, and
 * only the valid region is computed).
 *   A        device [G, M_cap, K] e4m3, packed
 *   sa       device fp32 [G][Kb][ld_sa], ld_sa >= M_cap
 *   B        device [G, N, K] e4m3, packed
 *   sb       device fp32 [G][Nb][Kb]
 *   masked_m device int32 [G]: valid rows of each group
 *   D        device [G, M_cap, N] bf16, packed
 *   expected_m  host hint of the typical count (0 = unknown); accepted for interface compatibility,
 *               the plan does not use it (measured: the tile width chosen from G, M_cap and N is best)
 * Group g computes rows [0, clamp(masked_m[g], 0, M_cap)); every other row of
 * D[g] is left untouched (bit for bit).  K % 16 == 0, G >= 1.
 * Debug mode (FG_CHECK_DEVICE=1, as for the contiguous form): a count
 * outside [0, M_cap], which the unchecked call clamps, returns FG_EINVAL
 * naming the group, and the GEMM is not launched.
 */
fg_status gemm_fp8_grouped_masked(const uint8_t* A, const float* sa, int64_t ld_sa,
                                  const uint8_t* B, const float* sb,
                                  const int32_t* masked_m,
                                  uint16_t* D, int G, int M_cap, int N, int K,
                                  int expected_m, void* stream);

/*
 * Per-token (1 x 128) FP8 cast of activations (the digest leaves casting to
 * the user, "GEMM arayuzu ve yerlesim kisitlari"; this is the library's own
 * helper).  For each row m and group kb:
 *     amax = max |x[m, 128kb : min(128kb+128, K)]|
 *     s    = max(amax, 1e-4f) / 448          (fp32, correctly rounded)
 *     q    = e4m3_RNE(x / s)                 (fp32 division, nearest-even)
 *   x   device fp32 [M, K], row stride ldx elements (ldx >= K, ldx % 4 == 0, 16-byte aligned)
 *   q   device [M, K] e4m3, packed (row stride K), 8-byte aligned
 *   sa  device fp32 [Kb][ld_sa], ld_sa >= M (written; the GEMM's activation-scale layout)
 * K % 16 == 0 (the last group holds K % 128 columns when K % 128 != 0).
 * Input values must be finite.
 */
fg_status fp8_cast_per_token(const float* x, int64_t ldx, uint8_t* q, float* sa, int64_t ld_sa,
                             int M, int K, void* stream);

/*
 * Per-block (128 x 128) FP8 cast of a weight matrix, same formula with amax
 * taken over each 128x128 block (the last row block covers N % 128 rows, the
 * last column block K % 128 columns).
 *   w   device fp32 [N, K], row stride ldw elements (ldw >= K, ldw % 4 == 0, 16-byte aligned)
 *   q   device [N, K] e4m3, packed, 4-byte aligned
 *   sb  device fp32 [Nb][Kb] (written; the GEMM's weight-scale layout)
 * K % 16 == 0.  For expert weights [G, N, K] with N % 128 == 0 one call on
 * [G*N, K] yields the [G][Nb][Kb] layout; otherwise call once per expert.
 */
fg_status fp8_cast_per_block(const float* w, int64_t ldw, uint8_t* q, float* sb,
                             int N, int K, void* stream);

/*
 * The same two casts from BF16 inputs (raw bf16 bit patterns).  Each input
 * is widened to fp32 exactly and then quantised as fp8_cast_per_token /
 * fp8_cast_per_block quantise that fp32 value (same formula, same outputs).
 *   x   device bf16 [M, K], row stride ldx elements (ldx >= K, ldx % 8 == 0), 16-byte aligned
 *   w   device bf16 [N, K], row stride ldw elements (ldw >= K, ldw % 4 == 0), 16-byte aligned
 * Other arguments, outputs and errors as for the fp32-input casts.
 */
fg_status fp8_cast_per_token_bf16(const uint16_t* x, int64_t ldx, uint8_t* q, float* sa, int64_t ld_sa,
                                  int M, int K, void* stream);
fg_status fp8_cast_per_block_bf16(const uint16_t* w, int64_t ldw, uint8_t* q, float* sb,
                                  int N, int K, void* stream);

/*
 * Power-of-two (UE8M0) scale factors.  The digest's layout section
 * ("GEMM arayuzu ve yerlesim kisitlari") gives the newer architecture's
 * factors as UE8M0 -- an unsigned exponent byte e, value 2^(e - 127) -- packed
 * four to a 32-bit integer.  Same granularity as the fp32 factors; four
 * consecutive K groups share an int32, K group 4i + j in byte j (least
 * significant first).  Kb4 = ceil(Kb / 4).
 *
 * Dense GEMM  D = bf16( sum_kb 2^(sa - 127) 2^(sb - 127) (A_kb . B_kb^T) )
 *   A   device [M, K] e4m3, row stride lda bytes (lda >= K, lda % 16 == 0), 16-byte aligned
 *   sa  device int32 [Kb4][ld_sa], ld_sa >= M: byte kb % 4 of sa[kb / 4][m] is row m's factor
 *       of K group kb
 *   B   device [N, K] e4m3, row stride ldb bytes (ldb >= K, ldb % 16 == 0), 16-byte aligned
 *   sb  device int32 [Nb][Kb4]: byte kb % 4 of sb[nb][kb / 4] is block (nb, kb)'s factor
 *   D   device [M, N] bf16, row stride ldd elements
 * The matrix cores apply the factors (gfx950's scaled FP8 MFMA) and add each
 * 128-deep slice into fp32 accumulators; the output is the same definition
 * as gemm_fp8_nt with factors 2^(e - 127).  Factor bytes 0 and 255 are not
 * meaningful inputs (the casts below never write them).  K % 16 == 0 (a
 * partial last K group when K % 128 != 0), lda, ldb <= 4 MiB.  Allocates
 * nothing; errors as for gemm_fp8_nt.
 */
fg_status gemm_fp8_nt_ue8m0(const uint8_t* A, int64_t lda, const int32_t* sa, int64_t ld_sa,
                            const uint8_t* B, int64_t ldb, const int32_t* sb,
                            uint16_t* D, int64_t ldd, int M, int N, int K, void* stream);

/*
 * Contiguous M-grouped GEMM (digest, "Dense ve Grouped GEMM") with
 * power-of-two factors: gemm_fp8_grouped_contiguous's layout and row mapping,
 * with the factors of gemm_fp8_nt_ue8m0.
 *   A          device [M_total, K] e4m3, packed
 *   sa         device int32 [Kb4][ld_sa], ld_sa >= M_total (packed as for gemm_fp8_nt_ue8m0)
 *   B          device [G, N, K] e4m3, packed
 *   sb         device int32 [G][Nb][Kb4]
 *   m_indices  device int32 [M_total]: expert of each row, -1 = padding row
 *   D          device [M_total, N] bf16, packed
 * Row m with m_indices[m] = e in [0, G) is computed with expert e's weights
 * as gemm_fp8_nt_ue8m0 computes it; padding rows of D are left untouched.
 * Each 128-row block holds one expert (or padding).  K % 16 == 0,
 * M_total % 128 == 0, G >= 1.  Allocates nothing; errors as for
 * gemm_fp8_grouped_contiguous.
 */
fg_status gemm_fp8_grouped_contiguous_ue8m0(const uint8_t* A, const int32_t* sa, int64_t ld_sa,
                                            const uint8_t* B, const int32_t* sb,
                                            const int32_t* m_indices,
                                            uint16_t* D, int M_total, int N, int K, int G, void* stream);

/*
 * Masked grouped GEMM (decode; digest, "Dense ve Grouped GEMM") with
 * power-of-two factors: gemm_fp8_grouped_masked's layout and row masking,
 * with the factors of gemm_fp8_nt_ue8m0 packed per group.
 *   A        device [G, M_cap, K] e4m3, packed
 *   sa       device int32 [G][Kb4][ld_sa], ld_sa >= M_cap (packed as for gemm_fp8_nt_ue8m0)
 *   B        device [G, N, K] e4m3, packed
 *   sb       device int32 [G][Nb][Kb4]
 *   masked_m device int32 [G]: valid rows of each group
 *   D        device [G, M_cap, N] bf16, packed
 *   expected_m  accepted for interface compatibility; not used
 * Group g computes rows [0, clamp(masked_m[g], 0, M_cap)) as gemm_fp8_nt_ue8m0
 * computes them; every other row of D[g] is left untouched (bit for bit).
 * K % 16 == 0, G >= 1.  Allocates nothing; errors as for
 * gemm_fp8_grouped_masked.
 */
fg_status gemm_fp8_grouped_masked_ue8m0(const uint8_t* A, const int32_t* sa, int64_t ld_sa,
                                        const uint8_t* B, const int32_t* sb,
                                        const int32_t* masked_m,
                                        uint16_t* D, int G, int M_cap, int N, int K,
                                        int expected_m, void* stream);

/*
 * Per-token (1 x 128) cast with power-of-two factors: as fp8_cast_per_token,
 * but the fp32 factor max(amax, 1e-4f) / 448 is rounded up to the next power
 * of two 2^(e - 127) (so no code saturates) and e is written as a byte:
 *   sa  device int32 [Kb4][ld_sa], ld_sa >= M; byte kb % 4 of sa[kb / 4][m] is
 *       written for every kb < Kb (bytes for K groups >= Kb are not written)
 */
fg_status fp8_cast_per_token_ue8m0(const float* x, int64_t ldx, uint8_t* q, int32_t* sa, int64_t ld_sa,
                                   int M, int K, void* stream);

/*
 * Per-block (128 x 128) cast with power-of-two factors (rounding as above):
 *   sb  device int32 [Nb][Kb4]; byte kb % 4 of sb[nb][kb / 4] is written for every kb < Kb
 */
fg_status fp8_cast_per_block_ue8m0(const float* w, int64_t ldw, uint8_t* q, int32_t* sb,
                                   int N, int K, void* stream);

/*
 * The two power-of-two-factor casts from BF16 inputs (raw bf16 bit patterns),
 * widened to fp32 exactly first, as fp8_cast_per_token_bf16 /
 * fp8_cast_per_block_bf16 do:
 *   x   device bf16 [M, K], row stride ldx elements (ldx >= K, ldx % 8 == 0), 16-byte aligned
 *   w   device bf16 [N, K], row stride ldw elements (ldw >= K, ldw % 4 == 0), 16-byte aligned
 * Other arguments, outputs and errors as for fp8_cast_per_token_ue8m0 /
 * fp8_cast_per_block_ue8m0.
 */
fg_status fp8_cast_per_token_ue8m0_bf16(const uint16_t* x, int64_t ldx, uint8_t* q, int32_t* sa, int64_t ld_sa,
                                        int M, int K, void* stream);
fg_status fp8_cast_per_block_ue8m0_bf16(const uint16_t* w, int64_t ldw, uint8_t* q, int32_t* sb,
                                        int N, int K, void* stream);

/* Row alignment of each expert segment in the contiguous layout: 128. */
int fg_get_mk_alignment_for_contiguous_layout(void);

/* Cap on the compute units the GEMM kernels spread their persistent workgroups
 * over (the digest's set_num_sms); 0 (the default) means all of them.
 * Results do not depend on the cap (every tile is computed whole by one
 * workgroup).  Process-wide, not thread-safe against concurrent launches. */
void fg_set_num_cus(int n);
int fg_get_num_cus(void);

/* Description of the last failure on this thread ("" after success). */
const char* fg_last_error(void);

/* Library version string. */
const char* fg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H */
