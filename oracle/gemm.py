"""Fine-grained-scaled FP8 GEMM, dense / M-grouped contiguous / M-grouped masked.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Operation (DeepGEMM digest, GeekNews topic 19459, "GEMM arayuzu ve yerlesim
kisitlari"): the NT GEMM D = A @ B.T with A [M, K] row-major and B [N, K]
(K-contiguous rows), and D = C + A @ B.T with an fp32 addend C (the digest's
naming convention for every GEMM kernel; ``gemm_nt_addend``).  The
fp32 accumulation is "promoted" once per 128-wide K slice (GeekNews topic
19444, opening bullets; 7minutos.es, "Detalles y beneficios tecnicos"):

    a[m,k] = dec(A[m,k]) * sa[k//128][m]
    b[n,k] = dec(B[n,k]) * sb[n//128][k//128]
    X[m,n] = sum_k a[m,k] * b[n,k]                (float64, the true value)
    D[m,n] = bf16_RNE(X[m,n])                      (expected output)
    S[m,n] = sum_k |a[m,k] * b[n,k]|              (magnitude for error bounds)

The promotion only changes where rounding happens, not the value computed,
so the oracle evaluates the definition.  Two forms are provided and
cross-checked in the tests:

(i)  ``gemm_blockwise``: per 128-K slice, the float64 product of the decoded
     codes (exact: every e4m3 value is a multiple of 2^-9 below 2^9, so a
     128-term slice sum has at most 43 significant bits), then scaled by
     sa*sb (exact in float64) and accumulated in float64.
(ii) ``gemm_dequant``: decode-and-scale both operands (exact in float64),
     then one float64 matmul.

Grouped forms ("Dense ve Grouped GEMM" of the same digest):

* contiguous: experts share N and K; each row r of A belongs to expert
  m_indices[r] and uses B[m_indices[r]], sb[m_indices[r]].  Reading for the
  padding rows the pages leave open: an index < 0 marks a padding row whose
  output is left untouched.
* masked: group g computes rows [0, min(max(mask[g], 0), M_cap)) of A[g]
  against B[g]; all other rows of D[g] are left untouched.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import decode, bf16_rne_bits

GROUP = 128


def _check_dense(A, sa, B, sb):
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B need the same K")
    Kb = -(-K // GROUP)  # a last, partial K group when K % 128 != 0
    Nb = -(-N // GROUP)
    if sa.shape[0] != Kb or sa.shape[1] < M:
        raise ValueError(f"sa must be [ceil(K/128), >=M], got {sa.shape}")
    if sb.shape != (Nb, Kb):
        raise ValueError(f"sb must be [ceil(N/128), ceil(K/128)], got {sb.shape}")
    return M, N, K, Kb


def gemm_blockwise(A, sa, B, sb, with_magnitude: bool = False):
    """Form (i).  A uint8 [M,K], sa f32 [K/128, >=M], B uint8 [N,K], sb f32 [Nb,Kb].

    Returns X float64 [M, N] (and S when ``with_magnitude``).
    """
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    sa = np.asarray(sa, np.float32)
    sb = np.asarray(sb, np.float32)
    M, N, K, Kb = _check_dense(A, sa, B, sb)
    a = decode(A)
    b = decode(B)
    nblk = np.arange(N) // GROUP
    X = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64) if with_magnitude else None
    for kb in range(Kb):
        ks = slice(kb * GROUP, min(K, (kb + 1) * GROUP))
        P = a[:, ks] @ b[:, ks].T  # exact slice partial
        scale = sa[kb, :M].astype(np.float64)[:, None] * sb[nblk, kb].astype(np.float64)[None, :]
        X += P * scale
        if with_magnitude:
            S += (np.abs(a[:, ks]) @ np.abs(b[:, ks]).T) * np.abs(scale)
    return (X, S) if with_magnitude else X


def gemm_dequant(A, sa, B, sb, with_magnitude: bool = False):
    """Form (ii): dequantise both operands exactly, then one float64 matmul
    (and, with ``with_magnitude``, S = |a| @ |b|.T of the same operands)."""
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    sa = np.asarray(sa, np.float32)
    sb = np.asarray(sb, np.float32)
    M, N, K, Kb = _check_dense(A, sa, B, sb)
    kblk = np.arange(K) // GROUP
    nblk = np.arange(N) // GROUP
    a = decode(A) * sa[kblk, :M].T.astype(np.float64)
    b = decode(B) * sb[nblk][:, kblk].astype(np.float64)
    X = a @ b.T
    if with_magnitude:
        return X, np.abs(a) @ np.abs(b).T
    return X


def gemm_nt(A, sa, B, sb, with_magnitude: bool = False):
    """Dense NT GEMM: float64 X (and S).  Use ``to_bf16`` for the D bits."""
    return gemm_blockwise(A, sa, B, sb, with_magnitude=with_magnitude)


def gemm_nt_addend(A, sa, B, sb, C, with_magnitude: bool = False):
    """D = C + A @ B.T (GeekNews topic 19459, "GEMM arayuzu ve yerlesim
    kisitlari": the kernels are named after D = C + A @ B).  Reading where the
    pages are silent: C is float32 [M, N], added once to the exact product
    before the single BF16 rounding of D; |C| joins the magnitude S."""
    C = np.asarray(C, np.float32).astype(np.float64)
    X, S = gemm_blockwise(A, sa, B, sb, with_magnitude=True)
    if C.shape != X.shape:
        raise ValueError(f"C has shape {C.shape}, expected {X.shape}")
    X = X + C
    return (X, S + np.abs(C)) if with_magnitude else X


def gemm_layout(layout: str, A, sa, B, sb, C=None, with_magnitude: bool = False):
    """The four storage layouts (GeekNews topic 19459, "Dense ve Grouped GEMM":
    fp8_gemm_{nt, nn, tn, tt}).  Reading: the first letter says whether the
    stored A is used as is ("n", A [M, K]) or transposed ("t", A stored
    [K, M]); the second the same for B, where "t" is the NT form's B [N, K]
    (D = A @ B.T) and "n" stores B as [K, N] (D = A @ B).  The scale factors
    belong to the logical operands -- A as [M, K] with sa [Kb][M], B as
    [N, K] with sb [Nb][Kb] -- whatever the storage.  A transpose of the
    stored codes gives the NT operands; C is the optional fp32 addend."""
    if layout not in ("nt", "nn", "tn", "tt"):
        raise ValueError(f"layout {layout!r}")
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    a = A.T if layout[0] == "t" else A
    b = B.T if layout[1] == "n" else B
    if C is None:
        return gemm_blockwise(a, sa, b, sb, with_magnitude=with_magnitude)
    return gemm_nt_addend(a, sa, b, sb, C, with_magnitude=with_magnitude)


def gemm_k_grouped_tn(A, sa, B, sb, ks, C=None, with_magnitude: bool = False):
    """K-grouped TN GEMM for MoE weight gradients (GeekNews topic 19459,
    "Dense ve Grouped GEMM": grouped along K, M and N fixed,
    k_grouped_fp8_gemm_tn_contiguous).  A is stored [K_total, M] and B
    [K_total, N]; group g owns the ks[g] consecutive K rows starting at
    sum(ks[:g]) and gives D[g] = C[g] + A_g^T @ B_g, [M, N].

    Readings where the pages are silent: every ks[g] is a multiple of 128
    (zero allowed: D[g] = C[g], or 0); the scale factors are those of the
    dense form over the whole K range -- sa [Kb_total][M] (1x128 along K) and
    sb [Nb][Kb_total] (128x128 blocks of the logical [N, K] operand) -- and
    group g uses their K groups sum(ks[:g])/128 ..; C is an optional fp32
    [G, M, N] addend."""
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    sa = np.asarray(sa, np.float32)
    sb = np.asarray(sb, np.float32)
    ks = [int(k) for k in ks]
    if any(k < 0 or k % GROUP for k in ks) or sum(ks) != A.shape[0] or B.shape[0] != A.shape[0]:
        raise ValueError(f"group sizes {ks} do not tile K_total = {A.shape[0]} in multiples of {GROUP}")
    M, N = A.shape[1], B.shape[1]
    G = len(ks)
    X = np.zeros((G, M, N))
    S = np.zeros((G, M, N))
    k0 = 0
    for g, k in enumerate(ks):
        kb0, kb1 = k0 // GROUP, (k0 + k) // GROUP
        if k:
            X[g], S[g] = gemm_blockwise(A[k0:k0 + k].T, sa[kb0:kb1], B[k0:k0 + k].T, sb[:, kb0:kb1],
                                        with_magnitude=True)
        if C is not None:
            c = np.asarray(C[g], np.float32).astype(np.float64)
            X[g] += c
            S[g] += np.abs(c)
        k0 += k
    return (X, S) if with_magnitude else X


def to_bf16(X) -> np.ndarray:
    """Expected BF16 output bits, D = bf16_RNE(X)."""
    return bf16_rne_bits(X)


def gemm_grouped_contiguous(A, sa, B, sb, m_indices, with_magnitude: bool = False):
    """Contiguous M-grouped GEMM.

    A uint8 [M_total, K]; sa f32 [K/128, >=M_total];
    B uint8 [G, N, K]; sb f32 [G, Nb, Kb]; m_indices int [M_total].
    Returns (X float64 [M_total, N], valid bool [M_total]) (+ S).
    Rows with m_indices < 0 are not valid: their X rows are 0 and the
    library must leave them untouched.
    """
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    sa = np.asarray(sa, np.float32)
    sb = np.asarray(sb, np.float32)
    idx = np.asarray(m_indices).astype(np.int64)
    G, N, K = B.shape
    M = A.shape[0]
    if idx.shape != (M,):
        raise ValueError("m_indices must have one entry per row of A")
    if (idx >= G).any():
        raise ValueError("expert index out of range")
    X = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64) if with_magnitude else None
    for e in np.unique(idx[idx >= 0]):
        rows = np.nonzero(idx == e)[0]
        res = gemm_blockwise(A[rows], sa[:, rows], B[e], sb[e], with_magnitude=with_magnitude)
        if with_magnitude:
            X[rows], S[rows] = res
        else:
            X[rows] = res
    valid = idx >= 0
    return (X, valid, S) if with_magnitude else (X, valid)


def gemm_grouped_masked(A, sa, B, sb, masked_m, with_magnitude: bool = False):
    """Masked M-grouped GEMM.

    A uint8 [G, M_cap, K]; sa f32 [G, K/128, >=M_cap];
    B uint8 [G, N, K]; sb f32 [G, Nb, Kb]; masked_m int [G].
    Returns (X float64 [G, M_cap, N], valid bool [G, M_cap]) (+ S).
    """
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    sa = np.asarray(sa, np.float32)
    sb = np.asarray(sb, np.float32)
    mask = np.asarray(masked_m).astype(np.int64)
    G, M_cap, K = A.shape
    N = B.shape[1]
    if mask.shape != (G,):
        raise ValueError("masked_m must have one entry per group")
    X = np.zeros((G, M_cap, N), dtype=np.float64)
    S = np.zeros((G, M_cap, N), dtype=np.float64) if with_magnitude else None
    valid = np.zeros((G, M_cap), dtype=bool)
    for g in range(G):
        rows = int(min(max(mask[g], 0), M_cap))
        valid[g, :rows] = True
        if rows == 0:
            continue
        res = gemm_blockwise(A[g, :rows], sa[g][:, :rows], B[g], sb[g], with_magnitude=with_magnitude)
        if with_magnitude:
            X[g, :rows], S[g, :rows] = res
        else:
            X[g, :rows] = res
    return (X, valid, S) if with_magnitude else (X, valid)
