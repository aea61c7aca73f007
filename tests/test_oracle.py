"""Pins for the CPU oracle: each check ties it to something other than itself.

* e4m3fn decode/encode and bf16 rounding against torch's own conversions
  (library routines) and against the formats' closed-form special values;
* the GEMM against exact rational brute force (``fractions.Fraction``) on
  tiny shapes, against a closed form, against integer matmul in an exactly
  representable regime, and through linearity in each block scale;
* the grouped forms against per-row brute force and their reduction to dense;
* the quantiser against torch's conversion of the same fp32 quotients and
  against its defining invariants;
* the power-of-two (UE8M0) factors against torch's log2/ceil, a hand-written
  packing layout, and their reduction to the fp32 mode when a factor is
  already a power of two.
"""

from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3, quant, gemm, metrics
import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# --------------------------------------------------------------------------
# e4m3fn codec


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x32, np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3.decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero is kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_closed_form_specials():
    d = e4m3.decode(np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0xB8, 0xFE, 0x7F, 0xFF], np.uint8))
    assert d[0] == 448.0
    assert d[1] == 2.0 ** -6  # smallest normal
    assert d[2] == 7 * 2.0 ** -9  # largest subnormal
    assert d[3] == 2.0 ** -9  # smallest subnormal
    assert d[4] == 1.0 and d[5] == -1.0 and d[6] == -448.0
    assert np.isnan(d[7]) and np.isnan(d[8])
    finite = e4m3.decode(np.arange(256, dtype=np.uint8))
    finite = finite[~np.isnan(finite)]
    assert len(finite) == 254 and np.abs(finite).max() == 448.0


def test_encode_ties_and_specials():
    vals = np.array([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 464.0, 449.0, 0.0, -0.0, -1e-10], np.float32)
    codes = e4m3.encode_rne(vals)
    assert list(codes) == [0x38, 0x3A, 0x02, 0x00, 0x7E, 0x7E, 0x00, 0x80, 0x80]
    with pytest.raises(OverflowError):
        e4m3.encode_rne(np.array([465.0], np.float32))


def test_encode_matches_torch_on_every_midpoint_and_random():
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    mids = (pos[:-1] + pos[1:]) / 2  # exact in fp32: adjacent values share an exponent step
    just = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)), np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(200_000) * rng.choice([1e-3, 0.05, 1, 30, 150], 200_000)).astype(np.float32)
    rnd = rnd[np.abs(rnd) < 448]
    x = np.concatenate([pos, mids, just, rnd]).astype(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(e4m3.encode_rne(x), torch_encode(x))


def test_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(e4m3.encode_rne(e4m3.decode(codes)), codes)


# --------------------------------------------------------------------------
# bf16 rounding


def torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x32, np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_closed_forms():
    bits = e4m3.bf16_rne_bits(np.array([257.0, 259.0, 1.0, -2.5, 0.0, -0.0, 1e40]))
    vals = e4m3.bf16_bits_to_f64(bits)
    assert list(vals[:4]) == [256.0, 260.0, 1.0, -2.5]
    assert bits[4] == 0x0000 and bits[5] == 0x8000
    assert np.isinf(vals[6])


def test_bf16_matches_torch_for_fp32_inputs():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300_000) * np.exp(rng.uniform(-60, 60, 300_000))).astype(np.float32)
    # exact ties: 8 significant bits plus a half
    ties = ((rng.integers(128, 256, 1000) * 2 + 1) * np.exp2(rng.integers(-30, 30, 1000))).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    assert np.array_equal(e4m3.bf16_rne_bits(x.astype(np.float64)), torch_bf16_bits(x))


def test_bf16_rounds_float64_directly():
    # 1 + 2^-8 + 2^-40 is above the tie: rounds up in one step; a detour via
    # fp32 would first drop 2^-40 and then tie to even (down).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert e4m3.bf16_bits_to_f64(e4m3.bf16_rne_bits(np.array([x])))[0] == 1.0 + 2.0 ** -7


# --------------------------------------------------------------------------
# quantiser


def test_quantize_per_token_matches_torch_conversion():
    A, _ = synth.dense_problem(64, 8, 512, seed=3)
    x = A.numpy()
    q, sa = quant.quantize_per_token(x)
    assert q.shape == x.shape and sa.shape == (4, 64) and sa.dtype == np.float32
    xt = torch.from_numpy(x).view(64, 4, 128)
    amax = xt.abs().amax(dim=2)
    s = torch.clamp(amax, min=torch.tensor(1e-4, dtype=torch.float32)) / 448.0
    assert np.array_equal(sa, s.T.numpy())
    ref = (xt / s[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 512).numpy()
    assert np.array_equal(q, ref)


def test_quantize_invariants_and_zero_group():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 384)).astype(np.float32) * np.float32(7.5)
    x[2, 128:256] = 0.0
    q, sa = quant.quantize_per_token(x)
    dq = e4m3.decode(q).reshape(5, 3, 128)
    # each non-zero group reaches the format maximum exactly once-or-more
    for m, kb in itertools.product(range(5), range(3)):
        if (m, kb) == (2, 1):
            assert (q.reshape(5, 3, 128)[m, kb] == 0).all()
            assert sa[kb, m] == np.float32(np.float32(1e-4) / np.float32(448))
            continue
        assert np.abs(dq[m, kb]).max() == 448.0
    # reconstruction error within half an e4m3 step (relative 2^-4) plus fp32 division rounding
    rec = dq * sa.T[:, :, None]
    err = np.abs(rec - x.reshape(5, 3, 128))
    tol = np.maximum(np.abs(x.reshape(5, 3, 128)) * 2.0 ** -4, 2.0 ** -10 * sa.T[:, :, None]) * (1 + 2.0 ** -20)
    assert (err <= tol).all()


def test_quantize_per_block_tail_rows_use_their_own_amax():
    _, B = synth.dense_problem(1, 2112, 256, seed=4)
    w = B.numpy()
    q, sb = quant.quantize_per_block(w)
    assert sb.shape == (17, 2)
    q_tail, sb_tail = quant.quantize_per_block(w[2048:])  # the 64-row tail on its own
    assert np.array_equal(sb[16], sb_tail[0]) and np.array_equal(q[2048:], q_tail)
    # each block's scale equals its own amax / 448
    for nb, kb in [(0, 0), (5, 1), (16, 1)]:
        blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
        assert sb[nb, kb] == np.float32(np.abs(blk).max()) / np.float32(448)
    # against torch's conversion of the same fp32 quotients
    sbt = torch.from_numpy(np.repeat(np.repeat(sb, 128, 0)[:2112], 128, 1))
    ref = (torch.from_numpy(w) / sbt).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


# --------------------------------------------------------------------------
# GEMM


def _random_problem(rng, M, N, K, codes_from=None):
    """Random finite codes and positive fp32 scales (no quantiser involved)."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    pool = finite if codes_from is None else np.asarray(codes_from, np.uint8)
    A = rng.choice(pool, (M, K))
    B = rng.choice(pool, (N, K))
    Kb, Nb = K // 128, -(-N // 128)
    sa = np.exp(rng.uniform(-8, 8, (Kb, M))).astype(np.float32)
    sb = np.exp(rng.uniform(-8, 8, (Nb, Kb))).astype(np.float32)
    return A, sa, B, sb


def _fraction_gemm(A, sa, B, sb):
    """Exact rational X and S, decoding with torch and looping over every term."""
    da, db = torch_decode(A), torch_decode(B)
    M, K = A.shape
    N = B.shape[0]
    X = np.empty((M, N), dtype=object)
    S = np.empty((M, N), dtype=object)
    fa = [[Fraction(float(da[m, k])) * Fraction(float(sa[k // 128, m])) for k in range(K)] for m in range(M)]
    fb = [[Fraction(float(db[n, k])) * Fraction(float(sb[n // 128, k // 128])) for k in range(K)] for n in range(N)]
    for m in range(M):
        for n in range(N):
            terms = [fa[m][k] * fb[n][k] for k in range(K)]
            X[m, n] = sum(terms, Fraction(0))
            S[m, n] = sum((abs(t) for t in terms), Fraction(0))
    return X, S


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 130, 128), (2, 260, 256), (3, 1, 384)])
def test_gemm_matches_exact_rational_bruteforce(M, N, K):
    rng = np.random.default_rng(M * 1000 + N + K)
    A, sa, B, sb = _random_problem(rng, M, N, K)
    X, S = gemm.gemm_nt(A, sa, B, sb, with_magnitude=True)
    Xe, Se = _fraction_gemm(A, sa, B, sb)
    for m, n in itertools.product(range(M), range(N)):
        assert abs(Fraction(float(X[m, n])) - Xe[m, n]) <= Fraction(2) ** -50 * Se[m, n]
        assert abs(Fraction(float(S[m, n])) - Se[m, n]) <= Fraction(2) ** -50 * Se[m, n]


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 130, 256), (2, 5, 384)])
def test_addend_matches_exact_rational_bruteforce(M, N, K):
    """D = C + A @ B.T against Fraction sums; C holds values of every size,
    including ones that cancel the product exactly."""
    rng = np.random.default_rng(M * 7 + N + K)
    A, sa, B, sb = _random_problem(rng, M, N, K)
    Xe, Se = _fraction_gemm(A, sa, B, sb)
    C = (rng.standard_normal((M, N)) * 10.0 ** rng.integers(-3, 4, (M, N))).astype(np.float32)
    C[0, 0] = np.float32(-float(Xe[0, 0]))  # cancellation: X = product - fp32(product)
    X, S = gemm.gemm_nt_addend(A, sa, B, sb, C, with_magnitude=True)
    for m, n in itertools.product(range(M), range(N)):
        c = Fraction(float(C[m, n]))
        assert abs(Fraction(float(X[m, n])) - (Xe[m, n] + c)) <= Fraction(2) ** -50 * (Se[m, n] + abs(c))
        assert Fraction(float(S[m, n])) - (Se[m, n] + abs(c)) <= Fraction(2) ** -50 * (Se[m, n] + abs(c))


def test_addend_bf16_rounds_the_sum_once():
    """bf16(C + P) is not bf16(C) + bf16(P): with P = 1 and C = 2^-8 + 2^-16
    the sum rounds up to 1 + 2^-7 while the separately rounded terms give 1."""
    A = np.full((1, 128), 0x38, np.uint8)  # 1.0
    B = np.zeros((1, 128), np.uint8)
    B[0, 0] = 0x38
    sa = np.ones((1, 1), np.float32)
    sb = np.ones((1, 1), np.float32)
    C = np.array([[2.0 ** -8 + 2.0 ** -16]], np.float32)
    X = gemm.gemm_nt_addend(A, sa, B, sb, C)
    assert X[0, 0] == 1 + 2.0 ** -8 + 2.0 ** -16
    bits = int(gemm.to_bf16(X)[0, 0])
    assert bits == 0x3F81  # 1 + 2^-7


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
def test_layouts_match_bruteforce_on_stored_arrays(layout):
    """Each layout against Fraction sums that index the stored arrays directly
    (A[k, m] when A is stored transposed, B[k, n] when B is stored [K, N])."""
    M, N, K = 3, 5, 256
    rng = np.random.default_rng(len(layout) + ord(layout[0]) * 3 + ord(layout[1]))
    A, sa, B, sb = _random_problem(rng, M, N, K)
    As = np.ascontiguousarray(A.T) if layout[0] == "t" else A
    Bs = np.ascontiguousarray(B.T) if layout[1] == "n" else B
    C = rng.standard_normal((M, N)).astype(np.float32)
    X, S = gemm.gemm_layout(layout, As, sa, Bs, sb, C=C, with_magnitude=True)
    da, db = torch_decode(As), torch_decode(Bs)
    for m, n in itertools.product(range(M), range(N)):
        terms = []
        for k in range(K):
            a = da[k, m] if layout[0] == "t" else da[m, k]
            b = db[k, n] if layout[1] == "n" else db[n, k]
            terms.append(Fraction(float(a)) * Fraction(float(sa[k // 128, m])) * Fraction(float(b))
                         * Fraction(float(sb[n // 128, k // 128])))
        c = Fraction(float(C[m, n]))
        se = sum((abs(t) for t in terms), Fraction(0)) + abs(c)
        assert abs(Fraction(float(X[m, n])) - (sum(terms, Fraction(0)) + c)) <= Fraction(2) ** -50 * se
    X0 = gemm.gemm_layout(layout, As, sa, Bs, sb)
    assert np.array_equal(X0, gemm.gemm_nt(A, sa, B, sb))


def test_k_grouped_tn_matches_bruteforce():
    """Three groups along K, one of them empty, against Fraction sums over the
    stored [K_total, .] arrays; the group's scale columns start at its first
    K group."""
    M, N, ks = 3, 130, [256, 0, 128]
    Kt = sum(ks)
    rng = np.random.default_rng(31)
    A, sa, B, sb = _random_problem(rng, M, N, Kt)  # NT codes, scales over K_total
    As, Bs = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    C = rng.standard_normal((len(ks), M, N)).astype(np.float32)
    X, S = gemm.gemm_k_grouped_tn(As, sa, Bs, sb, ks, C=C, with_magnitude=True)
    da, db = torch_decode(As), torch_decode(Bs)
    k0 = 0
    for g, kg in enumerate(ks):
        for m, n in itertools.product(range(M), (0, 1, 127, 128, 129)):
            terms = [Fraction(float(da[k, m])) * Fraction(float(sa[k // 128, m])) * Fraction(float(db[k, n]))
                     * Fraction(float(sb[n // 128, k // 128])) for k in range(k0, k0 + kg)]
            c = Fraction(float(C[g, m, n]))
            se = sum((abs(t) for t in terms), Fraction(0)) + abs(c)
            assert abs(Fraction(float(X[g, m, n])) - (sum(terms, Fraction(0)) + c)) <= Fraction(2) ** -50 * se
            assert abs(Fraction(float(S[g, m, n])) - se) <= Fraction(2) ** -50 * se
        k0 += kg
    # one group is the dense TN layout
    X1 = gemm.gemm_k_grouped_tn(As, sa, Bs, sb, [Kt])
    assert np.array_equal(X1[0], gemm.gemm_layout("tn", As, sa, Bs, sb))
    with pytest.raises(ValueError):
        gemm.gemm_k_grouped_tn(As, sa, Bs, sb, [200, 184])


@pytest.mark.parametrize("M,N,K", [(2, 3, 16), (3, 130, 176), (2, 5, 304)])
def test_k_tail_gemm_matches_bruteforce(M, N, K):
    """K % 128 != 0: the last K group is partial; Fraction sums over all K."""
    rng = np.random.default_rng(K + M)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    Kb, Nb = -(-K // 128), -(-N // 128)
    A = rng.choice(finite, (M, K))
    B = rng.choice(finite, (N, K))
    sa = np.exp(rng.uniform(-8, 8, (Kb, M))).astype(np.float32)
    sb = np.exp(rng.uniform(-8, 8, (Nb, Kb))).astype(np.float32)
    X, S = gemm.gemm_nt(A, sa, B, sb, with_magnitude=True)
    Xe, Se = _fraction_gemm(A, sa, B, sb)
    for m, n in itertools.product(range(M), range(N)):
        assert abs(Fraction(float(X[m, n])) - Xe[m, n]) <= Fraction(2) ** -50 * Se[m, n]
        assert abs(Fraction(float(S[m, n])) - Se[m, n]) <= Fraction(2) ** -50 * Se[m, n]
    assert np.allclose(X, gemm.gemm_dequant(A, sa, B, sb), rtol=0, atol=1e-12 * S.max())
    # the dequantised form's magnitude against the exact sums as well
    _, S2 = gemm.gemm_dequant(A, sa, B, sb, with_magnitude=True)
    for m, n in itertools.product(range(M), range(N)):
        assert abs(Fraction(float(S2[m, n])) - Se[m, n]) <= Fraction(2) ** -50 * Se[m, n]


def test_k_tail_quantisers_match_torch_on_their_own_columns():
    """The partial last group's factor is max(amax, 1e-4)/448 over its own
    columns, its codes torch's RNE of x / s; full groups are unaffected."""
    A, B = synth.dense_problem(5, 130, 208, seed=4)
    x, w = A.numpy(), B.numpy()
    q, sa = quant.quantize_per_token(x)
    assert q.shape == (5, 208) and sa.shape == (2, 5)
    tail = torch.from_numpy(x[:, 128:])
    s = torch.clamp(tail.abs().amax(dim=1), min=torch.tensor(1e-4, dtype=torch.float32)) / 448.0
    assert np.array_equal(sa[1], s.numpy())
    ref = (tail / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[:, 128:], ref)
    q0, sa0 = quant.quantize_per_token(x[:, :128])
    assert np.array_equal(q[:, :128], q0) and np.array_equal(sa[:1], sa0)
    qb, sb = quant.quantize_per_block(w)
    assert qb.shape == (130, 208) and sb.shape == (2, 2)
    for nb, rows in ((0, slice(0, 128)), (1, slice(128, 130))):
        blk = torch.from_numpy(w[rows, 128:])
        s = torch.clamp(blk.abs().amax(), min=torch.tensor(1e-4, dtype=torch.float32)) / 448.0
        assert sb[nb, 1] == s.item()
        ref = (blk / s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(qb[rows, 128:], ref)


def test_two_oracle_forms_agree():
    rng = np.random.default_rng(7)
    A, sa, B, sb = _random_problem(rng, 48, 300, 640)
    X1, S = gemm.gemm_blockwise(A, sa, B, sb, with_magnitude=True)
    X2 = gemm.gemm_dequant(A, sa, B, sb)
    assert (np.abs(X1 - X2) <= 1e-12 * S).all()
    X3, S3 = gemm.gemm_dequant(A, sa, B, sb, with_magnitude=True)
    assert np.array_equal(X3, X2)
    assert (np.abs(S3 - S) <= 1e-12 * S).all()


def test_gemm_closed_form_constant_codes():
    for c, d, K in [(0x38, 0x40, 256), (0x7E, 0xB0, 512), (0x01, 0x44, 128)]:  # 1*2, 448*-0.5, 2^-9*3
        A = np.full((4, K), c, np.uint8)
        B = np.full((6, K), d, np.uint8)
        sa = np.ones((K // 128, 4), np.float32)
        sb = np.ones((1, K // 128), np.float32)
        X = gemm.gemm_nt(A, sa, B, sb)
        cv, dv = e4m3.decode(np.array([c, d], np.uint8))
        assert (X == K * cv * dv).all()


def exact_regime_problem(rng, M, N, K):
    """Integer codes in [-4, 4], power-of-two scales: every fp32 step is exact."""
    ints = np.arange(-4, 5, dtype=np.float32)
    pool = torch_encode(ints)
    A, sa, B, sb = _random_problem(rng, M, N, K, codes_from=pool)
    sa = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), sa.shape)
    sb = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), sb.shape)
    return A, sa, B, sb


def test_gemm_exact_regime_matches_integer_matmul():
    rng = np.random.default_rng(11)
    M, N, K = 40, 200, 1024
    A, sa, B, sb = exact_regime_problem(rng, M, N, K)
    ia = torch_decode(A).astype(np.int64)
    ib = torch_decode(B).astype(np.int64)
    # scales are 2^e with e in {-1,0,1}: scale everything by 4 to stay integer
    total = np.zeros((M, N), np.int64)
    for kb in range(K // 128):
        ks = slice(kb * 128, kb * 128 + 128)
        p = ia[:, ks] @ ib[:, ks].T
        ea = (sa[kb] * 2).astype(np.int64)  # 1, 2, 4
        eb = (sb[np.arange(N) // 128, kb] * 2).astype(np.int64)
        total += p * ea[:, None] * eb[None, :]
    X = gemm.gemm_nt(A, sa, B, sb)
    assert np.array_equal(X * 4, total.astype(np.float64))


def test_gemm_linear_in_each_block_scale():
    rng = np.random.default_rng(13)
    A, sa, B, sb = _random_problem(rng, 6, 260, 384)
    ts = [np.float32(0.25), np.float32(1.5), np.float32(6.0)]
    # activation scale of (row 4, slice 1)
    xs = []
    for t in ts:
        s2 = sa.copy()
        s2[1, 4] = t
        xs.append(gemm.gemm_nt(A, s2, B, sb))
    for X in xs:  # other rows do not move
        assert np.array_equal(np.delete(X, 4, 0), np.delete(xs[0], 4, 0))
    slope1 = (xs[1][4] - xs[0][4]) / float(ts[1] - ts[0])
    slope2 = (xs[2][4] - xs[1][4]) / float(ts[2] - ts[1])
    assert np.allclose(slope1, slope2, rtol=1e-9, atol=1e-9 * np.abs(xs[2][4]).max())
    # slope is sb * (exact partial of that slice): check against the decoded slice product
    P = torch_decode(A)[4, 128:256] @ torch_decode(B)[:, 128:256].T
    assert np.allclose(slope1, P * sb[np.arange(260) // 128, 1], rtol=1e-9, atol=1e-12)
    # weight scale of block (nb=2, kb=0): only columns 256..259 move
    ys = []
    for t in ts:
        s2 = sb.copy()
        s2[2, 0] = t
        ys.append(gemm.gemm_nt(A, sa, B, s2))
    assert np.array_equal(ys[0][:, :256], ys[2][:, :256])
    assert not np.array_equal(ys[0][:, 256:], ys[2][:, 256:])


def test_contiguous_reduces_to_dense_and_bruteforce():
    rng = np.random.default_rng(17)
    idx = synth.contiguous_indices([130, 0, 100], pad_to=128)  # uneven groups, an empty one, padding
    M, N, K, G = idx.shape[0], 140, 256, 3
    A = rng.choice(np.arange(0x7F, dtype=np.uint8), (M, K))
    B = rng.choice(np.arange(0x7F, dtype=np.uint8), (G, N, K))
    sa = np.exp(rng.uniform(-3, 3, (2, M))).astype(np.float32)
    sb = np.exp(rng.uniform(-3, 3, (G, 2, 2))).astype(np.float32)
    X, valid = gemm.gemm_grouped_contiguous(A, sa, B, sb, idx)
    assert np.array_equal(valid, idx >= 0)
    assert (X[~valid] == 0).all()
    for e in range(G):
        rows = np.nonzero(idx == e)[0]
        if len(rows):
            assert np.array_equal(X[rows], gemm.gemm_nt(A[rows], sa[:, rows], B[e], sb[e]))
    # brute force a few rows, each with the expert its index names
    for r in [0, 129, 130, 256, 355]:
        e = idx[r]
        if e < 0:
            continue
        Xe, Se = _fraction_gemm(A[r:r + 1], sa[:, r:r + 1], B[e], sb[e])
        for n in range(N):
            assert abs(Fraction(float(X[r, n])) - Xe[0, n]) <= Fraction(2) ** -50 * Se[0, n]


def test_masked_reduces_to_dense_and_respects_mask():
    rng = np.random.default_rng(19)
    G, Mc, N, K = 4, 40, 130, 256
    A = rng.choice(np.arange(0x7F, dtype=np.uint8), (G, Mc, K))
    B = rng.choice(np.arange(0x7F, dtype=np.uint8), (G, N, K))
    sa = np.exp(rng.uniform(-3, 3, (G, 2, Mc))).astype(np.float32)
    sb = np.exp(rng.uniform(-3, 3, (G, 2, 2))).astype(np.float32)
    mask = np.array([0, 40, 17, -5], np.int32)
    X, valid = gemm.gemm_grouped_masked(A, sa, B, sb, mask)
    assert valid.sum(axis=1).tolist() == [0, 40, 17, 0]
    assert (X[~valid] == 0).all()
    assert np.array_equal(X[1], gemm.gemm_nt(A[1], sa[1], B[1], sb[1]))
    assert np.array_equal(X[2, :17], gemm.gemm_nt(A[2, :17], sa[2][:, :17], B[2], sb[2]))
    # mask above capacity is clamped
    X2, valid2 = gemm.gemm_grouped_masked(A, sa, B, sb, np.array([99, 0, 0, 0], np.int32))
    assert valid2[0].all() and np.array_equal(X2[0], X[1] * 0 + gemm.gemm_nt(A[0], sa[0], B[0], sb[0]))


# --------------------------------------------------------------------------
# metrics and planted mistakes (mistakes are planted in the oracle's inputs or
# results on the CPU, never in device code)


def test_metrics_accept_fp32_promotion_and_reject_dropped_slice():
    rng = np.random.default_rng(23)
    A, sa, B, sb = _random_problem(rng, 32, 256, 1024, codes_from=np.arange(0x70, dtype=np.uint8))
    X, S = gemm.gemm_nt(A, sa, B, sb, with_magnitude=True)
    Kb = 8
    # an fp32 emulation of the promoted accumulation (different rounding order)
    da, db = torch_decode(A).astype(np.float32), torch_decode(B).astype(np.float32)
    acc = np.zeros((32, 256), np.float32)
    for kb in range(Kb):
        ks = slice(kb * 128, kb * 128 + 128)
        P = (da[:, ks] @ db[:, ks].T).astype(np.float32)
        s = (sa[kb][:, None] * sb[np.arange(256) // 128, kb][None, :]).astype(np.float32)
        acc = (acc + P * s).astype(np.float32)
    y = e4m3.bf16_bits_to_f64(e4m3.bf16_rne_bits(acc.astype(np.float64)))
    rep = metrics.check_result(y, X, S, Kb)
    assert rep["ok"], rep
    # a dropped slice fails
    Xd = gemm.gemm_nt(A[:, :896], sa[:7], B[:, :896], sb[:, :7])
    assert not metrics.check_result(Xd, X, S, Kb)["ok"]
    # a transposed scale index (sb[kb][nb] instead of sb[nb][kb]) fails
    sbt = np.ascontiguousarray(sb.T[:2, :2])
    A2, sa2, B2 = A[:, :256], sa[:2], B[:, :256]
    Xt = gemm.gemm_nt(A2, sa2, B2, sbt)
    X2, S2 = gemm.gemm_nt(A2, sa2, B2, sb[:, :2], with_magnitude=True)
    if not np.array_equal(sbt, sb[:, :2]):
        assert not metrics.check_result(Xt, X2, S2, 2)["ok"]
    # a sign error fails
    assert not metrics.check_result(-y, X, S, Kb)["ok"]


@pytest.mark.parametrize("bits,ok", [(16, True), (12, False)])
def test_metrics_level_of_the_matrix_core_term(bits, ok):
    """A slice sum that aligns its 128 products to the largest one's exponent
    and truncates each to `bits` bits below it: with 16 bits (coarser than
    any error measured on the device) it stays inside the bound, with 12 the
    cancelling sums, where the 1e-2 term gives no room, fall outside."""
    rng = np.random.default_rng(31)
    M, N, K = 48, 64, 384
    A = rng.integers(0, 0x7F, (M, K), dtype=np.uint8)
    B = rng.integers(0, 0x7F, (N, K), dtype=np.uint8)
    A[:, ::2] |= 0x80  # half the products negative: sums cancel
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones((1, K // 128), np.float32)
    X, S = gemm.gemm_nt(A, sa, B, sb, with_magnitude=True)
    da, db = torch_decode(A).astype(np.float64), torch_decode(B).astype(np.float64)
    acc = np.zeros((M, N), np.float32)
    for kb in range(K // 128):
        ks = slice(kb * 128, kb * 128 + 128)
        prod = da[:, None, ks] * db[None, :, ks]  # exact
        top = np.floor(np.log2(np.maximum(np.abs(prod).max(axis=2, keepdims=True), 2.0 ** -40)))
        q = 2.0 ** (top - bits)
        P = (np.trunc(prod / q) * q).sum(axis=2).astype(np.float32)
        acc = (acc + P).astype(np.float32)
    y = e4m3.bf16_bits_to_f64(e4m3.bf16_rne_bits(acc.astype(np.float64)))
    assert metrics.check_result(y, X, S, K // 128)["ok"] == ok


def test_planted_decode_mistake_is_caught(monkeypatch):
    """Mutate the oracle's decode table (flip the sign of one code) and show
    the brute-force pin no longer passes."""
    bad = e4m3.DECODE_TABLE.copy()
    bad[0x40] = -bad[0x40]
    monkeypatch.setattr(e4m3, "DECODE_TABLE", bad)
    rng = np.random.default_rng(29)
    A, sa, B, sb = _random_problem(rng, 2, 3, 128, codes_from=np.array([0x40, 0x38], np.uint8))
    X, S = gemm.gemm_nt(A, sa, B, sb, with_magnitude=True)
    Xe, Se = _fraction_gemm(A, sa, B, sb)
    diffs = [abs(Fraction(float(X[m, n])) - Xe[m, n]) <= Fraction(2) ** -50 * Se[m, n] for m in range(2) for n in range(3)]
    assert not all(diffs)


def test_similarity_defect_definition():
    x = np.array([1.0, 2.0, 3.0])
    assert metrics.similarity_defect(x, x) == 0.0
    assert abs(metrics.similarity_defect(-x, x) - 2.0) < 1e-15
    assert metrics.similarity_defect(np.zeros(3), np.zeros(3)) == 0.0


# --------------------------------------------------------------------------
# power-of-two (UE8M0) scale factors


def test_ue8m0_round_up_closed_forms():
    """The byte is the exponent of the smallest power of two >= s, plus 127;
    checked against math.frexp-free closed forms and torch's log2/ceil."""
    s = np.float32([1.0, 1.5, 0.75, 2.0 ** -20, 3 * 2.0 ** -20, 448.0, 0.5000001, 2.0 ** 100])
    assert quant.ue8m0_round_up(s).tolist() == [127, 128, 127, 107, 109, 136, 127, 227]
    rng = np.random.default_rng(8)
    r = (rng.random(2000).astype(np.float32) + np.float32(1e-3)) * np.float32(2.0) ** rng.integers(-30, 30, 2000)
    r = r.astype(np.float32)
    want = torch.ceil(torch.log2(torch.from_numpy(r).double())).to(torch.int64).numpy() + 127
    assert np.array_equal(quant.ue8m0_round_up(r).astype(np.int64), want)
    assert quant.ue8m0_decode([127, 128, 100]).tolist() == [1.0, 2.0, 2.0 ** -27]


def test_ue8m0_pack_layout_and_roundtrip():
    """Group 4i + j lands in byte j of element i, along the K-group axis."""
    b = np.array([[1], [2], [3], [4], [5]], np.uint8)  # [Kb=5, M=1], K-group-major
    p = quant.pack_ue8m0(b, axis=0)
    assert p.shape == (2, 1) and p.view(np.uint32).ravel().tolist() == [0x04030201, 0x05]
    w = np.arange(12, dtype=np.uint8).reshape(2, 6)  # [Nb, Kb]
    pw = quant.pack_ue8m0(w, axis=1)
    assert pw.view(np.uint32).tolist() == [[0x03020100, 0x0504], [0x09080706, 0x0B0A]]
    rng = np.random.default_rng(1)
    for shape, axis in [((7, 33), 0), ((9, 13), 1), ((4, 4), 0)]:
        x = rng.integers(0, 256, shape).astype(np.uint8)
        assert np.array_equal(quant.unpack_ue8m0(quant.pack_ue8m0(x, axis), shape[axis], axis), x)


def test_ue8m0_quantize_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 384)).astype(np.float32) * np.float32(3.0)
    x[1, 0:128] = 0.0
    q, e = quant.quantize_per_token_ue8m0(x)
    assert e.shape == (3, 6) and e.dtype == np.uint8
    s = quant.ue8m0_decode(e).T  # [M, Kb]
    amax = np.maximum(np.abs(x.reshape(6, 3, 128)).max(axis=2), np.float32(1e-4))
    s32 = (amax / np.float32(448)).astype(np.float32)
    # the smallest power of two at or above the fp32 factor
    assert (s >= s32).all() and (s / 2 < s32).all()
    dq = e4m3.decode(q).reshape(6, 3, 128)
    assert (np.abs(dq) <= 448).all()
    # dividing by a power of two is exact, so the codes are torch's RNE of x * 2^-e
    ref = (torch.from_numpy(x.reshape(6, 3, 128)) / torch.from_numpy(s)[:, :, None]).to(torch.float8_e4m3fn)
    assert np.array_equal(q.reshape(6, 3, 128), ref.view(torch.uint8).numpy())
    rec = dq * s[:, :, None]
    tol = np.maximum(np.abs(x.reshape(6, 3, 128)) * 2.0 ** -4, 2.0 ** -10 * s[:, :, None])
    assert (np.abs(rec - x.reshape(6, 3, 128)) <= tol).all()


def test_ue8m0_equals_fp32_factors_when_already_a_power_of_two():
    """A group whose amax / 448 is a power of two gets the same factor and
    codes in both modes."""
    rng = np.random.default_rng(6)
    x = rng.uniform(-1, 1, (3, 256)).astype(np.float32)
    for m, kb, k in [(0, 0, -3), (1, 1, 0), (2, 0, 4)]:
        g = x[m, kb * 128:(kb + 1) * 128]
        g[:] = g / np.abs(g).max() * np.float32(448 * 2.0 ** k)
        g[5] = np.float32(448 * 2.0 ** k)
    qf, sf = quant.quantize_per_token(x)
    qe, e = quant.quantize_per_token_ue8m0(x)
    for m, kb in [(0, 0), (1, 1), (2, 0)]:
        assert quant.ue8m0_decode(e[kb, m]) == sf[kb, m]
        assert np.array_equal(qf[m, kb * 128:(kb + 1) * 128], qe[m, kb * 128:(kb + 1) * 128])


def test_ue8m0_per_block_tail_and_gemm_definition():
    """Per-block factors of a short tail block use its own amax; a GEMM on
    decoded UE8M0 factors is the same definition as with fp32 factors."""
    A, B = synth.dense_problem(16, 200, 256, seed=7)
    qb, eb = quant.quantize_per_block_ue8m0(B.numpy())
    assert eb.shape == (2, 2)
    qt, et = quant.quantize_per_block_ue8m0(B.numpy()[128:])
    assert np.array_equal(eb[1], et[0]) and np.array_equal(qb[128:], qt)
    qa, ea = quant.quantize_per_token_ue8m0(A.numpy())
    X = gemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb))
    # brute force in fp64 from the decoded operands
    a = e4m3.decode(qa) * np.repeat(quant.ue8m0_decode(ea).T, 128, axis=1)
    b = e4m3.decode(qb) * np.repeat(np.repeat(quant.ue8m0_decode(eb), 128, axis=0)[:200], 128, axis=1)
    assert np.allclose(X, a @ b.T, rtol=1e-12, atol=1e-12)


def test_ue8m0_k_tail_quantisers_on_their_own_columns():
    """K % 128 != 0 with power-of-two factors: the partial last group's factor
    is the smallest power of two at or above max(amax, 1e-4)/448 over its own
    columns (amax from torch), its codes torch's RNE of x / s; the full groups
    equal the quantisation of the first 128 columns alone."""
    A, B = synth.dense_problem(5, 130, 208, seed=9)
    x, w = A.numpy(), B.numpy()
    q, e = quant.quantize_per_token_ue8m0(x)
    assert q.shape == (5, 208) and e.shape == (2, 5)
    tail = torch.from_numpy(x[:, 128:])
    s32 = (torch.clamp(tail.abs().amax(dim=1), min=torch.tensor(1e-4, dtype=torch.float32)) / 448.0).numpy()
    s = quant.ue8m0_decode(e[1])
    assert (s >= s32).all() and (s / 2 < s32).all()
    ref = (tail / torch.from_numpy(s)[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[:, 128:], ref)
    q0, e0 = quant.quantize_per_token_ue8m0(x[:, :128])
    assert np.array_equal(q[:, :128], q0) and np.array_equal(e[:1], e0)
    qb, eb = quant.quantize_per_block_ue8m0(w)
    assert qb.shape == (130, 208) and eb.shape == (2, 2)
    for nb, rows in [(0, slice(0, 128)), (1, slice(128, 130))]:
        blk = torch.from_numpy(w[rows, 128:])
        s32 = float(max(blk.abs().max().item(), 1e-4)) / 448.0
        sbk = float(quant.ue8m0_decode(eb[nb, 1]))
        assert sbk >= np.float32(s32) and sbk / 2 < np.float32(s32)
        refb = (blk / sbk).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(qb[rows, 128:], refb)
    qb0, eb0 = quant.quantize_per_block_ue8m0(w[:, :128])
    assert np.array_equal(qb[:, :128], qb0) and np.array_equal(eb[:, :1], eb0)


def test_bf16_widening_matches_torch():
    """bf16 -> fp32 is exact: every pattern against torch's conversion."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = e4m3.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.isnan(got[~np.isfinite(ref) & np.isnan(ref)]).all()
