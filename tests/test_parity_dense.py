"""Dense NT GEMM on the GPU against the CPU oracle.

Tolerances: bit-exact in the exactly representable regime (integer codes,
power-of-two scales), otherwise the oracle's per-element bound
|y - X| <= 1e-2 |X| + (2^-14 + 2^-24 (Kb + 3)) S plus a similarity defect below
1e-3 (``oracle.metrics``)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, gemm as ogemm, quant
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_f32, dev_sa, dev_u8,
    exact_regime, oracle_dense, quantize_dense, run_dense, sentinel_like,
)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["big", "small"])
def tile_config(request, monkeypatch):
    """Force the 256x256 or the 128x128 kernel for shapes either could take."""
    monkeypatch.setenv("FG_FORCE_CONFIG", request.param)
    return request.param


def test_small_dense_config(gpu_lib):
    """128x256x512, N(0,1) inputs quantised with amax/448 scales, seed 0."""
    announce("dense 128x256x512 seed 0")
    M, N, K = synth.SMALL_DENSE.shapes[0]
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X, S = oracle_dense(qa, sa, qb, sb)
    rep = assert_close(bf16_to_f64(D), X, S, K // 128, "dense small")
    assert rep["similarity_defect"] < 1e-5


@pytest.mark.parametrize(
    "M,N,K",
    [(1, 1, 128), (3, 130, 128), (63, 130, 256), (65, 257, 384), (129, 2112, 512), (256, 300, 1024), (200, 1000, 2048)],
)
def test_exact_regime_bitwise(gpu_lib, tile_config, M, N, K):
    announce(f"dense exact regime {M}x{N}x{K} {tile_config}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (17, 136, 256), (100, 520, 640), (257, 1030, 1536), (512, 512, 7168)])
def test_random_shapes(gpu_lib, tile_config, M, N, K):
    announce(f"dense random {M}x{N}x{K} {tile_config}")
    A32, B32 = synth.dense_problem(M, N, K, seed=M + N + K)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(D), X, S, K // 128, f"dense {M}x{N}x{K}")


def test_strided_operands_and_untouched_padding(gpu_lib, tile_config):
    """lda > K, ldb > K, ld_sa > M, ldd > N: only D[:M, :N] is written."""
    announce(f"dense strided 70x200x384 {tile_config}")
    M, N, K = 70, 200, 384
    A32, B32 = synth.dense_problem(M, N, K, seed=5)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    Abuf = torch.zeros(M, K + 64, dtype=torch.uint8, device="cuda")
    Abuf[:, :K] = dev_u8(qa)
    Bbuf = torch.zeros(N, K + 32, dtype=torch.uint8, device="cuda")
    Bbuf[:, :K] = dev_u8(qb)
    Dbuf = sentinel_like((M + 3, N + 24))
    gpu_lib.gemm_fp8_nt(Abuf[:, :K], dev_sa(sa, ld=M + 30 + 2), Bbuf[:, :K], dev_f32(sb), Dbuf[:M, :N])
    torch.cuda.synchronize()
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(Dbuf[:M, :N]), X, S, K // 128, "strided")
    bits = bf16_bits(Dbuf)
    assert (bits[M:, :] == SENTINEL_BF16).all()
    assert (bits[:, N:] == SENTINEL_BF16).all()


def test_k_zero_writes_zeros(gpu_lib):
    announce("dense K=0")
    D = sentinel_like((33, 40))
    a = torch.zeros(33, 16, dtype=torch.uint8, device="cuda")[:, :0]
    b = torch.zeros(40, 16, dtype=torch.uint8, device="cuda")[:, :0]
    sa = torch.zeros(0, 36, dtype=torch.float32, device="cuda")[:, :33]
    sb = torch.zeros(1, 0, dtype=torch.float32, device="cuda")
    gpu_lib.gemm_fp8_nt(a, sa, b, sb, D)
    torch.cuda.synchronize()
    assert (bf16_bits(D) == 0).all()


def test_power_of_two_equivariance(gpu_lib, tile_config):
    """Doubling one row's activation scales doubles that row; doubling one
    weight block row doubles its 128 columns -- bit for bit."""
    announce(f"dense equivariance 96x384x512 {tile_config}")
    M, N, K = 96, 384, 512
    A32, B32 = synth.dense_problem(M, N, K, seed=9)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    base = bf16_to_f64(run_dense(gpu_lib, qa, sa, qb, sb))
    sa2 = sa.copy()
    sa2[:, 17] *= 2
    y = bf16_to_f64(run_dense(gpu_lib, qa, sa2, qb, sb))
    assert np.array_equal(y[17], 2 * base[17]) and np.array_equal(np.delete(y, 17, 0), np.delete(base, 17, 0))
    sb2 = sb.copy()
    sb2[1, :] *= 2
    y = bf16_to_f64(run_dense(gpu_lib, qa, sa, qb, sb2))
    assert np.array_equal(y[:, 128:256], 2 * base[:, 128:256])
    assert np.array_equal(y[:, :128], base[:, :128]) and np.array_equal(y[:, 256:], base[:, 256:])


def test_determinism_and_grid_invariance(gpu_lib, tile_config, monkeypatch):
    """Whole-tile scheduling: the CU cap changes which workgroup computes a
    tile, never how, so the bits are identical."""
    announce(f"dense grid invariance 640x1000x1024 {tile_config}")
    M, N, K = 640, 1000, 1024
    A32, B32 = synth.dense_problem(M, N, K, seed=21)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    ref = bf16_bits(run_dense(gpu_lib, qa, sa, qb, sb))
    assert np.array_equal(ref, bf16_bits(run_dense(gpu_lib, qa, sa, qb, sb)))
    try:
        for cus in (1, 7, 64):
            gpu_lib.set_num_cus(cus)
            assert gpu_lib.get_num_cus() == cus
            assert np.array_equal(ref, bf16_bits(run_dense(gpu_lib, qa, sa, qb, sb))), cus
    finally:
        gpu_lib.set_num_cus(0)


@pytest.mark.parametrize("M", [64, 128])
@pytest.mark.parametrize("N,K", [(2112, 7168), (4096, 7168), (7168, 2048)])
def test_small_m_decode_shapes_full(gpu_lib, M, N, K):
    """Small-M decode shapes, every output checked."""
    announce(f"dense small-M {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(D), X, S, K // 128, f"small-M {M}x{N}x{K}")


@pytest.mark.parametrize("shape", synth.DENSE_M4096.shapes, ids=lambda s: "x".join(map(str, s)))
def test_m4096_full_size_sampled(gpu_lib, shape):
    """Full-size M=4096 shapes in the benchmark's launch path (GPU cast, then
    GEMM).  The oracle quantises a sample of A rows and B row blocks on the
    CPU; the GPU's cast bytes must equal them there, and the GEMM outputs of
    the sampled rows x blocks must meet the tolerance."""
    M, N, K = shape
    announce(f"dense full-size sampled {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    a_dev = A32.cuda()
    b_dev = B32.cuda()
    qa_d, sa_d = gpu_lib.fp8_cast_per_token(a_dev)
    qb_d, sb_d = gpu_lib.fp8_cast_per_block(b_dev)
    D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d, D)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N + K)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    Nb = -(-N // 128)
    blocks = np.unique(np.concatenate([[0, Nb - 1], rng.choice(Nb, 3, replace=False)]))
    qa, sa = quant.quantize_per_token(A32.numpy()[rows])
    assert np.array_equal(qa_d[torch.from_numpy(rows).cuda()].cpu().numpy(), qa)
    assert np.array_equal(sa_d[:, torch.from_numpy(rows).cuda()].cpu().numpy(), sa)
    Dh = D[torch.from_numpy(rows).cuda()]
    for nb in blocks:
        cols = slice(nb * 128, min(N, nb * 128 + 128))
        qb, sb = quant.quantize_per_block(B32.numpy()[cols])
        assert np.array_equal(qb_d[cols].cpu().numpy(), qb)
        assert np.array_equal(sb_d[nb].cpu().numpy(), sb[0])
        X, S = ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
        assert_close(bf16_to_f64(Dh[:, cols]), X, S, K // 128, f"{shape} block {nb}")
