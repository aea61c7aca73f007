"""The large kernel at tile widths that are not a multiple of the 128-column
weight-scale block (256x224 and 256x160), forced with FG_FORCE_BN.

With these widths a wave's columns can cross a weight-block boundary, so the
kernel picks the weight scale per 16-column subtile.  The exact regime (integer
codes, power-of-two scales drawn independently per block) is compared bit for
bit, so a scale taken from the wrong block shows up as a wrong element; the
equivariance test doubles one weight-block row of scales at a time and checks
that exactly its 128 columns double."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, quant
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_f32, dev_sa, dev_u8,
    exact_regime, oracle_dense, quantize_dense, run_dense, sentinel_like,
)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[224, 160, 256])
def width(request, monkeypatch):
    monkeypatch.setenv("FG_FORCE_CONFIG", "big")
    monkeypatch.setenv("FG_FORCE_BN", str(request.param))
    return request.param


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (70, 300, 256), (256, 896, 512), (300, 1000, 384), (513, 2112, 256)])
def test_dense_exact_regime_bitwise(gpu_lib, width, M, N, K):
    announce(f"width {width}: dense exact regime {M}x{N}x{K}")
    rng = np.random.default_rng(M * 5 + N + K + width)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


@pytest.mark.parametrize("M,N,K", [(40, 232, 256), (257, 1030, 1536), (512, 7168, 1024)])
def test_dense_random(gpu_lib, width, M, N, K):
    announce(f"width {width}: dense random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=N + K)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(D), X, S, K // 128, f"width {width} dense {M}x{N}x{K}")


def test_weight_block_equivariance(gpu_lib, width):
    """Doubling the scales of weight block nb doubles columns [128 nb, 128 nb + 128)
    and nothing else, for every block of a width that straddles them."""
    M, N, K = 64, 896, 256
    announce(f"width {width}: weight-block equivariance {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=31)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    base = bf16_to_f64(run_dense(gpu_lib, qa, sa, qb, sb))
    for nb in range(N // 128):
        sb2 = sb.copy()
        sb2[nb, :] *= 2
        y = bf16_to_f64(run_dense(gpu_lib, qa, sa, qb, sb2))
        cols = slice(128 * nb, 128 * nb + 128)
        assert np.array_equal(y[:, cols], 2 * base[:, cols]), nb
        rest = np.ones(N, bool)
        rest[cols] = False
        assert np.array_equal(y[:, rest], base[:, rest]), nb


def test_contiguous_exact_regime_bitwise(gpu_lib, width):
    announce(f"width {width}: contiguous exact regime")
    rng = np.random.default_rng(width)
    idx = synth.contiguous_indices([200, 60, 0, 300], pad_to=128)
    M, N, K, G = idx.shape[0], 520, 384, 4
    qa, sa, _, _ = exact_regime(rng, M, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = sentinel_like((M, N))
    gpu_lib.gemm_fp8_grouped_contiguous(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb),
                                        torch.from_numpy(idx.astype(np.int32)).cuda(), D)
    torch.cuda.synchronize()
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_masked_exact_regime_bitwise(gpu_lib, width):
    announce(f"width {width}: masked exact regime")
    rng = np.random.default_rng(width + 1)
    G, Mc, N, K = 5, 256, 700, 256
    mask = np.array([0, 1, 129, 256, 77], np.int32)
    qa, sa, qb, sb = exact_regime(rng, Mc, N, K, groups=(G, G))
    D = sentinel_like((G, Mc, N))
    gpu_lib.gemm_fp8_grouped_masked(dev_u8(qa), dev_sa(sa, groups=True), dev_u8(qb), dev_f32(sb),
                                    torch.from_numpy(mask).cuda(), D)
    torch.cuda.synchronize()
    X, valid = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_masked_random(gpu_lib, width):
    announce(f"width {width}: masked random 4x256x7168x512")
    G, Mc, N, K = 4, 256, 7168, 512
    A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=width)
    qa, sa = zip(*(quant.quantize_per_token(a) for a in A32.numpy()))
    qa, sa = np.stack(qa), np.stack(sa)
    qb, sb = zip(*(quant.quantize_per_block(b) for b in B32.numpy()))
    qb, sb = np.stack(qb), np.stack(sb)
    D = sentinel_like((G, Mc, N))
    gpu_lib.gemm_fp8_grouped_masked(dev_u8(qa), dev_sa(sa, groups=True), dev_u8(qb), dev_f32(sb),
                                    torch.from_numpy(np.asarray(mask, np.int32)).cuda(), D)
    torch.cuda.synchronize()
    X, valid, S = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask, with_magnitude=True)
    assert_close(bf16_to_f64(D)[valid], X[valid], S[valid], K // 128, f"width {width} masked")
    assert (bf16_bits(D)[~valid] == SENTINEL_BF16).all()


@pytest.mark.parametrize("with_c", [False, True])
def test_unaligned_output_rows(gpu_lib, width, with_c):
    """An output whose rows start 2 bytes past a 16-byte boundary and are an odd
    number of elements apart, N not a multiple of 8: the epilogue's element-wise
    stores (the vector ones need 16- or 8-byte alignment).  Exact regime, bit for
    bit, with and without the fp32 addend; the padding around D is untouched."""
    M, N, K = 300, 517, 384
    announce(f"width {width}: unaligned output rows {M}x{N}x{K} C={with_c}")
    rng = np.random.default_rng(width + 3 * with_c)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    ldd = N + 3
    buf = sentinel_like((M + 2, ldd))
    flat = buf.view(-1)[1:1 + M * ldd]
    D = flat.view(M, ldd)[:, :N]
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    if with_c:
        C = (rng.integers(-1024, 1025, (M, N)) / 4.0).astype(np.float32)
        gpu_lib.gemm_fp8_nt_c(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), dev_f32(C), D)
        X = X + C
    else:
        gpu_lib.gemm_fp8_nt(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), D)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))
    bits = bf16_bits(buf).reshape(-1)
    inside = np.zeros(bits.size, bool)
    for m in range(M):
        inside[1 + m * ldd: 1 + m * ldd + N] = True
    assert (bits[~inside] == SENTINEL_BF16).all()
