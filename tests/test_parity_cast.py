"""FP8 cast kernels on the GPU: byte-exact codes and bit-exact scales against
the oracle quantiser (both sides divide in fp32 and round to nearest even)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, gemm as ogemm, quant
from tests.helpers import announce, assert_close, bf16_to_f64

pytestmark = pytest.mark.gpu


def special_values(rng, shape):
    """N(0,1) with planted zero groups, ties, subnormal-range and huge-range groups."""
    x = rng.standard_normal(shape).astype(np.float32)
    flat = x.reshape(-1, 128)
    if flat.shape[0] > 4:
        flat[0] = 0.0  # amax = 0 -> floor scale, q = 0
        flat[1] *= np.float32(1e-30)  # tiny magnitudes
        flat[2] *= np.float32(1e30)
        flat[3, :] = np.float32(-0.0)
        flat[3, 5] = np.float32(448.0)  # exact-representable values after scaling (s = 1)
        flat[3, 6] = np.float32(1.0625)  # ties at s = 1
        flat[3, 7] = np.float32(-1.1875)
        flat[3, 8] = np.float32(2.0 ** -10)
        flat[3, 9] = np.float32(3 * 2.0 ** -10)
    return x


# 1000 x 4352 has 34000 row groups: the launch takes the 8-lane split; the others the 16-lane one.
@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (129, 7168), (1000, 2048), (1000, 4352)])
def test_per_token_bytes(gpu_lib, M, K):
    announce(f"cast per-token {M}x{K}")
    rng = np.random.default_rng(M + K)
    x = special_values(rng, (M, K))
    q_ref, s_ref = quant.quantize_per_token(x)
    q, sa = gpu_lib.fp8_cast_per_token(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_per_token_strided_input(gpu_lib):
    announce("cast per-token strided")
    rng = np.random.default_rng(1)
    xb = rng.standard_normal((50, 640)).astype(np.float32)
    x = torch.from_numpy(xb).cuda()[:, :512]
    q_ref, s_ref = quant.quantize_per_token(xb[:, :512])
    sa = torch.full((4, 60), -1.0, device="cuda")
    q, sa_v = gpu_lib.fp8_cast_per_token(x, sa=sa[:, :50])
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sa[:, :50].cpu().numpy(), s_ref)
    assert (sa[:, 50:].cpu().numpy() == -1.0).all()


@pytest.mark.parametrize("N,K", [(1, 128), (130, 256), (2112, 7168), (256, 1536)])
def test_per_block_bytes(gpu_lib, N, K):
    announce(f"cast per-block {N}x{K}")
    rng = np.random.default_rng(N * K)
    w = special_values(rng, (N, K))
    q_ref, s_ref = quant.quantize_per_block(w)
    q, sb = gpu_lib.fp8_cast_per_block(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sb.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_cast_then_gemm_end_to_end(gpu_lib):
    """fp32 -> GPU casts -> GPU GEMM against oracle quantise -> oracle GEMM."""
    announce("cast+gemm end to end 256x2112x1024")
    M, N, K = 256, 2112, 1024
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token(A32.cuda())
    qb_d, sb_d = gpu_lib.fp8_cast_per_block(B32.cuda())
    D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d, D)
    torch.cuda.synchronize()
    qa, sa = quant.quantize_per_token(A32.numpy())
    qb, sb = quant.quantize_per_block(B32.numpy())
    X, S = ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, K // 128, "end to end")


# ------------------------------------------------------------- bf16 inputs


def bf16_values(rng, shape) -> np.ndarray:
    """bf16 bit patterns of special_values (rounded to bf16 by torch)."""
    x = special_values(rng, shape)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (129, 7168), (257, 1024), (600, 7168)])
def test_per_token_bf16_input_bytes(gpu_lib, M, K):
    """bf16 input quantises exactly as its fp32 widening does in the oracle."""
    announce(f"cast per-token bf16 {M}x{K}")
    bits = bf16_values(np.random.default_rng(M * 3 + K), (M, K))
    q_ref, s_ref = quant.quantize_per_token(e4m3.bf16_bits_to_f32(bits))
    q, sa = gpu_lib.fp8_cast_per_token(dev_bf16(bits))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(128, 128), (2112, 512), (300, 1024)])
def test_per_block_bf16_input_bytes(gpu_lib, N, K):
    announce(f"cast per-block bf16 {N}x{K}")
    bits = bf16_values(np.random.default_rng(N + K), (N, K))
    q_ref, s_ref = quant.quantize_per_block(e4m3.bf16_bits_to_f32(bits))
    q, sb = gpu_lib.fp8_cast_per_block(dev_bf16(bits))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sb.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_bf16_input_strided_rows(gpu_lib):
    """A bf16 view with a padded row stride (ldx > K)."""
    M, K = 40, 256
    bits = bf16_values(np.random.default_rng(5), (M, K))
    buf = torch.zeros(M, K + 64, dtype=torch.bfloat16, device="cuda")
    buf[:, :K] = dev_bf16(bits)
    announce("cast per-token bf16 strided")
    q, sa = gpu_lib.fp8_cast_per_token(buf[:, :K])
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quantize_per_token(e4m3.bf16_bits_to_f32(bits))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
