"""FP8 cast kernels on the GPU: byte-exact codes and bit-exact scales against
the oracle quantiser (both sides divide in fp32 and round to nearest even)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, quant
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


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (129, 7168), (1000, 2048)])
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
