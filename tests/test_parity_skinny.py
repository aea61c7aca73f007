"""The dense GEMM for few activation rows (M <= 128: the weight-streaming
kernel), on the GPU against the CPU oracle.

Every column-tile width, a range of K splits and both activation-fragment
heights are forced with FG_SKINNY.
The exact regime (integer codes, power-of-two scales) is compared bit for
bit, which also pins the split-K reduction: a partial added twice or left out
changes the result.  Random inputs use the oracle's per-element bound."""

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

# (column fragments, K splits[, activation fragments]): 64-row fragments by
# default, rows beyond 64 in a second row part; the third field 8 selects
# 128-row fragments in one part (M > 64 only, at most 2 column fragments)
PLANS = ["1,1", "2,1", "4,1", "1,2", "2,4", "1,8", "2,3", "2,2,8", "1,3,8"]


@pytest.fixture(params=PLANS)
def plan(request, monkeypatch):
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.setenv("FG_SKINNY", request.param)
    return request.param


def _usable(plan: str, M: int, K: int) -> bool:
    cf, sp, *rest = map(int, plan.split(","))
    mf = rest[0] if rest else 4
    if mf == 8 and (M <= 64 or cf > 2):
        return False
    return -(-K // 128) >= sp


@pytest.mark.parametrize(
    "M,N,K",
    [(1, 16, 128), (16, 100, 512), (33, 130, 1024), (64, 2112, 1152), (65, 300, 640), (100, 136, 2048), (128, 520, 896)],
)
def test_exact_regime_bitwise(gpu_lib, plan, M, N, K):
    if not _usable(plan, M, K):
        pytest.skip("plan does not apply to this shape")
    announce(f"skinny {plan} exact regime {M}x{N}x{K}")
    rng = np.random.default_rng(M * 31 + N + K)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


@pytest.mark.parametrize("M,N,K", [(7, 200, 768), (64, 1000, 1536), (128, 4104, 1024)])
def test_random(gpu_lib, plan, M, N, K):
    if not _usable(plan, M, K):
        pytest.skip("plan does not apply to this shape")
    announce(f"skinny {plan} random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=M + 3 * N + K)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(D), X, S, K // 128, f"skinny {plan} {M}x{N}x{K}")


def test_repeated_calls_are_bitwise_identical(gpu_lib, monkeypatch):
    """The split-K arrival counters are left at zero by every launch: the same
    call gives the same bits again, for several splits."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    M, N, K = 96, 777, 2048
    A32, B32 = synth.dense_problem(M, N, K, seed=11)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    for plan in ("2,1", "2,4", "1,16"):
        monkeypatch.setenv("FG_SKINNY", plan)
        announce(f"skinny repeat {plan}")
        first = bf16_bits(run_dense(gpu_lib, qa, sa, qb, sb))
        for _ in range(3):
            assert np.array_equal(bf16_bits(run_dense(gpu_lib, qa, sa, qb, sb)), first)


def test_strided_and_unaligned_output(gpu_lib, monkeypatch):
    """lda > K, ld_sa > M, an output row stride that is not a multiple of 4
    (element-wise stores) and untouched padding."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.setenv("FG_SKINNY", "2,2")
    announce("skinny strided 50x90x512")
    M, N, K = 50, 90, 512
    A32, B32 = synth.dense_problem(M, N, K, seed=4)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    Abuf = torch.zeros(M, K + 48, dtype=torch.uint8, device="cuda")
    Abuf[:, :K] = dev_u8(qa)
    Dbuf = sentinel_like((M + 2, N + 7))
    gpu_lib.gemm_fp8_nt(Abuf[:, :K], dev_sa(sa, ld=M + 14), dev_u8(qb), dev_f32(sb), Dbuf[:M, :N])
    torch.cuda.synchronize()
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(Dbuf[:M, :N]), X, S, K // 128, "skinny strided")
    bits = bf16_bits(Dbuf)
    assert (bits[M:, :] == SENTINEL_BF16).all()
    assert (bits[:, N:] == SENTINEL_BF16).all()


@pytest.mark.parametrize("shape", synth.DENSE_SMALL_M.shapes, ids=lambda s: "x".join(map(str, s)))
def test_small_m_decode_full_size(gpu_lib, monkeypatch, shape):
    """The decode shapes at full size with the library's own plan; the output
    is checked in full against the oracle (M rows are few)."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("FG_SKINNY", raising=False)
    M, N, K = shape
    announce(f"skinny decode full size {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(D), X, S, K // 128, f"decode {M}x{N}x{K}")
