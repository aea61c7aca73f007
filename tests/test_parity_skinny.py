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
# 128-row fragments in one part (M > 64 only, one column fragment)
PLANS = ["1,1", "2,1", "4,1", "1,2", "2,4", "1,8", "2,3", "4,3", "1,2,8", "1,3,8"]


@pytest.fixture(params=PLANS)
def plan(request, monkeypatch):
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.setenv("FG_SKINNY", request.param)
    return request.param


def _usable(plan: str, M: int, K: int) -> bool:
    cf, sp, *rest = map(int, plan.split(","))
    mf = rest[0] if rest else 4
    if mf == 8 and (M <= 64 or cf > 1):
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


def test_workspace_rules(gpu_lib, monkeypatch):
    """gemm_fp8_nt_ws: a workspace below fg_nt_workspace_bytes is rejected
    before anything runs; NULL selects gemm_fp8_nt's unsplit plan (same bits
    as the C entry point gemm_fp8_nt); a workspace that already served other
    shapes gives the same bits as a fresh zero-filled one."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("FG_SKINNY", raising=False)
    M, N, K = 64, 2112, 2048
    announce(f"skinny workspace rules {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=13)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    a, s_a, b, s_b = dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb)
    need = gpu_lib.nt_workspace_bytes(M, N, K)
    assert need > 64 * 1024  # the decode plan splits K
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    D = sentinel_like((M, N))
    with pytest.raises(gpu_lib.FP8GemmError, match="workspace of"):
        gpu_lib.gemm_fp8_nt(a, s_a, b, s_b, D, workspace=small)
    torch.cuda.synchronize()
    assert (bf16_bits(D) == SENTINEL_BF16).all()  # nothing was launched
    unsplit = sentinel_like((M, N))
    gpu_lib.gemm_fp8_nt_unsplit(a, s_a, b, s_b, unsplit)
    lib = gpu_lib.load_library()
    null_ws = sentinel_like((M, N))
    st = lib.gemm_fp8_nt_ws(a.data_ptr(), K, s_a.data_ptr(), s_a.stride(0), b.data_ptr(), K, s_b.data_ptr(),
                            null_ws.data_ptr(), N, M, N, K, None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.fg_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(null_ws), bf16_bits(unsplit))
    X, S = oracle_dense(qa, sa, qb, sb)
    assert_close(bf16_to_f64(unsplit), X, S, K // 128, "unsplit plan")
    # a workspace reused across shapes keeps its counters at zero
    ws = torch.zeros(gpu_lib.load_library().fg_nt_workspace_max_bytes(), dtype=torch.uint8, device="cuda")
    fresh = bf16_bits(run_dense(gpu_lib, qa, sa, qb, sb))
    for (m2, n2, k2) in [(32, 4096, 7168), (128, 300, 4096), (M, N, K)]:
        A2, B2 = synth.dense_problem(m2, n2, k2, seed=m2 + n2)
        q2 = quantize_dense(A2, B2)
        D2 = torch.empty(m2, n2, dtype=torch.bfloat16, device="cuda")
        gpu_lib.gemm_fp8_nt(dev_u8(q2[0]), dev_sa(q2[1]), dev_u8(q2[2]), dev_f32(q2[3]), D2, workspace=ws)
    Dw = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt(a, s_a, b, s_b, Dw, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(Dw), fresh)
    assert (ws[:64 * 1024] == 0).all()  # counters left at zero


# Row counts around the 16-row fragment and 64-row part boundaries, widths
# around the 32- and 64-column tiles and one weight-scale block, K with a
# partial last slice: the planner's own choice of tile width and K split.
SWEEP = [(m, n, k) for m in (1, 15, 17, 63, 65, 127) for n, k in ((31, 144), (65, 1040), (130, 2320), (2112, 4112))]


@pytest.mark.parametrize("M,N,K", SWEEP, ids=lambda v: str(v))
def test_default_plan_sweep_bitwise(gpu_lib, monkeypatch, M, N, K):
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("FG_SKINNY", raising=False)
    announce(f"skinny default plan {M}x{N}x{K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    D = run_dense(gpu_lib, qa, sa, qb, sb)
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))
