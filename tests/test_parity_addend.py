"""D = C + A . B^T (an fp32 addend C) on the GPU against the CPU oracle.

Every kernel that serves the dense call is forced in turn: the few-row
kernel at each column width and activation height (the addend call never
splits K: it takes no workspace), the 128x128 kernel and the large kernel
at each tile width.  In the exact regime (integer codes, power-of-two
scales, C on a 1/4 grid) the result is compared bit for bit; random inputs
use the oracle's per-element bound with |C| in the magnitude.  With C = 0 the
call must give the bits of gemm_fp8_nt, since it runs the same kernels."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_f32, dev_sa, dev_u8, exact_regime,
    quantize_dense, sentinel_like,
)

pytestmark = pytest.mark.gpu

KERNELS = {
    "skinny-1x1": {"FG_SKINNY": "1,1"},
    "skinny-2x1": {"FG_SKINNY": "2,1"},
    "skinny-4x1": {"FG_SKINNY": "4,1"},
    "skinny-1x2-128rows": {"FG_SKINNY": "1,2,8"},
    "small": {"FG_FORCE_CONFIG": "small"},
    "big-256": {"FG_FORCE_CONFIG": "big", "FG_FORCE_BN": "256"},
    "big-224": {"FG_FORCE_CONFIG": "big", "FG_FORCE_BN": "224"},
    "big-160": {"FG_FORCE_CONFIG": "big", "FG_FORCE_BN": "160"},
}
ENV_KEYS = ("FG_SKINNY", "FG_FORCE_CONFIG", "FG_FORCE_BN")


@pytest.fixture(params=list(KERNELS))
def kernel(request, monkeypatch):
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)
    for k, v in KERNELS[request.param].items():
        monkeypatch.setenv(k, v)
    return request.param


def _applies(kernel: str, M: int, K: int) -> bool:
    if not kernel.startswith("skinny"):
        return True
    cf, sp, *rest = map(int, KERNELS[kernel]["FG_SKINNY"].split(","))
    if rest and rest[0] == 8 and M <= 64:
        return False  # 128-row fragments only for more than 64 rows
    return M <= 128 and K // 128 >= sp


def grid_addend(rng, M, N) -> np.ndarray:
    """fp32 values on a 1/4 grid in [-256, 256]: sums with the exact-regime
    products stay exact in fp32."""
    return (rng.integers(-1024, 1025, (M, N)) / 4.0).astype(np.float32)


def run_c(fg, qa, sa, qb, sb, C, out=None, C_dev=None):
    M, N = qa.shape[0], qb.shape[0]
    D = out if out is not None else sentinel_like((M, N))
    Cd = C_dev if C_dev is not None else dev_f32(C)
    fg.gemm_fp8_nt_c(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), Cd, D)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (33, 130, 512), (64, 300, 256), (128, 520, 896),
                                   (300, 1000, 640), (513, 2112, 256)])
def test_exact_regime_bitwise(gpu_lib, kernel, M, N, K):
    if not _applies(kernel, M, K):
        pytest.skip("plan does not apply to this shape")
    announce(f"addend {kernel} exact regime {M}x{N}x{K}")
    rng = np.random.default_rng(M + 3 * N + K)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    C = grid_addend(rng, M, N)
    D = run_c(gpu_lib, qa, sa, qb, sb, C)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(ogemm.gemm_nt_addend(qa, sa, qb, sb, C)))


@pytest.mark.parametrize("M,N,K", [(7, 200, 768), (128, 1000, 1536), (257, 1030, 1024)])
def test_random(gpu_lib, kernel, M, N, K):
    if not _applies(kernel, M, K):
        pytest.skip("plan does not apply to this shape")
    announce(f"addend {kernel} random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=5 * M + N + K)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    rng = np.random.default_rng(M + N)
    C = (rng.standard_normal((M, N)) * 10.0 ** rng.integers(-2, 3, (M, N))).astype(np.float32)
    D = run_c(gpu_lib, qa, sa, qb, sb, C)
    X, S = ogemm.gemm_nt_addend(qa, sa, qb, sb, C, with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, K // 128 + 1, f"addend {kernel} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 2112, 1024), (300, 700, 512)])
def test_zero_addend_gives_gemm_bits(gpu_lib, kernel, M, N, K):
    """Same kernels, same summation order: C = 0 reproduces the bits of the
    C entry point gemm_fp8_nt (neither splits K)."""
    if not _applies(kernel, M, K):
        pytest.skip("plan does not apply to this shape")
    announce(f"addend {kernel} zero C {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=17)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D0 = sentinel_like((M, N))
    gpu_lib.gemm_fp8_nt_unsplit(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), D0)
    D1 = run_c(gpu_lib, qa, sa, qb, sb, np.zeros((M, N), np.float32))
    assert np.array_equal(bf16_bits(D1), bf16_bits(D0))


@pytest.mark.parametrize("ldc_pad", [0, 1, 6])
def test_strided_addend_and_output(gpu_lib, kernel, ldc_pad):
    """C and D as views of wider buffers; ldc = N + 1 forces element loads.
    D's padding keeps its sentinel."""
    M, N, K = (50, 90, 512) if kernel.startswith("skinny") else (300, 200, 256)
    if not _applies(kernel, M, K):
        pytest.skip("plan does not apply to this shape")
    announce(f"addend {kernel} strided ldc=N+{ldc_pad}")
    rng = np.random.default_rng(ldc_pad)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    C = grid_addend(rng, M, N)
    Cbuf = torch.full((M, N + ldc_pad), float("nan"), dtype=torch.float32, device="cuda")
    Cbuf[:, :N] = dev_f32(C)
    Dbuf = sentinel_like((M + 3, N + 8))
    run_c(gpu_lib, qa, sa, qb, sb, C, out=Dbuf[:M, :N], C_dev=Cbuf[:, :N])
    assert np.array_equal(bf16_bits(Dbuf[:M, :N]), ogemm.to_bf16(ogemm.gemm_nt_addend(qa, sa, qb, sb, C)))
    bits = bf16_bits(Dbuf)
    assert (bits[M:, :] == SENTINEL_BF16).all() and (bits[:, N:] == SENTINEL_BF16).all()


def test_k_zero_writes_rounded_addend(gpu_lib, monkeypatch):
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)
    announce("addend K=0")
    M, N = 70, 130
    rng = np.random.default_rng(1)
    C = rng.standard_normal((M, N)).astype(np.float32)
    D = sentinel_like((M, N))
    A = torch.zeros(M, 16, dtype=torch.uint8, device="cuda")[:, :0]
    B = torch.zeros(N, 16, dtype=torch.uint8, device="cuda")[:, :0]
    sa = torch.zeros(0, 72, dtype=torch.float32, device="cuda")[:, :M]
    sb = torch.zeros(2, 0, dtype=torch.float32, device="cuda")
    gpu_lib.gemm_fp8_nt_c(A, sa, B, sb, dev_f32(C), D)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(C.astype(np.float64)))


def test_rejects_missing_addend(gpu_lib):
    """A NULL C is an argument error, reported before anything is launched."""
    lib = gpu_lib.load_library()
    st = lib.gemm_fp8_nt_c(None, 128, None, 4, None, 128, None, None, 8, None, 8, 4, 8, 128, None)
    assert st == 1  # FG_EINVAL
    assert b"C" in lib.fg_last_error()


def test_full_size_sampled(gpu_lib, monkeypatch):
    """The dense M=4096 workload's first shape with the library's own plan;
    sampled rows x column blocks against the oracle."""
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)
    M, N, K = synth.DENSE_M4096.shapes[0]
    announce(f"addend full size {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    rng = np.random.default_rng(9)
    C = rng.standard_normal((M, N)).astype(np.float32)
    D = run_c(gpu_lib, qa, sa, qb, sb, C)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 6, replace=False)]))
    for nb in np.unique(np.concatenate([[0, -(-N // 128) - 1], rng.choice(N // 128, 2, replace=False)])):
        cols = slice(nb * 128, min(N, nb * 128 + 128))
        X, S = ogemm.gemm_nt_addend(qa[rows], sa[:, rows], qb[cols], sb[nb:nb + 1], C[rows][:, cols],
                                    with_magnitude=True)
        y = bf16_to_f64(D[torch.from_numpy(rows).cuda(), cols])
        assert_close(y, X, S, K // 128 + 1, f"addend full size block {nb}")
