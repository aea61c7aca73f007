"""Shared test utilities: move oracle-quantised problems to the GPU, run the
library, compare against the oracle.  Test-only code (imports both sides)."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import e4m3, gemm as ogemm, metrics, quant

SENTINEL_BF16 = 0x7FC1  # a NaN pattern no GEMM result can produce


def announce(msg: str) -> None:
    """Name the case about to touch the GPU, unbuffered."""
    sys.stderr.write(f"[gpu-case] {msg}\n")
    sys.stderr.flush()


def dev_u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_sa(sa: np.ndarray, ld: int | None = None, groups: bool = False) -> torch.Tensor:
    """Activation scales [.., Kb, rows] into a padded [.., Kb, ld] device buffer, returned as a view."""
    rows = sa.shape[-1]
    ld = ld or max(4, (rows + 3) // 4 * 4)
    buf = np.full(sa.shape[:-1] + (ld,), np.nan, np.float32)  # padding never read
    buf[..., :rows] = sa
    t = torch.from_numpy(buf).cuda()
    return t[..., :rows]


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return e4m3.bf16_bits_to_f64(bits)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sentinel_like(shape, device="cuda") -> torch.Tensor:
    return torch.full(shape, SENTINEL_BF16, dtype=torch.int16, device=device).view(torch.bfloat16)


def quantize_dense(A32, B32):
    qa, sa = quant.quantize_per_token(np.asarray(A32))
    qb, sb = quant.quantize_per_block(np.asarray(B32))
    return qa, sa, qb, sb


def assert_close(y: np.ndarray, X: np.ndarray, S: np.ndarray, Kb: int, what: str) -> dict:
    rep = metrics.check_result(y, X, S, Kb)
    assert rep["ok"], f"{what}: {rep}"
    return rep


def run_dense(fg, qa, sa, qb, sb, out=None) -> torch.Tensor:
    M = qa.shape[0]
    N = qb.shape[0]
    D = out if out is not None else sentinel_like((M, N))
    fg.gemm_fp8_nt(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), D)
    torch.cuda.synchronize()
    return D


def exact_regime(rng, M, N, K, groups=None):
    """Integer codes in [-4, 4] and scales in {1/2, 1, 2}: every fp32 step exact."""
    ints = np.arange(-4, 5, dtype=np.float32)
    pool = e4m3.encode_rne(ints)
    shapeA = (M, K) if groups is None else (groups[0], M, K)
    shapeB = (N, K) if groups is None else (groups[1], N, K)
    A = rng.choice(pool, shapeA)
    B = rng.choice(pool, shapeB)
    Kb, Nb = -(-K // 128), -(-N // 128)
    pw = np.array([0.5, 1.0, 2.0], np.float32)
    sa = rng.choice(pw, shapeA[:-2] + (Kb, M))
    sb = rng.choice(pw, shapeB[:-2] + (Nb, Kb))
    return A, sa, B, sb


def oracle_dense(qa, sa, qb, sb):
    return ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
