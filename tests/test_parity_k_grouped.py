"""The K-grouped TN GEMM (weight gradients) on the GPU against the CPU oracle.

Groups of ks[g] consecutive K rows, some empty, with the scale factors of
their own K groups, as one persistent launch over every group's tiles: on
K-major copies in the workspace, or (no workspace) on the operands as
stored.  A group that used another group's rows, columns or factors changes
the bits.  The exact regime is compared bit for bit on both paths; random
inputs use the oracle's bound."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_f32, dev_sa, dev_u8, exact_regime,
    quantize_dense,
)

pytestmark = pytest.mark.gpu

ENV_KEYS = ("FG_SKINNY", "FG_FORCE_CONFIG", "FG_FORCE_BN")


@pytest.fixture(autouse=True)
def default_plan(monkeypatch):
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)


# "copy": a workspace from torch's allocator; "direct": an empty one
@pytest.fixture(params=["copy", "direct"])
def path(request):
    return request.param


def run_kg(fg, As, sa, Bs, sb, ks, C=None, path="copy"):
    """The GEMM on device copies of the stored operands; on the direct path
    with operands it does not take (M or N not a multiple of 16), checks the
    FG_EALIGN error with D untouched and returns None."""
    M, N = As.shape[1], Bs.shape[1]
    D = torch.full((len(ks), M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(0, dtype=torch.uint8, device="cuda") if path == "direct" else None
    args = (dev_u8(As), dev_sa(sa), dev_u8(Bs), dev_f32(sb), ks, D)
    if path == "direct" and (M % 16 or N % 16) and sum(ks):
        with pytest.raises(fg.FP8GemmError, match="without a workspace"):
            fg.gemm_fp8_k_grouped_tn_contiguous(*args, C=None if C is None else dev_f32(C), workspace=ws)
        torch.cuda.synchronize()
        return None
    fg.gemm_fp8_k_grouped_tn_contiguous(*args, C=None if C is None else dev_f32(C), workspace=ws)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("M,N,ks", [(1, 1, [128]), (64, 200, [128, 0, 256]), (128, 130, [256, 128, 384]),
                                    (300, 1000, [384, 128]), (513, 130, [256, 256, 0, 128]),
                                    (16, 16, [128, 0]), (144, 272, [128, 0, 256]), (256, 528, [384, 128, 0, 256]),
                                    (1040, 160, [128, 128, 128]), (64, 48, [0, 128] * 150),
                                    (32, 32, [128] * 260)],
                         ids=lambda v: str(v).replace(" ", ""))
@pytest.mark.parametrize("with_c", [False, True], ids=["no-C", "C"])
def test_exact_regime_bitwise(gpu_lib, path, M, N, ks, with_c):
    announce(f"k-grouped {path} exact {M}x{N} ks={len(ks)} groups C={with_c}")
    Kt = sum(ks)
    rng = np.random.default_rng(M + N + Kt + len(ks))
    A, sa, B, sb = exact_regime(rng, M, N, Kt)
    As, Bs = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    C = (rng.integers(-1024, 1025, (len(ks), M, N)) / 4.0).astype(np.float32) if with_c else None
    D = run_kg(gpu_lib, As, sa, Bs, sb, ks, C, path=path)
    if D is None:
        return
    X = ogemm.gemm_k_grouped_tn(As, sa, Bs, sb, ks, C=C)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


@pytest.mark.parametrize("M,N", [(257, 1030), (272, 1040)])
def test_random_inputs(gpu_lib, path, M, N):
    ks = [512, 0, 1024, 128]
    announce(f"k-grouped {path} random {M}x{N} ks={ks}")
    A32, B32 = synth.dense_problem(M, N, sum(ks), seed=37)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    As, Bs = np.ascontiguousarray(qa.T), np.ascontiguousarray(qb.T)
    C = np.random.default_rng(5).standard_normal((len(ks), M, N)).astype(np.float32)
    D = run_kg(gpu_lib, As, sa, Bs, sb, ks, C, path=path)
    if D is None:
        return
    X, S = ogemm.gemm_k_grouped_tn(As, sa, Bs, sb, ks, C=C, with_magnitude=True)
    for g, k in enumerate(ks):
        assert_close(bf16_to_f64(D[g]), X[g], S[g], max(k // 128, 1) + 1, f"k-grouped random group {g}")


@pytest.mark.parametrize("M,N", [(300, 700), (304, 704)])
def test_one_group_is_the_tn_layout(gpu_lib, M, N):
    """One group equals the TN layout, bit for bit: on copies (both) and,
    where the operands allow it, on the operands as stored (both)."""
    K = 1024
    announce(f"k-grouped one group = tn {M}x{N}")
    A32, B32 = synth.dense_problem(M, N, K, seed=41)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    As, Bs = np.ascontiguousarray(qa.T), np.ascontiguousarray(qb.T)
    for path in (["copy", "direct"] if M % 16 == 0 and N % 16 == 0 else ["copy"]):
        D1 = run_kg(gpu_lib, As, sa, Bs, sb, [K], path=path)
        D0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(0, dtype=torch.uint8, device="cuda") if path == "direct" else None
        gpu_lib.gemm_fp8_tn(dev_u8(As), dev_sa(sa), dev_u8(Bs), dev_f32(sb), D0, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(D1[0]), bf16_bits(D0)), path


def test_all_groups_empty(gpu_lib):
    """K_total = 0: D[g] = bf16(C[g]), or zeros without C."""
    M, N, ks = 70, 90, [0, 0, 0]
    announce("k-grouped all empty")
    As = np.zeros((0, M), np.uint8)
    Bs = np.zeros((0, N), np.uint8)
    sa = np.zeros((0, M), np.float32)
    sb = np.zeros((1, 0), np.float32)
    C = np.random.default_rng(6).standard_normal((3, M, N)).astype(np.float32)
    D = torch.full((3, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_k_grouped_tn_contiguous(
        torch.zeros(16, M, dtype=torch.uint8, device="cuda")[:0], torch.zeros(0, 72, device="cuda")[:, :M],
        torch.zeros(16, N, dtype=torch.uint8, device="cuda")[:0], torch.zeros(1, 0, device="cuda"), ks, D,
        C=dev_f32(C))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(ogemm.gemm_k_grouped_tn(As, sa, Bs, sb, ks, C=C)))


def test_bad_group_sizes_and_workspace_are_rejected(gpu_lib):
    M, N = 64, 256
    rng = np.random.default_rng(8)
    A, sa, B, sb = exact_regime(rng, M, N, 256)
    As, Bs = dev_u8(np.ascontiguousarray(A.T)), dev_u8(np.ascontiguousarray(B.T))
    D = torch.full((2, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # the binding checks that ks tiles K_total
        gpu_lib.gemm_fp8_k_grouped_tn_contiguous(As, dev_sa(sa), Bs, dev_f32(sb), [200, 100], D)
    # through the C ABI: a group size that is not a multiple of 128 fails
    # before any pointer is used
    import ctypes

    lib = gpu_lib.load_library()
    ks = (ctypes.c_int * 2)(200, 56)
    st = lib.gemm_fp8_k_grouped_tn_contiguous(None, M, None, M, None, N, None, ctypes.cast(ks, ctypes.c_void_p), 2,
                                              None, None, M, N, None, 0, None)
    assert st == 2  # FG_EALIGN
    ws = torch.empty(gpu_lib.k_grouped_workspace_bytes(M, N, 256) - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.FP8GemmError, match="workspace"):
        gpu_lib.gemm_fp8_k_grouped_tn_contiguous(As, dev_sa(sa), Bs, dev_f32(sb), [128, 128], D, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(D.float()).all()


def test_direct_path_with_empty_groups_and_addend(gpu_lib):
    """Without a workspace (NULL through the C ABI): empty groups (first,
    middle, last) get bf16(C[g]) from the fill kernel, and 256 groups with K
    rows take one launch."""
    import ctypes

    M, N = 48, 80
    ks = [0] + [128] * 128 + [0] + [128] * 128 + [0]
    Kt = sum(ks)
    announce(f"k-grouped direct {M}x{N} {len(ks)} groups")
    rng = np.random.default_rng(14)
    A, sa, B, sb = exact_regime(rng, M, N, Kt)
    As, Bs = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    C = (rng.integers(-1024, 1025, (len(ks), M, N)) / 4.0).astype(np.float32)
    Ad, Bd, sad, sbd, Cd = dev_u8(As), dev_u8(Bs), dev_sa(sa), dev_f32(sb), dev_f32(C)
    D = torch.full((len(ks), M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    kv = (ctypes.c_int * len(ks))(*ks)
    lib = gpu_lib.load_library()
    st = lib.gemm_fp8_k_grouped_tn_contiguous(Ad.data_ptr(), M, sad.data_ptr(), sad.stride(0), Bd.data_ptr(), N,
                                              sbd.data_ptr(), ctypes.cast(kv, ctypes.c_void_p), len(ks),
                                              Cd.data_ptr(), D.data_ptr(), M, N, None, 0, None)
    torch.cuda.synchronize()
    assert st == 0
    X = ogemm.gemm_k_grouped_tn(As, sa, Bs, sb, ks, C=C)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


def test_weight_gradient_size_sampled(gpu_lib, path):
    """Eight experts of 512 tokens each, M = 4096, N = 7168 (240 GFLOP), on
    both paths; sampled (group, rows, column blocks)."""
    M, N, ks = 4096, 7168, [512] * 8
    Kt = sum(ks)
    announce(f"k-grouped {path} weight-gradient size {M}x{N} ks={ks}")
    A32, B32 = synth.dense_problem(M, N, Kt, seed=0)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    del A32, B32
    As, Bs = np.ascontiguousarray(qa.T), np.ascontiguousarray(qb.T)
    D = run_kg(gpu_lib, As, sa, Bs, sb, ks, path=path)
    rng = np.random.default_rng(10)
    for g in (0, 3, 7):
        k0 = sum(ks[:g])
        kb0, kb1 = k0 // 128, (k0 + ks[g]) // 128
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 4, replace=False)]))
        for nb in (0, int(rng.integers(1, N // 128 - 1)), N // 128 - 1):
            cols = slice(nb * 128, nb * 128 + 128)
            X, S = ogemm.gemm_nt(qa[rows][:, k0:k0 + ks[g]], sa[kb0:kb1][:, rows], qb[cols][:, k0:k0 + ks[g]],
                                 sb[nb:nb + 1, kb0:kb1], with_magnitude=True)
            y = bf16_to_f64(D[g][torch.from_numpy(rows).cuda(), cols])
            assert_close(y, X, S, kb1 - kb0, f"k-grouped group {g} block {nb}")
