"""Host-side boundary tests (no GPU): the C library loads, exports every
symbol the header declares, and rejects bad arguments with the documented
status codes before touching the device."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import moe_grouped_gemm_e4m3_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gemm.h")

FG_OK, FG_EINVAL, FG_EALIGN, FG_EUNSUPPORTED, FG_EHIP = 0, 1, 2, 3, 4


def header_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([A-Za-z_]\w*)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    return fg.load_library()


def test_header_symbols_exported(lib):
    names = header_functions()
    assert len(names) >= 10
    assert set(names) == set(fg.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_alignment(lib):
    assert lib.fg_version().startswith(b"fp8gemm")
    assert lib.fg_get_mk_alignment_for_contiguous_layout() == 128
    assert fg.get_mk_alignment_for_contiguous_layout() == 128


# fake device addresses: never dereferenced, the checks fail before any launch
P16 = 0x10000
P8 = 0x10008
P4 = 0x10004


def dense(lib, A=P16, lda=512, sa=P16, ld_sa=64, B=P16, ldb=512, sb=P16, D=P16, ldd=256, M=64, N=256, K=512):
    return lib.gemm_fp8_nt(A, lda, sa, ld_sa, B, ldb, sb, D, ldd, M, N, K, None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(M=-1), FG_EINVAL, "negative"),
        (dict(N=-3), FG_EINVAL, "negative"),
        (dict(K=-128), FG_EINVAL, "negative"),
        (dict(K=100), FG_EALIGN, "K=100"),
        (dict(A=None), FG_EINVAL, "A is NULL"),
        (dict(B=None), FG_EINVAL, "B is NULL"),
        (dict(sa=None), FG_EINVAL, "sa is NULL"),
        (dict(sb=None), FG_EINVAL, "sb is NULL"),
        (dict(D=None), FG_EINVAL, "D is NULL"),
        (dict(A=P8), FG_EALIGN, "A is not 16-byte"),
        (dict(B=P4), FG_EALIGN, "B is not 16-byte"),
        (dict(D=P8 + 1), FG_EALIGN, "D is not 2-byte"),
        (dict(sa=P4 + 2), FG_EALIGN, "sa is not 4-byte"),
        (dict(sb=P4 + 2), FG_EALIGN, "sb is not 4-byte"),
        (dict(lda=500), FG_EINVAL, "lda=500"),
        (dict(lda=520), FG_EALIGN, "lda=520"),
        (dict(ldb=520), FG_EALIGN, "ldb=520"),
        (dict(ldd=200), FG_EINVAL, "ldd=200"),
        (dict(ld_sa=32), FG_EINVAL, "ld_sa=32"),
        (dict(lda=(1 << 22) + 16, ldb=(1 << 22) + 16), FG_EUNSUPPORTED, "4 MiB"),
        (dict(M=(1 << 30) + 1, ld_sa=1 << 31), FG_EUNSUPPORTED, "2^30"),
    ],
)
def test_dense_argument_errors(lib, kw, status, needle):
    st = dense(lib, **kw)
    assert st == status
    assert needle in lib.fg_last_error().decode()


def dense_ws(lib, ws=P16 * 16, ws_bytes=1 << 20, **kw):
    a = dict(A=P16, lda=512, sa=P16, ld_sa=64, B=P16, ldb=512, sb=P16, D=P16, ldd=256, M=64, N=256, K=512)
    a.update(kw)
    return lib.gemm_fp8_nt_ws(a["A"], a["lda"], a["sa"], a["ld_sa"], a["B"], a["ldb"], a["sb"], a["D"], a["ldd"],
                              a["M"], a["N"], a["K"], ws, ws_bytes, None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(ws_bytes=-1), FG_EINVAL, "negative"),
        (dict(ws=None, ws_bytes=4096), FG_EINVAL, "workspace is NULL"),
        (dict(ws=P16 * 16 + 16), FG_EALIGN, "256-byte aligned"),
        (dict(K=100), FG_EALIGN, "K=100"),
        (dict(A=None), FG_EINVAL, "A is NULL"),
        (dict(M=-2), FG_EINVAL, "negative"),
    ],
)
def test_dense_workspace_argument_errors(lib, kw, status, needle):
    """gemm_fp8_nt_ws checks its workspace arguments on the host before any
    device query (the too-small case needs the device's plan: a GPU test)."""
    assert dense_ws(lib, **kw) == status
    assert needle in lib.fg_last_error().decode()


def test_workspace_queries_on_the_host(lib):
    assert lib.fg_nt_workspace_max_bytes() == (8 << 20) + (64 << 10)
    assert lib.fg_nt_workspace_bytes(-1, 64, 128) == -1
    assert lib.fg_nt_workspace_bytes(64, -1, 128) == -1
    # sizes the calls reject have no workspace size (and no overflow)
    assert lib.fg_layout_workspace_bytes(b"tn", 64, 64, (1 << 22) + 16) == -1
    assert lib.fg_k_grouped_workspace_bytes((1 << 30) + 1, 64, 128) == -1
    assert lib.fg_layout_workspace_bytes(b"tn", 3, 5, 256) == 768 + 1280  # each copy rounded to 256 bytes


def test_empty_problems_are_noops(lib):
    # no pointers at all: nothing may be touched or launched
    assert lib.gemm_fp8_nt(None, 0, None, 0, None, 0, None, None, 0, 0, 128, 256, None) == FG_OK
    assert lib.fg_last_error() == b""
    assert lib.gemm_fp8_nt(None, 0, None, 0, None, 0, None, None, 0, 16, 0, 256, None) == FG_OK
    assert lib.gemm_fp8_grouped_contiguous(None, None, 0, None, None, None, None, 0, 64, 256, 4, None) == FG_OK
    assert lib.gemm_fp8_grouped_masked(None, None, 0, None, None, None, None, 4, 0, 64, 256, 0, None) == FG_OK
    assert lib.fp8_cast_per_token(None, 0, None, None, 0, 0, 256, None) == FG_OK
    assert lib.fp8_cast_per_block(None, 0, None, None, 0, 256, None) == FG_OK


def test_error_string_cleared_on_next_call(lib):
    assert dense(lib, K=100) == FG_EALIGN
    assert lib.fg_last_error() != b""
    assert lib.gemm_fp8_nt(None, 0, None, 0, None, 0, None, None, 0, 0, 1, 128, None) == FG_OK
    assert lib.fg_last_error() == b""


def contig(lib, A=P16, sa=P16, ld_sa=256, B=P16, sb=P16, idx=P16, D=P16, M=256, N=256, K=512, G=4):
    return lib.gemm_fp8_grouped_contiguous(A, sa, ld_sa, B, sb, idx, D, M, N, K, G, None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(G=0), FG_EINVAL, "G=0"),
        (dict(G=-2), FG_EINVAL, "G=-2"),
        (dict(M=200), FG_EALIGN, "M_total=200"),
        (dict(K=130), FG_EALIGN, "K=130"),
        (dict(idx=None), FG_EINVAL, "m_indices is NULL"),
        (dict(idx=P4 + 2), FG_EALIGN, "m_indices"),
        (dict(A=None), FG_EINVAL, "A is NULL"),
        (dict(ld_sa=128), FG_EINVAL, "ld_sa=128"),
        (dict(D=P8 + 1), FG_EALIGN, "D is not"),
    ],
)
def test_contiguous_argument_errors(lib, kw, status, needle):
    assert contig(lib, **kw) == status
    assert needle in lib.fg_last_error().decode()


def masked(lib, A=P16, sa=P16, ld_sa=256, B=P16, sb=P16, mask=P16, D=P16, G=4, Mc=256, N=256, K=512):
    return lib.gemm_fp8_grouped_masked(A, sa, ld_sa, B, sb, mask, D, G, Mc, N, K, 0, None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(G=0), FG_EINVAL, "G=0"),
        (dict(Mc=-1), FG_EINVAL, "negative"),
        (dict(K=72), FG_EALIGN, "K=72"),
        (dict(mask=None), FG_EINVAL, "masked_m is NULL"),
        (dict(B=None), FG_EINVAL, "B is NULL"),
        (dict(ld_sa=100), FG_EINVAL, "ld_sa=100"),
        (dict(sa=P4 + 1), FG_EALIGN, "sa is not 4-byte"),
    ],
)
def test_masked_argument_errors(lib, kw, status, needle):
    assert masked(lib, **kw) == status
    assert needle in lib.fg_last_error().decode()


def test_cast_argument_errors(lib):
    assert lib.fp8_cast_per_token(P16, 512, P8, P4, 64, 64, 500, None) == FG_EALIGN
    assert lib.fp8_cast_per_token(None, 512, P8, P4, 64, 64, 512, None) == FG_EINVAL
    assert lib.fp8_cast_per_token(P8, 512, P8, P4, 64, 64, 512, None) == FG_EALIGN
    assert lib.fp8_cast_per_token(P16, 500, P8, P4, 64, 64, 512, None) == FG_EINVAL
    assert lib.fp8_cast_per_token(P16, 512, P8, P4, 32, 64, 512, None) == FG_EINVAL
    assert lib.fp8_cast_per_token(P16, 512, P4, P4, 64, 64, 512, None) == FG_EALIGN
    assert lib.fp8_cast_per_block(P16, 256, P4, P4, 130, 200, None) == FG_EALIGN
    assert lib.fp8_cast_per_block(P16, 255, P4, P4, 130, 256, None) == FG_EINVAL
    assert lib.fp8_cast_per_block(P16, 256, None, P4, 130, 256, None) == FG_EINVAL
    assert lib.fp8_cast_per_block(P16, 256, P4, P4, -1, 256, None) == FG_EINVAL


def test_k_tail_alignment_rules(lib):
    """K % 16 == 0 is enough for the fp32- and power-of-two-factor calls (a
    partial last K group); K % 16 != 0 fails everywhere.  Checked before
    anything touches a device."""
    for K in (8, 100, 1028):
        assert dense(lib, K=K, lda=512, ldb=512) == FG_EALIGN
        assert "multiple of 16" in lib.fg_last_error().decode()
        assert contig(lib, K=K) == FG_EALIGN
        assert masked(lib, K=K) == FG_EALIGN
        assert lib.fp8_cast_per_token(P16, 512, P8, P4, 64, 64, K, None) == FG_EALIGN
        assert lib.fp8_cast_per_block(P16, 512, P4, P4, 130, K, None) == FG_EALIGN
        assert lib.gemm_fp8_nt_ue8m0(P16, 512, P4, 64, P16, 512, P4, P16, 256, 64, 256, K, None) == FG_EALIGN
        assert "multiple of 16" in lib.fg_last_error().decode()
        assert lib.gemm_fp8_grouped_contiguous_ue8m0(P16, P4, 256, P16, P4, P4, P16, 256, 256, K, 2,
                                                     None) == FG_EALIGN
        assert lib.gemm_fp8_grouped_masked_ue8m0(P16, P4, 64, P16, P4, P4, P16, 2, 64, 256, K, 0,
                                                 None) == FG_EALIGN
        assert lib.fp8_cast_per_token_ue8m0(P16, 512, P8, P4, 64, 64, K, None) == FG_EALIGN
        assert lib.fp8_cast_per_block_ue8m0(P16, 512, P4, P4, 130, K, None) == FG_EALIGN


def test_num_cus_setter(lib):
    lib.fg_set_num_cus(7)
    assert lib.fg_get_num_cus() == 7
    lib.fg_set_num_cus(0)
    lib.fg_set_num_cus(-5)  # non-positive means "all"
    lib.fg_set_num_cus(0)


def test_python_wrappers_reject_cpu_tensors():
    import torch

    a = torch.zeros(4, 128, dtype=torch.uint8)
    with pytest.raises((TypeError, ValueError)):
        fg.gemm_fp8_nt(a, torch.zeros(1, 4), a, torch.zeros(1, 1), torch.zeros(4, 4, dtype=torch.bfloat16))


def test_python_ue8m0_wrappers_reject_cpu_tensors():
    """The power-of-two-factor wrappers check dtypes and devices before any
    call into the library (CPU tensors never reach a kernel)."""
    import torch

    a = torch.zeros(2, 128, 128, dtype=torch.uint8)
    i32 = torch.zeros(2, 1, 128, dtype=torch.int32)
    mask = torch.zeros(2, dtype=torch.int32)
    d = torch.zeros(2, 128, 128, dtype=torch.bfloat16)
    with pytest.raises((TypeError, ValueError)):
        fg.gemm_fp8_grouped_masked_ue8m0(a, i32, a, torch.zeros(2, 1, 1, dtype=torch.int32), mask, d)
    with pytest.raises((TypeError, ValueError)):
        fg.gemm_fp8_grouped_contiguous_ue8m0(a[0], i32[0], a, torch.zeros(2, 1, 1, dtype=torch.int32),
                                             torch.zeros(128, dtype=torch.int32), d[0])
    with pytest.raises((TypeError, ValueError)):
        fg.fp8_cast_per_token_ue8m0(torch.zeros(4, 128, dtype=torch.bfloat16))
    with pytest.raises((TypeError, ValueError)):
        fg.fp8_cast_per_block_ue8m0(torch.zeros(4, 128))
