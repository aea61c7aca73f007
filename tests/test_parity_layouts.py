"""The NN, TN and TT storage layouts on the GPU against the CPU oracle.

Two paths serve an operand stored MN-major: with a workspace, a byte
transpose into it followed by the NT kernels on the copy; without one, the
large-tile kernel staging it as stored (the transposing LDS reads build the
MFMA fragments).  A wrong
byte anywhere in either changes the GEMM result: in the exact regime (integer
codes, power-of-two scales, an addend on a 1/4 grid) every layout is compared
bit for bit on both paths, for the few-row, 128x128 and large-tile kernels,
with ragged shapes that leave partial tiles and K tails, and with row strides
that force the transpose's byte-wise paths or pad the direct path's rows with
NaN bytes it must never read."""

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

LAYOUTS = ["nn", "tn", "tt"]
ENV_KEYS = ("FG_SKINNY", "FG_FORCE_CONFIG", "FG_FORCE_BN", "FG_LAYOUT_COPY")
# "copy": a workspace from torch's allocator, copies forced (FG_LAYOUT_COPY=1;
# by default the plan may skip them where the large tiles fill the device);
# "direct": an empty workspace (operands staged as stored)
PATHS = ["copy", "direct"]


@pytest.fixture(autouse=True)
def default_plan(monkeypatch):
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)


@pytest.fixture(params=PATHS)
def path(request, monkeypatch):
    if request.param == "copy":
        monkeypatch.setenv("FG_LAYOUT_COPY", "1")
    return request.param


def direct_ok(layout, M, N, lda=None, ldb=None):
    """The direct path's rule: each MN-major operand has a row stride and a
    column count that are multiples of 16."""
    ok = True
    if layout[0] == "t":
        ok &= M % 16 == 0 and (lda or M) % 16 == 0
    if layout[1] == "n":
        ok &= N % 16 == 0 and (ldb or N) % 16 == 0
    return ok


def stored(layout, A, B):
    """NT codes A [M, K], B [N, K] -> the arrays the layout stores."""
    As = np.ascontiguousarray(A.T) if layout[0] == "t" else A
    Bs = np.ascontiguousarray(B.T) if layout[1] == "n" else B
    return As, Bs


def dev_padded(a: np.ndarray, pad: int) -> torch.Tensor:
    """A view of a wider device buffer (row stride = columns + pad); the padding
    holds 0x7F (NaN) bytes that must never be read into the result."""
    buf = torch.full((a.shape[0], a.shape[1] + pad), 0x7F, dtype=torch.uint8, device="cuda")
    buf[:, : a.shape[1]] = dev_u8(a)
    return buf[:, : a.shape[1]]


def call(fg, layout, As, sa, Bs, sb, C=None, out=None, pad=(0, 0), path="copy"):
    M = sa.shape[1]
    N = Bs.shape[1] if layout[1] == "n" else Bs.shape[0]
    D = out if out is not None else sentinel_like((M, N))
    Ad = dev_padded(As, pad[0]) if pad[0] else dev_u8(As)
    Bd = dev_padded(Bs, pad[1]) if pad[1] else dev_u8(Bs)
    ws = torch.empty(0, dtype=torch.uint8, device="cuda") if path == "direct" else None
    getattr(fg, "gemm_fp8_" + layout)(Ad, dev_sa(sa), Bd, dev_f32(sb), D, C=None if C is None else dev_f32(C),
                                      workspace=ws)
    torch.cuda.synchronize()
    return D


def call_or_reject(fg, layout, As, sa, Bs, sb, path, ok, **kw):
    """call(); on the direct path with operands it does not take, check the
    FG_EALIGN error and that D is untouched, and return None."""
    if path == "direct" and not ok:
        M = sa.shape[1]
        N = Bs.shape[1] if layout[1] == "n" else Bs.shape[0]
        D = kw.pop("out", None)
        D = D if D is not None else sentinel_like((M, N))
        with pytest.raises(fg.FP8GemmError, match="without a workspace"):
            call(fg, layout, As, sa, Bs, sb, out=D, path=path, **kw)
        assert (bf16_bits(D) == SENTINEL_BF16).all()
        return None
    return call(fg, layout, As, sa, Bs, sb, path=path, **kw)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (37, 200, 512), (128, 130, 256), (300, 1000, 640),
                                   (513, 2112, 256), (1100, 1300, 384), (144, 272, 384), (528, 1040, 640),
                                   (400, 2064, 272), (784, 16, 128)])
@pytest.mark.parametrize("with_c", [False, True], ids=["no-C", "C"])
def test_exact_regime_bitwise(gpu_lib, path, layout, M, N, K, with_c):
    announce(f"layout {layout} {path} exact regime {M}x{N}x{K} C={with_c}")
    rng = np.random.default_rng(M + 7 * N + K + len(layout))
    A, sa, B, sb = exact_regime(rng, M, N, K)
    As, Bs = stored(layout, A, B)
    C = (rng.integers(-1024, 1025, (M, N)) / 4.0).astype(np.float32) if with_c else None
    D = call_or_reject(gpu_lib, layout, As, sa, Bs, sb, path, direct_ok(layout, M, N), C=C)
    if D is not None:
        assert np.array_equal(bf16_bits(D), ogemm.to_bf16(ogemm.gemm_layout(layout, As, sa, Bs, sb, C=C)))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,pad", [(150, 290, (1, 3)), (150, 290, (5, 16)), (150, 290, (16, 7)),
                                     (160, 288, (16, 32)), (160, 288, (48, 16))])
def test_strided_operands(gpu_lib, path, layout, M, N, pad):
    """Row strides that are not multiples of 16 on the stored operands (byte-wise
    transpose loads), padded 16-byte rows on the direct path, NaN bytes in the
    padding, and an output view with a sentinel border."""
    K = 384
    announce(f"layout {layout} {path} strided {M}x{N} pad={pad}")
    rng = np.random.default_rng(sum(pad))
    A, sa, B, sb = exact_regime(rng, M, N, K)
    As, Bs = stored(layout, A, B)
    # the K-major operand of nn / tt keeps the NT rule (stride a multiple of 16)
    pa = pad[0] if layout[0] == "t" else 16
    pb = pad[1] if layout[1] == "n" else 16
    Dbuf = sentinel_like((M + 2, N + 5))
    ok = direct_ok(layout, M, N, M + pa, N + pb)
    if call_or_reject(gpu_lib, layout, As, sa, Bs, sb, path, ok, out=Dbuf[:M, :N], pad=(pa, pb)) is None:
        return
    assert np.array_equal(bf16_bits(Dbuf[:M, :N]), ogemm.to_bf16(ogemm.gemm_layout(layout, As, sa, Bs, sb)))
    bits = bf16_bits(Dbuf)
    assert (bits[M:, :] == SENTINEL_BF16).all() and (bits[:, N:] == SENTINEL_BF16).all()


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N", [(257, 1030), (272, 1040)])
def test_random_inputs(gpu_lib, path, layout, M, N):
    K = 1024
    announce(f"layout {layout} {path} random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=23)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    As, Bs = stored(layout, qa, qb)
    C = np.random.default_rng(2).standard_normal((M, N)).astype(np.float32)
    D = call_or_reject(gpu_lib, layout, As, sa, Bs, sb, path, direct_ok(layout, M, N), C=C)
    if D is None:
        return
    X, S = ogemm.gemm_layout(layout, As, sa, Bs, sb, C=C, with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, K // 128 + 1, f"layout {layout} random")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_same_bits_as_nt(gpu_lib, layout):
    """The layouts run the NT kernels on a transposed copy: same bits as the
    NT entry point (neither splits K)."""
    M, N, K = 64, 2112, 1024
    announce(f"layout {layout} equals nt")
    A32, B32 = synth.dense_problem(M, N, K, seed=29)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D0 = sentinel_like((M, N))
    gpu_lib.gemm_fp8_nt_unsplit(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), D0)
    As, Bs = stored(layout, qa, qb)
    D1 = call(gpu_lib, layout, As, sa, Bs, sb)
    assert np.array_equal(bf16_bits(D1), bf16_bits(D0))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_direct_same_bits_as_transposed(gpu_lib, monkeypatch, layout):
    """Staging an MN-major operand as stored and transposing it first feed the
    same bytes to the same MFMAs in the same order: identical bits."""
    M, N, K = 1040, 2064, 1280
    announce(f"layout {layout} direct equals transposed")
    A32, B32 = synth.dense_problem(M, N, K, seed=31)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    As, Bs = stored(layout, qa, qb)
    C = np.random.default_rng(3).standard_normal((M, N)).astype(np.float32)
    monkeypatch.setenv("FG_FORCE_CONFIG", "big")
    D1 = call(gpu_lib, layout, As, sa, Bs, sb, C, path="direct")
    D0 = call(gpu_lib, layout, As, sa, Bs, sb, C, path="copy")
    assert np.array_equal(bf16_bits(D1), bf16_bits(D0))
    X, S = ogemm.gemm_layout(layout, As, sa, Bs, sb, C=C, with_magnitude=True)
    assert_close(bf16_to_f64(D1), X, S, K // 128 + 1, f"layout {layout} direct")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_planned_path_with_workspace(gpu_lib, monkeypatch, layout):
    """With a workspace and the default plan, at a size where the plan skips
    the copies (16 x 28 tiles of 256 x 256 on the device), at one where it
    keeps them (16 x 9 tiles), and at the first size with row strides the
    copy-free path cannot take (8 bytes of padding: the copies again): the
    same bits as the forced copies, and the exact-regime value."""
    for (M, N, K, pad) in [(4096, 7168, 256, 0), (4096, 2112, 256, 0), (4096, 7168, 256, 8)]:
        announce(f"layout {layout} planned path {M}x{N}x{K} pad {pad}")
        rng = np.random.default_rng(M + N + pad)
        A, sa, B, sb = exact_regime(rng, M, N, K)
        As, Bs = stored(layout, A, B)
        # only the MN-major operands take the odd stride (a K-major one keeps the NT rule)
        pads = (pad if layout[0] == "t" else 0, pad if layout[1] == "n" else 0)
        monkeypatch.setenv("FG_LAYOUT_COPY", "1")
        D0 = call(gpu_lib, layout, As, sa, Bs, sb, pad=pads)
        monkeypatch.delenv("FG_LAYOUT_COPY")
        D1 = call(gpu_lib, layout, As, sa, Bs, sb, pad=pads)
        assert np.array_equal(bf16_bits(D1), bf16_bits(D0))
        assert np.array_equal(bf16_bits(D1), ogemm.to_bf16(ogemm.gemm_layout(layout, As, sa, Bs, sb)))


def test_direct_path_needs_no_workspace(gpu_lib):
    """Through the C ABI: a NULL workspace of 0 bytes runs the direct path."""
    import ctypes

    M, N, K = 2048, 4096, 256
    rng = np.random.default_rng(12)
    A, sa, B, sb = exact_regime(rng, M, N, K)
    As, Bs = stored("tn", A, B)
    Ad, Bd, sad, sbd = dev_u8(As), dev_u8(Bs), dev_sa(sa), dev_f32(sb)
    D = sentinel_like((M, N))
    lib = gpu_lib.load_library()
    st = lib.gemm_fp8_tn(Ad.data_ptr(), M, sad.data_ptr(), sad.stride(0), Bd.data_ptr(), N, sbd.data_ptr(), None, 0,
                         D.data_ptr(), N, M, N, K, None, 0, None)
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(ogemm.gemm_layout("tn", As, sa, Bs, sb)))


def test_workspace_too_small_is_rejected(gpu_lib):
    M, N, K = 64, 256, 256
    rng = np.random.default_rng(3)
    A, sa, B, sb = exact_regime(rng, M, N, K)
    As, Bs = stored("tn", A, B)
    need = gpu_lib.layout_workspace_bytes("tn", M, N, K)
    assert need == M * K + N * K
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    D = sentinel_like((M, N))
    with pytest.raises(gpu_lib.FP8GemmError, match="workspace"):
        gpu_lib.gemm_fp8_tn(dev_u8(As), dev_sa(sa), dev_u8(Bs), dev_f32(sb), D, workspace=ws)
    torch.cuda.synchronize()
    assert (bf16_bits(D) == SENTINEL_BF16).all()


def test_full_size_tn_sampled(gpu_lib, path):
    """TN (both operands stored [K, .], the weight-gradient form) at the dense
    4096 x 7168 x 2048 size, on both paths; sampled rows x column blocks."""
    M, N, K = synth.DENSE_M4096.shapes[4]
    announce(f"layout tn {path} full size {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    As, Bs = stored("tn", qa, qb)
    D = call(gpu_lib, "tn", As, sa, Bs, sb, path=path)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 6, replace=False)]))
    for nb in np.unique(np.concatenate([[0, N // 128 - 1], rng.choice(N // 128, 2, replace=False)])):
        cols = slice(nb * 128, nb * 128 + 128)
        X, S = ogemm.gemm_nt(qa[rows], sa[:, rows], qb[cols], sb[nb:nb + 1], with_magnitude=True)
        y = bf16_to_f64(D[torch.from_numpy(rows).cuda(), cols])
        assert_close(y, X, S, K // 128, f"tn full size block {nb}")
