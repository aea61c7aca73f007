"""K tails (K % 128 != 0, K % 16 == 0) on the GPU against the CPU oracle.

The last K group is partial: it holds the K % 128 remaining columns and has
its own factors.  Every kernel reads a 128-wide slice, so the columns past K
must enter the sums as zeros.  Packed operands (row stride K) put the next
row's codes there; strided ones put 0x7F bytes (NaN in e4m3) in the padding,
which would poison any result they reached.  In the exact regime (integer
codes, power-of-two factors) every result is compared bit for bit, for the
few-row (with and without a K split), 128x128 and large-tile kernels, the
grouped forms, the addend and the storage layouts; N(0,1) problems are
checked against the oracle's bound; the casts are compared byte for byte."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, quant
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_f32, dev_sa, dev_u8, exact_regime,
    quantize_dense, sentinel_like,
)

pytestmark = pytest.mark.gpu

ENV_KEYS = ("FG_SKINNY", "FG_FORCE_CONFIG", "FG_FORCE_BN")
TAIL_KS = [16, 48, 176, 304, 1040]


@pytest.fixture(autouse=True)
def default_plan(monkeypatch):
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)


def kb_of(K: int) -> int:
    return -(-K // 128)


def nan_padded(a: np.ndarray, pad: int) -> torch.Tensor:
    """A view of a wider device buffer whose padding columns hold 0x7F (NaN)."""
    buf = torch.full((a.shape[0], a.shape[1] + pad), 0x7F, dtype=torch.uint8, device="cuda")
    buf[:, : a.shape[1]] = dev_u8(a)
    return buf[:, : a.shape[1]]


def run(fg, qa, sa, qb, sb, pad=0):
    M, N = qa.shape[0], qb.shape[0]
    D = sentinel_like((M, N))
    A = nan_padded(qa, pad) if pad else dev_u8(qa)
    B = nan_padded(qb, pad) if pad else dev_u8(qb)
    fg.gemm_fp8_nt(A, dev_sa(sa), B, dev_f32(sb), D)
    torch.cuda.synchronize()
    return D


# (M, N, plan): the few-row kernel unsplit and split, the 128x128 and the
# large-tile kernel
PLANS = [
    (7, 136, {}),
    (64, 520, {"FG_SKINNY": "2,2"}),
    (128, 300, {"FG_SKINNY": "1,4"}),
    (200, 260, {"FG_FORCE_CONFIG": "small"}),
    (300, 520, {"FG_FORCE_CONFIG": "big"}),
    (300, 520, {"FG_FORCE_CONFIG": "big", "FG_FORCE_BN": "160"}),
]


@pytest.mark.parametrize("K", TAIL_KS)
@pytest.mark.parametrize("M,N,env", PLANS)
def test_dense_tail_exact_bitwise(gpu_lib, monkeypatch, M, N, env, K):
    if "FG_SKINNY" in env and kb_of(K) < 4 * int(env["FG_SKINNY"].split(",")[1]):
        env = {}  # too few K slices to split; the default plan
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    announce(f"k-tail dense exact {M}x{N}x{K} {env}")
    rng = np.random.default_rng(M + 5 * N + 11 * K)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    for pad in (0, 32):
        D = run(gpu_lib, qa, sa, qb, sb, pad=pad)
        assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X)), f"pad={pad}"


@pytest.mark.parametrize("M,N,K", [(1, 64, 16), (64, 2112, 1040), (128, 4096, 7056), (257, 1030, 1424),
                                   (512, 512, 7184)])
def test_dense_tail_random(gpu_lib, M, N, K):
    announce(f"k-tail dense random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=M + N + K)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    D = run(gpu_lib, qa, sa, qb, sb)
    X, S = ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, kb_of(K), f"dense {M}x{N}x{K}")


def test_dense_tail_equals_zero_padded(gpu_lib):
    """A GEMM over K = 128j + t equals the same GEMM over K padded with zero
    codes to 128(j+1), with the same factors (the zeros add nothing)."""
    announce("k-tail dense vs zero-padded")
    M, N, K = 256, 384, 688
    A32, B32 = synth.dense_problem(M, N, K, seed=3)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    Kp = kb_of(K) * 128
    qa_p = np.zeros((M, Kp), np.uint8)
    qa_p[:, :K] = qa
    qb_p = np.zeros((N, Kp), np.uint8)
    qb_p[:, :K] = qb
    D = run(gpu_lib, qa, sa, qb, sb)
    Dp = run(gpu_lib, qa_p, sa, qb_p, sb)
    assert np.array_equal(bf16_bits(D), bf16_bits(Dp))


def test_addend_tail_exact(gpu_lib):
    announce("k-tail addend 96x200x400")
    rng = np.random.default_rng(9)
    M, N, K = 96, 200, 400
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    C = (rng.integers(-64, 64, (M, N)) / 4.0).astype(np.float32)
    D = sentinel_like((M, N))
    gpu_lib.gemm_fp8_nt_c(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb), dev_f32(C), D)
    torch.cuda.synchronize()
    X = ogemm.gemm_nt_addend(qa, sa, qb, sb, C)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layouts_tail_exact(gpu_lib, layout):
    announce(f"k-tail layout {layout} 70x260x208")
    rng = np.random.default_rng(len(layout) + ord(layout[0]))
    M, N, K = 70, 260, 208
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    As = np.ascontiguousarray(qa.T) if layout[0] == "t" else qa
    Bs = np.ascontiguousarray(qb.T) if layout[1] == "n" else qb
    D = sentinel_like((M, N))
    getattr(gpu_lib, "gemm_fp8_" + layout)(dev_u8(As), dev_sa(sa), dev_u8(Bs), dev_f32(sb), D)
    torch.cuda.synchronize()
    X = ogemm.gemm_layout(layout, As, sa, Bs, sb)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


def test_contiguous_tail_exact(gpu_lib):
    announce("k-tail contiguous rows=[130,0,250] N=136 K=336")
    rng = np.random.default_rng(21)
    rows, N, K = [130, 0, 250], 136, 336
    idx = synth.contiguous_indices(rows)
    G, Mt = len(rows), len(idx)
    qa, sa, _, _ = exact_regime(rng, Mt, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = sentinel_like((Mt, N))
    gpu_lib.gemm_fp8_grouped_contiguous(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb),
                                        torch.from_numpy(np.asarray(idx, np.int32)).cuda(), D)
    torch.cuda.synchronize()
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_masked_tail_exact(gpu_lib):
    announce("k-tail masked G=4 Mc=160 N=200 K=592")
    rng = np.random.default_rng(22)
    G, Mc, N, K = 4, 160, 200, 592
    qa, sa, qb, sb = exact_regime(rng, Mc, N, K, groups=(G, G))
    mask = [160, 0, 77, 129]
    D = sentinel_like((G, Mc, N))
    gpu_lib.gemm_fp8_grouped_masked(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb),
                                    torch.from_numpy(np.asarray(mask, np.int32)).cuda(), D)
    torch.cuda.synchronize()
    X, valid = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


@pytest.mark.parametrize("M,K", [(1, 16), (5, 48), (129, 176), (300, 7184), (512, 8208)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cast_per_token_tail_bytes(gpu_lib, M, K, dtype):
    announce(f"k-tail cast per-token {M}x{K} {dtype}")
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, -1] *= np.float32(40.0)  # the tail group's amax differs from the full groups'
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.to(torch.float32).numpy()  # exact widening
    q_ref, s_ref = quant.quantize_per_token(x)
    q, sa = gpu_lib.fp8_cast_per_token(xt.cuda())
    torch.cuda.synchronize()
    assert tuple(sa.shape) == (kb_of(K), M)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(1, 16), (130, 176), (2112, 1040), (256, 7184)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cast_per_block_tail_bytes(gpu_lib, N, K, dtype):
    announce(f"k-tail cast per-block {N}x{K} {dtype}")
    rng = np.random.default_rng(N + 3 * K)
    w = rng.standard_normal((N, K)).astype(np.float32)
    w[0, -1] = np.float32(75.0)
    wt = torch.from_numpy(w)
    if dtype == "bf16":
        wt = wt.to(torch.bfloat16)
        w = wt.to(torch.float32).numpy()
    q_ref, s_ref = quant.quantize_per_block(w)
    q, sb = gpu_lib.fp8_cast_per_block(wt.cuda())
    torch.cuda.synchronize()
    assert tuple(sb.shape) == (-(-N // 128), kb_of(K))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sb.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_cast_then_gemm_tail(gpu_lib):
    """The device casts feed the GEMM at a tail K: the result is within the
    oracle's bound of the oracle run on the oracle's own codes."""
    announce("k-tail cast+gemm 192x384x1360")
    M, N, K = 192, 384, 1360
    A32, B32 = synth.dense_problem(M, N, K, seed=8)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token(A32.cuda())
    qb_d, sb_d = gpu_lib.fp8_cast_per_block(B32.cuda())
    D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d, D)
    torch.cuda.synchronize()
    qa, sa, qb, sb = quantize_dense(A32, B32)
    X, S = ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, kb_of(K), "cast+gemm tail")


# ---------------------------------------------------------------------------
# Power-of-two (UE8M0) factors with a K tail: the casts byte for byte, the
# dense, contiguous and masked GEMMs bit for bit in the exact regime (for each
# tile shape) and within the bound on N(0,1) inputs.

from tests.test_parity_ue8m0 import (  # noqa: E402
    run as run_ue8m0, run_contig as run_contig_ue8m0, run_masked as run_masked_ue8m0, to_bytes,
)

UE8M0_TILES = ["256x224", "256x160", "128x256", "256x256"]


@pytest.mark.parametrize("M,K", [(5, 48), (129, 176), (300, 7184), (512, 8208)])
def test_ue8m0_cast_per_token_tail_bytes(gpu_lib, M, K):
    announce(f"k-tail ue8m0 cast per-token {M}x{K}")
    rng = np.random.default_rng(M + K + 1)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, -1] *= np.float32(40.0)
    q_ref, e_ref = quant.quantize_per_token_ue8m0(x)
    q, sa = gpu_lib.fp8_cast_per_token_ue8m0(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert tuple(sa.shape) == ((kb_of(K) + 3) // 4, M)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(quant.unpack_ue8m0(sa.cpu().numpy(), kb_of(K), axis=0), e_ref)


@pytest.mark.parametrize("N,K", [(1, 16), (130, 176), (256, 7184)])
def test_ue8m0_cast_per_block_tail_bytes(gpu_lib, N, K):
    announce(f"k-tail ue8m0 cast per-block {N}x{K}")
    rng = np.random.default_rng(N + K + 2)
    w = rng.standard_normal((N, K)).astype(np.float32)
    w[:, -3] *= np.float32(40.0)
    q_ref, e_ref = quant.quantize_per_block_ue8m0(w)
    q, sb = gpu_lib.fp8_cast_per_block_ue8m0(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert tuple(sb.shape) == (-(-N // 128), (kb_of(K) + 3) // 4)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(quant.unpack_ue8m0(sb.cpu().numpy(), kb_of(K), axis=1), e_ref)


@pytest.mark.parametrize("tile", UE8M0_TILES)
@pytest.mark.parametrize("K", [48, 1040])
def test_ue8m0_dense_tail_exact_regime_bitwise(gpu_lib, monkeypatch, tile, K):
    monkeypatch.setenv("FG_UE8M0_TILE", tile)
    M, N = 300, 520
    announce(f"k-tail ue8m0 dense {tile} {M}x{N}x{K}")
    rng = np.random.default_rng(K + len(tile))
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    D = run_ue8m0(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb))
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(ogemm.gemm_nt(qa, sa, qb, sb)))


def test_ue8m0_dense_tail_random(gpu_lib):
    M, N, K = 257, 1030, 1360
    announce(f"k-tail ue8m0 dense random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=17)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quant.quantize_per_block_ue8m0(B32.numpy())
    D = run_ue8m0(gpu_lib, qa, ea, qb, eb)
    X, S = ogemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, kb_of(K), "ue8m0 tail random")


@pytest.mark.parametrize("tile", UE8M0_TILES)
def test_ue8m0_contiguous_tail_exact_regime_bitwise(gpu_lib, monkeypatch, tile):
    monkeypatch.setenv("FG_UE8M0_TILE", tile)
    announce(f"k-tail ue8m0 contiguous {tile}")
    rng = np.random.default_rng(11 + len(tile))
    idx = synth.contiguous_indices([200, 60, 128, 1], pad_to=128)
    M, N, K, G = idx.shape[0], 264, 1040, 4
    qa, sa, _, _ = exact_regime(rng, M, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = run_contig_ue8m0(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb), idx)
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


@pytest.mark.parametrize("tile", UE8M0_TILES)
def test_ue8m0_masked_tail_exact_regime_bitwise(gpu_lib, monkeypatch, tile):
    monkeypatch.setenv("FG_UE8M0_TILE", tile)
    announce(f"k-tail ue8m0 masked {tile}")
    rng = np.random.default_rng(13 + len(tile))
    G, Mc, N, K = 4, 200, 300, 176
    qa, sa, qb, sb = exact_regime(rng, Mc, N, K, groups=(G, G))
    mask = [200, 0, 130, 7]
    D = run_masked_ue8m0(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb), mask)
    X, valid = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()
