"""Power-of-two (UE8M0) factors on the GPU against the CPU oracle: the two
casts, and the dense, contiguous and masked GEMMs, on the scaled MFMA and
(256x256 tiles) on the fp32-factor kernel with the factor bytes decoded.

The casts must match the oracle byte for byte (codes and factor bytes).  The
GEMM is compared bit for bit in the exact regime -- its factors {1/2, 1, 2}
are powers of two already -- for each of its tile shapes (FG_UE8M0_TILE), and within
the oracle's per-element bound on random inputs.  Doubling one factor (its
byte + 1) must double exactly the outputs it touches."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, quant
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_u8, exact_regime, sentinel_like,
)

pytestmark = pytest.mark.gpu


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_sa_packed(e: np.ndarray, pad: int = 4) -> torch.Tensor:
    """UE8M0 bytes [Kb, M] -> a [ceil(Kb/4), M] view of a padded int32 buffer."""
    p = quant.pack_ue8m0(e, axis=0)
    kb4, M = p.shape
    ld = max(4, (M + pad - 1) // pad * pad)
    buf = np.full((kb4, ld), -1, np.int32)  # padding never read
    buf[:, :M] = p
    return dev_i32(buf)[:, :M]


def to_bytes(s: np.ndarray) -> np.ndarray:
    """Power-of-two fp32 factors -> UE8M0 bytes (exact)."""
    e = quant.ue8m0_round_up(s)
    assert np.array_equal(quant.ue8m0_decode(e), s)
    return e


def run(fg, qa, ea, qb, eb, out=None):
    M, N = qa.shape[0], qb.shape[0]
    D = out if out is not None else sentinel_like((M, N))
    fg.gemm_fp8_nt_ue8m0(dev_u8(qa), dev_sa_packed(ea), dev_u8(qb), dev_i32(quant.pack_ue8m0(eb, axis=1)), D)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("M,K", [(1, 128), (37, 640), (256, 1536), (130, 512), (300, 14336)])
def test_cast_per_token_bytes(gpu_lib, M, K):
    announce(f"ue8m0 cast per token {M}x{K}")
    A32, _ = synth.dense_problem(M, 8, K, seed=M + K)
    x = A32.numpy().copy()
    x[0, :128] = 0.0  # an all-zero group
    q_ref, e_ref = quant.quantize_per_token_ue8m0(x)
    q, sa = gpu_lib.fp8_cast_per_token_ue8m0(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    got = quant.unpack_ue8m0(sa.cpu().numpy(), K // 128, axis=0)
    assert np.array_equal(got, e_ref)


@pytest.mark.parametrize("N,K", [(128, 128), (2112, 640), (300, 1024)])
def test_cast_per_block_bytes(gpu_lib, N, K):
    announce(f"ue8m0 cast per block {N}x{K}")
    _, B32 = synth.dense_problem(1, N, K, seed=N + K)
    q_ref, e_ref = quant.quantize_per_block_ue8m0(B32.numpy())
    q, sb = gpu_lib.fp8_cast_per_block_ue8m0(B32.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(quant.unpack_ue8m0(sb.cpu().numpy(), K // 128, axis=1), e_ref)


@pytest.fixture(params=["256x224", "256x160", "128x256", "256x256"])
def width(request, monkeypatch):
    """The tile shapes, forced with FG_UE8M0_TILE (256x256 runs on the
    fp32-factor kernel with each factor byte decoded, the others on the
    scaled MFMA); the value is the tile width (used to vary the seeds)."""
    monkeypatch.delenv("FG_FORCE_BN", raising=False)
    monkeypatch.setenv("FG_UE8M0_TILE", request.param)
    return int(request.param.split("x")[1])


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (70, 300, 256), (256, 896, 512), (300, 1000, 640), (513, 2112, 256)])
def test_gemm_exact_regime_bitwise(gpu_lib, width, M, N, K):
    announce(f"ue8m0 gemm width {width} exact regime {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K + width)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    D = run(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb))
    X = ogemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(X))


@pytest.mark.parametrize("M,N,K", [(40, 232, 256), (257, 1030, 1536), (512, 7168, 1024)])
def test_gemm_random(gpu_lib, width, M, N, K):
    announce(f"ue8m0 gemm width {width} random {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=N + K)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quant.quantize_per_block_ue8m0(B32.numpy())
    D = run(gpu_lib, qa, ea, qb, eb)
    X, S = ogemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), with_magnitude=True)
    assert_close(bf16_to_f64(D), X, S, K // 128, f"ue8m0 width {width} {M}x{N}x{K}")


def test_gemm_factor_equivariance(gpu_lib, width):
    """Raising one activation factor byte by one doubles that row exactly; one
    weight block's bytes by one double its 128 columns exactly."""
    M, N, K = 64, 640, 384
    A32, B32 = synth.dense_problem(M, N, K, seed=41)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quant.quantize_per_block_ue8m0(B32.numpy())
    announce(f"ue8m0 gemm width {width} equivariance")
    base = bf16_to_f64(run(gpu_lib, qa, ea, qb, eb))
    ea2 = ea.copy()
    ea2[:, 5] += 1
    y = bf16_to_f64(run(gpu_lib, qa, ea2, qb, eb))
    assert np.array_equal(y[5], 2 * base[5])
    assert np.array_equal(np.delete(y, 5, 0), np.delete(base, 5, 0))
    for nb in range(N // 128):
        eb2 = eb.copy()
        eb2[nb, :] += 1
        y = bf16_to_f64(run(gpu_lib, qa, ea, qb, eb2))
        cols = slice(128 * nb, 128 * nb + 128)
        assert np.array_equal(y[:, cols], 2 * base[:, cols]), nb
        rest = np.ones(N, bool)
        rest[cols] = False
        assert np.array_equal(y[:, rest], base[:, rest]), nb


def test_gemm_width_256_request_falls_back(gpu_lib, monkeypatch):
    """The scaled-MFMA kernel has no 256-wide tile; asking it for one with
    FG_FORCE_BN gives the 224-wide result."""
    M, N, K = 300, 700, 384
    rng = np.random.default_rng(7)
    qa, sa, qb, sb = exact_regime(rng, M, N, K)
    announce("ue8m0 gemm width 256 request")
    monkeypatch.setenv("FG_FORCE_BN", "256")
    D = run(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb))
    assert np.array_equal(bf16_bits(D), ogemm.to_bf16(ogemm.gemm_nt(qa, sa, qb, sb)))


def test_gemm_strided_output_and_tails(gpu_lib):
    announce("ue8m0 gemm strided output")
    M, N, K = 300, 200, 256
    A32, B32 = synth.dense_problem(M, N, K, seed=43)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quant.quantize_per_block_ue8m0(B32.numpy())
    Dbuf = sentinel_like((M + 3, N + 8))
    run(gpu_lib, qa, ea, qb, eb, out=Dbuf[:M, :N])
    X, S = ogemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), with_magnitude=True)
    assert_close(bf16_to_f64(Dbuf[:M, :N]), X, S, K // 128, "ue8m0 strided")
    bits = bf16_bits(Dbuf)
    assert (bits[M:, :] == SENTINEL_BF16).all() and (bits[:, N:] == SENTINEL_BF16).all()


@pytest.mark.parametrize("shape", synth.DENSE_M4096.shapes, ids=lambda s: "x".join(map(str, s)))
def test_full_size_gpu_cast_sampled(gpu_lib, monkeypatch, shape):
    """GPU casts + GEMM at the dense M=4096 sizes; sampled rows x column
    blocks against the oracle, which quantises those rows and blocks itself
    (the GPU's codes and factor bytes must equal its own)."""
    monkeypatch.delenv("FG_FORCE_BN", raising=False)
    M, N, K = shape
    announce(f"ue8m0 full size {M}x{N}x{K}")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token_ue8m0(A32.cuda())
    qb_d, sb_d = gpu_lib.fp8_cast_per_block_ue8m0(B32.cuda())
    D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt_ue8m0(qa_d, sa_d, qb_d, sb_d, D)
    torch.cuda.synchronize()
    Kb = K // 128
    ea_d = quant.unpack_ue8m0(sa_d.cpu().numpy(), Kb, axis=0)
    eb_d = quant.unpack_ue8m0(sb_d.cpu().numpy(), Kb, axis=1)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 6, replace=False)]))
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy()[rows])
    assert np.array_equal(qa_d[torch.from_numpy(rows).cuda()].cpu().numpy(), qa)
    assert np.array_equal(ea_d[:, rows], ea)
    for nb in np.unique(np.concatenate([[0, -(-N // 128) - 1], rng.choice(N // 128, 2, replace=False)])):
        cols = slice(nb * 128, min(N, nb * 128 + 128))
        qb, eb = quant.quantize_per_block_ue8m0(B32.numpy()[cols])
        assert np.array_equal(eb_d[nb:nb + 1], eb)
        X, S = ogemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), with_magnitude=True)
        y = bf16_to_f64(D[torch.from_numpy(rows).cuda(), cols])
        assert_close(y, X, S, Kb, f"ue8m0 full size block {nb}")


# ---------------------------------------------------------------------------
# Masked grouped GEMM with UE8M0 factors: each group as the dense definition
# with factors 2^(e - 127), rows past the group's count untouched.


def run_masked(fg, qa, ea, qb, eb, mask):
    """qa [G, Mc, K], ea bytes [G, Kb, Mc], qb [G, N, K], eb bytes [G, Nb, Kb]."""
    G, Mc, K = qa.shape
    N = qb.shape[1]
    kb4 = (K // 128 + 3) // 4
    ld = (Mc + 3) // 4 * 4 + 4
    buf = np.full((G, kb4, ld), -1, np.int32)  # padding never read
    for g in range(G):
        buf[g, :, :Mc] = quant.pack_ue8m0(ea[g], axis=0)
    sa = dev_i32(buf)[:, :, :Mc]
    sb = dev_i32(np.stack([quant.pack_ue8m0(eb[g], axis=1) for g in range(G)]))
    D = sentinel_like((G, Mc, N))
    fg.gemm_fp8_grouped_masked_ue8m0(dev_u8(qa), sa, dev_u8(qb), sb,
                                     torch.tensor(list(mask), dtype=torch.int32, device="cuda"), D)
    torch.cuda.synchronize()
    return D


def test_masked_exact_regime_bitwise(gpu_lib, width):
    """Counts of 0, 1, partial, more than one 128-row tile, the capacity, above
    it and negative; K = 640 leaves the last packed word half used."""
    announce(f"ue8m0 masked width {width} exact regime")
    rng = np.random.default_rng(width)
    G, Mc, N, K = 7, 200, 300, 640
    qa, sa, qb, sb = exact_regime(rng, Mc, N, K, groups=(G, G))
    mask = [200, 0, 33, 130, 1, 999, -5]
    D = run_masked(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb), mask)
    X, valid = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_masked_random(gpu_lib, width):
    announce(f"ue8m0 masked width {width} random")
    G, Mc, N, K = 4, 256, 1024, 1024
    g = torch.Generator().manual_seed(width)
    A32 = torch.randn(G, Mc, K, generator=g).numpy()
    B32 = torch.randn(G, N, K, generator=g).numpy()
    qs = [quant.quantize_per_token_ue8m0(a) for a in A32]
    ws = [quant.quantize_per_block_ue8m0(b) for b in B32]
    qa, ea = np.stack([q for q, _ in qs]), np.stack([e for _, e in qs])
    qb, eb = np.stack([q for q, _ in ws]), np.stack([e for _, e in ws])
    mask = [256, 1, 130, 64]
    D = run_masked(gpu_lib, qa, ea, qb, eb, mask)
    X, valid, S = ogemm.gemm_grouped_masked(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), mask,
                                            with_magnitude=True)
    bits = bf16_bits(D)
    assert (bits[~valid] == SENTINEL_BF16).all()
    assert_close(bf16_to_f64(D)[valid], X[valid], S[valid], K // 128, f"ue8m0 masked width {width}")


def test_masked_full_equals_dense(gpu_lib, width):
    """With every count at the capacity each group equals the dense call on
    its operands bit for bit (same tile shape, same summation order)."""
    announce(f"ue8m0 masked width {width} vs dense")
    G, Mc, N, K = 3, 130, 264, 512
    g = torch.Generator().manual_seed(6)
    A32 = torch.randn(G, Mc, K, generator=g).numpy()
    B32 = torch.randn(G, N, K, generator=g).numpy()
    qs = [quant.quantize_per_token_ue8m0(a) for a in A32]
    ws = [quant.quantize_per_block_ue8m0(b) for b in B32]
    qa, ea = np.stack([q for q, _ in qs]), np.stack([e for _, e in qs])
    qb, eb = np.stack([q for q, _ in ws]), np.stack([e for _, e in ws])
    Dm = bf16_bits(run_masked(gpu_lib, qa, ea, qb, eb, [Mc] * G))
    for e in range(G):
        assert np.array_equal(Dm[e], bf16_bits(run(gpu_lib, qa[e], ea[e], qb[e], eb[e]))), e


def test_promotion_and_scaled_mfma_kernels_agree(gpu_lib, monkeypatch):
    """The scaled MFMA adds a slice's exact dot product, times its power-of-two
    factor, into the fp32 accumulator with one rounding; the promotion kernel
    rounds the dot product to fp32 first.  The two differ only where that
    dot product has more than 24 significant bits, which random e4m3 rows of
    128 rarely give: on these dense and masked operands the bits are equal
    (a regression to a wrong factor byte or block would change most of them)."""
    M, N, K = 300, 520, 1024
    A32, B32 = synth.dense_problem(M, N, K, seed=77)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quant.quantize_per_block_ue8m0(B32.numpy())
    G, Mc = 3, 200
    g = torch.Generator().manual_seed(78)
    A3 = torch.randn(G, Mc, K, generator=g).numpy()
    B3 = torch.randn(G, N, K, generator=g).numpy()
    qs = [quant.quantize_per_token_ue8m0(a) for a in A3]
    ws = [quant.quantize_per_block_ue8m0(b) for b in B3]
    qa3, ea3 = np.stack([q for q, _ in qs]), np.stack([e for _, e in qs])
    qb3, eb3 = np.stack([q for q, _ in ws]), np.stack([e for _, e in ws])
    mask = [200, 77, 0]
    out = {}
    for tile in ("256x224", "256x256"):
        monkeypatch.setenv("FG_UE8M0_TILE", tile)
        announce(f"ue8m0 kernels agree {tile}")
        out[tile] = (bf16_bits(run(gpu_lib, qa, ea, qb, eb)), bf16_bits(run_masked(gpu_lib, qa3, ea3, qb3, eb3, mask)))
    assert np.array_equal(out["256x224"][0], out["256x256"][0])
    assert np.array_equal(out["256x224"][1], out["256x256"][1])


@pytest.mark.parametrize("shape", synth.MASKED_16x256.shapes, ids=lambda s: "x".join(map(str, s)))
def test_masked_decode_full_size(gpu_lib, monkeypatch, shape):
    """16 experts x capacity 256 with the seed-0 counts: GPU casts with UE8M0
    factors and the masked GEMM; sampled valid rows of every group against the
    oracle on the same codes, every invalid row untouched."""
    monkeypatch.delenv("FG_FORCE_BN", raising=False)
    monkeypatch.delenv("FG_UE8M0_TILE", raising=False)
    G, Mc, N, K = shape
    Kb, kb4 = K // 128, (K // 128 + 3) // 4
    announce(f"ue8m0 masked full-size {G}x{Mc} N={N} K={K}")
    A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=0)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token_ue8m0(A32.cuda().view(G * Mc, K))
    qa_d = qa_d.view(G, Mc, K)
    sa_g = torch.empty(G, kb4, Mc, dtype=torch.int32, device="cuda")
    sa_g.copy_(sa_d.reshape(kb4, G, Mc).permute(1, 0, 2))
    qb_d, sb_d = gpu_lib.fp8_cast_per_block_ue8m0(B32.cuda().view(G * N, K))
    qb_d, sb_d = qb_d.view(G, N, K), sb_d.view(G, N // 128, kb4)
    D = sentinel_like((G, Mc, N))
    gpu_lib.gemm_fp8_grouped_masked_ue8m0(qa_d, sa_g, qb_d, sb_d, torch.from_numpy(mask).cuda(), D)
    torch.cuda.synchronize()
    bits = bf16_bits(D)
    ea_d = quant.unpack_ue8m0(sa_d.cpu().numpy(), Kb, axis=0).reshape(Kb, G, Mc)
    eb_d = quant.unpack_ue8m0(sb_d.cpu().numpy().reshape(G * (N // 128), kb4), Kb, axis=1).reshape(G, N // 128, Kb)
    rng = np.random.default_rng(2)
    for g in range(G):
        v = int(mask[g])
        assert (bits[g, v:] == SENTINEL_BF16).all(), g
        if v == 0:
            continue
        rows = np.unique(np.concatenate([[0, v - 1], rng.choice(v, min(v, 4), replace=False)]))
        qa, ea = quant.quantize_per_token_ue8m0(A32.numpy()[g, rows])
        assert np.array_equal(qa_d[g, torch.from_numpy(rows).cuda()].cpu().numpy(), qa)
        assert np.array_equal(ea_d[:, g, rows], ea)
        nbs = range(N // 128) if g < 2 else rng.choice(N // 128, 2, replace=False)
        for nb in nbs:
            cols = slice(nb * 128, nb * 128 + 128)
            qb, eb = quant.quantize_per_block_ue8m0(B32.numpy()[g, cols])
            assert np.array_equal(eb_d[g, nb:nb + 1], eb)
            X, S = ogemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), with_magnitude=True)
            y = bf16_to_f64(D[g, torch.from_numpy(rows).cuda(), cols])
            assert_close(y, X, S, Kb, f"ue8m0 masked group {g} block {nb}")


# ---------------------------------------------------------------------------
# Contiguous grouped GEMM with UE8M0 factors: each row as the dense definition
# with its expert's weights, padding rows untouched.


def run_contig(fg, qa, ea, qb, eb, idx):
    """qa [M, K], ea bytes [Kb, M], qb [G, N, K], eb bytes [G, Nb, Kb]."""
    M, N = qa.shape[0], qb.shape[1]
    G = qb.shape[0]
    sb = dev_i32(np.stack([quant.pack_ue8m0(eb[g], axis=1) for g in range(G)]))
    D = sentinel_like((M, N))
    fg.gemm_fp8_grouped_contiguous_ue8m0(dev_u8(qa), dev_sa_packed(ea), dev_u8(qb), sb,
                                         torch.from_numpy(np.asarray(idx, np.int32)).cuda(), D)
    torch.cuda.synchronize()
    return D


def quantize_experts_ue8m0(B32):
    ws = [quant.quantize_per_block_ue8m0(b) for b in B32]
    return np.stack([q for q, _ in ws]), np.stack([e for _, e in ws])


def test_contig_index_past_experts_is_padding(gpu_lib):
    """As for the fp32-factor kernel: blocks indexed G or above are padding."""
    announce("ue8m0 contiguous indices past the experts")
    rng = np.random.default_rng(19)
    G, N, K = 2, 264, 640
    idx = np.repeat(np.asarray([G, 0, 1000, 1, G + 1, 1 << 30], np.int32), 128)
    M = idx.shape[0]
    qa, sa, _, _ = exact_regime(rng, M, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = run_contig(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb), idx)
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, np.where(idx >= G, -1, idx))
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_contig_exact_regime_bitwise(gpu_lib, width):
    """Expert blocks of 256, 128, 0, 128 and 128 rows (the 256-row tile over
    rows 256..511 holds two experts and runs as two segments; the last tile is
    half past M_total); N = 264 leaves a ragged column tile, K = 640 a
    half-used packed word."""
    announce(f"ue8m0 contiguous width {width} exact regime")
    rng = np.random.default_rng(width + 1)
    idx = synth.contiguous_indices([200, 60, 0, 128, 1], pad_to=128)
    M, N, K, G = idx.shape[0], 264, 640, 5
    qa, sa, _, _ = exact_regime(rng, M, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = run_contig(gpu_lib, qa, to_bytes(sa), qb, to_bytes(sb), idx)
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


@pytest.mark.parametrize("rows,N,K", [([130, 0, 100, 1], 520, 384), ([384], 136, 1024)])
def test_contig_random(gpu_lib, width, rows, N, K):
    announce(f"ue8m0 contiguous width {width} rows={rows} N={N} K={K}")
    A32, B32, idx = synth.contiguous_problem(rows, N, K, seed=len(rows) + width)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quantize_experts_ue8m0(B32.numpy())
    D = run_contig(gpu_lib, qa, ea, qb, eb, idx)
    X, valid, S = ogemm.gemm_grouped_contiguous(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), idx,
                                                with_magnitude=True)
    assert (bf16_bits(D)[~valid] == SENTINEL_BF16).all()
    assert_close(bf16_to_f64(D)[valid], X[valid], S[valid], K // 128, f"ue8m0 contiguous width {width}")


def test_contig_equals_dense_per_group(gpu_lib, width):
    """Each expert's rows equal the dense call on them bit for bit."""
    announce(f"ue8m0 contiguous width {width} vs dense")
    A32, B32, idx = synth.contiguous_problem([256, 128, 384], 384, 768, seed=8)
    qa, ea = quant.quantize_per_token_ue8m0(A32.numpy())
    qb, eb = quantize_experts_ue8m0(B32.numpy())
    Dc = bf16_bits(run_contig(gpu_lib, qa, ea, qb, eb, idx))
    for e in range(3):
        rows = np.nonzero(idx == e)[0]
        assert np.array_equal(Dc[rows], bf16_bits(run(gpu_lib, qa[rows], ea[:, rows], qb[e], eb[e]))), e


def test_contig_8_experts_full_size_sampled(gpu_lib, monkeypatch):
    """8 experts x 4096 rows, N=4096, K=7168 with UE8M0 factors: GPU casts and
    the grouped GEMM; the oracle quantises sampled rows and column blocks
    itself and checks the GPU's codes, factor bytes and outputs."""
    monkeypatch.delenv("FG_FORCE_BN", raising=False)
    monkeypatch.delenv("FG_UE8M0_TILE", raising=False)
    G, R, N, K = synth.CONTIGUOUS_8x4096.shapes[0]
    Kb, kb4 = K // 128, (K // 128 + 3) // 4
    announce(f"ue8m0 contiguous full-size {G}x{R} N={N} K={K}")
    A32, B32, idx = synth.contiguous_problem([R] * G, N, K, seed=0)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token_ue8m0(A32.cuda())
    qb_d, sb_d = gpu_lib.fp8_cast_per_block_ue8m0(B32.cuda().view(G * N, K))
    qb_d, sb_d = qb_d.view(G, N, K), sb_d.view(G, N // 128, kb4)
    D = torch.empty(G * R, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_grouped_contiguous_ue8m0(qa_d, sa_d, qb_d, sb_d, torch.from_numpy(idx).cuda(), D)
    torch.cuda.synchronize()
    ea_d = quant.unpack_ue8m0(sa_d.cpu().numpy(), Kb, axis=0)
    eb_d = quant.unpack_ue8m0(sb_d.cpu().numpy().reshape(G * (N // 128), kb4), Kb, axis=1).reshape(G, N // 128, Kb)
    rng = np.random.default_rng(1)
    blocks = [0, N // 128 - 1, int(rng.integers(1, N // 128 - 1))]
    for e in range(G):
        rows = np.sort(rng.choice(np.arange(e * R, (e + 1) * R), 6, replace=False))
        qa, ea = quant.quantize_per_token_ue8m0(A32.numpy()[rows])
        assert np.array_equal(qa_d[torch.from_numpy(rows).cuda()].cpu().numpy(), qa)
        assert np.array_equal(ea_d[:, rows], ea)
        Dr = D[torch.from_numpy(rows).cuda()]
        for nb in blocks:
            cols = slice(nb * 128, nb * 128 + 128)
            qb, eb = quant.quantize_per_block_ue8m0(B32.numpy()[e, cols])
            assert np.array_equal(eb_d[e, nb:nb + 1], eb)
            X, S = ogemm.gemm_nt(qa, quant.ue8m0_decode(ea), qb, quant.ue8m0_decode(eb), with_magnitude=True)
            assert_close(bf16_to_f64(Dr[:, cols]), X, S, Kb, f"ue8m0 expert {e} block {nb}")


# ---------------------------------------------------------------------------
# BF16 inputs: widened to fp32 exactly, then cast as that fp32 value is.

from tests.test_parity_cast import bf16_values, dev_bf16  # noqa: E402
from oracle import e4m3  # noqa: E402


@pytest.mark.parametrize("M,K", [(3, 384), (128, 7184), (600, 7168)])
def test_cast_per_token_bf16_input_bytes(gpu_lib, M, K):
    """600 x 7168 has 33600 row groups (the 8-lane split); 7184 a K tail."""
    announce(f"ue8m0 cast per token bf16 {M}x{K}")
    bits = bf16_values(np.random.default_rng(M + K + 5), (M, K))
    q_ref, e_ref = quant.quantize_per_token_ue8m0(e4m3.bf16_bits_to_f32(bits))
    q, sa = gpu_lib.fp8_cast_per_token_ue8m0(dev_bf16(bits))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(quant.unpack_ue8m0(sa.cpu().numpy(), -(-K // 128), axis=0), e_ref)


@pytest.mark.parametrize("N,K", [(136, 176), (2112, 512)])
def test_cast_per_block_bf16_input_bytes(gpu_lib, N, K):
    announce(f"ue8m0 cast per block bf16 {N}x{K}")
    bits = bf16_values(np.random.default_rng(N + K + 6), (N, K))
    q_ref, e_ref = quant.quantize_per_block_ue8m0(e4m3.bf16_bits_to_f32(bits))
    q, sb = gpu_lib.fp8_cast_per_block_ue8m0(dev_bf16(bits))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(quant.unpack_ue8m0(sb.cpu().numpy(), -(-K // 128), axis=1), e_ref)
