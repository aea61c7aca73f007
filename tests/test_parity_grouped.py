"""Contiguous and masked M-grouped GEMMs on the GPU against the CPU oracle.

Indexing and masking are checked bit for bit: D is pre-filled with a NaN
sentinel and every row the oracle marks invalid must still hold it."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, quant
from tests.helpers import (
    SENTINEL_BF16, announce, assert_close, bf16_bits, bf16_to_f64, dev_f32, dev_sa, dev_u8,
    exact_regime, sentinel_like,
)

pytestmark = pytest.mark.gpu


def quantize_grouped_B(B32: np.ndarray):
    qs, ss = zip(*(quant.quantize_per_block(b) for b in B32))
    return np.stack(qs), np.stack(ss)


def run_contig(fg, qa, sa, qb, sb, idx):
    M, N = qa.shape[0], qb.shape[1]
    D = sentinel_like((M, N))
    fg.gemm_fp8_grouped_contiguous(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb),
                                   torch.from_numpy(np.asarray(idx, np.int32)).cuda(), D)
    torch.cuda.synchronize()
    return D


def run_masked(fg, qa, sa, qb, sb, mask, expected_m=0):
    G, Mc, K = qa.shape
    N = qb.shape[1]
    D = sentinel_like((G, Mc, N))
    fg.gemm_fp8_grouped_masked(dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb),
                               torch.from_numpy(np.asarray(mask, np.int32)).cuda(), D, expected_m=expected_m)
    torch.cuda.synchronize()
    return D


# ---------------------------------------------------------------- contiguous


@pytest.mark.parametrize("rows,N,K", [([130, 0, 100], 256, 256), ([1, 255, 128, 64], 520, 384), ([384], 136, 1024)])
def test_contiguous_uneven_groups(gpu_lib, rows, N, K):
    announce(f"contiguous rows={rows} N={N} K={K}")
    A32, B32, idx = synth.contiguous_problem(rows, N, K, seed=len(rows) + N)
    qa, sa = quant.quantize_per_token(A32.numpy())
    qb, sb = quantize_grouped_B(B32.numpy())
    D = run_contig(gpu_lib, qa, sa, qb, sb, idx)
    X, valid, S = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx, with_magnitude=True)
    y = bf16_to_f64(D)
    assert_close(y[valid], X[valid], S[valid], K // 128, "contiguous")
    assert (bf16_bits(D)[~valid] == SENTINEL_BF16).all()


def test_contiguous_exact_regime_bitwise(gpu_lib):
    announce("contiguous exact regime")
    rng = np.random.default_rng(3)
    idx = synth.contiguous_indices([200, 60, 0, 128], pad_to=128)
    M, N, K, G = idx.shape[0], 264, 512, 4
    qa, sa, _, _ = exact_regime(rng, M, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = run_contig(gpu_lib, qa, sa, qb, sb, idx)
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


@pytest.mark.parametrize("G,seed", [(32, 1), (64, 2)])
def test_contiguous_many_experts_bitwise(gpu_lib, G, seed):
    """Many experts with random row counts (zeros included), each segment
    padded to 128 rows: exact bits for every expert's rows, padding rows
    untouched.  Two-expert 256-row tiles and padding-only blocks occur
    throughout."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, 300, G)
    rows[::7] = 0
    idx = synth.contiguous_indices(rows, pad_to=128)
    M, N, K = idx.shape[0], 392, 384
    announce(f"contiguous {G} experts, {M} rows")
    qa, sa, _, _ = exact_regime(rng, M, N, K)
    _, _, qb, sb = exact_regime(rng, 1, N, K, groups=(1, G))
    D = run_contig(gpu_lib, qa, sa, qb, sb, idx)
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


@pytest.mark.parametrize("K", [512, 0])
def test_contiguous_index_past_experts_is_padding(gpu_lib, K):
    """Blocks whose index is G or larger are padding: their rows stay
    untouched and no weight past B is addressed; the other rows are exact.
    Block layout (128 rows each): G, 0, 1000, 1, (two blocks in one 256-row
    tile), then a tile of two blocks past the experts."""
    announce(f"contiguous indices past the experts K={K}")
    rng = np.random.default_rng(17)
    G, N = 2, 264
    blocks = [G, 0, 1000, 1, G + 1, 1 << 30]
    idx = np.repeat(np.asarray(blocks, np.int32), 128)
    idx[130:140] = -1  # padding rows inside a valid block
    M = idx.shape[0]
    qa, sa, _, _ = exact_regime(rng, M, N, max(K, 128))
    _, _, qb, sb = exact_regime(rng, 1, N, max(K, 128), groups=(1, G))
    qa, sa, qb, sb = qa[:, :K], sa[:K // 128], qb[:, :, :K], sb[:, :, :K // 128]
    if K:
        D = run_contig(gpu_lib, qa, sa, qb, sb, idx)
    else:  # empty operands as plain device tensors
        D = sentinel_like((M, N))
        gpu_lib.gemm_fp8_grouped_contiguous(
            torch.zeros(M, 0, dtype=torch.uint8, device="cuda"), torch.zeros(0, M, device="cuda"),
            torch.zeros(G, N, 0, dtype=torch.uint8, device="cuda"), torch.zeros(G, -(-N // 128), 0, device="cuda"),
            torch.from_numpy(idx).cuda(), D)
        torch.cuda.synchronize()
    ref_idx = np.where(idx >= G, -1, idx)
    X, valid = ogemm.gemm_grouped_contiguous(qa, sa, qb, sb, ref_idx)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_contiguous_equals_dense_per_group(gpu_lib, monkeypatch):
    """Bit for bit against the large-tile dense kernel, which adds the slices
    in the same order (the few-row dense kernel adds per-wave K partials)."""
    monkeypatch.setenv("FG_FORCE_CONFIG", "big")
    announce("contiguous vs dense per group")
    A32, B32, idx = synth.contiguous_problem([256, 128, 384], 384, 768, seed=8)
    qa, sa = quant.quantize_per_token(A32.numpy())
    qb, sb = quantize_grouped_B(B32.numpy())
    Dc = bf16_bits(run_contig(gpu_lib, qa, sa, qb, sb, idx))
    for e in range(3):
        rows = np.nonzero(idx == e)[0]
        Dd = torch.empty(len(rows), 384, dtype=torch.bfloat16, device="cuda")
        gpu_lib.gemm_fp8_nt(dev_u8(qa[rows]), dev_sa(sa[:, rows]), dev_u8(qb[e]), dev_f32(sb[e]), Dd)
        torch.cuda.synchronize()
        assert np.array_equal(Dc[rows], bf16_bits(Dd))


def test_contiguous_8_experts_full_size_sampled(gpu_lib):
    """8 experts x 4096 rows, N=4096, K=7168: GPU cast + grouped GEMM; the
    oracle checks sampled rows of every expert against sampled column blocks."""
    G, R, N, K = synth.CONTIGUOUS_8x4096.shapes[0]
    announce(f"contiguous full-size {G}x{R} N={N} K={K}")
    A32, B32, idx = synth.contiguous_problem([R] * G, N, K, seed=0)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token(A32.cuda())
    qb_d, sb_d = gpu_lib.fp8_cast_per_block(B32.cuda().view(G * N, K))
    qb_d = qb_d.view(G, N, K)
    sb_d = sb_d.view(G, N // 128, K // 128)
    D = torch.empty(G * R, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_grouped_contiguous(qa_d, sa_d, qb_d, sb_d, torch.from_numpy(idx).cuda(), D)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    blocks = [0, N // 128 - 1, int(rng.integers(1, N // 128 - 1))]
    for e in range(G):
        rows = np.sort(rng.choice(np.arange(e * R, (e + 1) * R), 6, replace=False))
        qa, sa = quant.quantize_per_token(A32.numpy()[rows])
        assert np.array_equal(qa_d[torch.from_numpy(rows).cuda()].cpu().numpy(), qa)
        Dr = D[torch.from_numpy(rows).cuda()]
        for nb in blocks:
            cols = slice(nb * 128, nb * 128 + 128)
            qb, sb = quant.quantize_per_block(B32.numpy()[e, cols])
            assert np.array_equal(qb_d[e, cols].cpu().numpy(), qb)
            X, S = ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
            assert_close(bf16_to_f64(Dr[:, cols]), X, S, K // 128, f"expert {e} block {nb}")


# -------------------------------------------------------------------- masked


@pytest.mark.parametrize(
    "mask,Mc,N,K",
    [
        ([0, 1, 127, 128, 129, 255, 256, 64], 256, 256, 256),
        ([300, -4, 40, 0], 100, 136, 384),
        ([0, 0, 0], 64, 128, 128),
    ],
)
def test_masked_edges(gpu_lib, mask, Mc, N, K):
    announce(f"masked mask={mask} Mc={Mc} N={N} K={K}")
    G = len(mask)
    g = torch.Generator().manual_seed(G + Mc)
    A32 = torch.randn(G, Mc, K, generator=g).numpy()
    B32 = torch.randn(G, N, K, generator=g).numpy()
    qs = [quant.quantize_per_token(a) for a in A32]
    qa = np.stack([q for q, _ in qs])
    sa = np.stack([s for _, s in qs])
    qb, sb = quantize_grouped_B(B32)
    D = run_masked(gpu_lib, qa, sa, qb, sb, mask)
    X, valid, S = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask, with_magnitude=True)
    bits = bf16_bits(D)
    assert (bits[~valid] == SENTINEL_BF16).all()
    if valid.any():
        y = bf16_to_f64(D)
        assert_close(y[valid], X[valid], S[valid], K // 128, "masked")


@pytest.mark.parametrize("G,Mc,N", [(16, 256, 1040), (12, 512, 520), (70, 256, 264)],
                         ids=["16x256", "12x512", "70x256"])
def test_masked_order_over_rounds(gpu_lib, G, Mc, N):
    """Launches with more (group, tile) units than workgroups: under CU caps
    that leave partial last rounds, every valid row is exact and every other
    row untouched, with the same bits under every cap."""
    K = 256
    announce(f"masked order over rounds G={G} Mc={Mc} N={N}")
    rng = np.random.default_rng(G + Mc)
    mask = rng.integers(0, Mc + 1, G)
    mask[:3] = [0, Mc, 1]
    qa, sa, qb, sb = exact_regime(rng, Mc, N, K, groups=(G, G))
    X, valid = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask)
    ref = None
    try:
        for cus in (0, 1, 3, 7, 40):
            gpu_lib.set_num_cus(cus)
            bits = bf16_bits(run_masked(gpu_lib, qa, sa, qb, sb, mask))
            assert (bits[~valid] == SENTINEL_BF16).all(), cus
            assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid])), cus
            if ref is None:
                ref = bits
            assert np.array_equal(bits, ref), cus
    finally:
        gpu_lib.set_num_cus(0)


def test_masked_exact_regime_bitwise(gpu_lib):
    announce("masked exact regime")
    rng = np.random.default_rng(4)
    G, Mc, N, K = 5, 96, 200, 640
    qa, sa, qb, sb = exact_regime(rng, Mc, N, K, groups=(G, G))
    mask = [96, 0, 33, 95, 1]
    D = run_masked(gpu_lib, qa, sa, qb, sb, mask)
    X, valid = ogemm.gemm_grouped_masked(qa, sa, qb, sb, mask)
    bits = bf16_bits(D)
    assert np.array_equal(bits[valid], ogemm.to_bf16(X[valid]))
    assert (bits[~valid] == SENTINEL_BF16).all()


def test_masked_full_equals_dense(gpu_lib, monkeypatch):
    monkeypatch.setenv("FG_FORCE_CONFIG", "big")  # the large-tile dense kernel: same summation order
    announce("masked mask==M_cap vs dense")
    rng = np.random.default_rng(6)
    G, Mc, N, K = 3, 130, 264, 512
    g = torch.Generator().manual_seed(6)
    A32 = torch.randn(G, Mc, K, generator=g).numpy()
    B32 = torch.randn(G, N, K, generator=g).numpy()
    qs = [quant.quantize_per_token(a) for a in A32]
    qa = np.stack([q for q, _ in qs])
    sa = np.stack([s for _, s in qs])
    qb, sb = quantize_grouped_B(B32)
    Dm = bf16_bits(run_masked(gpu_lib, qa, sa, qb, sb, [Mc] * G))
    for e in range(G):
        Dd = torch.empty(Mc, N, dtype=torch.bfloat16, device="cuda")
        gpu_lib.gemm_fp8_nt(dev_u8(qa[e]), dev_sa(sa[e]), dev_u8(qb[e]), dev_f32(sb[e]), Dd)
        torch.cuda.synchronize()
        assert np.array_equal(Dm[e], bf16_bits(Dd))


@pytest.mark.parametrize("shape", synth.MASKED_16x256.shapes, ids=lambda s: "x".join(map(str, s)))
def test_masked_decode_full_size(gpu_lib, shape):
    """16 experts x capacity 256, seed-0 counts; GPU cast + masked GEMM; the
    oracle checks sampled valid rows of every group (all column blocks of a
    few groups, sampled blocks of the rest) and every invalid row is untouched."""
    G, Mc, N, K = shape
    announce(f"masked full-size {G}x{Mc} N={N} K={K}")
    A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=0)
    qa_d, sa_d = gpu_lib.fp8_cast_per_token(A32.cuda().view(G * Mc, K))
    qa_d = qa_d.view(G, Mc, K)
    sa_full = sa_d  # [Kb, G*Mc] view: regroup per expert into [G, Kb, ld]
    sa_g = torch.empty(G, K // 128, Mc, dtype=torch.float32, device="cuda")
    sa_g.copy_(sa_full.reshape(K // 128, G, Mc).permute(1, 0, 2))
    qb_d, sb_d = gpu_lib.fp8_cast_per_block(B32.cuda().view(G * N, K))
    qb_d, sb_d = qb_d.view(G, N, K), sb_d.view(G, N // 128, K // 128)
    D = sentinel_like((G, Mc, N))
    gpu_lib.gemm_fp8_grouped_masked(qa_d, sa_g, qb_d, sb_d, torch.from_numpy(mask).cuda(), D, expected_m=int(mask.mean()))
    torch.cuda.synchronize()
    bits = bf16_bits(D)
    rng = np.random.default_rng(2)
    for g in range(G):
        v = int(mask[g])
        assert (bits[g, v:] == SENTINEL_BF16).all(), g
        if v == 0:
            continue
        rows = np.unique(np.concatenate([[0, v - 1], rng.choice(v, min(v, 4), replace=False)]))
        qa, sa = quant.quantize_per_token(A32.numpy()[g, rows])
        assert np.array_equal(qa_d[g, torch.from_numpy(rows).cuda()].cpu().numpy(), qa)
        nbs = range(N // 128) if g < 2 else rng.choice(N // 128, 2, replace=False)
        for nb in nbs:
            cols = slice(nb * 128, nb * 128 + 128)
            qb, sb = quant.quantize_per_block(B32.numpy()[g, cols])
            X, S = ogemm.gemm_nt(qa, sa, qb, sb, with_magnitude=True)
            y = bf16_to_f64(D[g, torch.from_numpy(rows).cuda(), cols])
            assert_close(y, X, S, K // 128, f"group {g} block {nb}")


def test_device_check_mode(gpu_lib, monkeypatch):
    """FG_CHECK_DEVICE=1: valid metadata runs as usual; an expert index
    outside [-1, G), a block holding two experts, and a count outside
    [0, M_cap] are reported as FG_EINVAL naming the position, and the GEMM is
    not launched (D keeps its sentinel).  B is allocated with one expert more
    than G, so even the out-of-range index would stay inside it."""
    monkeypatch.setenv("FG_CHECK_DEVICE", "1")
    announce("device check mode")
    G, N, K = 3, 256, 256
    A32, B32, idx = synth.contiguous_problem([128, 200, 60], N, K, seed=40)
    qa, sa = quant.quantize_per_token(A32.numpy())
    qb, sb = quantize_grouped_B(B32.numpy())
    qb_x = np.concatenate([qb, qb[:1]])  # G + 1 experts of storage
    sb_x = np.concatenate([sb, sb[:1]])
    a, s_a, b, s_b = dev_u8(qa), dev_sa(sa), dev_u8(qb_x), dev_f32(sb_x)
    ok = run_contig(gpu_lib, qa, sa, qb, sb, idx)
    for bad, needle in [((5, G), "m_indices\\[5\\] = 3"), ((130, -5), "m_indices\\[130\\] = -5"),
                        ((257, 0), "m_indices\\[257\\] = 0")]:
        row, val = bad
        idx_bad = idx.copy()
        idx_bad[row] = val
        D = sentinel_like((idx.shape[0], N))
        with pytest.raises(gpu_lib.FP8GemmError, match=needle):
            gpu_lib.gemm_fp8_grouped_contiguous(a, s_a, b[:G], s_b[:G], torch.from_numpy(idx_bad).cuda(), D)
        torch.cuda.synchronize()
        assert (bf16_bits(D) == SENTINEL_BF16).all()
    # the valid call in check mode equals the unchecked one
    D = sentinel_like((idx.shape[0], N))
    gpu_lib.gemm_fp8_grouped_contiguous(a, s_a, b[:G], s_b[:G], torch.from_numpy(idx).cuda(), D)
    torch.cuda.synchronize()
    mapped = idx >= 0
    assert np.array_equal(bf16_bits(D)[mapped], bf16_bits(ok)[mapped])
    # masked counts
    Gm, Mc = 4, 128
    rng = np.random.default_rng(41)
    qa_m, sa_m, qb_m, sb_m = exact_regime(rng, Mc, N, K, groups=(Gm, Gm))
    for mask, needle in [([5, 0, 129, 3], "masked_m\\[2\\] = 129"), ([5, -1, 7, 3], "masked_m\\[1\\] = -1")]:
        D = sentinel_like((Gm, Mc, N))
        with pytest.raises(gpu_lib.FP8GemmError, match=needle):
            gpu_lib.gemm_fp8_grouped_masked(dev_u8(qa_m), dev_sa(sa_m, groups=True), dev_u8(qb_m), dev_f32(sb_m),
                                            torch.tensor(mask, dtype=torch.int32, device="cuda"), D)
        torch.cuda.synchronize()
        assert (bf16_bits(D) == SENTINEL_BF16).all()
    Dm = run_masked(gpu_lib, qa_m, sa_m, qb_m, sb_m, [5, 0, 128, 3])
    Xm, valid = ogemm.gemm_grouped_masked(qa_m, sa_m, qb_m, sb_m, [5, 0, 128, 3])
    assert np.array_equal(bf16_bits(Dm)[valid], ogemm.to_bf16(Xm[valid]))
    # the check reads a result back, so it refuses a capturing stream
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    D = sentinel_like((idx.shape[0], N))
    idx_d = torch.from_numpy(idx).cuda()
    torch.cuda.synchronize()
    with pytest.raises(gpu_lib.FP8GemmError, match="captured"):
        with torch.cuda.graph(g, stream=s):
            gpu_lib.gemm_fp8_grouped_contiguous(a, s_a, b[:G], s_b[:G], idx_d, D, stream=s)
    torch.cuda.synchronize()
