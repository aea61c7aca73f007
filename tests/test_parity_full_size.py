"""Every output element of the full-size dense M=4096 shapes and of the
contiguous 8 x 4096-row MoE GEMM against the oracle.

The operands go through the benchmark's launch path: the GPU cast kernels
quantise the fp32 sources (their codes and factors must equal the oracle
quantiser's, byte for byte, over the whole tensors), then the GEMM runs with
the library's own plan.  The oracle evaluates its dequantised form, in row
chunks, with the magnitude S for the per-element bound; the similarity
defect is taken over all elements.  This covers every tile of every round,
the raster bands, the tile width each shape runs at and the last-round
tiles, at their real counts.  CPU work: about a minute per workload on a
16-core host."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, metrics, quant
from tests.helpers import announce, bf16_to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHUNK = 1024  # oracle rows per call


class Totals:
    """Per-element bound over chunks, and the similarity defect's sums."""

    def __init__(self):
        self.n = self.bad = 0
        self.sxy = self.sxx = 0.0

    def add(self, y, X, S, Kb):
        rep = metrics.check_result(y, X, S, Kb)
        self.n += rep["n"]
        self.bad += rep["n_bad"]
        self.sxy += float(np.sum(y * X))
        self.sxx += float(np.sum(y * y + X * X))

    def check(self, what):
        defect = 1.0 - 2.0 * self.sxy / self.sxx
        assert self.bad == 0, f"{what}: {self.bad} of {self.n} elements outside the bound"
        assert defect < 1e-3, f"{what}: similarity defect {defect}"
        return defect


def _cast_and_compare(fg, a32, b32):
    """GPU casts of the full tensors; codes and factors equal the oracle's."""
    qa, sa = quant.quantize_per_token(a32.numpy())
    qb, sb = quant.quantize_per_block(b32.numpy())
    qa_d, sa_d = fg.fp8_cast_per_token(a32.cuda())
    qb_d, sb_d = fg.fp8_cast_per_block(b32.cuda())
    assert np.array_equal(qa_d.cpu().numpy(), qa)
    assert np.array_equal(sa_d.cpu().numpy(), sa)
    assert np.array_equal(qb_d.cpu().numpy(), qb)
    assert np.array_equal(sb_d.cpu().numpy(), sb)
    return (qa, sa, qb, sb), (qa_d, sa_d, qb_d, sb_d)


@pytest.mark.parametrize("shape", synth.DENSE_M4096.shapes, ids=lambda s: "x".join(map(str, s)))
def test_dense_m4096_every_element(gpu_lib, monkeypatch, shape):
    for k in ("FG_SKINNY", "FG_FORCE_CONFIG", "FG_FORCE_BN"):
        monkeypatch.delenv(k, raising=False)
    M, N, K = shape
    announce(f"full-size dense {M}x{N}x{K}, every element")
    A32, B32 = synth.dense_problem(M, N, K, seed=0)
    (qa, sa, qb, sb), (qa_d, sa_d, qb_d, sb_d) = _cast_and_compare(gpu_lib, A32, B32)
    D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d, D)
    torch.cuda.synchronize()
    y = bf16_to_f64(D)
    del qa_d, qb_d, D
    tot = Totals()
    for r0 in range(0, M, CHUNK):
        rows = slice(r0, min(M, r0 + CHUNK))
        X, S = ogemm.gemm_dequant(qa[rows], sa[:, rows], qb, sb, with_magnitude=True)
        tot.add(y[rows], X, S, -(-K // 128))
    tot.check(f"dense {M}x{N}x{K}")


def test_contiguous_8x4096_every_element(gpu_lib, monkeypatch):
    for k in ("FG_FORCE_BN",):
        monkeypatch.delenv(k, raising=False)
    G, rows, N, K = synth.CONTIGUOUS_8x4096.shapes[0]
    announce(f"full-size contiguous {G}x{rows}x{N}x{K}, every element")
    A32, B32, idx = synth.contiguous_problem([rows] * G, N, K, seed=0)
    (qa, sa, qb, sb), (qa_d, sa_d, qb_d, sb_d) = _cast_and_compare(gpu_lib, A32, B32.reshape(G * N, K))
    qb, sb = qb.reshape(G, N, K), sb.reshape(G, N // 128, -1)
    D = torch.empty(idx.shape[0], N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_grouped_contiguous(qa_d, sa_d, qb_d.view(G, N, K), sb_d.view(G, N // 128, -1),
                                        torch.from_numpy(idx).cuda(), D)
    torch.cuda.synchronize()
    y = bf16_to_f64(D)
    del qa_d, qb_d, D
    tot = Totals()
    for e in range(G):
        er = np.nonzero(idx == e)[0]
        for r0 in range(0, er.size, CHUNK):
            r = er[r0:r0 + CHUNK]
            X, S = ogemm.gemm_dequant(qa[r], sa[:, r], qb[e], sb[e], with_magnitude=True)
            tot.add(y[r], X, S, -(-K // 128))
    tot.check("contiguous 8x4096")


@pytest.mark.parametrize("shape", synth.MASKED_16x256.shapes, ids=lambda s: "x".join(map(str, s)))
def test_masked_16x256_every_element(gpu_lib, shape):
    """Masked decode at full size: every valid row against the oracle, every
    row past a group's count untouched (sentinel)."""
    from tests.helpers import SENTINEL_BF16, bf16_bits, dev_f32, dev_sa, dev_u8, sentinel_like

    G, Mc, N, K = shape
    announce(f"full-size masked {G}x{Mc}x{N}x{K}, every element")
    A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=0)
    qs = [quant.quantize_per_token(a) for a in A32.numpy()]
    qa = np.stack([q for q, _ in qs])
    sa = np.stack([s for _, s in qs])
    qbs = [quant.quantize_per_block(b) for b in B32.numpy()]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    D = sentinel_like((G, Mc, N))
    gpu_lib.gemm_fp8_grouped_masked(dev_u8(qa), dev_sa(sa, groups=True), dev_u8(qb), dev_f32(sb),
                                    torch.from_numpy(mask.astype(np.int32)).cuda(), D)
    torch.cuda.synchronize()
    bits = bf16_bits(D)
    y = bf16_to_f64(D)
    tot = Totals()
    for g in range(G):
        v = int(mask[g])
        assert (bits[g, v:] == SENTINEL_BF16).all(), g
        if v:
            X, S = ogemm.gemm_dequant(qa[g, :v], sa[g][:, :v], qb[g], sb[g], with_magnitude=True)
            tot.add(y[g, :v], X, S, -(-K // 128))
    tot.check(f"masked {G}x{Mc}x{N}x{K}")
