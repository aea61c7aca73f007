"""Hand-worked examples under tests/golden/ (each file states its source and
derivation): the oracle must reproduce them on the CPU, and the HIP kernels
on the GPU.  The values are worked out by hand from the definitions, not
computed by either implementation."""

from __future__ import annotations

import os

import numpy as np
import pytest

from oracle import e4m3, gemm as ogemm, quant

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    """key: value lines of a fixture; '#' lines are its commentary."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def cast_row():
    g = load("cast_worked_example.txt")
    v = np.array([float(t) for t in g["values_v"].split()], np.float32)
    x = np.tile(v / np.float32(g["divisor"]), 128 // v.size)[None, :]
    codes = np.tile(np.array([int(t, 16) for t in g["codes_v"].split()], np.uint8), 128 // v.size)[None, :]
    return g, x, codes


def gemm_case():
    g = load("gemm_worked_example.txt")
    M, N, K = int(g["M"]), int(g["N"]), int(g["K"])
    A = np.full((M, K), int(g["a_code"], 16), np.uint8)
    B = np.full((N, K), int(g["b_code"], 16), np.uint8)
    sa = np.array([[float(t) for t in part.split()] for part in g["sa"].split("|")], np.float32)  # [Kb, M]
    sb = np.array([[float(t) for t in g["sb"].split()]], np.float32)  # [Nb, Kb]
    rows = [int(t, 16) for t in g["expected_bf16_rows"].split()]
    expected = np.repeat(np.array(rows, np.uint16)[:, None], N, axis=1)
    return A, sa, B, sb, expected


# ------------------------------------------------------------------ oracle


def test_oracle_cast_worked_example():
    g, x, codes = cast_row()
    q, sa = quant.quantize_per_token(x)
    assert np.array_equal(q, codes)
    assert sa.shape == (1, 1) and sa[0, 0] == np.float32(g["scale"])
    qe, e = quant.quantize_per_token_ue8m0(x)
    assert np.array_equal(qe, codes)
    assert int(e[0, 0]) == int(g["ue8m0_byte"])


def test_oracle_decodes_the_worked_codes():
    g, _, _ = cast_row()
    v = [float(t) for t in g["values_v"].split()]
    assert e4m3.decode(np.array([int(t, 16) for t in g["codes_v"].split()], np.uint8)).tolist() == v


def test_oracle_gemm_worked_example():
    A, sa, B, sb, expected = gemm_case()
    assert np.array_equal(ogemm.to_bf16(ogemm.gemm_nt(A, sa, B, sb)), expected)


def test_oracle_ue8m0_pack_worked_example():
    g = load("ue8m0_pack_worked_example.txt")
    b = np.array([int(t, 16) for t in g["bytes"].split()], np.uint8)
    assert b.tolist() == [127 + int(t) for t in g["exponents"].split()]
    packed = quant.pack_ue8m0(b[None, :], axis=1)
    assert packed.shape == (1, 1)
    assert int(packed.view(np.uint32)[0, 0]) == int(g["packed_hex"], 16)


# ------------------------------------------------------------------ kernels


@pytest.mark.gpu
def test_kernels_cast_worked_example(gpu_lib):
    import torch

    g, x, codes = cast_row()
    q, sa = gpu_lib.fp8_cast_per_token(torch.from_numpy(x).cuda())
    qe, sae = gpu_lib.fp8_cast_per_token_ue8m0(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), codes)
    assert float(sa[0, 0].item()) == float(g["scale"])
    assert np.array_equal(qe.cpu().numpy(), codes)
    assert int(sae[0, 0].item()) & 0xFF == int(g["ue8m0_byte"])


@pytest.mark.gpu
def test_kernels_gemm_worked_example(gpu_lib, monkeypatch):
    """On the few-row kernel (the default at M = 2) and on the large-tile one."""
    import torch

    from tests.helpers import bf16_bits, dev_f32, dev_sa, dev_u8

    A, sa, B, sb, expected = gemm_case()
    for force in (None, "big"):
        if force:
            monkeypatch.setenv("FG_FORCE_CONFIG", force)
        D = torch.empty(A.shape[0], B.shape[0], dtype=torch.bfloat16, device="cuda")
        gpu_lib.gemm_fp8_nt(dev_u8(A), dev_sa(sa), dev_u8(B), dev_f32(sb), D)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(D), expected), force
