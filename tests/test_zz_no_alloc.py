"""gemm_fp8_nt_noalloc (split-K buffers in the library's static scratch
array) against gemm_fp8_nt_ws (the same plan with a caller's workspace),
through the C ABI: bit for bit on two calls in a row, the second smaller,
for decode shapes whose plans split K (and one that does not)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.helpers import announce, bf16_bits, dev_f32, dev_sa, dev_u8, quantize_dense, sentinel_like

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    A32, B32 = synth.dense_problem(M, N, K, seed=seed)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    return dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb)


def _call(lib, name, op, D, *extra):
    a, sa, b, sb = op
    M, K = a.shape
    N = b.shape[0]
    st = getattr(lib, name)(a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0), b.data_ptr(), b.stride(0),
                            sb.data_ptr(), D.data_ptr(), D.stride(0), M, N, K, *extra,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.fg_last_error()


@pytest.mark.parametrize("first,second", [((128, 4096, 7168), (64, 2112, 2048)),
                                          ((64, 2112, 7168), (16, 520, 1024)),
                                          ((96, 1000, 4096), (1, 300, 512))])
def test_noalloc_matches_workspace_entry(gpu_lib, monkeypatch, first, second):
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("FG_SKINNY", raising=False)
    lib = gpu_lib.load_library()
    announce(f"no-alloc {first} then {second}")
    for shape, seed in ((first, 1), (second, 2)):
        M, N, K = shape
        op = _operands(M, N, K, seed)
        need = lib.fg_nt_workspace_bytes(M, N, K)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        ref = sentinel_like((M, N))
        _call(lib, "gemm_fp8_nt_ws", op, ref, ws.data_ptr(), ws.numel())
        got = sentinel_like((M, N))
        _call(lib, "gemm_fp8_nt_noalloc", op, got)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(got), bf16_bits(ref)), shape
        # a second call on the same scratch gives the same bits again
        _call(lib, "gemm_fp8_nt_noalloc", op, got)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(got), bf16_bits(ref)), shape


def test_noalloc_argument_errors(gpu_lib):
    lib = gpu_lib.load_library()
    st = lib.gemm_fp8_nt_noalloc(0x10000, 512, 0x10000, 64, 0x10000, 512, 0x10000, 0x10000, 256, 64, 256, 100, None)
    assert st == 2 and b"K=100" in lib.fg_last_error()
    st = lib.gemm_fp8_nt_noalloc(None, 0, None, 0, None, 0, None, None, 0, 0, 256, 512, None)
    assert st == 0  # empty: nothing launched
