"""MI355X (gfx950) FP8 e4m3 fine-grained-scaled GEMM: Python binding.

A thin ctypes layer over ``libfp8gemm.so`` (C ABI in ``include/fp8gemm.h``).
Each function takes torch CUDA tensors, checks dtypes and devices, and passes
raw pointers, sizes and the current HIP stream to the C entry point of the
same name.  Every step of the computation runs in the library's HIP kernels;
there is no host or PyTorch fallback: if the library cannot be loaded, every
call raises.

Layouts (Kb = ceil(K/128), Nb = ceil(N/128)):
  A   e4m3 [M, K] (uint8 or torch.float8_e4m3fn), rows K-contiguous
  sa  fp32 [Kb, M] view of a [Kb, ld_sa] buffer (activation scales, K-group-major)
  B   e4m3 [N, K]                      sb  fp32 [Nb, Kb]
  D   bf16 [M, N]
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8gemm.so")

__all__ = [
    "FP8GemmError",
    "load_library",
    "library_path",
    "gemm_fp8_nt",
    "gemm_fp8_nt_unsplit",
    "nt_workspace_bytes",
    "nt_workspace",
    "gemm_fp8_nt_c",
    "gemm_fp8_nn",
    "gemm_fp8_tn",
    "gemm_fp8_tt",
    "layout_workspace_bytes",
    "gemm_fp8_k_grouped_tn_contiguous",
    "k_grouped_workspace_bytes",
    "gemm_fp8_grouped_contiguous",
    "gemm_fp8_grouped_masked",
    "fp8_cast_per_token",
    "fp8_cast_per_block",
    "gemm_fp8_nt_ue8m0",
    "gemm_fp8_grouped_contiguous_ue8m0",
    "gemm_fp8_grouped_masked_ue8m0",
    "fp8_cast_per_token_ue8m0",
    "fp8_cast_per_block_ue8m0",
    "empty_activation_scales_ue8m0",
    "get_mk_alignment_for_contiguous_layout",
    "set_num_cus",
    "get_num_cus",
    "aligned_scale_ld",
    "empty_activation_scales",
    "EXPORTED_SYMBOLS",
]

FG_STATUS = {0: "FG_OK", 1: "FG_EINVAL", 2: "FG_EALIGN", 3: "FG_EUNSUPPORTED", 4: "FG_EHIP"}

# name -> (restype, argtypes); one entry per declaration in include/fp8gemm.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SIGNATURES = {
    "gemm_fp8_nt": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _I, _I, _I, _P]),
    "gemm_fp8_nt_ws": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _I, _I, _I, _P, _I64, _P]),
    "gemm_fp8_nt_noalloc": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _I, _I, _I, _P]),
    "fg_nt_workspace_bytes": (_I64, [_I, _I, _I]),
    "fg_nt_workspace_max_bytes": (_I64, []),
    "gemm_fp8_nt_c": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _I, _I, _I, _P]),
    "gemm_fp8_nn": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _I, _I, _I, _P, _I64, _P]),
    "gemm_fp8_tn": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _I, _I, _I, _P, _I64, _P]),
    "gemm_fp8_tt": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _I, _I, _I, _P, _I64, _P]),
    "fg_layout_workspace_bytes": (_I64, [ctypes.c_char_p, _I, _I, _I]),
    "gemm_fp8_k_grouped_tn_contiguous": (
        _I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I, _P, _P, _I, _I, _P, _I64, _P]),
    "fg_k_grouped_workspace_bytes": (_I64, [_I, _I, _I64]),
    "gemm_fp8_grouped_contiguous": (_I, [_P, _P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "gemm_fp8_grouped_masked": (_I, [_P, _P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fp8_cast_per_token": (_I, [_P, _I64, _P, _P, _I64, _I, _I, _P]),
    "fp8_cast_per_block": (_I, [_P, _I64, _P, _P, _I, _I, _P]),
    "gemm_fp8_nt_ue8m0": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _I, _I, _I, _P]),
    "gemm_fp8_grouped_contiguous_ue8m0": (_I, [_P, _P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "gemm_fp8_grouped_masked_ue8m0": (_I, [_P, _P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fp8_cast_per_token_ue8m0": (_I, [_P, _I64, _P, _P, _I64, _I, _I, _P]),
    "fp8_cast_per_block_ue8m0": (_I, [_P, _I64, _P, _P, _I, _I, _P]),
    "fp8_cast_per_token_bf16": (_I, [_P, _I64, _P, _P, _I64, _I, _I, _P]),
    "fp8_cast_per_block_bf16": (_I, [_P, _I64, _P, _P, _I, _I, _P]),
    "fp8_cast_per_token_ue8m0_bf16": (_I, [_P, _I64, _P, _P, _I64, _I, _I, _P]),
    "fp8_cast_per_block_ue8m0_bf16": (_I, [_P, _I64, _P, _P, _I, _I, _P]),
    "fg_get_mk_alignment_for_contiguous_layout": (_I, []),
    "fg_set_num_cus": (None, [_I]),
    "fg_get_num_cus": (_I, []),
    "fg_last_error": (ctypes.c_char_p, []),
    "fg_version": (ctypes.c_char_p, []),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


class FP8GemmError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        self.status = status
        self.status_name = FG_STATUS.get(status, str(status))
        super().__init__(f"{fn}: {self.status_name}: {msg}")


def library_path() -> str:
    return os.environ.get("FG_LIBRARY", LIB_PATH)


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle; raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} not found: build it with `python -m moe_grouped_gemm_e4m3_amd.build` (no fallback path exists)"
        )
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _call(name: str, *args):
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise FP8GemmError(name, st, lib.fg_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _fp8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8 or float8_e4m3fn, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    return t


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError(f"{name} must be a float32 CUDA tensor")
    return t


def _unit_inner(t: torch.Tensor, name: str):
    if t.dim() >= 1 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")


def _ld(t: torch.Tensor) -> int:
    """Row stride of a 2-D tensor in elements.  A single row's stride is
    arbitrary in torch (a broadcast or sliced view can report 0), so one row
    reports its own length."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def aligned_scale_ld(rows: int) -> int:
    """Leading dimension for activation scales: rows rounded up to 4 floats."""
    return max(4, (rows + 3) // 4 * 4)


def empty_activation_scales(rows: int, K: int, device="cuda", groups: int | None = None) -> torch.Tensor:
    """A [Kb, rows] (or [G, Kb, rows]) view of a padded [.., Kb, ld_sa] fp32 buffer."""
    ld = aligned_scale_ld(rows)
    Kb = -(-K // 128)  # a partial last K group when K % 128 != 0
    if groups is None:
        return torch.empty(Kb, ld, dtype=torch.float32, device=device)[:, :rows]
    return torch.empty(groups, Kb, ld, dtype=torch.float32, device=device)[:, :, :rows]


def nt_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes gemm_fp8_nt's K-split plan needs for (M, N, K) (0: no split)."""
    n = load_library().fg_nt_workspace_bytes(M, N, K)
    if n < 0:
        raise ValueError(f"sizes {(M, N, K)} not accepted, or the device cannot be queried")
    return n


# Split-K workspaces of gemm_fp8_nt, one per (device, stream): zero-filled
# once (the library keeps the counters at zero between calls) and kept for the
# life of the process, so a graph that captured one keeps a valid buffer.
_NT_WS: dict = {}


def nt_workspace(device=None, stream=None) -> torch.Tensor:
    """The cached split-K workspace of `stream` (current stream by default),
    created zero-filled by torch's allocator on first use."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    key = (dev.index, _stream(stream))
    ws = _NT_WS.get(key)
    if ws is None:
        ws = torch.zeros(load_library().fg_nt_workspace_max_bytes(), dtype=torch.uint8, device=dev)
        _NT_WS[key] = ws
    return ws


def gemm_fp8_nt(A, sa, B, sb, D, stream=None, workspace=None):
    """D[M,N] = bf16(A . B^T) with 1x128 activation and 128x128 weight scales.

    Calls gemm_fp8_nt_ws: for few rows (M <= 128) the K range may be split
    over workgroups, with the partials in `workspace` (a uint8 CUDA tensor
    whose first 64 KiB are zero; by default the cached one of the stream)."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    if D.dtype != torch.bfloat16 or not D.is_cuda:
        raise TypeError("D must be a bfloat16 CUDA tensor")
    for t, n in ((A, "A"), (B, "B"), (sa, "sa"), (D, "D")):
        _unit_inner(t, n)
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous [Nb, Kb]")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(D.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} D{tuple(D.shape)}")
    ws_ptr, ws_bytes = None, 0
    if workspace is None and M <= 128 and nt_workspace_bytes(M, N, K) > 0:
        workspace = nt_workspace(D.device, stream)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous uint8 CUDA tensor")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    _call(
        "gemm_fp8_nt_ws",
        _ptr(A), _ld(A), _ptr(sa), _ld(sa), _ptr(B), _ld(B), _ptr(sb),
        _ptr(D), _ld(D), M, N, K, ws_ptr, ws_bytes, _stream(stream),
    )
    return D


def gemm_fp8_nt_unsplit(A, sa, B, sb, D, stream=None):
    """gemm_fp8_nt's C entry point itself: never splits K, needs no workspace."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    if D.dtype != torch.bfloat16 or not D.is_cuda:
        raise TypeError("D must be a bfloat16 CUDA tensor")
    for t, n in ((A, "A"), (B, "B"), (sa, "sa"), (D, "D")):
        _unit_inner(t, n)
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous [Nb, Kb]")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(D.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} D{tuple(D.shape)}")
    _call(
        "gemm_fp8_nt",
        _ptr(A), _ld(A), _ptr(sa), _ld(sa), _ptr(B), _ld(B), _ptr(sb),
        _ptr(D), _ld(D), M, N, K, _stream(stream),
    )
    return D


def gemm_fp8_nt_c(A, sa, B, sb, C, D, stream=None):
    """D[M,N] = bf16(C + A . B^T): gemm_fp8_nt with an fp32 addend C [M, N]."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb, C = _f32(sa, "sa"), _f32(sb, "sb"), _f32(C, "C")
    if D.dtype != torch.bfloat16 or not D.is_cuda:
        raise TypeError("D must be a bfloat16 CUDA tensor")
    for t, n in ((A, "A"), (B, "B"), (sa, "sa"), (C, "C"), (D, "D")):
        _unit_inner(t, n)
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous [Nb, Kb]")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(D.shape) != (M, N) or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)} D{tuple(D.shape)}")
    _call(
        "gemm_fp8_nt_c",
        _ptr(A), _ld(A), _ptr(sa), _ld(sa), _ptr(B), _ld(B), _ptr(sb),
        _ptr(C), _ld(C), _ptr(D), _ld(D), M, N, K, _stream(stream),
    )
    return D


def layout_workspace_bytes(layout: str, M: int, N: int, K: int) -> int:
    """Device workspace bytes gemm_fp8_<layout> needs (0 for "nt")."""
    n = load_library().fg_layout_workspace_bytes(layout.encode(), M, N, K)
    if n < 0:
        raise ValueError(f"layout {layout!r} or sizes {(M, N, K)} not accepted")
    return n


def _gemm_layout(layout, A, sa, B, sb, D, C, stream, workspace):
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    if C is not None:
        C = _f32(C, "C")
    if D.dtype != torch.bfloat16 or not D.is_cuda:
        raise TypeError("D must be a bfloat16 CUDA tensor")
    for t, n in ((A, "A"), (B, "B"), (sa, "sa"), (C, "C"), (D, "D")):
        if t is not None:
            _unit_inner(t, n)
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous [Nb, Kb]")
    K, M = A.shape if layout[0] == "t" else A.shape[::-1]
    N = B.shape[1] if layout[1] == "n" else B.shape[0]
    kb = B.shape[0] if layout[1] == "n" else B.shape[1]
    if kb != K or tuple(D.shape) != (M, N) or (C is not None and tuple(C.shape) != (M, N)):
        raise ValueError(f"{layout}: shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} D{tuple(D.shape)}")
    need = layout_workspace_bytes(layout, M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=D.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 CUDA tensor")
    _call(
        "gemm_fp8_" + layout,
        _ptr(A), _ld(A), _ptr(sa), _ld(sa), _ptr(B), _ld(B), _ptr(sb),
        _ptr(C), _ld(C) if C is not None else 0, _ptr(D), _ld(D), M, N, K,
        _ptr(workspace), workspace.numel(), _stream(stream),
    )
    return D


def gemm_fp8_nn(A, sa, B, sb, D, C=None, stream=None, workspace=None):
    """D[M,N] = bf16(C + A . B), A [M, K], B stored [K, N].  Scales as for
    gemm_fp8_nt (sb: 128x128 blocks of the logical [N, K] operand).  The
    workspace (layout_workspace_bytes) comes from torch's allocator if not
    given; an empty one (0 bytes) runs without copies, on the operands as
    stored (MN-major ones then need 16-byte rows and M, N multiples of 16)."""
    return _gemm_layout("nn", A, sa, B, sb, D, C, stream, workspace)


def gemm_fp8_tn(A, sa, B, sb, D, C=None, stream=None, workspace=None):
    """D[M,N] = bf16(C + A^T . B), A stored [K, M], B stored [K, N]."""
    return _gemm_layout("tn", A, sa, B, sb, D, C, stream, workspace)


def gemm_fp8_tt(A, sa, B, sb, D, C=None, stream=None, workspace=None):
    """D[M,N] = bf16(C + A^T . B^T), A stored [K, M], B [N, K]."""
    return _gemm_layout("tt", A, sa, B, sb, D, C, stream, workspace)


def k_grouped_workspace_bytes(M: int, N: int, K_total: int) -> int:
    """Device workspace bytes gemm_fp8_k_grouped_tn_contiguous needs."""
    n = load_library().fg_k_grouped_workspace_bytes(M, N, K_total)
    if n < 0:
        raise ValueError(f"sizes {(M, N, K_total)} not accepted")
    return n


def gemm_fp8_k_grouped_tn_contiguous(A, sa, B, sb, ks, D, C=None, stream=None, workspace=None):
    """D[g] = bf16(C[g] + A_g^T . B_g) for groups of ks[g] consecutive K rows.

    A [K_total, M] and B [K_total, N] (uint8 / e4m3, row-contiguous); sa fp32
    [K_total/128, M] view; sb fp32 [Nb, K_total/128]; ks: host sequence of
    group sizes (multiples of 128); D bf16 [G, M, N] and C fp32 [G, M, N]
    contiguous.  The workspace comes from torch's allocator if not given; an
    empty one (0 bytes) runs without copies, on A and B as stored (they then
    need 16-byte rows and M, N multiples of 16)."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    if C is not None:
        C = _f32(C, "C")
        if not C.is_contiguous():
            raise ValueError("C must be contiguous [G, M, N]")
    if D.dtype != torch.bfloat16 or not D.is_cuda or not D.is_contiguous():
        raise TypeError("D must be a contiguous bfloat16 CUDA tensor [G, M, N]")
    for t, n in ((A, "A"), (B, "B"), (sa, "sa")):
        _unit_inner(t, n)
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous [Nb, Kb_total]")
    ks = [int(k) for k in ks]
    G = len(ks)
    K_total, M = A.shape
    N = B.shape[1]
    if B.shape[0] != K_total or sum(ks) != K_total or tuple(D.shape) != (G, M, N) or (
            C is not None and tuple(C.shape) != (G, M, N)):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} D{tuple(D.shape)} ks={ks}")
    need = k_grouped_workspace_bytes(M, N, K_total)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=D.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 CUDA tensor")
    ks_host = (ctypes.c_int * G)(*ks)
    _call(
        "gemm_fp8_k_grouped_tn_contiguous",
        _ptr(A), _ld(A), _ptr(sa), _ld(sa), _ptr(B), _ld(B), _ptr(sb),
        ctypes.cast(ks_host, ctypes.c_void_p), G, _ptr(C), _ptr(D), M, N,
        _ptr(workspace), workspace.numel(), _stream(stream),
    )
    return D


def gemm_fp8_grouped_contiguous(A, sa, B, sb, m_indices, D, stream=None):
    """Contiguous M-grouped GEMM: row r of A uses expert m_indices[r] (-1 = padding, untouched)."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    if m_indices.dtype != torch.int32 or not m_indices.is_cuda or not m_indices.is_contiguous():
        raise TypeError("m_indices must be a contiguous int32 CUDA tensor")
    if D.dtype != torch.bfloat16 or not D.is_contiguous():
        raise TypeError("D must be a contiguous bfloat16 CUDA tensor")
    if not (A.is_contiguous() and B.is_contiguous() and sb.is_contiguous()):
        raise ValueError("A, B and sb must be contiguous")
    _unit_inner(sa, "sa")
    M, K = A.shape
    G, N, K2 = B.shape
    if K2 != K or tuple(D.shape) != (M, N) or m_indices.shape[0] != M:
        raise ValueError("shape mismatch")
    _call(
        "gemm_fp8_grouped_contiguous",
        _ptr(A), _ptr(sa), _ld(sa), _ptr(B), _ptr(sb), _ptr(m_indices), _ptr(D),
        M, N, K, G, _stream(stream),
    )
    return D


def gemm_fp8_grouped_masked(A, sa, B, sb, masked_m, D, expected_m: int = 0, stream=None):
    """Masked M-grouped GEMM: group g computes rows [0, masked_m[g]) of A[g]; other rows of D untouched."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    if masked_m.dtype != torch.int32 or not masked_m.is_cuda or not masked_m.is_contiguous():
        raise TypeError("masked_m must be a contiguous int32 CUDA tensor")
    if D.dtype != torch.bfloat16 or not D.is_contiguous():
        raise TypeError("D must be a contiguous bfloat16 CUDA tensor")
    if not (A.is_contiguous() and B.is_contiguous() and sb.is_contiguous()):
        raise ValueError("A, B and sb must be contiguous")
    G, Mc, K = A.shape
    N = B.shape[1]
    if sa.dim() != 3 or sa.shape[0] != G or sa.stride(2) != 1 or sa.stride(0) != sa.shape[1] * sa.stride(1):
        raise ValueError("sa must be a [G, Kb, M_cap] view of a [G, Kb, ld_sa] buffer")
    if B.shape != (G, N, K) or tuple(D.shape) != (G, Mc, N) or masked_m.shape[0] != G:
        raise ValueError("shape mismatch")
    _call(
        "gemm_fp8_grouped_masked",
        _ptr(A), _ptr(sa), sa.stride(1), _ptr(B), _ptr(sb), _ptr(masked_m), _ptr(D),
        G, Mc, N, K, int(expected_m), _stream(stream),
    )
    return D


def _f32_or_bf16(t: torch.Tensor, name: str) -> tuple[torch.Tensor, str]:
    """Cast input and the entry-point suffix for its dtype."""
    if t.dtype == torch.bfloat16 and t.is_cuda:
        return t, "_bf16"
    return _f32(t, name), ""


def fp8_cast_per_token(x, q=None, sa=None, stream=None):
    """1x128 cast of fp32 or bf16 activations [M, K] -> (q uint8 [M, K], sa fp32 [Kb, M] view)."""
    x, sfx = _f32_or_bf16(x, "x")
    _unit_inner(x, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = empty_activation_scales(M, K, device=x.device)
    q = _fp8(q, "q")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _unit_inner(sa, "sa")
    _call("fp8_cast_per_token" + sfx, _ptr(x), _ld(x), _ptr(q), _ptr(sa), _ld(sa), M, K, _stream(stream))
    return q, sa


def fp8_cast_per_block(w, q=None, sb=None, stream=None):
    """128x128 cast of fp32 or bf16 weights [N, K] -> (q uint8 [N, K], sb fp32 [Nb, Kb])."""
    w, sfx = _f32_or_bf16(w, "w")
    _unit_inner(w, "w")
    N, K = w.shape
    if q is None:
        q = torch.empty(N, K, dtype=torch.uint8, device=w.device)
    if sb is None:
        sb = torch.empty((N + 127) // 128, -(-K // 128), dtype=torch.float32, device=w.device)
    q = _fp8(q, "q")
    if not (q.is_contiguous() and sb.is_contiguous()):
        raise ValueError("q and sb must be contiguous")
    _call("fp8_cast_per_block" + sfx, _ptr(w), _ld(w), _ptr(q), _ptr(sb), N, K, _stream(stream))
    return q, sb


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_cuda:
        raise TypeError(f"{name} must be an int32 CUDA tensor of packed UE8M0 factors")
    return t


def empty_activation_scales_ue8m0(rows: int, K: int, device="cuda") -> torch.Tensor:
    """A [ceil(Kb/4), rows] view of a padded int32 buffer for packed UE8M0 activation factors."""
    kb4 = (-(-K // 128) + 3) // 4
    return torch.empty(kb4, aligned_scale_ld(rows), dtype=torch.int32, device=device)[:, :rows]


def gemm_fp8_nt_ue8m0(A, sa, B, sb, D, stream=None):
    """D[M,N] = bf16(A . B^T) with packed power-of-two (UE8M0) factors:
    sa int32 [ceil(Kb/4), M] view (row stride ld_sa), sb int32 [Nb, ceil(Kb/4)]."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _i32(sa, "sa"), _i32(sb, "sb")
    if D.dtype != torch.bfloat16 or not D.is_cuda:
        raise TypeError("D must be a bfloat16 CUDA tensor")
    for t, n in ((A, "A"), (B, "B"), (sa, "sa"), (D, "D")):
        _unit_inner(t, n)
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous [Nb, ceil(Kb/4)]")
    M, K = A.shape
    N = B.shape[0]
    kb4 = (-(-K // 128) + 3) // 4
    if B.shape[1] != K or tuple(D.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} D{tuple(D.shape)}")
    if K and (tuple(sa.shape) != (kb4, M) or tuple(sb.shape) != ((N + 127) // 128, kb4)):
        raise ValueError("factor shapes must be sa [ceil(Kb/4), M] and sb [Nb, ceil(Kb/4)]")
    _call(
        "gemm_fp8_nt_ue8m0",
        _ptr(A), _ld(A), _ptr(sa), _ld(sa), _ptr(B), _ld(B), _ptr(sb),
        _ptr(D), _ld(D), M, N, K, _stream(stream),
    )
    return D


def gemm_fp8_grouped_contiguous_ue8m0(A, sa, B, sb, m_indices, D, stream=None):
    """Contiguous M-grouped GEMM with packed power-of-two (UE8M0) factors: sa
    int32 [ceil(Kb/4), M_total] view (row stride ld_sa), sb int32 [G, Nb,
    ceil(Kb/4)]; row r of A uses expert m_indices[r] (-1 = padding, untouched)."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _i32(sa, "sa"), _i32(sb, "sb")
    if m_indices.dtype != torch.int32 or not m_indices.is_cuda or not m_indices.is_contiguous():
        raise TypeError("m_indices must be a contiguous int32 CUDA tensor")
    if D.dtype != torch.bfloat16 or not D.is_contiguous():
        raise TypeError("D must be a contiguous bfloat16 CUDA tensor")
    if not (A.is_contiguous() and B.is_contiguous() and sb.is_contiguous()):
        raise ValueError("A, B and sb must be contiguous")
    _unit_inner(sa, "sa")
    M, K = A.shape
    G, N, K2 = B.shape
    kb4 = (-(-K // 128) + 3) // 4
    if K2 != K or tuple(D.shape) != (M, N) or m_indices.shape[0] != M:
        raise ValueError("shape mismatch")
    if K and (tuple(sa.shape) != (kb4, M) or tuple(sb.shape) != (G, (N + 127) // 128, kb4)):
        raise ValueError("factor shapes must be sa [ceil(Kb/4), M_total] and sb [G, Nb, ceil(Kb/4)]")
    _call(
        "gemm_fp8_grouped_contiguous_ue8m0",
        _ptr(A), _ptr(sa), _ld(sa), _ptr(B), _ptr(sb), _ptr(m_indices), _ptr(D),
        M, N, K, G, _stream(stream),
    )
    return D


def gemm_fp8_grouped_masked_ue8m0(A, sa, B, sb, masked_m, D, expected_m: int = 0, stream=None):
    """Masked M-grouped GEMM with packed power-of-two (UE8M0) factors: sa int32
    [G, ceil(Kb/4), M_cap] view of a [G, ceil(Kb/4), ld_sa] buffer, sb int32
    [G, Nb, ceil(Kb/4)]; group g computes rows [0, masked_m[g]), other rows of D untouched."""
    A, B = _fp8(A, "A"), _fp8(B, "B")
    sa, sb = _i32(sa, "sa"), _i32(sb, "sb")
    if masked_m.dtype != torch.int32 or not masked_m.is_cuda or not masked_m.is_contiguous():
        raise TypeError("masked_m must be a contiguous int32 CUDA tensor")
    if D.dtype != torch.bfloat16 or not D.is_contiguous():
        raise TypeError("D must be a contiguous bfloat16 CUDA tensor")
    if not (A.is_contiguous() and B.is_contiguous() and sb.is_contiguous()):
        raise ValueError("A, B and sb must be contiguous")
    G, Mc, K = A.shape
    N = B.shape[1]
    kb4 = (-(-K // 128) + 3) // 4
    if sa.dim() != 3 or sa.shape[0] != G or sa.stride(2) != 1 or sa.stride(0) != sa.shape[1] * sa.stride(1):
        raise ValueError("sa must be a [G, ceil(Kb/4), M_cap] view of a [G, ceil(Kb/4), ld_sa] buffer")
    if B.shape != (G, N, K) or tuple(D.shape) != (G, Mc, N) or masked_m.shape[0] != G:
        raise ValueError("shape mismatch")
    if K and (tuple(sa.shape) != (G, kb4, Mc) or tuple(sb.shape) != (G, (N + 127) // 128, kb4)):
        raise ValueError("factor shapes must be sa [G, ceil(Kb/4), M_cap] and sb [G, Nb, ceil(Kb/4)]")
    _call(
        "gemm_fp8_grouped_masked_ue8m0",
        _ptr(A), _ptr(sa), sa.stride(1), _ptr(B), _ptr(sb), _ptr(masked_m), _ptr(D),
        G, Mc, N, K, int(expected_m), _stream(stream),
    )
    return D


def fp8_cast_per_token_ue8m0(x, q=None, sa=None, stream=None):
    """1x128 cast of fp32 or bf16 activations with power-of-two factors ->
    (q uint8 [M, K], sa int32 [ceil(Kb/4), M] view)."""
    x, sfx = _f32_or_bf16(x, "x")
    _unit_inner(x, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = empty_activation_scales_ue8m0(M, K, device=x.device)
    q = _fp8(q, "q")
    sa = _i32(sa, "sa")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _unit_inner(sa, "sa")
    _call("fp8_cast_per_token_ue8m0" + sfx, _ptr(x), _ld(x), _ptr(q), _ptr(sa), _ld(sa), M, K, _stream(stream))
    return q, sa


def fp8_cast_per_block_ue8m0(w, q=None, sb=None, stream=None):
    """128x128 cast of fp32 or bf16 weights with power-of-two factors ->
    (q uint8 [N, K], sb int32 [Nb, ceil(Kb/4)])."""
    w, sfx = _f32_or_bf16(w, "w")
    _unit_inner(w, "w")
    N, K = w.shape
    if q is None:
        q = torch.empty(N, K, dtype=torch.uint8, device=w.device)
    if sb is None:
        sb = torch.empty((N + 127) // 128, (-(-K // 128) + 3) // 4, dtype=torch.int32, device=w.device)
    q = _fp8(q, "q")
    sb = _i32(sb, "sb")
    if not (q.is_contiguous() and sb.is_contiguous()):
        raise ValueError("q and sb must be contiguous")
    _call("fp8_cast_per_block_ue8m0" + sfx, _ptr(w), _ld(w), _ptr(q), _ptr(sb), N, K, _stream(stream))
    return q, sb


def get_mk_alignment_for_contiguous_layout() -> int:
    return load_library().fg_get_mk_alignment_for_contiguous_layout()


def set_num_cus(n: int) -> None:
    load_library().fg_set_num_cus(int(n))


def get_num_cus() -> int:
    return load_library().fg_get_num_cus()
