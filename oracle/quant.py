"""Fine-grained FP8 quantisation (the cast helpers), reference form.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages call the scaling "fine-grained, as proposed in DeepSeek-V3"
(GeekNews topic 19444, opening bullets; 7minutos.es, "Detalles y beneficios
tecnicos") and fix the factor type as FP32 on SM90 (DeepGEMM digest, GeekNews
topic 19459, "GEMM arayuzu ve yerlesim kisitlari", which also leaves the FP8
cast to the user).  They give no granularity and no formula.  Readings taken:

* activations: one scale per row and 128-wide K group  (1 x 128);
* weights:     one scale per 128 x 128 block (the last N block may be short);
* amax is the largest |x| in the group, s = max(amax, 1e-4) / 448 computed in
  fp32 (the 1e-4 floor only keeps an all-zero group finite);
* q = e4m3fn_RNE( fp32(x / s) ) with an IEEE fp32 division.

All arithmetic that decides a code is done in fp32, as the GPU does it.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import encode_rne

GROUP = 128
E4M3_MAX = np.float32(448.0)
AMAX_FLOOR = np.float32(1e-4)


def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    return (np.maximum(amax, AMAX_FLOOR) / E4M3_MAX).astype(np.float32)


def _encode_scaled(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    y = (np.asarray(x, dtype=np.float32) / s).astype(np.float32)  # fp32 division
    return encode_rne(y)


def _pad_k(x: np.ndarray) -> np.ndarray:
    """Zero columns up to the next multiple of 128.  A partial last K group
    (K % 128 != 0) is quantised on its own elements: zeros never raise an
    amax, and the codes of the added columns are dropped again."""
    K = x.shape[-1]
    Kp = -(-K // GROUP) * GROUP
    if Kp == K:
        return x
    out = np.zeros(x.shape[:-1] + (Kp,), np.float32)
    out[..., :K] = x
    return out


def quantize_per_token(x) -> tuple[np.ndarray, np.ndarray]:
    """1x128 quantisation of activations.

    x: float32 [M, K].  When K % 128 != 0 the last group holds the K % 128
    remaining columns and its factor comes from their amax alone.
    Returns (q uint8 [M, K], sa float32 [ceil(K/128), M]) -- the scales are
    returned K-group-major ("transposed"), the layout the GEMM consumes.
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    xp = _pad_k(x)
    Kb = xp.shape[1] // GROUP
    xg = xp.reshape(M, Kb, GROUP)
    amax = np.abs(xg).max(axis=2) if M else np.zeros((0, Kb), np.float32)
    s = _scale_from_amax(amax)  # [M, Kb]
    q = _encode_scaled(xg, s[:, :, None]).reshape(M, Kb * GROUP)[:, :K]
    return np.ascontiguousarray(q), np.ascontiguousarray(s.T)


def quantize_per_block(w) -> tuple[np.ndarray, np.ndarray]:
    """128x128 quantisation of weights.

    w: float32 [N, K]; N is arbitrary (the last row block covers N % 128
    rows when N is not a multiple of 128), and so is K (the last column block
    covers K % 128 columns).
    Returns (q uint8 [N, K], sb float32 [ceil(N/128), ceil(K/128)]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    wp = _pad_k(w)
    Kb = wp.shape[1] // GROUP
    Nb = -(-N // GROUP)
    q = np.empty((N, Kb * GROUP), dtype=np.uint8)
    sb = np.empty((Nb, Kb), dtype=np.float32)
    for nb in range(Nb):
        rows = slice(nb * GROUP, min(N, (nb + 1) * GROUP))
        blk = wp[rows].reshape(-1, Kb, GROUP)  # [r, Kb, 128]
        amax = np.abs(blk).max(axis=(0, 2))  # [Kb]
        s = _scale_from_amax(amax)
        sb[nb] = s
        q[rows] = _encode_scaled(blk, s[None, :, None]).reshape(-1, Kb * GROUP)
    return np.ascontiguousarray(q[:, :K]), sb


# ---------------------------------------------------------------------------
# Power-of-two (UE8M0) scale factors.
#
# The digest's layout section ("GEMM arayuzu ve yerlesim kisitlari", DeepGEMM
# digest, GeekNews topic 19459) says the newer architecture takes its scale
# factors as UE8M0 -- an unsigned 8-bit exponent, value 2**(e - 127) -- with
# four of them packed into one 32-bit integer.  It gives no rounding rule and
# no packing axis.  Readings taken:
#
# * same granularity as the fp32 factors (1 x 128 activations, 128 x 128
#   weights);
# * the factor is the fp32 one, max(amax, 1e-4) / 448, rounded UP to a power
#   of two, so that |x / s| <= 448 still holds and no code saturates;
# * q = e4m3fn_RNE(x / s), an exact scaling by a power of two before the
#   rounding;
# * four consecutive K groups of one row (activations) or one weight block
#   row (weights) share an int32, K group 4i + j in byte j (least significant
#   byte first); bytes past the last K group are unspecified.
# ---------------------------------------------------------------------------

UE8M0_BIAS = 127


def ue8m0_round_up(s) -> np.ndarray:
    """UE8M0 byte of the smallest power of two >= s, for positive normal fp32 s."""
    m, e = np.frexp(np.asarray(s, dtype=np.float64))  # s = m * 2**e, 0.5 <= m < 1 (exact)
    e = np.where(m == 0.5, e - 1, e)  # s is itself 2**(e - 1)
    return (e + UE8M0_BIAS).astype(np.uint8)


def ue8m0_decode(b) -> np.ndarray:
    """UE8M0 bytes -> float32 powers of two (exact)."""
    return np.ldexp(np.float32(1.0), np.asarray(b, dtype=np.int32) - UE8M0_BIAS).astype(np.float32)


def quantize_per_token_ue8m0(x) -> tuple[np.ndarray, np.ndarray]:
    """1x128 quantisation with power-of-two factors.

    A partial last K group (K % 128 != 0) takes its factor from its own
    columns, as in quantize_per_token.
    Returns (q uint8 [M, K], UE8M0 bytes uint8 [ceil(K/128), M]) --
    K-group-major, unpacked (see pack_ue8m0)."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    xp = _pad_k(x)
    Kb = xp.shape[1] // GROUP
    xg = xp.reshape(M, Kb, GROUP)
    amax = np.abs(xg).max(axis=2) if M else np.zeros((0, Kb), np.float32)
    e = ue8m0_round_up(_scale_from_amax(amax))  # [M, Kb]
    q = _encode_scaled(xg, ue8m0_decode(e)[:, :, None]).reshape(M, Kb * GROUP)[:, :K]
    return np.ascontiguousarray(q), np.ascontiguousarray(e.T)


def quantize_per_block_ue8m0(w) -> tuple[np.ndarray, np.ndarray]:
    """128x128 quantisation with power-of-two factors.

    The last row and column blocks may be partial (N % 128, K % 128), each
    with its own factor, as in quantize_per_block.
    Returns (q uint8 [N, K], UE8M0 bytes uint8 [ceil(N/128), ceil(K/128)])."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    wp = _pad_k(w)
    Kb = wp.shape[1] // GROUP
    Nb = -(-N // GROUP)
    q = np.empty((N, Kb * GROUP), dtype=np.uint8)
    eb = np.empty((Nb, Kb), dtype=np.uint8)
    for nb in range(Nb):
        rows = slice(nb * GROUP, min(N, (nb + 1) * GROUP))
        blk = wp[rows].reshape(-1, Kb, GROUP)
        e = ue8m0_round_up(_scale_from_amax(np.abs(blk).max(axis=(0, 2))))
        eb[nb] = e
        q[rows] = _encode_scaled(blk, ue8m0_decode(e)[None, :, None]).reshape(-1, Kb * GROUP)
    return np.ascontiguousarray(q[:, :K]), eb


def pack_ue8m0(b, axis: int) -> np.ndarray:
    """Pack UE8M0 bytes four to an int32 along `axis` (the K-group axis):
    element i holds groups 4i .. 4i+3, group 4i + j in byte j.  Missing bytes
    of the last element are 0."""
    b = np.moveaxis(np.asarray(b, dtype=np.uint8), axis, -1)
    n = b.shape[-1]
    padded = np.zeros(b.shape[:-1] + (-(-n // 4) * 4,), np.uint8)
    padded[..., :n] = b
    words = padded.reshape(b.shape[:-1] + (-1, 4)).astype(np.uint32)
    packed = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    return np.ascontiguousarray(np.moveaxis(packed.view(np.int32), -1, axis))


def unpack_ue8m0(p, n: int, axis: int) -> np.ndarray:
    """Inverse of pack_ue8m0 for n K groups."""
    p = np.moveaxis(np.asarray(p, dtype=np.int32), axis, -1).view(np.uint32)
    parts = [((p >> (8 * j)) & 0xFF).astype(np.uint8) for j in range(4)]
    b = np.stack(parts, axis=-1).reshape(p.shape[:-1] + (-1,))[..., :n]
    return np.ascontiguousarray(np.moveaxis(b, -1, axis))
