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


def quantize_per_token(x) -> tuple[np.ndarray, np.ndarray]:
    """1x128 quantisation of activations.

    x: float32 [M, K] with K % 128 == 0.
    Returns (q uint8 [M, K], sa float32 [K/128, M]) -- the scales are returned
    K-group-major ("transposed"), the layout the GEMM consumes.
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    Kb = K // GROUP
    xg = x.reshape(M, Kb, GROUP)
    amax = np.abs(xg).max(axis=2) if M else np.zeros((0, Kb), np.float32)
    s = _scale_from_amax(amax)  # [M, Kb]
    q = _encode_scaled(xg, s[:, :, None]).reshape(M, K)
    return q, np.ascontiguousarray(s.T)


def quantize_per_block(w) -> tuple[np.ndarray, np.ndarray]:
    """128x128 quantisation of weights.

    w: float32 [N, K] with K % 128 == 0; N is arbitrary (the last row block
    covers N % 128 rows when N is not a multiple of 128).
    Returns (q uint8 [N, K], sb float32 [ceil(N/128), K/128]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    Kb = K // GROUP
    Nb = -(-N // GROUP)
    q = np.empty((N, K), dtype=np.uint8)
    sb = np.empty((Nb, Kb), dtype=np.float32)
    for nb in range(Nb):
        rows = slice(nb * GROUP, min(N, (nb + 1) * GROUP))
        blk = w[rows].reshape(-1, Kb, GROUP)  # [r, Kb, 128]
        amax = np.abs(blk).max(axis=(0, 2))  # [Kb]
        s = _scale_from_amax(amax)
        sb[nb] = s
        q[rows] = _encode_scaled(blk, s[None, :, None]).reshape(-1, K)
    return q, sb
