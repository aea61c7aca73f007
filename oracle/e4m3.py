"""e4m3fn codec and bf16 rounding, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the operand format only as E4M3 (DeepGEMM digest, GeekNews
topic 19459, section on the v3.2 MQA kernels) and say the output is BF16.
The reading taken here is the OCP "e4m3fn" variant that gfx950 implements:

    code = s eeee mmm,   bias 7
    e == 0          -> (-1)^s * m * 2^-9           (subnormals, incl. +-0)
    e == 15, m == 7 -> NaN  (0x7F, 0xFF)
    otherwise       -> (-1)^s * (1 + m/8) * 2^(e-7)

No infinities; the largest finite magnitude is 448 (code 0x7E).
"""

from __future__ import annotations

import numpy as np

NAN_CODES = (0x7F, 0xFF)
MAX_FINITE = 448.0


def _decode_code(code: int) -> float:
    """Value of one 8-bit e4m3fn code, straight from the bit fields."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: float64 value of every code 0..255 (NaN for 0x7F / 0xFF).
DECODE_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """Decode an array of uint8 e4m3fn codes to float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes]


# Magnitudes of codes 0x00..0x7E are strictly increasing with the code, so the
# nearest code can be found by bisection.  480 is appended as the (non-finite)
# neighbour above 448 so that the rounding boundary 464 is placed correctly;
# landing on it means the value is not representable.
_POS_GRID = np.concatenate([DECODE_TABLE[:0x7F], [480.0]])
_CHUNK = 1 << 20


def encode_rne(values) -> np.ndarray:
    """Round float values to the nearest e4m3fn code, ties to the even code.

    The input is taken exactly as given (callers pass fp32 values).  The sign
    of the input, including that of zero, is kept in the sign bit.  A
    magnitude at or above 464 (the midpoint between 448 and the first value
    past it) has no finite e4m3fn neighbour: it raises, since the method never
    produces one (|x/s| <= 448 * (1 + 2^-23) by construction of s).
    """
    v = np.asarray(values)
    if v.size > _CHUNK:  # same element-wise rule, evaluated in cache-sized pieces
        flat = v.reshape(-1)
        out = np.empty(flat.shape, np.uint8)
        for i in range(0, flat.size, _CHUNK):
            out[i:i + _CHUNK] = encode_rne(flat[i:i + _CHUNK])
        return out.reshape(v.shape)
    v = v.astype(np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN input to e4m3 encode")
    mag = np.abs(v)
    hi = np.searchsorted(_POS_GRID, mag, side="left")  # grid[hi-1] < mag <= grid[hi]
    hi = np.minimum(hi, len(_POS_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_GRID[lo]
    d_hi = _POS_GRID[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == _POS_GRID[hi], hi, code)
    if (code >= 0x7F).any():
        raise OverflowError("value rounds past the largest finite e4m3fn (448)")
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def bf16_rne_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16, nearest-even, return the uint16 bits.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's exponent
    range.  The rounding is done on the exact float64 input (no intermediate
    fp32 rounding): x = f * 2^e with f in [0.5, 1); the bf16 value is
    rint(f * 2^8) * 2^(e-8), with the quantum floored at the bf16 subnormal
    step 2^-133.  Results above the bf16 range become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    e = np.maximum(e, -125)  # below 2^-126 the quantum stays 2^-133
    q = np.rint(np.ldexp(x, 8 - e))  # np.rint rounds half to even
    r = np.ldexp(q, e - 8)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)  # exact: r has <= 8 significant bits
    r32 = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, x), r32).astype(np.float32)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32, exactly (the 16 bits are the upper half
    of the fp32 pattern).  The casts take bf16 inputs through this widening."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
