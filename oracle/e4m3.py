"""E4M3 codec (OCP 8-bit floating point, E4M3FN variant).

The pages only say that the FP8 scheme gives "more mantissa bits" to its
values ([arch blog] heading "More Mantissa bits of fp8") and that the
checkpoint is "blockwise FP8" ([aguasto] "Quantization").  Reading: every
tensor uses the 4-exponent-bit / 3-mantissa-bit format as defined by the OCP
8-bit floating point specification (E4M3FN): bias 7, subnormals, no
infinities, S.1111.111 is NaN, largest finite value 448.

Encoding is round-to-nearest with ties to the even mantissa, sign preserved,
saturating to +-448 (no value above 448 is produced).
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
MIN_SUBNORMAL = 2.0 ** -9


def decode_value(code: int) -> float:
    """Value of one byte, straight from the format's field definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** -6          # subnormal: 0.M x 2^(1-bias)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


DECODE = np.array([decode_value(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values (table lookup)."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def _encode_chunk(v: np.ndarray) -> np.ndarray:
    c = v.astype(np.float64)
    nan = np.isnan(c)
    inf = np.isinf(c)
    a = np.where(nan | inf, 0.0, np.abs(c))
    _, e = np.frexp(a)                   # a = f * 2^e with f in [0.5, 1), so floor(log2 a) = e - 1
    big_e = e - 1
    normal = a >= MIN_NORMAL
    # Normal range: a in [2^E, 2^(E+1)) keeps 3 fraction bits, i.e. it is
    # rounded to a multiple of 2^(E-3): q = rint(a / 2^(E-3)) lies in [8, 16].
    # Subnormal range: multiples of 2^-9, q = rint(a * 2^9) in [0, 8].
    # rint rounds ties to the even integer, which is the even mantissa.
    q = np.rint(np.ldexp(a, np.where(normal, 3 - big_e, 9)))
    carry = normal & (q == 16)           # rounded up into the next binade
    big_e = big_e + carry
    q = np.where(carry, 8, q).astype(np.int32)
    code = np.where(normal, ((big_e + 7) << 3) | (q - 8), q)   # biased exponent field, 3-bit mantissa
    code = np.where(inf, 0x7E, np.minimum(code, 0x7E))   # saturate: nothing above 448 (0x7E); 0x7F is NaN
    code = np.where(np.signbit(c), code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def encode(v: np.ndarray) -> np.ndarray:
    """fp64 (or fp32) values -> uint8 E4M3FN codes, RNE, saturating.

    Rounding is the textbook one for a binary float format: a magnitude a in
    [2^E, 2^(E+1)) with E >= -6 keeps 3 fraction bits, i.e. is rounded to a
    multiple of 2^(E-3); below 2^-6 the grid is the subnormal spacing 2^-9.
    Ties go to the even multiple, which is the even mantissa.  NaN inputs are
    outside the method's domain and encode to 0x7F.  (Processed in chunks only
    to keep the temporaries small.)"""
    v = np.asarray(v)
    out = np.empty(v.shape, dtype=np.uint8)
    fv = v.reshape(-1)
    fo = out.reshape(-1)
    step = 1 << 20
    for i in range(0, fv.size, step):
        fo[i:i + step] = _encode_chunk(fv[i:i + step])
    return out


def finite_positive_grid() -> tuple[np.ndarray, np.ndarray]:
    """(values, codes) of the 127 finite non-negative codes 0x00..0x7E, ascending."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return DECODE[codes], codes


def half_ulp(mag: np.ndarray) -> np.ndarray:
    """Half the spacing of the E4M3 grid at magnitude ``mag`` (<= 448):
    2^(E-4) for mag in [2^E, 2^(E+1)), E >= -6; 2^-10 below 2^-6."""
    mag = np.asarray(mag, dtype=np.float64)
    _, e = np.frexp(np.maximum(mag, MIN_NORMAL))
    return np.ldexp(1.0, (e - 1) - 4)
