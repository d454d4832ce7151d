"""Fine-granularity (tile / block) FP8 quantisation with fp32 scales.

[arch blog] headings "Fine granularity quantization" and "Online
Quantization"; [aguasto] "Quantization" (blockwise FP8 checkpoint).  The
section bodies are missing from the page, so the oracle takes this reading:

* activations: one scale per row per 128 consecutive columns (1x128 tile),
  computed at run time from the tile itself ("online");
* weights: one scale per 128x128 block;
* per tile/block: amax = max |v| (exact), s = fp32(amax / 448) with a
  correctly rounded fp32 division, q_i = E4M3(fp32(v_i / s)) with a correctly
  rounded fp32 division; an all-zero tile gets s = 1 and codes 0x00;
* a tile so small that amax / 448 falls below the smallest normal fp32
  (amax < 448 * 2^-126) takes s = 2^-126 (the quotient then still lies within
  +-448, and the scale stays a normal number with a finite reciprocal).

Power-of-two ("UE8M0") variant ([arch blog] heading "More customized data
format and scaling factor"; the section body is missing, so this is a
reading): s is the smallest power of two with amax / s <= 448, i.e.
s = 2^k, k = ceil(log2(amax / 448)) decided exactly, clamped to [-127, 127]
(the range of an 8-bit biased exponent); v_i / s is then exact and only the
E4M3 rounding remains.  All-zero tiles keep s = 1.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

TILE = 128
F448 = np.float32(448.0)


def _pow2_scales(amax: np.ndarray) -> np.ndarray:
    """Smallest 2^k (k in [-127, 127]) with amax <= 448 * 2^k, decided with exact comparisons."""
    a = amax.astype(np.float64)                   # fp32 values are exact in fp64
    with np.errstate(divide="ignore"):
        k = np.ceil(np.log2(np.where(a > 0, a, 1.0) / 448.0)).astype(np.int64)   # estimate
    k = np.where(a > np.ldexp(448.0, k), k + 1, k)                              # fix the estimate
    k = np.where(a <= np.ldexp(448.0, k - 1), k - 1, k)                         # both ways
    k = np.clip(k, -127, 127)
    return np.where(a == 0, 1.0, np.ldexp(1.0, k)).astype(np.float32)


def _scales(amax: np.ndarray, ue8m0: bool = False) -> np.ndarray:
    amax = amax.astype(np.float32)
    if ue8m0:
        return _pow2_scales(amax)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.maximum((amax / F448).astype(np.float32), np.float32(2.0 ** -126))
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quant_1x128(v: np.ndarray, ue8m0: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """v fp32 [rows, cols] (cols % 128 == 0) -> (codes u8 [rows, cols], scales f32 [rows, cols/128])."""
    v = np.asarray(v, dtype=np.float32)
    rows, cols = v.shape
    assert cols % TILE == 0
    tiles = v.reshape(rows, cols // TILE, TILE)
    amax = np.max(np.abs(tiles), axis=-1)
    s = _scales(amax, ue8m0)
    quot = (tiles / s[..., None]).astype(np.float32)     # fp32 / fp32, IEEE correctly rounded
    codes = e4m3.encode(quot).reshape(rows, cols)
    return codes, s


def quant_128x128(w: np.ndarray, ue8m0: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """w fp32 [R, C] (both % 128 == 0) -> (codes u8 [R, C], scales f32 [R/128, C/128])."""
    w = np.asarray(w, dtype=np.float32)
    r, c = w.shape
    assert r % TILE == 0 and c % TILE == 0
    blocks = w.reshape(r // TILE, TILE, c // TILE, TILE)
    amax = np.max(np.abs(blocks), axis=(1, 3))
    s = _scales(amax, ue8m0)
    quot = (blocks / s[:, None, :, None]).astype(np.float32)
    codes = e4m3.encode(quot).reshape(r, c)
    return codes, s


def dequant_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 values of 1x128-tile codes."""
    rows, cols = codes.shape
    vals = e4m3.decode(codes).reshape(rows, cols // TILE, TILE)
    return (vals * scales.astype(np.float64)[..., None]).reshape(rows, cols)


def dequant_128x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 values of 128x128-block codes."""
    r, c = codes.shape
    vals = e4m3.decode(codes).reshape(r // TILE, TILE, c // TILE, TILE)
    return (vals * scales.astype(np.float64)[:, None, :, None]).reshape(r, c)
