"""RMSNorm in front of the MoE FFN (test infrastructure: only tests/, the smoke
check and the benchmark's CPU baseline use this package).

[R1 card] llm-architectures-explained, "DeepSeek-R1", facts table rows "Norm
placement" and "Norm type": pre-norm blocks with RMSNorm, the
post-attention norm sitting right before the MLP; [arch blog] onlylabs,
"DeepSeek v3 and R1 Model Architecture", "Architecture Overview" (RMSNorm).
The pages name the norm but give no formula, precision or epsilon.  Reading
(RMSNorm as usually defined, with a fixed rounding sequence):

  inv_t = fp32( 1 / sqrt( (sum_i x_ti^2) / d + eps ) )   computed in fp64
  y_ti  = bf16( fp32( fp32(x_ti * inv_t) * gamma_i ) )   two fp32 products, one bf16 rounding

The sum of squares is the exact sum rounded once to fp64 (squares of bf16
values are exact; math.fsum sums exactly), so it does not depend on the order
of the additions; the division, the square root and the reciprocal are IEEE
fp64 operations.

x and gamma are bf16 values, eps an fp32 value.  y (bf16) is what the layer
hands on: the router reads it and fp8_quant_1x128 quantises it, so the fused
kernel's codes and scales are quant_1x128(y).
"""
from __future__ import annotations

import math

import numpy as np


def round_bf16(v: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32 (normal range)."""
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(f, 8)), e - 8).astype(np.float32)


def inv_rms(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-row fp32 1/RMS of bf16-valued rows x [T, d]."""
    x64 = np.asarray(x, dtype=np.float64)
    d = x64.shape[1]
    ss = np.array([math.fsum(r) for r in x64 * x64])   # exact squares, exactly summed, rounded once
    e64 = float(np.float32(eps))
    return (1.0 / np.sqrt(ss / d + e64)).astype(np.float32)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y bf16-valued fp32 [T, d] from bf16-valued x [T, d] and gamma [d]."""
    x32 = np.asarray(x, dtype=np.float32)
    inv = inv_rms(x32, eps)
    t = (x32 * inv[:, None]).astype(np.float32)
    y = (t * np.asarray(gamma, dtype=np.float32)[None, :]).astype(np.float32)
    return round_bf16(y)
