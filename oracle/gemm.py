"""Block-scaled FP8 (grouped) GEMM, exactly: decode to fp64, scale, matmul.

[arch blog] headings "Fine granularity quantization" and "Better Accumulation
Precision"; [aguasto] "Quantization".  Reading: C = A . B^T where A holds
1x128-tile codes with scales a_s [M, K/128] and B holds 128x128-block codes
with scales b_s [N/128, K/128]; the products are accumulated at a precision
above the operands'.  The oracle forms the exact fp64 values of both operands
(an e4m3 value times an fp32 scale is exact in fp64) and multiplies them with
an fp64 matmul, so each 128-wide K block's scales enter exactly once, as in
the per-block scale promotion, without any tiling of its own.
"""
from __future__ import annotations

import numpy as np

from . import quant


def gemm_blockscaled(a_q: np.ndarray, a_s: np.ndarray, b_q: np.ndarray, b_s: np.ndarray) -> np.ndarray:
    """a_q u8 [M, K], a_s f32 [M, K/128], b_q u8 [N, K], b_s f32 [N/128, K/128] -> fp64 [M, N]."""
    a = quant.dequant_1x128(a_q, a_s)
    b = quant.dequant_128x128(b_q, b_s)
    return a @ b.T


def grouped_gemm_blockscaled(a_q: np.ndarray, a_s: np.ndarray, a_gather: np.ndarray | None,
                             b_q: np.ndarray, b_s: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Rows offsets[g]..offsets[g+1] of the (gathered) A multiply group g's B.

    a_gather[m] is the source row of logical row m (None: identity).
    b_q u8 [G, N, K], b_s f32 [G, N/128, K/128].  Returns fp64 [M, N]."""
    offsets = np.asarray(offsets)
    rows = np.arange(offsets[-1]) if a_gather is None else np.asarray(a_gather)
    g_count = b_q.shape[0]
    out = np.zeros((int(offsets[-1]), b_q.shape[1]), dtype=np.float64)
    for g in range(g_count):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            src = rows[lo:hi]
            out[lo:hi] = gemm_blockscaled(a_q[src], a_s[src], b_q[g], b_s[g])
    return out
