"""FP8 backward of the experts' grouped GEMMs: the input gradient (dgrad) and the
weight gradient (wgrad), with transposed tile quantisation.

[arch blog] "First ever FP8 Precision OSS LLM pre-training": the model is trained with its
matrix multiplications in FP8 (the section's body is cut off after the motivation), with the
FP8 headings "Fine granularity quantization", "Online Quantization" and "Better Accumulation
Precision".  The pages do not spell the backward out; the oracle's readings, for one GEMM of
the forward C = A . W^T (A [M, K] quantised 1x128 along K, W [N, K] in 128x128 blocks), are:

* dgrad: dA = dC . W.  The incoming gradient dC [M, N] is quantised 1x128 along its
  contraction dimension N (the forward's activation rule, online), and W enters through the
  same 128x128 blocks as in the forward, read transposed (a 128x128 block of W is the
  transposed block of W^T, with the same scale), so dgrad is a forward-shaped grouped GEMM
  with W^T in place of W;
* wgrad: for each group g of rows (one expert's tokens), dW_g = dC_g^T . A_g, a contraction
  over the group's rows.  Both operands are therefore quantised along rows: in 128x1 tiles
  (per column, per 128 consecutive rows of one group; a group's last tile holds what is left,
  and tiles never cross groups) - the "transposed" tiles.  Each is stored transposed, [N, Mp],
  with every group's rows padded with zeros to a multiple of 128 (Mp = sum over groups of
  ceil(M_g / 128) * 128), so a 128x1 tile is a 1x128 tile of the transposed matrix;
* every product is exact in fp64 and the sums are fp64; outputs are the fp64 results.
"""
from __future__ import annotations

import numpy as np

from . import gemm, quant


def padded_offsets(offsets: np.ndarray) -> np.ndarray:
    """Row offsets after padding every group to a multiple of 128 rows."""
    off = np.asarray(offsets, dtype=np.int64)
    sizes = -(-(off[1:] - off[:-1]) // 128) * 128
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def quant_128x1_grouped(v: np.ndarray, offsets: np.ndarray, ue8m0: bool = False):
    """v fp32 [M, N] (M = offsets[-1]) -> (codes u8 [N, Mp], scales f32 [N, Mp / 128], padded offsets).

    Group g's rows go to columns po[g] .. po[g] + M_g - 1 of the transposed output (zeros after
    them up to po[g + 1]); each run of 128 of them is one quantisation tile."""
    v = np.asarray(v, dtype=np.float32)
    off = np.asarray(offsets)
    po = padded_offsets(off)
    n = v.shape[1]
    t = np.zeros((n, int(po[-1])), dtype=np.float32)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        t[:, po[g]:po[g] + hi - lo] = v[lo:hi].T
    codes, scales = quant.quant_1x128(t, ue8m0)
    return codes, scales, po


def wgrad_grouped(a_t: np.ndarray, a_ts: np.ndarray, b_t: np.ndarray, b_ts: np.ndarray,
                  padded: np.ndarray) -> np.ndarray:
    """dW_g = A_g^T-operand times B_g-operand over group g's (padded) rows, exactly.

    a_t u8 [Na, Mp] with scales [Na, Mp / 128] and b_t u8 [Nb, Mp] with [Nb, Mp / 128], both the
    transposed 128x1-tile quantisations of quant_128x1_grouped.  Returns fp64 [G, Na, Nb] with
    out[g][i][j] = sum over the group's rows m of A[m][i] * B[m][j]."""
    a = quant.dequant_1x128(a_t, a_ts)
    b = quant.dequant_1x128(b_t, b_ts)
    G = len(padded) - 1
    out = np.zeros((G, a.shape[0], b.shape[0]), dtype=np.float64)
    for g in range(G):
        lo, hi = int(padded[g]), int(padded[g + 1])
        if hi > lo:
            out[g] = a[:, lo:hi] @ b[:, lo:hi].T
    return out


def transpose_weight(w_q: np.ndarray, w_s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The 128x128-block quantisation of W^T from that of W: codes transposed, block scales
    transposed (block (i, j) of W is block (j, i) of W^T)."""
    return np.ascontiguousarray(np.swapaxes(w_q, -1, -2)), np.ascontiguousarray(np.swapaxes(w_s, -1, -2))


def dgrad_grouped(dc_q: np.ndarray, dc_s: np.ndarray, w_q: np.ndarray, w_s: np.ndarray,
                  offsets: np.ndarray) -> np.ndarray:
    """dA = dC . W per group: dc (1x128 codes [M, N] with scales [M, N / 128]), the forward's
    weights w_q u8 [G, N, K] with scales [G, N / 128, K / 128].  Returns fp64 [M, K]."""
    wt_q, wt_s = transpose_weight(w_q, w_s)
    return gemm.grouped_gemm_blockscaled(dc_q, dc_s, None, wt_q, wt_s, offsets)
