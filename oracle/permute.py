"""Sorting token-expert assignments by expert, and the inverse combine.

The pages state the problem, not an algorithm: each token activates only part
of the network ([aguasto] "Theoretical weight-memory footprint"; [arch blog]
"More Aggressive Mixture-of-Expert"), so each expert's FFN runs on the rows
routed to it.  The oracle groups the T*k assignments a = t*k + j by expert
with a counting sort, which is stable, so within an expert rows keep the
order of a (token, then slot).
"""
from __future__ import annotations

import numpy as np


def permute(topk_idx: np.ndarray, n_experts: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """topk_idx int [T, k] -> (offsets int32 [E+1], sorted_assign int32 [T*k], assign_pos int32 [T*k]).

    offsets[e]..offsets[e+1] is expert e's row range in the sorted order;
    sorted_assign[p] = the assignment a at sorted position p;
    assign_pos[a] = the sorted position of assignment a."""
    flat = np.asarray(topk_idx).reshape(-1)
    counts = [0] * n_experts
    for e in flat.tolist():
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    nxt = offsets[:-1].copy()
    sorted_assign = [0] * len(flat)
    for a, e in enumerate(flat.tolist()):
        sorted_assign[nxt[e]] = a
        nxt[e] += 1
    assign_pos = [0] * len(flat)
    for p, a in enumerate(sorted_assign):
        assign_pos[a] = p
    return (np.array(offsets, dtype=np.int32), np.array(sorted_assign, dtype=np.int32),
            np.array(assign_pos, dtype=np.int32))


def gather_rows(rows: np.ndarray, sorted_assign: np.ndarray, top_k: int) -> np.ndarray:
    """Row of token t for each sorted position (t = a // k)."""
    return rows[np.asarray(sorted_assign) // top_k]


def unpermute(y_sorted: np.ndarray, assign_pos: np.ndarray, top_k: int) -> np.ndarray:
    """Pure inverse: [T*k, ...] in sorted order -> [T, k, ...] in (token, slot) order."""
    y = np.asarray(y_sorted)
    out = y[np.asarray(assign_pos)]
    return out.reshape((-1, top_k) + y.shape[1:])


def combine(y_sorted: np.ndarray, assign_pos: np.ndarray, topk_w: np.ndarray,
            shared_y: np.ndarray | None) -> np.ndarray:
    """out_t = sum_j w_tj * y[assign_pos(t, j)] (+ shared_y_t), in fp64."""
    t, k = topk_w.shape
    per_slot = unpermute(np.asarray(y_sorted, np.float64), assign_pos, k)      # [T, k, d]
    out = np.einsum("tk,tkd->td", np.asarray(topk_w, np.float64), per_slot)
    if shared_y is not None:
        out = out + np.asarray(shared_y, np.float64)
    return out
