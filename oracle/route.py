"""Gating: affinity scores, routing-only bias, group-limited top-k, weights.

[arch blog] "Local Balanced Routing to Experts": tokens go to experts by their
token-to-expert affinity; a bias term is added to the gating value and is used
only for routing.  [R1 card] "Every architecture field": 256 routed experts,
8 active.  The pages do not give the scoring function, the grouping or the
weight normalisation; the oracle's readings are:

* affinity s_e = sigmoid(x . w_e) (router logits accumulated in fp64 from the
  bf16 operands, rounded to fp32; sigmoid in fp64 on that fp32 logit, rounded
  to fp32);
* biased score b_e = fp32(s_e + bias_e), used for selection only;
* experts form n_group contiguous groups of E / n_group ids; a group's score is
  the fp32 sum of its two largest b (its largest b when a group has one
  expert); the topk_group groups with the highest group score are kept, ties
  to the lower group index; experts of dropped groups can never be chosen;
* the top_k experts by b among the kept ones, ties to the lower expert index;
  slot j holds the j-th best (descending b, ties to the lower index);
* weights use the unbiased s: w_j = fp32(s_j / S) * routed_scale, where S is
  the fp32 sum of s over slots 0..k-1 taken in slot order.
All selection arithmetic is IEEE fp32 (numpy float32); comparisons treat -0
and +0 as equal.
"""
from __future__ import annotations

import numpy as np


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """x [T, d] and w_router [E, d] hold bf16 values (as fp32) -> fp32 logits [T, E]."""
    return (np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T).astype(np.float32)


def sigmoid_scores(logits: np.ndarray) -> np.ndarray:
    l64 = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-l64))).astype(np.float32)


def biased(scores: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    s = np.asarray(scores, dtype=np.float32)
    if bias is None:
        return s.copy()
    return (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def group_scores(b: np.ndarray, n_group: int, rule: str = "top2_sum") -> np.ndarray:
    """b fp32 [T, E] -> fp32 [T, n_group]."""
    t, e = b.shape
    g = b.reshape(t, n_group, e // n_group)
    srt = -np.sort(-g, axis=-1)          # descending within each group
    if rule == "max" or g.shape[-1] == 1:
        return srt[..., 0].astype(np.float32)
    assert rule == "top2_sum"
    return (srt[..., 0] + srt[..., 1]).astype(np.float32)


def kept_groups(gscore: np.ndarray, topk_group: int) -> np.ndarray:
    """Indices [T, topk_group] of kept groups: highest score first, ties to the lower index."""
    order = np.argsort(-gscore, axis=-1, kind="stable")
    return order[:, :topk_group]


def select(scores: np.ndarray, bias: np.ndarray | None, n_group: int, topk_group: int, top_k: int,
           routed_scale: float = 1.0, group_rule: str = "top2_sum") -> tuple[np.ndarray, np.ndarray]:
    """fp32 scores [T, E] -> (topk_idx int32 [T, k], topk_w fp32 [T, k])."""
    s = np.asarray(scores, dtype=np.float32)
    t, e = s.shape
    b = biased(s, bias)
    gs = group_scores(b, n_group, group_rule)
    keep = kept_groups(gs, topk_group)
    group_of = np.arange(e) // (e // n_group)
    allowed = np.zeros((t, n_group), dtype=bool)
    np.put_along_axis(allowed, keep, True, axis=1)
    masked = np.where(allowed[:, group_of], b, np.float32(-np.inf)).astype(np.float32)
    order = np.argsort(-masked, axis=-1, kind="stable")   # descending b, ties to the lower index
    idx = order[:, :top_k].astype(np.int32)
    w = np.take_along_axis(s, idx, axis=1).astype(np.float32)
    total = np.zeros(t, dtype=np.float32)
    for j in range(top_k):                                  # slot-ordered fp32 sum
        total = (total + w[:, j]).astype(np.float32)
    wn = (w / total[:, None]).astype(np.float32)
    wn = (wn * np.float32(routed_scale)).astype(np.float32)
    return idx, wn


def route(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None, n_group: int, topk_group: int,
          top_k: int, routed_scale: float = 1.0, group_rule: str = "top2_sum"):
    """Scores from x, then select.  Returns (scores, topk_idx, topk_w)."""
    sc = sigmoid_scores(router_logits(x, w_router))
    idx, w = select(sc, bias, n_group, topk_group, top_k, routed_scale, group_rule)
    return sc, idx, w
