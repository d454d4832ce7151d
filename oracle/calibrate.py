"""Routing-bias adjustment toward target expert loads.

[arch blog] "Local Balanced Routing to Experts": the routing-only bias of an
expert is adjusted when that expert is overloaded or underloaded.  The page
gives no step size or schedule; reading: after each routing pass over a batch,
bias_e += gamma * sign(target_e - load_e) in fp32, with gamma decaying
geometrically.  This builds the load-skewed workload: targets are a Zipf load
profile, and experts with target 0 are pinned at a bias of -10 so they are
never chosen (scores lie in (0, 1)).
"""
from __future__ import annotations

import numpy as np

from . import route


def loads(topk_idx: np.ndarray, n_experts: int) -> np.ndarray:
    return np.bincount(np.asarray(topk_idx).reshape(-1), minlength=n_experts)


def update(bias: np.ndarray, topk_idx: np.ndarray, n_experts: int, gamma: float) -> np.ndarray:
    """One balancing step of the routing bias after a batch: the target of every expert is the
    mean load T*k/E, so an overloaded expert's bias drops by gamma, an underloaded one's rises by
    gamma, and an expert exactly at the mean keeps its bias (fp32 add)."""
    ld = loads(topk_idx, n_experts)
    mean = np.asarray(topk_idx).size / n_experts
    return adjust(bias, ld, np.full(n_experts, mean), gamma)


def adjust(bias: np.ndarray, load: np.ndarray, target: np.ndarray, gamma: float) -> np.ndarray:
    step = np.sign(np.asarray(target, np.float64) - load).astype(np.float32)
    return (bias + np.float32(gamma) * step).astype(np.float32)


def calibrate(scores: np.ndarray, target: np.ndarray, n_group: int, topk_group: int, top_k: int,
              iters: int = 600, gamma0: float = 2e-2, gamma1: float = 1e-4) -> tuple[np.ndarray, np.ndarray]:
    """Returns (bias fp32 [E], final loads on ``scores``)."""
    e = scores.shape[1]
    empty = np.asarray(target) == 0
    bias = np.where(empty, np.float32(-10.0), np.float32(0.0)).astype(np.float32)
    ratio = (gamma1 / gamma0) ** (1.0 / max(iters - 1, 1))
    gamma = gamma0
    for _ in range(iters):
        idx, _ = route.select(scores, bias, n_group, topk_group, top_k)
        ld = loads(idx, e)
        bias = adjust(bias, ld, target, gamma)
        bias[empty] = np.float32(-10.0)
        gamma *= ratio
    idx, _ = route.select(scores, bias, n_group, topk_group, top_k)
    return bias, loads(idx, e)
