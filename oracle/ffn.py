"""The MoE FFN layer forward in blockwise FP8, and the dense gated FFN.

Structure ([R1 card] "Every architecture field"; [arch blog] "Architecture
Overview", "More Aggressive Mixture-of-Expert", "Structural change"):
256 routed experts, 8 active per token, 1 always-activated shared expert; each
expert is a gated MLP using SwiGLU; the first layers are dense gated MLPs
(d_ff 18432).  Readings where the pages are silent:

* SwiGLU: h = silu(x W_gate^T) * (x W_up^T), y = h W_down^T, with
  silu(z) = z / (1 + e^-z); W13 = [W_gate; W_up] stacked on output rows;
* FP8 data flow: x -> 1x128 codes; gate/up GEMM exact in fp64; h rounded to
  fp32, then requantised 1x128; down GEMM exact in fp64;
* combine: out_t = sum_j w_tj y_tj + y_shared_t (shared weight 1) in fp64,
  then rounded to bf16 (round to nearest, ties to even).

Options: ``ue8m0`` switches every 1x128 quantisation (x and h) to power-of-two
scales (the weights must then be quantised the same way, quantize_expert(...,
ue8m0=True)); ``norm`` = (gamma, eps) applies the RMSNorm of norm.py to x
first, and the layer (router included) then sees the normalised bf16 rows.
"""
from __future__ import annotations

from typing import Callable, NamedTuple

import numpy as np

from . import gemm, norm as norm_mod, permute, quant, route


class QuantExpert(NamedTuple):
    w13_q: np.ndarray   # u8 [2*width, hidden]
    w13_s: np.ndarray   # f32 [2*width/128, hidden/128]
    w2_q: np.ndarray    # u8 [hidden, width]
    w2_s: np.ndarray    # f32 [hidden/128, width/128]


def quantize_expert(w13: np.ndarray, w2: np.ndarray, ue8m0: bool = False) -> QuantExpert:
    a, b = quant.quant_128x128(w13, ue8m0)
    c, d = quant.quant_128x128(w2, ue8m0)
    return QuantExpert(a, b, c, d)


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def round_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (8 significant bits), ties to even; returned as fp32.
    (Normal range only: the layer's outputs are far from bf16's limits.)"""
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)                     # v = f * 2^e, |f| in [0.5, 1)
    q = np.rint(np.ldexp(f, 8))            # 8 significant bits, ties to even
    return np.ldexp(q, e - 8).astype(np.float32)


def expert_forward(a_q: np.ndarray, a_s: np.ndarray, w: QuantExpert, ue8m0: bool = False) -> dict:
    """One gated expert on 1x128-quantised rows.  Returns h (fp32), h_q, h_s, y (fp64)."""
    gu = gemm.gemm_blockscaled(a_q, a_s, w.w13_q, w.w13_s)
    width = w.w13_q.shape[0] // 2
    h = (silu(gu[:, :width]) * gu[:, width:]).astype(np.float32)
    h_q, h_s = quant.quant_1x128(h, ue8m0)
    y = gemm.gemm_blockscaled(h_q, h_s, w.w2_q, w.w2_s)
    return {"h": h, "h_q": h_q, "h_s": h_s, "y": y}


def moe_ffn(x: np.ndarray, n_experts: int, top_k: int, n_group: int, topk_group: int,
            experts: Callable[[int], QuantExpert], w_router: np.ndarray | None = None,
            bias: np.ndarray | None = None, scores: np.ndarray | None = None, n_shared: int = 1,
            routed_scale: float = 1.0, group_rule: str = "top2_sum", ue8m0: bool = False,
            norm: tuple | None = None) -> dict:
    """x: bf16 values as fp32 [T, hidden].  experts(e) gives routed expert e's
    quantised weights; experts(n_experts) the shared expert (or the dense MLP
    when n_experts == 0).  scores (fp32 [T, E]) replaces the router when given.
    Returns every intermediate and ``out`` (bf16 values as fp32 [T, hidden])."""
    x = np.asarray(x, dtype=np.float32)
    t, d = x.shape
    r: dict = {}
    if norm is not None:
        x = norm_mod.rmsnorm(x, norm[0], norm[1])
        r["x_norm"] = x
    x_q, x_s = quant.quant_1x128(x, ue8m0)
    r.update(x_q=x_q, x_s=x_s)
    acc = np.zeros((t, d), dtype=np.float64)
    if n_experts > 0:
        if scores is None:
            scores = route.sigmoid_scores(route.router_logits(x, w_router))
        idx, w = route.select(scores, bias, n_group, topk_group, top_k, routed_scale, group_rule)
        offsets, sorted_assign, assign_pos = permute.permute(idx, n_experts)
        r.update(scores=scores, topk_idx=idx, topk_w=w, offsets=offsets, sorted_assign=sorted_assign,
                 assign_pos=assign_pos)
        rows = permute.gather_rows(np.arange(t), sorted_assign, top_k)   # token of each sorted row
        y_sorted = np.zeros((t * top_k, d), dtype=np.float64)
        h_q = None
        h_s = None
        for e in range(n_experts):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi == lo:
                continue
            src = rows[lo:hi]
            res = expert_forward(x_q[src], x_s[src], experts(e), ue8m0)
            if h_q is None:
                width = res["h_q"].shape[1]
                h_q = np.zeros((t * top_k, width), dtype=np.uint8)
                h_s = np.zeros((t * top_k, width // 128), dtype=np.float32)
            h_q[lo:hi], h_s[lo:hi] = res["h_q"], res["h_s"]
            y_sorted[lo:hi] = res["y"]
        r.update(h_q=h_q, h_s=h_s, y_sorted=y_sorted)
        acc += permute.combine(y_sorted, assign_pos, w, None)
    if n_shared:
        res = expert_forward(x_q, x_s, experts(n_experts), ue8m0)
        r.update(shared_h_q=res["h_q"], shared_h_s=res["h_s"], y_shared=res["y"])
        acc += res["y"]
    r["out_f64"] = acc
    r["out"] = round_bf16(acc)
    return r
