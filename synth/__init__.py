"""Seeded synthetic inputs for the blockwise-FP8 MoE FFN layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random numbers and describes workload shapes: it
holds none of the layer's arithmetic (no quantisation, routing, permutation or
GEMM), so that neither the oracle nor the HIP path can leak into the other
through it.

Layer shapes follow the DeepSeek-R1 card (llm-architectures-explained,
section "Every architecture field"): d_model 7168, 256 routed experts with 8
active, d_expert 2048, one shared expert of width 2048, and the dense first
layers with d_ff 18432.  "9 out of 257 (1 shared)" active experts is the
onlylabs post "DeepSeek v3 and R1 Model Architecture", table in section "More
Aggressive Mixture-of-Expert".

Every random stream is ``numpy.random.PCG64(SeedSequence([seed, cfg_id,
tensor_id, expert_id]))`` with seed 0.  Full-size expert weights (11.3 G
values at V3 shapes) are too many for numpy's generator in a test's time
budget; for those, ``torch_expert_weight`` draws them with torch's generator on
the target device under a seed derived the same way.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED = 0

# tensor ids of the per-tensor random streams
T_X, T_WR, T_WGATE, T_WUP, T_WDOWN, T_CAL, T_SCORES, T_BIAS = range(8)


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """One workload: a MoE FFN layer (n_experts > 0) or a dense gated FFN
    (n_experts == 0, the dense MLP plays the role of the shared expert)."""
    name: str
    cfg_id: int
    tokens: int
    hidden: int
    inter: int            # routed expert width (d_expert)
    n_experts: int        # routed experts (0: dense layer)
    top_k: int
    n_shared: int         # 0 or 1 always-on gated MLP
    inter_shared: int     # its width
    n_group: int
    topk_group: int
    routed_scale: float = 1.0
    skewed: bool = False  # router bias calibrated to a Zipf load profile

    @property
    def assignments(self) -> int:
        return self.tokens * self.top_k

    def fp8_flops(self) -> float:
        """Algorithmic expert FLOPs (multiply and add counted as 2):
        3 matrices of hidden x width per token-expert pair."""
        routed = 6.0 * self.hidden * self.inter * self.tokens * self.top_k
        shared = 6.0 * self.hidden * self.inter_shared * self.tokens * self.n_shared
        return routed + shared

    def router_flops(self) -> float:
        return 2.0 * self.tokens * self.hidden * self.n_experts

    def expert_bytes(self, width: int) -> int:
        """FP8 codes plus fp32 128x128 block scales of one gated expert."""
        codes = 3 * self.hidden * width
        scales = 4 * (2 * width // 128) * (self.hidden // 128) + 4 * (self.hidden // 128) * (width // 128)
        return codes + scales


TINY = MoeShape("tiny", 0, 64, 256, 128, 16, 2, 1, 128, 4, 2)
V3_DECODE = MoeShape("v3_decode", 1, 64, 7168, 2048, 256, 8, 1, 2048, 8, 4)
DENSE_FFN = MoeShape("dense_ffn", 2, 4096, 7168, 0, 0, 0, 1, 18432, 1, 1)
V3_PREFILL = MoeShape("v3_prefill", 3, 4096, 7168, 2048, 256, 8, 1, 2048, 8, 4)
V3_SKEW = MoeShape("v3_skew", 4, 16384, 7168, 2048, 256, 8, 1, 2048, 8, 4, skewed=True)
# One GPU's share of an expert-parallel V3 prefill (8 GPUs, one expert group each): its 32
# local experts receive about T*k rows, ~1024 per expert at T = 4096 per GPU; the shared
# expert is replicated.  Emulated as a layer with 32 experts in 8 groups of 4, 4 kept.
V3_EP_LOCAL = MoeShape("v3_ep_local", 5, 4096, 7168, 2048, 32, 8, 1, 2048, 8, 4)
SHAPES = {s.name: s for s in (TINY, V3_DECODE, DENSE_FFN, V3_PREFILL, V3_SKEW, V3_EP_LOCAL)}


def with_tokens(shape: MoeShape, tokens: int) -> MoeShape:
    return dataclasses.replace(shape, tokens=tokens)


def rng(cfg_id: int, tensor_id: int, expert_id: int = 0, seed: int = SEED) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id, expert_id])))


def stream_seed(cfg_id: int, tensor_id: int, expert_id: int = 0, seed: int = SEED) -> int:
    """A 63-bit seed for torch's generator, derived from the same key."""
    state = np.random.SeedSequence([seed, cfg_id, tensor_id, expert_id]).generate_state(1, np.uint64)
    return int(state[0]) & ((1 << 63) - 1)


# --- bf16 storage helpers (input preparation; IEEE round-to-nearest-even) ---

def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --- draws ---

def gen_x(shape: MoeShape, tokens: int | None = None, tensor_id: int = T_X) -> np.ndarray:
    """Activations x ~ N(0, 1), stored as bf16 bits [T, hidden]."""
    t = shape.tokens if tokens is None else tokens
    v = rng(shape.cfg_id, tensor_id).standard_normal((t, shape.hidden), dtype=np.float32)
    return f32_to_bf16_bits(v)


def gen_router_w(shape: MoeShape) -> np.ndarray:
    """Router weights ~ N(0, 0.02) (0.02 is the standard deviation), bf16 bits [E, hidden]."""
    v = rng(shape.cfg_id, T_WR).standard_normal((shape.n_experts, shape.hidden), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(v)


def gen_expert_w(shape: MoeShape, expert: int) -> tuple[np.ndarray, np.ndarray]:
    """fp32 weights of one gated expert, N(0, 1/sqrt(d_in)) (standard deviation).

    Returns (w13 [2*width, hidden] = [gate; up] stacked on rows, w2 [hidden, width]).
    expert == n_experts is the shared expert (or the dense MLP)."""
    width = shape.inter_shared if expert == shape.n_experts else shape.inter
    d = shape.hidden
    g = rng(shape.cfg_id, T_WGATE, expert).standard_normal((width, d), dtype=np.float32)
    u = rng(shape.cfg_id, T_WUP, expert).standard_normal((width, d), dtype=np.float32)
    w = rng(shape.cfg_id, T_WDOWN, expert).standard_normal((d, width), dtype=np.float32)
    s_in = np.float32(1.0 / math.sqrt(d))
    s_dn = np.float32(1.0 / math.sqrt(width))
    return np.concatenate([g * s_in, u * s_in], axis=0), w * s_dn


def torch_expert_weight(shape: MoeShape, expert: int, which: str, device):
    """The same weights' distribution drawn with torch on ``device`` (fp32).

    which = "w13" ([2*width, hidden]) or "w2" ([hidden, width]).  Used for V3
    shapes, where numpy's generator is too slow; a given (shape, expert,
    which, device type) always yields the same values."""
    import torch
    width = shape.inter_shared if expert == shape.n_experts else shape.inter
    d = shape.hidden
    tid = T_WGATE if which == "w13" else T_WDOWN
    gen = torch.Generator(device=device)
    gen.manual_seed(stream_seed(shape.cfg_id, tid, expert))
    if which == "w13":
        w = torch.randn((2 * width, d), generator=gen, device=device, dtype=torch.float32)
        return w.mul_(1.0 / math.sqrt(d))
    w = torch.randn((d, width), generator=gen, device=device, dtype=torch.float32)
    return w.mul_(1.0 / math.sqrt(width))


def gen_scores(n_tokens: int, n_experts: int, cfg_id: int = 0, ties: bool = False) -> np.ndarray:
    """Stand-alone gating scores in (0, 1) (fp32) for routing tests.

    With ``ties`` the values are drawn from a coarse grid of 16 levels so that
    equal scores, equal group scores and equal biased scores are common."""
    r = rng(cfg_id, T_SCORES, 1 if ties else 0)
    if ties:
        return ((r.integers(1, 16, size=(n_tokens, n_experts)).astype(np.float32)) / np.float32(16.0)).astype(np.float32)
    v = r.random((n_tokens, n_experts), dtype=np.float32)
    return np.clip(v, np.float32(1e-6), np.float32(1.0 - 1e-6)).astype(np.float32)


def gen_bias(n_experts: int, cfg_id: int = 0, scale: float = 0.1) -> np.ndarray:
    """A small random routing bias (fp32) for routing tests."""
    return (rng(cfg_id, T_BIAS).standard_normal(n_experts, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def zipf_targets(n_tokens: int, top_k: int, n_experts: int, s: float = 1.2, cap: float = 20.0,
                 n_empty: int = 16, cfg_id: int = 4) -> np.ndarray:
    """Target per-expert loads (rows) for the load-skewed prefill workload.

    Experts are ranked by a seeded permutation.  The first n_experts - n_empty
    ranks get loads proportional to r^-s, capped at ``cap`` times the mean and
    water-filled so the loads sum to n_tokens * top_k; the last n_empty ranks
    are empty.  No load may exceed n_tokens (a token picks an expert once).
    Returns float64 [n_experts] indexed by expert id."""
    total = float(n_tokens * top_k)
    mean = total / n_experts
    hi = min(cap * mean, float(n_tokens))
    n_live = n_experts - n_empty
    ranks = np.arange(1, n_live + 1, dtype=np.float64)
    base = ranks ** (-s)
    lo_c, hi_c = 0.0, total / base.min()
    for _ in range(200):  # bisection on the Zipf constant c so that sum(min(hi, c r^-s)) = total
        c = 0.5 * (lo_c + hi_c)
        if np.minimum(hi, c * base).sum() < total:
            lo_c = c
        else:
            hi_c = c
    loads = np.minimum(hi, hi_c * base)
    perm = rng(cfg_id, T_CAL, 1).permutation(n_experts)
    out = np.zeros(n_experts, dtype=np.float64)
    out[perm[:n_live]] = loads
    return out


def skew_bias() -> np.ndarray:
    """The load-skewed workload's routing bias (fp32 [256]), stored as bit
    patterns in tests/golden/v3_skew_bias.txt (written by the oracle's
    calibration script beside it)."""
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                        "v3_skew_bias.txt")
    with open(path) as f:
        words = [int(line, 16) for line in f if line.strip() and not line.startswith("#")]
    return np.array(words, dtype=np.uint32).view(np.float32)
