"""Shared helpers of the GPU parity tests: building layers on the device and
on the oracle side from the same fp32 weights, and the comparison bars."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import synth
from oracle import e4m3, ffn, norm, permute, quant, route

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> fp32 numpy values."""
    return t.float().cpu().numpy()


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits): 2^(floor(log2|v|) - 8)."""
    _, e = np.frexp(np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126))
    return np.ldexp(1.0, e - 1 - 8)


def output_bar(got: np.ndarray, ref_bf16: np.ndarray, ref_f64: np.ndarray) -> tuple[float, float, float]:
    """The output bar of the layer.

    * relative L2 of the bf16 output against the oracle's bf16-rounded output
      (bf16 rounding alone costs ~1.7e-3 in L2 against the unrounded value);
    * per element, the computation error: |out - oracle_fp64| minus the bf16
      output format's own rounding allowance (half an ulp of the oracle's value),
      over the RMS of the output.  (A correctly rounded element above ~5 x RMS
      already sits up to 2e-2 x RMS from the fp64 value; against the rounded
      output, a 1-ulp rounding disagreement is up to 4e-2 x RMS there.)
    Also returns max |out - bf16(oracle)| / RMS, for the record."""
    got = np.asarray(got, np.float64)
    rb = np.asarray(ref_bf16, np.float64)
    rf = np.asarray(ref_f64, np.float64)
    if rf.size == 0:
        return 0.0, 0.0, 0.0
    rms = max(float(np.sqrt(np.mean(rf ** 2))), 1e-300)
    rel = float(np.linalg.norm(got - rb) / max(np.linalg.norm(rb), 1e-300))
    comp = np.maximum(np.abs(got - rf) - bf16_half_ulp(rf), 0.0)
    mx = float(comp.max() / rms)
    mx_rounded = float(np.abs(got - rb).max() / rms)
    return rel, mx, mx_rounded


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """The bf16 spacing at |v| (normal range): 2^(floor(log2|v|) - 7)."""
    return 2.0 * bf16_half_ulp(v)


def ulp_stats(got: np.ndarray, ref_bf16: np.ndarray) -> tuple[float, float]:
    """(fraction of elements more than 1 bf16 ulp from the rounded oracle, largest distance in ulps)."""
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref_bf16, np.float64)) / bf16_ulp(ref_bf16)
    if d.size == 0:
        return 0.0, 0.0
    return float((d > 1.0).mean()), float(d.max())


def assert_output(got, ref: dict, what="", rows=None):
    rb, rf = ref["out"], ref["out_f64"]
    if rows is not None:
        rb, rf = rb[rows], rf[rows]
    rel, mx, mxr = output_bar(got, rb, rf)
    frac1, mxu = ulp_stats(got, rb)
    say(f"  {what}: rel L2 {rel:.3e} (vs bf16 oracle), per-element {mx:.3e} x RMS beyond bf16 rounding "
        f"({mxr:.3e} vs the rounded oracle); {frac1 * 100:.4f}% of elements > 1 bf16 ulp, max {mxu:.1f} ulp")
    assert rel <= 1e-3, f"{what}: relative L2 {rel:.3e} > 1e-3"
    assert mx <= 2e-2, f"{what}: per-element error {mx:.3e} x RMS > 2e-2"


def check_requant(got_q: np.ndarray, got_s: np.ndarray, gu: np.ndarray, absdot: np.ndarray, ue8m0: bool = False,
                  scale_rtol: float = 2e-6, max_flip: float = 2e-4) -> None:
    """The GPU's requantised h = silu(gate) * up (codes, 1x128 scales) against the oracle's.

    gu: the oracle's exact gate/up GEMM [M, 2W] (fp64); absdot: sum_k |a_k b_k| of each of its
    elements.  Both sides round h to fp32 and quantise it, but the GPU accumulates the 128-wide K
    blocks in fp32 (the oracle in fp64), so its gate and up values are off by at most
    gamma * absdot, gamma = 256 * 2^-24 (a 128-term fp32 sum inside each block, one scale product
    and one fused multiply-add per block, with room to spare), and silu, the product and the
    division by the scale add a few fp32 ulps of the quotient h/s.  A code can therefore differ
    from the oracle's only where the oracle's quotient lies within that error of an e4m3 rounding
    midpoint.  So: scales within scale_rtol (UE8M0: equal except where amax sits on a power-of-two
    boundary); codes equal except for at most max_flip of them; every code that differs is either
    the same value (+0 / -0) or the other neighbour of the oracle's quotient, whose distance to the
    midpoint between the two is within the error bound."""
    from oracle.ffn import silu
    W = gu.shape[1] // 2
    g, u = gu[:, :W], gu[:, W:]
    h = (silu(g) * u).astype(np.float32)
    want_q, want_s = quant.quant_1x128(h, ue8m0)
    if ue8m0:
        assert (got_s != want_s).mean() <= 1e-3
    else:
        assert np.allclose(got_s, want_s, rtol=scale_rtol, atol=0), \
            float(np.max(np.abs(got_s / want_s - 1.0)))
    same_s = np.repeat(got_s == want_s, 128, axis=1) if ue8m0 else np.ones(h.shape, bool)
    mism = (got_q != want_q) & same_s
    assert mism.mean() <= max_flip, mism.mean()
    if not mism.any():
        say(f"    requantised h: {h.size} codes, all equal to the oracle's")
        return
    r, c = np.nonzero(mism)
    s_ref = want_s[r, c // 128].astype(np.float64)
    quot = h[r, c].astype(np.float64) / s_ref
    gv, wv = e4m3.decode(got_q[r, c]), e4m3.decode(want_q[r, c])
    grid, _ = e4m3.finite_positive_grid()
    gi = np.searchsorted(grid, np.abs(gv))
    wi = np.searchsorted(grid, np.abs(wv))
    same_value = gv == wv                                                   # +0 and -0
    neighbours = (np.sign(gv) * np.sign(wv) >= 0) & (np.abs(gi - wi) == 1)
    neighbours |= (np.minimum(gi, wi) == 0) & (np.maximum(gi, wi) == 1)     # 0 and the smallest subnormal
    gamma = 256 * 2.0 ** -24
    zg = g[r, c]
    sg = 1.0 / (1.0 + np.exp(-zg))
    dsilu = sg * (1.0 + zg * (1.0 - sg))                                    # d silu / dz
    err_h = gamma * (np.abs(dsilu * u[r, c]) * absdot[r, c] + np.abs(silu(zg)) * absdot[r, W + c])
    bound = err_h / s_ref + 16 * 2.0 ** -24 * np.abs(quot) + 2.0 ** -149 / s_ref   # (subnormal h: one ulp)
    dist = np.abs(quot - (gv + wv) / 2.0)
    ok = same_value | (neighbours & (dist <= bound))
    say(f"    requantised h: {mism.sum()} of {h.size} codes differ ({mism.mean():.2e}): {same_value.sum()} +-0, "
        f"{(neighbours & ~same_value).sum()} neighbours; midpoint distance / error bound at most "
        f"{float(np.max(np.where(same_value, 0, dist / bound))):.3f}")
    for i in np.flatnonzero(~ok)[:10]:
        say(f"      row {r[i]} col {c[i]}: gpu {got_q[r[i], c[i]]:#04x} ({gv[i]}), oracle {want_q[r[i], c[i]]:#04x} "
            f"({wv[i]}), quotient {quot[i]!r}, bound {bound[i]:.3e}, h {h[r[i], c[i]]!r}")
    assert ok.all()


# The FP8 MFMA returns a 128-term block sum within this fraction of the block's sum of |products|
# (measured on MI355X: up to ~1.4e-5 on Gaussian-quantised tiles; the grouped-GEMM tests hold the
# FP8 path to it).
FP8_MFMA_REL = 5e-5
# The exact (bf16 MFMA) gate/up path: fp32 accumulation of 128-term blocks, one scale product and one
# fused multiply-add per block (see check_requant).
GAMMA_EXACT = 256 * 2.0 ** -24


def expert_error_bound(x_q, x_s, ex: ffn.QuantExpert, ue8m0: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """For rows (x_q, x_s) of one expert: (bound on |y_gpu - y_oracle| per output element, |y_oracle|).

    The GPU's h may differ from the oracle's only in codes whose quotient h/s lies within the
    exact path's error of an e4m3 rounding midpoint (see check_requant); each such code may move
    by its larger neighbour step.  The down GEMM (FP8 MFMA) adds FP8_MFMA_REL of sum_c |h_c w_c|.
    Built from the oracle's own steps (dequantisation, quantisation, silu) in fp64."""
    from oracle.ffn import silu
    A = quant.dequant_1x128(x_q, x_s)
    W13 = quant.dequant_128x128(ex.w13_q, ex.w13_s)
    gu = A @ W13.T
    ad = np.abs(A) @ np.abs(W13).T
    W = W13.shape[0] // 2
    del W13
    g, u = gu[:, :W], gu[:, W:]
    h = (silu(g) * u).astype(np.float32)
    h_q, h_s = quant.quant_1x128(h, ue8m0)
    srep = np.repeat(h_s.astype(np.float64), 128, axis=1)
    mag = np.abs(h.astype(np.float64)) / srep
    sg = 1.0 / (1.0 + np.exp(-g))
    err = GAMMA_EXACT * (np.abs(sg * (1.0 + g * (1.0 - sg)) * u) * ad[:, :W] + np.abs(silu(g)) * ad[:, W:]) / srep
    # a tile scale off by the amax element's relative error moves every quotient of the tile by as much
    amax_rel = np.repeat((err * (mag >= 447.0)).reshape(h.shape[0], -1, 128).max(-1) / 448.0, 128, axis=1)
    err = err + (16 * 2.0 ** -24 + amax_rel) * mag + 2.0 ** -149 / srep      # (h subnormal: one ulp of it)
    grid, _ = e4m3.finite_positive_grid()
    i = np.searchsorted(grid, np.abs(e4m3.decode(h_q)))
    up = np.where(i + 1 < grid.size, grid[np.minimum(i + 1, grid.size - 1)], np.inf)
    dn = np.where(i > 0, grid[np.maximum(i - 1, 0)], -np.inf)
    v = grid[i]
    near = (np.abs(mag - (v + up) / 2.0) <= err) | (np.abs(mag - (v + dn) / 2.0) <= err)
    step = np.maximum(np.where(np.isfinite(up), up - v, 0.0), np.where(np.isfinite(dn), v - dn, 0.0))
    flip = np.where(near, step, 0.0) * srep
    W2 = np.abs(quant.dequant_128x128(ex.w2_q, ex.w2_s))
    H = quant.dequant_1x128(h_q, h_s)
    y_abs = np.abs(H) @ W2.T
    return FP8_MFMA_REL * y_abs + flip @ W2.T, y_abs


def assert_within_error_bound(layer, x_vals, got, ref, rows=None, chunks=8) -> None:
    """Every output element against a per-element bound on the GPU's deviation from the oracle's fp64
    output: half a bf16 ulp of the result (output rounding), the fp32 combine's rounding
    ((k + 2) 2^-24 sum |terms|), |w_gpu - w_oracle| |y| for each routed term, and each expert's
    expert_error_bound weighted by its routing weight (the shared expert by 1)."""
    s = layer.s
    rows = np.arange(x_vals.shape[0]) if rows is None else np.flatnonzero(rows)
    xr = x_vals[rows] if layer.norm is None else norm.rmsnorm(x_vals[rows], *layer.norm)
    x_q, x_s = quant.quant_1x128(xr, layer.ue8m0)
    T = rows.size
    if s.n_experts:
        idx, w = ref["topk_idx"][rows], ref["topk_w"][rows].astype(np.float64)
        dw = np.abs(got["topk_w"][rows].astype(np.float64) - w) if "topk_w" in got else np.zeros_like(w)
        jobs = [(e, np.flatnonzero((idx == e).any(1))) for e in np.unique(idx)]
    else:
        jobs = []
    if s.n_shared:
        jobs.append((s.n_experts, np.arange(T)))

    def one(job):
        e, r = job
        return e, r, expert_error_bound(x_q[r], x_s[r], layer.expert(int(e)), layer.ue8m0)
    bound = np.zeros((T, s.hidden))
    terms = np.zeros((T, s.hidden))
    with ThreadPoolExecutor(chunks) as ex:
        for e, r, (b, y_abs) in ex.map(one, jobs):
            if e == s.n_experts and s.n_shared:
                wt, dwt = np.ones(r.size), np.zeros(r.size)
            else:
                j = np.argmax(idx[r] == e, axis=1)
                wt, dwt = w[r, j], dw[r, j]
            bound[r] += wt[:, None] * b + dwt[:, None] * y_abs
            terms[r] += wt[:, None] * y_abs
    out = np.asarray(got["out"][rows], np.float64)
    k = s.top_k if s.n_experts else 0
    bound += bf16_half_ulp(out) + (k + 2) * 2.0 ** -24 * terms
    dev = np.abs(out - ref["out_f64"][rows])
    ratio = dev / bound
    say(f"    per-element bound: deviation / bound at most {ratio.max():.3f} (median {np.median(ratio):.3f}) "
        f"over {dev.size} elements")
    assert np.all(dev <= bound), f"{int((dev > bound).sum())} elements outside the bound"


class Layer:
    """One layer's weights on both sides.  Small shapes draw numpy weights
    (synth.gen_expert_w); V3 shapes draw them on the device with torch.  The
    GPU side quantises with fp8_quant_128x128 (then packs the codes into the
    GEMMs' fragment order), the oracle with its own quant_128x128, from the
    same fp32 values."""

    def __init__(self, shape: synth.MoeShape, device_draw: bool | None = None, bias: np.ndarray | None = None,
                 ue8m0: bool = False, norm_gamma: np.ndarray | None = None, norm_eps: float = 1e-6):
        """ue8m0: power-of-two scales everywhere (weights, x, h); norm_gamma: bf16 bits [hidden] of
        an RMSNorm applied to x first."""
        import sparse_moe_ffn_sigmoid_amd as moe
        self.s = shape
        self.ue8m0 = ue8m0
        self.norm = None if norm_gamma is None else (synth.bf16_bits_to_f32(norm_gamma), norm_eps)
        self.device_draw = shape.hidden >= 4096 if device_draw is None else device_draw
        self.cfg = moe.MoeConfig.of(shape, ue8m0=ue8m0, norm_eps=norm_eps)
        E = shape.n_experts
        self._np_cache: dict[int, tuple[np.ndarray, np.ndarray]] = {}
        self._oracle: dict[int, ffn.QuantExpert] = {}
        w13q, w13s, w2q, w2s = [], [], [], []
        for e in range(E + (1 if shape.n_shared else 0)):
            w13, w2 = self._fp32_dev(e)
            a, b = moe.quantize_pack_128x128(w13, ue8m0=ue8m0)
            c, d = moe.quantize_pack_128x128(w2, ue8m0=ue8m0)
            del w13, w2
            w13q.append(a); w13s.append(b); w2q.append(c); w2s.append(d)
        kw = {}
        if E:
            kw = dict(w13_q=torch.stack(w13q[:E]), w13_s=torch.stack(w13s[:E]), w2_q=torch.stack(w2q[:E]),
                      w2_s=torch.stack(w2s[:E]))
            del w13q[:E], w13s[:E], w2q[:E], w2s[:E]
        if shape.n_shared:
            kw.update(sh_w13_q=w13q[-1], sh_w13_s=w13s[-1], sh_w2_q=w2q[-1], sh_w2_s=w2s[-1])
        if norm_gamma is not None:
            kw["norm_w"] = to_dev(norm_gamma)
        self.wr_bits = synth.gen_router_w(shape) if E else None
        self.bias = bias
        if E:
            kw["w_router"] = to_dev(self.wr_bits)
            if bias is not None:
                kw["bias"] = to_dev(bias.astype(np.float32))
        self.weights = moe.MoeWeights(**kw)
        torch.cuda.synchronize()

    def _fp32_host(self, e: int) -> tuple[np.ndarray, np.ndarray]:
        if self.device_draw:
            w13 = synth.torch_expert_weight(self.s, e, "w13", DEV).cpu().numpy()
            w2 = synth.torch_expert_weight(self.s, e, "w2", DEV).cpu().numpy()
            return w13, w2
        return synth.gen_expert_w(self.s, e)

    def _fp32_dev(self, e: int):
        if self.device_draw:
            return synth.torch_expert_weight(self.s, e, "w13", DEV), synth.torch_expert_weight(self.s, e, "w2", DEV)
        w13, w2 = synth.gen_expert_w(self.s, e)
        return to_dev(w13), to_dev(w2)

    def oracle_experts(self, ids) -> None:
        """Quantise the given experts on the oracle side (threads: numpy releases the GIL)."""
        todo = sorted(set(int(i) for i in ids) - set(self._oracle))
        host = {e: self._fp32_host(e) for e in todo}           # device draws happen on this thread
        with ThreadPoolExecutor(16) as ex:
            res = ex.map(lambda e: (e, ffn.quantize_expert(*host[e], ue8m0=self.ue8m0)), todo)
            for e, q in res:
                self._oracle[e] = q
                del host[e]

    def expert(self, e: int) -> ffn.QuantExpert:
        if e not in self._oracle:
            self.oracle_experts([e])
        return self._oracle[e]

    def oracle_forward(self, x_vals: np.ndarray, scores: np.ndarray | None = None, chunks: int = 1) -> dict:
        """The oracle layer on x_vals (bf16 values).  With chunks > 1 the tokens (independent given
        their routing) are split into that many groups run in parallel threads, after every expert
        they need has been quantised; the routing, output and score arrays are joined."""
        s = self.s
        if s.n_experts:
            if scores is None:
                xr = x_vals if self.norm is None else norm.rmsnorm(x_vals, *self.norm)
                scores = route.sigmoid_scores(route.router_logits(xr, synth.bf16_bits_to_f32(self.wr_bits)))
            idx, _ = route.select(scores, self.bias, s.n_group, s.topk_group, s.top_k, s.routed_scale)
            self.oracle_experts(list(np.unique(idx)) + [s.n_experts] if s.n_shared else list(np.unique(idx)))
        else:
            self.oracle_experts([0])

        def run(rows):
            return ffn.moe_ffn(x_vals[rows], s.n_experts, s.top_k, s.n_group, s.topk_group, self.expert,
                               scores=None if scores is None else scores[rows], bias=self.bias,
                               n_shared=s.n_shared, routed_scale=s.routed_scale, ue8m0=self.ue8m0, norm=self.norm)
        if chunks <= 1 or x_vals.shape[0] < 2:
            return run(np.arange(x_vals.shape[0]))
        parts = [p for p in np.array_split(np.arange(x_vals.shape[0]), chunks) if p.size]
        with ThreadPoolExecutor(len(parts)) as ex:
            res = list(ex.map(run, parts))
        keys = ("out", "out_f64") + (("scores", "topk_idx", "topk_w") if s.n_experts else ())
        return {k: np.concatenate([r[k] for r in res]) for k in keys}


def run_layer(layer, xb, scores=None, deterministic=False):
    """moe_ffn_forward on bf16 bits xb [T, hidden]; returns the output values and the routing."""
    import sparse_moe_ffn_sigmoid_amd as moe
    s = layer.s
    T = xb.shape[0]
    x = to_dev(xb)
    if s.n_experts:
        sc = to_dev(scores) if scores is not None else torch.empty((T, s.n_experts), dtype=torch.float32, device=DEV)
        ti = torch.empty((T, s.top_k), dtype=torch.int32, device=DEV)
        tw = torch.empty((T, s.top_k), dtype=torch.float32, device=DEV)
    else:
        sc = ti = tw = None
    out = moe.moe_ffn_forward(x, layer.cfg, layer.weights, scores=sc, scores_given=scores is not None, topk_idx=ti,
                              topk_w=tw, deterministic=deterministic)
    torch.cuda.synchronize()
    r = {"out": bf16_np(out)}
    if s.n_experts:
        r.update(scores=sc.cpu().numpy(), topk_idx=ti.cpu().numpy(), topk_w=tw.cpu().numpy())
    return r


def compare_router_run(layer, xb, got, tokens=None, chunks=1):
    """Router on the device: compare tokens whose expert sets agree; the rest must be near-ties."""
    s = layer.s
    xv = synth.bf16_bits_to_f32(xb)
    tok = np.arange(xb.shape[0]) if tokens is None else np.asarray(tokens)
    ref = layer.oracle_forward(xv[tok], chunks=chunks)
    if not s.n_experts:
        assert_output(got["out"][tok], ref, f"{s.name} dense")
        assert_within_error_bound(layer, xv[tok], {"out": got["out"][tok]}, ref, chunks=max(chunks, 4))
        return
    gi = np.sort(got["topk_idx"][tok], 1)
    wi = np.sort(ref["topk_idx"], 1)
    same = (gi == wi).all(1)
    say(f"  {s.name}: expert sets equal on {same.mean() * 100:.2f}% of {len(tok)} tokens")
    assert same.mean() >= 0.97
    b = route.biased(ref["scores"], layer.bias)
    for i in np.flatnonzero(~same):
        assert abs(float(b[i, gi[i]].astype(np.float64).sum() - b[i, wi[i]].astype(np.float64).sum())) < 1e-4
    assert_output(got["out"][tok][same], ref, f"{s.name} (router on device)", rows=same)
    # the GPU's slots in the oracle's slot order (equal sets; the slot order follows the scores)
    sub = {"out": got["out"][tok]}
    if s.n_experts:
        order = np.argsort(got["topk_idx"][tok], 1)
        back = np.argsort(np.argsort(ref["topk_idx"], 1), 1)
        sub["topk_w"] = np.take_along_axis(np.take_along_axis(got["topk_w"][tok], order, 1), back, 1)
    assert_within_error_bound(layer, xv[tok], sub, ref, rows=same, chunks=max(chunks, 4))


# ---- sampled tokens at V3 size ----

def tile_edges(offsets, bm=128):
    """Sorted positions of the first and the last row of the m tiles of every group (of its first
    two and last two tiles when it has more): a group of n rows has ceil(n / bm) tiles over which
    its rows are split evenly in whole 16-row blocks (the tile kernel's split), keyed by the
    group's tile row counts (its tile shape)."""
    shapes = {}
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        n = hi - lo
        if n == 0:
            continue
        c = -(-n // bm)
        rb = ((-(-n // c)) + 15) // 16 * 16 if c > 1 else bm
        edges, rows = [], []
        for j in range(c):
            a, b = lo + j * rb, min(lo + (j + 1) * rb, hi)
            if j < 2 or j >= c - 2:
                edges += [a, b - 1]
            rows.append(b - a)
        shapes.setdefault(tuple(rows), []).append(edges)
    return shapes


def pick_tokens(idx, E, n_min, seed, max_shapes=24):
    """Tokens whose assignments sit at the first and last rows of the m tiles of one group per tile
    shape (up to max_shapes shapes, spread over the smallest to the largest), topped up with random
    tokens to at least n_min."""
    T, k = idx.shape
    off, sa, _ = permute.permute(idx, E)
    shapes = tile_edges(off)
    keys = sorted(shapes, key=lambda t: (len(t), t))
    if len(keys) > max_shapes:
        keys = [keys[i] for i in np.linspace(0, len(keys) - 1, max_shapes).round().astype(int)]
    toks = set()
    for key in keys:
        for p in shapes[key][0]:
            toks.add(int(sa[p]) // k)
    r = np.random.default_rng(seed)
    while len(toks) < n_min:
        toks.add(int(r.integers(T)))
    say(f"  {len(toks)} tokens: tile edges of {len(keys)} of {len(shapes)} tile shapes "
        f"(e.g. {keys[0]}, {keys[len(keys) // 2]}, {keys[-1]}) + random")
    return sorted(toks)
