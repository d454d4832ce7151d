"""Shared helpers of the GPU parity tests: building layers on the device and
on the oracle side from the same fp32 weights, and the comparison bars."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import synth
from oracle import ffn, norm, route

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


def assert_output(got, ref: dict, what="", rows=None):
    rb, rf = ref["out"], ref["out_f64"]
    if rows is not None:
        rb, rf = rb[rows], rf[rows]
    rel, mx, mxr = output_bar(got, rb, rf)
    say(f"  {what}: rel L2 {rel:.3e} (vs bf16 oracle), per-element {mx:.3e} x RMS beyond bf16 rounding "
        f"({mxr:.3e} vs the rounded oracle)")
    assert rel <= 1e-3, f"{what}: relative L2 {rel:.3e} > 1e-3"
    assert mx <= 2e-2, f"{what}: per-element error {mx:.3e} x RMS > 2e-2"


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

    def oracle_forward(self, x_vals: np.ndarray, scores: np.ndarray | None = None) -> dict:
        s = self.s
        if s.n_experts:
            if scores is None:
                xr = x_vals if self.norm is None else norm.rmsnorm(x_vals, *self.norm)
                scores = route.sigmoid_scores(route.router_logits(xr, synth.bf16_bits_to_f32(self.wr_bits)))
            idx, _ = route.select(scores, self.bias, s.n_group, s.topk_group, s.top_k, s.routed_scale)
            self.oracle_experts(list(np.unique(idx)) + [s.n_experts] if s.n_shared else list(np.unique(idx)))
        else:
            self.oracle_experts([0])
        return ffn.moe_ffn(x_vals, s.n_experts, s.top_k, s.n_group, s.topk_group, self.expert, scores=scores,
                           bias=self.bias, n_shared=s.n_shared, routed_scale=s.routed_scale, ue8m0=self.ue8m0,
                           norm=self.norm)


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


def compare_router_run(layer, xb, got, tokens=None):
    """Router on the device: compare tokens whose expert sets agree; the rest must be near-ties."""
    s = layer.s
    xv = synth.bf16_bits_to_f32(xb)
    tok = np.arange(xb.shape[0]) if tokens is None else np.asarray(tokens)
    ref = layer.oracle_forward(xv[tok])
    if not s.n_experts:
        assert_output(got["out"][tok], ref, f"{s.name} dense")
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
