"""Pins for the oracle's full layer: brute-force dense evaluation of every
expert on every token masked by the routing, closed forms of SwiGLU and the
bf16 rounding, the pages' shape constants, and the dense-layer special case."""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import synth
from oracle import ffn, route


@pytest.fixture(scope="module")
def tiny():
    s = synth.TINY
    x = synth.bf16_bits_to_f32(synth.gen_x(s))
    wr = synth.bf16_bits_to_f32(synth.gen_router_w(s))
    experts = [ffn.quantize_expert(*synth.gen_expert_w(s, e)) for e in range(s.n_experts + 1)]
    return s, x, wr, experts


def _dense_masked(s, x, experts, idx, w, ue8m0=False):
    """Every expert on every token; each output weighted by the token's routing
    weight for that expert, or 0 when the expert was not chosen."""
    from oracle import quant
    x_q, x_s = quant.quant_1x128(x, ue8m0)
    mask = np.zeros((x.shape[0], s.n_experts))
    for t in range(x.shape[0]):
        for j in range(s.top_k):
            mask[t, idx[t, j]] = float(w[t, j])
    out = np.zeros(x.shape, np.float64)
    for e in range(s.n_experts):
        y = ffn.expert_forward(x_q, x_s, experts[e], ue8m0)["y"]   # per-row quantisation: tokens are independent
        out += mask[:, e:e + 1] * y
    out += ffn.expert_forward(x_q, x_s, experts[s.n_experts], ue8m0)["y"]
    return out


@pytest.mark.parametrize("bias_scale", [0.0, 0.5])
def test_tiny_layer_equals_dense_masked_evaluation(tiny, bias_scale):
    s, x, wr, experts = tiny
    bias = synth.gen_bias(s.n_experts, scale=bias_scale) if bias_scale else None
    r = ffn.moe_ffn(x, s.n_experts, s.top_k, s.n_group, s.topk_group, lambda e: experts[e], w_router=wr, bias=bias)
    want = _dense_masked(s, x, experts, r["topk_idx"], r["topk_w"])
    assert np.allclose(r["out_f64"], want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["out"], ffn.round_bf16(want))


def test_ue8m0_layer_with_prenorm_equals_dense_masked_evaluation(tiny):
    """The power-of-two-scale variant with the RMSNorm in front: same brute-force pin, on the
    normalised rows (the router sees them too), with every quantisation power-of-two."""
    from oracle import norm
    s, x, wr, _ = tiny
    experts = [ffn.quantize_expert(*synth.gen_expert_w(s, e), ue8m0=True) for e in range(s.n_experts + 1)]
    gamma = norm.round_bf16(np.random.default_rng(3).uniform(0.5, 1.5, s.hidden).astype(np.float32))
    r = ffn.moe_ffn(x, s.n_experts, s.top_k, s.n_group, s.topk_group, lambda e: experts[e], w_router=wr,
                    ue8m0=True, norm=(gamma, 1e-6))
    xn = norm.rmsnorm(x, gamma, 1e-6)
    assert np.array_equal(r["x_norm"], xn)
    sc = route.sigmoid_scores(route.router_logits(xn, wr))
    idx, w = route.select(sc, None, s.n_group, s.topk_group, s.top_k)
    assert np.array_equal(r["topk_idx"], idx)
    assert np.all(np.frexp(r["x_s"])[0] == 0.5) and np.all(np.frexp(r["h_s"][r["h_s"] > 0])[0] == 0.5)
    want = _dense_masked(s, xn, experts, idx, w, ue8m0=True)
    assert np.allclose(r["out_f64"], want, rtol=1e-12, atol=1e-12)


def test_given_scores_replace_the_router(tiny):
    s, x, wr, experts = tiny
    sc = synth.gen_scores(s.tokens, s.n_experts, cfg_id=9)
    r = ffn.moe_ffn(x, s.n_experts, s.top_k, s.n_group, s.topk_group, lambda e: experts[e], scores=sc)
    idx, w = route.select(sc, None, s.n_group, s.topk_group, s.top_k)
    assert np.array_equal(r["topk_idx"], idx)
    want = _dense_masked(s, x, experts, idx, w)
    assert np.allclose(r["out_f64"], want, rtol=1e-12, atol=1e-12)


def test_token_subset_independence(tiny):
    s, x, wr, experts = tiny
    full = ffn.moe_ffn(x, s.n_experts, s.top_k, s.n_group, s.topk_group, lambda e: experts[e], w_router=wr)
    sub = [3, 17, 40]
    part = ffn.moe_ffn(x[sub], s.n_experts, s.top_k, s.n_group, s.topk_group, lambda e: experts[e], w_router=wr)
    assert np.array_equal(part["out"], full["out"][sub])


def test_dense_layer_special_case():
    s = synth.MoeShape("dense_small", 2, 8, 256, 0, 0, 0, 1, 384, 1, 1)
    x = synth.bf16_bits_to_f32(synth.gen_x(s))
    ex = ffn.quantize_expert(*synth.gen_expert_w(s, 0))
    r = ffn.moe_ffn(x, 0, 0, 1, 1, lambda e: ex)
    from oracle import quant
    x_q, x_s = quant.quant_1x128(x)
    assert np.array_equal(r["out"], ffn.round_bf16(ffn.expert_forward(x_q, x_s, ex)["y"]))


def test_swiglu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 2.5])
    assert ffn.silu(z)[0] == 0.0
    assert ffn.silu(z)[1] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert ffn.silu(z)[3] == pytest.approx(40.0, rel=1e-15)
    assert abs(ffn.silu(z)[4]) < 1e-15
    r = np.random.default_rng(0).standard_normal(1000) * 4
    assert np.allclose(ffn.silu(r), r * expit(r), rtol=1e-14, atol=1e-300)
    assert np.allclose(ffn.silu(r) - ffn.silu(-r), r, rtol=1e-13, atol=1e-13)   # silu(z) - silu(-z) = z


def test_round_bf16_matches_library_cast():
    r = np.random.default_rng(1)
    v = (r.standard_normal(200000) * np.exp2(r.integers(-20, 20, 200000))).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ffn.round_bf16(v.astype(np.float64)), lib)
    # fp64 inputs just above a bf16 midpoint round up (no double rounding through fp32)
    mid = 1.0 + 2.0 ** -8
    assert ffn.round_bf16(np.array([mid]))[0] == 1.0
    assert ffn.round_bf16(np.array([mid + 2.0 ** -40]))[0] == np.float32(1.0 + 2.0 ** -7)


def test_page_shape_constants():
    s = synth.V3_PREFILL
    # DeepSeek-R1 card, "Every architecture field"
    assert (s.hidden, s.n_experts, s.top_k, s.inter, s.n_shared, s.inter_shared) == (7168, 256, 8, 2048, 1, 2048)
    assert synth.DENSE_FFN.inter_shared == 18432
    # "9 out of 257 (1 shared)" active experts (onlylabs, table in "More Aggressive Mixture-of-Expert")
    assert s.top_k + s.n_shared == 9 and s.n_experts + s.n_shared == 257
    # a gated expert holds three matrices: 3 * 7168 * 2048 codes (the page's 29.36M counts two)
    assert 3 * 7168 * 2048 == 44_040_192 and 2 * 7168 * 2048 == 29_360_128
    assert s.expert_bytes(2048) == 44_040_192 + 4 * (32 * 56 + 56 * 16)
    # FLOPs of one MoE layer per token: 9 experts x 3 matrices x 2 FLOP per MAC
    assert synth.with_tokens(s, 1).fp8_flops() == 9 * 6 * 7168 * 2048


def test_fp8_fidelity_informational(tiny):
    """parity unpinned: the pages' statement of FP8 accuracy against bf16 is cut
    off, so this only reports the layer's error against unquantised fp64 math."""
    s, x, wr, experts = tiny
    r = ffn.moe_ffn(x, s.n_experts, s.top_k, s.n_group, s.topk_group, lambda e: experts[e], w_router=wr)
    ref = np.zeros_like(r["out_f64"])
    for t in range(s.tokens):
        for e, wt in list(zip(r["topk_idx"][t], r["topk_w"][t])) + [(s.n_experts, 1.0)]:
            w13, w2 = synth.gen_expert_w(s, int(e))
            gu = x[t].astype(np.float64) @ w13.astype(np.float64).T
            h = ffn.silu(gu[:s.inter]) * gu[s.inter:]
            ref[t] += float(wt) * (h @ w2.astype(np.float64).T)
    rel = np.linalg.norm(r["out_f64"] - ref) / np.linalg.norm(ref)
    print(f"FP8 layer vs unquantised fp64: relative L2 {rel:.3e}")
    assert rel < 0.2


def test_expert_forward_hand_computed_single_token():
    """One token through one gated expert, worked out by hand on small-integer codes: two 128-wide
    K blocks with different activation scales, a weight block with scale 1/2, the gate rows before
    the up rows, silu(z) = z / (1 + e^-z), h rounded to fp32 and requantised 1x128, then the down
    projection.  The expected numbers are written out below with plain Python arithmetic (no
    matmul, no oracle helper), so a dropped term, a swapped gate/up half, a wrong scale or a
    transposed operand anywhere in the chain shows up."""
    from oracle.ffn import QuantExpert
    f32 = np.float32
    d, W = 256, 128
    # x: tile 0 has amax 448 (s = 1), tile 1 amax 7 (s = 7/448 = 1/64): codes are the values / s
    E4 = {448.0: 0x7E, 2.0: 0x40, -3.0: 0xC4, 1.0: 0x38, 32.0: 0x60}   # e4m3 bytes of these values
    a_q = np.zeros((1, d), np.uint8)
    a_q[0, 0], a_q[0, 1], a_q[0, 2], a_q[0, 3] = E4[448.0], E4[2.0], E4[-3.0], E4[1.0]
    a_q[0, 128], a_q[0, 129] = E4[448.0], E4[32.0]                    # x = 7 and 0.5 at scale 1/64
    a_s = np.array([[1.0, 1.0 / 64]], np.float32)
    # W13 [2W, d]: gate block (rows 0..127) scale 1, up block (rows 128..255) scale 1/2
    w13 = np.zeros((2 * W, d), np.uint8)
    w13[0, 1], w13[0, 3], w13[0, 128], w13[0, 129] = E4[1.0], E4[1.0], E4[1.0], E4[2.0]   # g0 = 2+1+7+2*0.5 = 11
    w13[1, 2] = E4[1.0]                                                                 # g1 = -3
    w13[2, 0] = E4[1.0]                                                                 # g2 = 448
    w13[127, 127] = w13[255, 255] = E4[448.0]                     # block amax (x is 0 there)
    w13[W + 0, 1] = E4[2.0]                                       # u0 = 2 * (2 * 1/2) = 2
    w13[W + 1, 3], w13[W + 1, 129] = E4[2.0], E4[32.0]            # u1 = 1*1 + 0.5*16 = 9
    w13_s = np.array([[1.0, 1.0], [0.5, 0.5]], np.float32)
    # W2 [d, W]: one block per 128 output rows; block 0 scale 1, block 1 scale 2
    w2 = np.zeros((d, W), np.uint8)
    w2[0, 0], w2[0, 1] = E4[1.0], E4[2.0]                         # y0 = h0 + 2 h1
    w2[1, 1] = E4[-3.0]                                           # y1 = -3 h1
    w2[128, 0] = E4[32.0]                                         # y128 = 2 * 32 h0
    w2[127, 127] = w2[255, 127] = E4[448.0]
    w2_s = np.array([[1.0], [2.0]], np.float32)
    r = ffn.expert_forward(a_q, a_s, QuantExpert(w13, w13_s, w2, w2_s))

    g0, g1, u0, u1 = 11.0, -3.0, 2.0, 9.0                          # g2 = 448 has u2 = 0
    h0 = f32(g0 / (1.0 + math.exp(-g0)) * u0)
    h1 = f32(g1 / (1.0 + math.exp(-g1)) * u1)
    assert r["h"][0, 0] == h0 and r["h"][0, 1] == h1 and not r["h"][0, 2:].any()
    s = f32(h0 / f32(448.0))                                      # amax is h0
    assert r["h_s"][0, 0] == s
    # h0 / s lands on 448 (code 0x7E); h1 / s = -1.2805 / 0.049106 = -26.076, whose nearest e4m3
    # values are -26 (1.625 x 2^4, code 0xDD) and -28: -26
    q1 = f32(h1 / s)
    assert -26.25 < q1 < -25.9 and r["h_q"][0, 0] == 0x7E and r["h_q"][0, 1] == 0xDD and not r["h_q"][0, 2:].any()
    v0, v1 = 448.0 * float(s), -26.0 * float(s)                    # dequantised h
    want = np.zeros(d)
    want[0], want[1], want[128] = v0 + 2.0 * v1, -3.0 * v1, 2.0 * 32.0 * v0
    assert np.array_equal(r["y"][0], want)
