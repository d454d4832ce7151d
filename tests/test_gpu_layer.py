"""End-to-end GPU parity of moe_ffn_forward against the oracle.

Small shapes are compared on every token; V3 shapes (decode T=64, prefill
T=4096, load-skewed prefill T=16384, dense FFN T=4096) run in the launch
configuration the benchmark times and are compared on sampled tokens (tokens
are independent given their routing).  The bar: bf16 output within relative
L2 1e-3 and per-element 2e-2 x RMS of the bf16-rounded oracle; routing
bit-exact when both sides route the same given scores; with the router on
the device, expert sets must agree except within rounding of a tie."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import quant, route

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_ffn_sigmoid_amd as moe
    from gpu_util import DEV, Layer, assert_output, assert_within_error_bound, bf16_np, pick_tokens, say, to_dev
    from gpu_util import compare_router_run as _compare_router_run
    from gpu_util import run_layer as _run

MID_A = synth.MoeShape("mid_a", 10, 200, 512, 256, 32, 4, 1, 256, 4, 2)
MID_B = synth.MoeShape("mid_b", 11, 1024, 384, 256, 16, 4, 1, 384, 4, 4)
MID_LARGE = synth.MoeShape("mid_large", 12, 2304, 256, 128, 16, 4, 1, 128, 4, 2)   # 9216 assignments
NO_SHARED = synth.MoeShape("no_shared", 13, 100, 256, 128, 16, 2, 0, 0, 4, 2)
DENSE_SMALL = synth.MoeShape("dense_small", 14, 300, 512, 0, 0, 0, 1, 640, 1, 1)
MID_C = synth.MoeShape("mid_c", 15, 384, 256, 128, 64, 6, 1, 256, 8, 4)          # 36 rows per expert: 64-row tiles
MID_D = synth.MoeShape("mid_d", 17, 256, 512, 256, 32, 2, 1, 256, 4, 2)          # 16 rows per expert: 32-row streaming tiles


@pytest.fixture(scope="module")
def tiny():
    return Layer(synth.TINY)


def test_tiny_router_on_device(tiny):
    say("forward tiny, router on device")
    xb = synth.gen_x(synth.TINY)
    _compare_router_run(tiny, xb, _run(tiny, xb))


def test_tiny_scores_given_bit_exact_routing(tiny):
    say("forward tiny, scores given")
    s = synth.TINY
    xb = synth.gen_x(s)
    sc = synth.gen_scores(s.tokens, s.n_experts, cfg_id=21)
    got = _run(tiny, xb, scores=sc)
    ref = tiny.oracle_forward(synth.bf16_bits_to_f32(xb), scores=sc)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    assert np.array_equal(got["topk_w"].view(np.uint32), ref["topk_w"].view(np.uint32))
    assert_output(got["out"], ref, "tiny scores given")
    assert_within_error_bound(tiny, synth.bf16_bits_to_f32(xb), got, ref)


def test_tiny_deterministic_repeat(tiny):
    say("forward tiny, deterministic repeat")
    xb = synth.gen_x(synth.TINY)
    a = _run(tiny, xb, deterministic=True)
    b = _run(tiny, xb, deterministic=True)
    assert np.array_equal(a["out"], b["out"])


def test_forward_stages_events_optional(tiny):
    """moe_ffn_forward_stages with every stage event, with NULL entries (not recorded) and with
    none gives moe_ffn_forward's output bit for bit; the recorded events come in stage order."""
    import ctypes
    from sparse_moe_ffn_sigmoid_amd import _lib
    say("forward_stages with all, some and no stage events")
    xb = synth.gen_x(synth.TINY)
    ref = _run(tiny, xb)["out"]
    x = to_dev(xb)
    T = x.shape[0]
    ws = moe.alloc_workspace(T, tiny.cfg, DEV)
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    c, wc = tiny.cfg.c(), tiny.weights.c()
    n_ev = _lib.MOE_FWD_STAGE_EVENTS
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in evs:
        e.record()                                # creates the event; the library records it again
    torch.cuda.synchronize()
    for keep in (tuple(range(n_ev)), (2, 3), ()):
        out = torch.empty_like(x)
        arr = (ctypes.c_void_p * n_ev)(*[evs[j].cuda_event if j in keep else None for j in range(n_ev)])
        st = lib.moe_ffn_forward_stages(ctypes.c_void_p(x.data_ptr()), T, ctypes.byref(c), ctypes.byref(wc),
                                        ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(out.data_ptr()),
                                        None, None, None, 0, arr, n_ev, stream)
        assert st == 0, lib.moe_last_error().decode()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_np(out), ref)
        for a, b in zip(keep, keep[1:]):
            assert evs[a].elapsed_time(evs[b]) >= 0.0


def test_large_batch_is_bit_reproducible():
    """The combine is slot-ordered at every batch size: repeated runs agree bit for bit."""
    say("forward mid_large twice: bit-reproducible")
    layer = Layer(MID_LARGE)
    xb = synth.gen_x(MID_LARGE)
    a, b = _run(layer, xb), _run(layer, xb)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["topk_idx"], b["topk_idx"])


@pytest.mark.parametrize("shape", [MID_A, MID_B, MID_C, MID_D, MID_LARGE, NO_SHARED, DENSE_SMALL])
def test_mid_shapes(shape):
    say(f"forward {shape.name} T={shape.tokens} d={shape.hidden} E={shape.n_experts} k={shape.top_k}")
    layer = Layer(shape)
    xb = synth.gen_x(shape)
    _compare_router_run(layer, xb, _run(layer, xb))
    if shape.n_experts:
        sc = synth.gen_scores(shape.tokens, shape.n_experts, cfg_id=shape.cfg_id)
        got = _run(layer, xb, scores=sc, deterministic=True)
        ref = layer.oracle_forward(synth.bf16_bits_to_f32(xb), scores=sc)
        assert np.array_equal(got["topk_idx"], ref["topk_idx"])
        assert_output(got["out"], ref, f"{shape.name} scores given, deterministic")
        assert_within_error_bound(layer, synth.bf16_bits_to_f32(xb), got, ref)


def test_ragged_tails_empty_experts_and_hot_expert():
    shape = dataclasses.replace(MID_A, name="mid_skew", tokens=333)
    say("forward mid_skew: empty experts, one hot expert, ragged tails")
    bias = np.zeros(shape.n_experts, np.float32)
    bias[[3, 9, 17]] = -10.0                       # never chosen
    bias[5] = 2.0                                  # chosen by every token whose group survives
    layer = Layer(shape, bias=bias)
    xb = synth.gen_x(shape)
    got = _run(layer, xb)
    assert not np.isin(got["topk_idx"], [3, 9, 17]).any()
    _compare_router_run(layer, xb, got)


def test_single_token_and_empty_batch(tiny):
    say("forward T=1 and T=0")
    xb = synth.gen_x(synth.TINY)[:1]
    _compare_router_run(tiny, xb, _run(tiny, xb))
    out = moe.moe_ffn_forward(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), tiny.cfg, tiny.weights,
                              workspace=torch.empty(256, dtype=torch.uint8, device=DEV))
    assert out.shape == (0, 256)


ROUTER_SPLIT = synth.MoeShape("router_split", 21, 512, 4096, 128, 16, 4, 1, 128, 4, 2)


@pytest.mark.parametrize("T,ue8m0", [(1, False), (64, False), (512, False), (64, True)])
def test_forward_router_scores_split_over_k(T, ue8m0):
    """Batches of up to 512 tokens with a hidden dimension of 4096 or more: the forward's router
    splits the hidden dimension over four workgroups and adds their partial logits in a fixed
    order; the layer input's 1x128 quantisation runs in the same launch as that sum (fp32 or
    power-of-two scales).  Its scores against the oracle's (the bound of the single-pass router),
    the same routing as the oracle's except at near-ties, and the layer output."""
    s = dataclasses.replace(ROUTER_SPLIT, tokens=T)
    say(f"forward router with the hidden dimension split: T={T}, hidden {s.hidden}, ue8m0 {ue8m0}")
    layer = Layer(s, ue8m0=ue8m0)
    xb = synth.gen_x(s)
    got = _run(layer, xb)
    want = route.sigmoid_scores(route.router_logits(synth.bf16_bits_to_f32(xb),
                                                    synth.bf16_bits_to_f32(synth.gen_router_w(s))))
    assert np.abs(got["scores"] - want).max() <= 2e-5
    _compare_router_run(layer, xb, got)
    # x's codes and scales, read from the forward's workspace (after the bf16 normalised-rows
    # region, 256-byte aligned: codes [T][hidden], then scales [T][hidden / 128]), bit-exact
    # against the oracle's quantiser; the workspace is filled with 0xA5 first
    ws = moe.alloc_workspace(T, layer.cfg, DEV).fill_(0xA5)
    moe.moe_ffn_forward(to_dev(xb), layer.cfg, layer.weights, workspace=ws)
    torch.cuda.synchronize()
    d = s.hidden
    align = lambda v: (v + 255) // 256 * 256
    o_q = align(T * d * 2)
    o_s = o_q + align(T * d)
    wsn = ws.cpu().numpy()
    want_q, want_s = quant.quant_1x128(synth.bf16_bits_to_f32(xb), ue8m0)
    assert np.array_equal(wsn[o_q:o_q + T * d].reshape(T, d), want_q)
    assert np.array_equal(wsn[o_s:o_s + T * (d // 128) * 4].view(np.float32).reshape(T, d // 128).view(np.uint32),
                          np.asarray(want_s, np.float32).view(np.uint32))


ROUTER_LDS = synth.MoeShape("router_lds", 22, 1100, 1152, 128, 256, 8, 1, 128, 8, 4)


@pytest.mark.parametrize("T,hidden,E,whole", [
    (700, 1152, 256, True),     # 6 token tiles (the last of 60 tokens), K split 16 ways: 1 or 2 chunks of 64
    (1100, 1152, 256, True),    # 9 token tiles (the last of 76 tokens), K split 16 ways
    (1536, 2560, 256, False),   # 12 token tiles, K split 16 ways: 2 or 3 chunks (an odd count's last chunk)
    (2048, 256, 256, True),     # the split capped by the hidden dimension: 4 ways of one chunk
    (8192, 256, 1024, False),   # 64 token tiles x 4 expert tiles: no split, the sigmoid in the kernel
])
def test_forward_router_scores_large_batch(T, hidden, E, whole):
    """Batches above 512 tokens with a multiple of 256 experts: the forward's router stages 128
    tokens x 256 experts through LDS, its hidden dimension split over workgroups whose partial
    logits are added in a fixed order.  Every score against the oracle's (the bound of the
    single-pass router); the layer against the oracle on every token, or on the first and last 128
    tokens."""
    s = dataclasses.replace(ROUTER_LDS, tokens=T, hidden=hidden, n_experts=E)
    say(f"forward router, LDS-staged: T={T}, hidden {hidden}, E={E}")
    layer = Layer(s)
    xb = synth.gen_x(s)
    got = _run(layer, xb)
    want = route.sigmoid_scores(route.router_logits(synth.bf16_bits_to_f32(xb),
                                                    synth.bf16_bits_to_f32(synth.gen_router_w(s))))
    assert np.abs(got["scores"] - want).max() <= 2e-5
    toks = None if whole else np.r_[0:128, T - 128:T]
    _compare_router_run(layer, xb, got, tokens=toks, chunks=4)
    again = _run(layer, xb)
    assert np.array_equal(again["scores"], got["scores"]) and np.array_equal(again["out"], got["out"])


# ---- V3 shapes, in the benchmark's launch configuration, on sampled tokens ----

@pytest.fixture(scope="module")
def v3():
    say("building the V3 layer (257 experts, device-drawn weights)")
    return Layer(synth.V3_PREFILL)


def _v3_run(v3, shape):
    bias = synth.skew_bias() if shape.skewed else None
    v3.bias = bias
    v3.weights.bias = to_dev(bias) if bias is not None else None
    xb = synth.gen_x(shape)
    got = _run(v3, xb)
    counts = np.bincount(got["topk_idx"].reshape(-1), minlength=256)
    say(f"  loads: max/mean {counts.max() / counts.mean():.1f}, empty experts {(counts == 0).sum()}")
    return xb, got


@pytest.mark.timeout(400)
def test_v3_decode_every_token(v3):
    """The decode step (T = 64): every token against the oracle."""
    shape = synth.V3_DECODE
    say(f"forward {shape.name} T={shape.tokens}: all tokens against the oracle")
    xb, got = _v3_run(v3, shape)
    _compare_router_run(v3, xb, got, chunks=8)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("shape", [synth.V3_PREFILL, synth.V3_SKEW])
def test_v3_prefill_sampled_tokens(v3, shape):
    say(f"forward {shape.name} T={shape.tokens} (sampled oracle check)")
    xb, got = _v3_run(v3, shape)
    # every score of the batch (the router's K split at this size) against the oracle's router
    want = route.sigmoid_scores(route.router_logits(synth.bf16_bits_to_f32(xb), synth.bf16_bits_to_f32(v3.wr_bits)))
    assert np.abs(got["scores"] - want).max() <= 2e-5
    toks = pick_tokens(got["topk_idx"], 256, 32, shape.cfg_id)
    _compare_router_run(v3, xb, got, tokens=toks, chunks=8)
    v3.bias = None
    v3.weights.bias = None


@pytest.mark.timeout(300)
def test_dense_ffn_sampled_tokens():
    s = synth.DENSE_FFN
    say(f"forward {s.name} T={s.tokens} (sampled oracle check)")
    layer = Layer(s)
    xb = synth.gen_x(s)
    got = _run(layer, xb)
    # 128-row tiles: the first and last row of a spread of tiles, the batch's first and last rows
    toks = sorted(set([0, s.tokens - 1] + [t for m in range(0, s.tokens, 384) for t in (m, m + 127)]))
    _compare_router_run(layer, xb, got, tokens=toks, chunks=8)


@pytest.mark.timeout(300)
def test_ep_local_sampled_tokens():
    """One GPU's share of an expert-parallel V3 prefill: 32 local experts, ~1024 rows each."""
    s = synth.V3_EP_LOCAL
    say(f"forward {s.name} T={s.tokens} E={s.n_experts} (sampled oracle check)")
    layer = Layer(s)
    xb = synth.gen_x(s)
    got = _run(layer, xb)
    counts = np.bincount(got["topk_idx"].reshape(-1), minlength=s.n_experts)
    say(f"  rows per expert: min {counts.min()}, max {counts.max()}")
    _compare_router_run(layer, xb, got, tokens=pick_tokens(got["topk_idx"], s.n_experts, 32, s.cfg_id), chunks=8)
