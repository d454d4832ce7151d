"""GPU parity of the steps next to the layer: the RMSNorm fused with the 1x128
quantisation, the routing-bias balancing step, and the power-of-two (UE8M0)
scale variant, each against the oracle.  Codes, scales, normalised bf16 rows,
loads and biases are compared bit for bit; layers with the RMSNorm and / or
UE8M0 scales use the layer's output bar."""
import numpy as np
import pytest
import torch

import synth
from oracle import calibrate, e4m3, gemm, norm, quant

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_ffn_sigmoid_amd as moe
    from gpu_util import (DEV, FP8_MFMA_REL, Layer, check_requant, compare_router_run, pick_tokens, run_layer, say,
                          to_dev)


def _gamma_bits(d, seed):
    g = np.random.default_rng(seed).uniform(0.25, 2.0, d).astype(np.float32)
    return synth.f32_to_bf16_bits(g)


# ---- UE8M0 quantisation ----

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(5, 128), (37, 384), (512, 7168)])
def test_quant_1x128_ue8m0_bit_exact(dtype, rows, cols):
    say(f"quant_1x128 UE8M0 {dtype} {rows}x{cols}")
    r = np.random.default_rng(rows + cols)
    v = (r.standard_normal((rows, cols)) * np.exp2(r.integers(-30, 30, (rows, 1)))).astype(np.float32)
    v[0, :128] = 0.0
    v[1, :] = np.float32(1e-41)                               # clamped exponent
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(v)
        v = synth.bf16_bits_to_f32(bits)
        xd = to_dev(bits)
    else:
        xd = to_dev(v)
    q, s = moe.fp8_quant_1x128(xd, ue8m0=True)
    want_q, want_s = quant.quant_1x128(v, ue8m0=True)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), want_q)


def test_quant_128x128_ue8m0_bit_exact():
    say("quant_128x128 UE8M0 512x768")
    r = np.random.default_rng(21)
    w = (r.standard_normal((512, 768)) * np.exp2(r.integers(-12, 12, (512, 1)))).astype(np.float32)
    q, s = moe.fp8_quant_128x128(to_dev(w), ue8m0=True)
    want_q, want_s = quant.quant_128x128(w, ue8m0=True)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), want_q)


# ---- RMSNorm + quantisation ----

def _norm_case(T, d, seed, scale=1.0):
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        (np.random.default_rng(seed).standard_normal((T, d)) * scale).astype(np.float32)))
    return synth.f32_to_bf16_bits(x), x


@pytest.mark.parametrize("ue8m0", [False, True])
@pytest.mark.parametrize("T,d,scale", [(1, 128, 1.0), (37, 7168, 1.0), (64, 256, 3e-3), (300, 1024, 40.0),
                                       (9, 8320, 1.0)])
def test_rmsnorm_quant_bit_exact(T, d, scale, ue8m0):
    say(f"rmsnorm+quant T={T} d={d} scale={scale} ue8m0={ue8m0}")
    xb, xv = _norm_case(T, d, T * 31 + d, scale)
    gb = _gamma_bits(d, d)
    eps = 1e-6
    y, q, s = moe.fp8_rmsnorm_quant_1x128(to_dev(xb), to_dev(gb), eps, ue8m0=ue8m0)
    want_y = norm.rmsnorm(xv, synth.bf16_bits_to_f32(gb), eps)
    want_q, want_s = quant.quant_1x128(want_y, ue8m0=ue8m0)
    assert np.array_equal(y.float().cpu().numpy(), want_y)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), want_q)
    y2, q2, s2 = moe.fp8_rmsnorm_quant_1x128(to_dev(xb), to_dev(gb), eps, want_y=False, ue8m0=ue8m0)
    assert y2 is None and torch.equal(q2, q) and torch.equal(s2, s)


def test_rmsnorm_quant_empty_and_composition():
    say("rmsnorm+quant: T = 0; fused == norm then fp8_quant_1x128")
    y, q, s = moe.fp8_rmsnorm_quant_1x128(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV),
                                          to_dev(_gamma_bits(256, 1)))
    assert y.shape == (0, 256) and q.shape == (0, 256)
    xb, _ = _norm_case(50, 512, 3)
    y, q, s = moe.fp8_rmsnorm_quant_1x128(to_dev(xb), to_dev(_gamma_bits(512, 2)))
    q2, s2 = moe.fp8_quant_1x128(y)
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_rmsnorm_quant_v3_prefill_rows_sampled():
    """The V3 prefill shape (T = 4096, d = 7168) in one launch, checked on sampled rows."""
    T, d = 4096, 7168
    say(f"rmsnorm+quant T={T} d={d}, sampled rows")
    xb = synth.gen_x(synth.V3_PREFILL)
    xv = synth.bf16_bits_to_f32(xb)
    gb = _gamma_bits(d, 7)
    y, q, s = moe.fp8_rmsnorm_quant_1x128(to_dev(xb), to_dev(gb), 1e-6)
    rows = np.random.default_rng(0).choice(T, 96, replace=False)
    want_y = norm.rmsnorm(xv[rows], synth.bf16_bits_to_f32(gb), 1e-6)
    want_q, want_s = quant.quant_1x128(want_y)
    assert np.array_equal(y.float().cpu().numpy()[rows], want_y)
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy()[rows], want_q)


# ---- routing-bias balancing step ----

@pytest.mark.parametrize("T,k,E", [(0, 8, 256), (1, 1, 1), (64, 8, 256), (4096, 8, 256), (999, 6, 64),
                                   (16384, 8, 1024)])
def test_bias_update_bit_exact(T, k, E):
    say(f"bias update T={T} k={k} E={E}")
    r = np.random.default_rng(T + E)
    idx = (r.zipf(1.5, (T, k)) % E).astype(np.int32) if T else np.zeros((0, k), np.int32)
    bias = (r.standard_normal(E) * 0.1).astype(np.float32)
    bias[:3] = np.float32(-0.0)
    b = to_dev(bias)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    moe.moe_bias_update(to_dev(idx), E, 1e-3, b, counts)
    want = calibrate.update(bias, idx, E, 1e-3)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert np.array_equal(counts.cpu().numpy(), calibrate.loads(idx, E))


def test_bias_update_loads_at_the_mean_keep_their_bias():
    say("bias update: loads exactly at the mean")
    E, k = 16, 4
    idx = np.tile(np.arange(E, dtype=np.int32), 3).reshape(-1, k)      # every expert loaded 3 times
    idx[0, 0], idx[1, 0] = 5, 5                                        # expert 5 up, experts 0 and 4 down
    bias = np.linspace(-1, 1, E).astype(np.float32)
    b = to_dev(bias)
    moe.moe_bias_update(to_dev(idx), E, 0.25, b)
    assert np.array_equal(b.cpu().numpy(), calibrate.update(bias, idx, E, 0.25))


# ---- UE8M0 in the SwiGLU requantisation epilogue ----

def _ue8m0_case(seed, mg, N, K):
    r = np.random.default_rng(seed)
    M = sum(mg)
    a_q, a_s = quant.quant_1x128(r.standard_normal((M, K)).astype(np.float32), ue8m0=True)
    bq = [quant.quant_128x128((r.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32), ue8m0=True) for _ in mg]
    b_q, b_s = np.stack([x[0] for x in bq]), np.stack([x[1] for x in bq])
    off = np.concatenate([[0], np.cumsum(mg)]).astype(np.int32)
    return a_q, a_s, b_q, b_s, off


# Power-of-two scales enter the GEMMs without a per-block promotion: as the FP8 MFMA's E8M0 scale
# operands (down GEMM) or in the exact bf16 conversion (SwiGLU GEMM).  Group sizes pick the
# weight-streaming kernel (<= 10 rows per group on average) or the LDS tile kernel.
@pytest.mark.parametrize("mg,W,K", [([7, 0, 130, 64], 256, 512), ([3, 5, 0, 9, 2], 256, 384),
                                    ([161, 120, 150], 2048, 7168)])
def test_grouped_gemm_swiglu_ue8m0(mg, W, K):
    say(f"grouped GEMM SwiGLU+quant with UE8M0 scales groups={mg} W={W} K={K}")
    a_q, a_s, b_q, b_s, off = _ue8m0_case(31 + K, mg, 2 * W, K)
    M = int(off[-1])
    h_q, h_s = moe.fp8_grouped_gemm_blockscaled(to_dev(a_q), to_dev(a_s), moe.moe_pack_weights(to_dev(b_q)),
                                                to_dev(b_s), to_dev(off), moe.MOE_EPI_SWIGLU_QUANT, m_max=M,
                                                ue8m0=True)
    gu = gemm.grouped_gemm_blockscaled(a_q, a_s, None, b_q, b_s, off)
    got_s = h_s.cpu().numpy()
    assert np.all(np.frexp(got_s)[0] == 0.5)                          # powers of two
    check_requant(h_q.cpu().numpy(), got_s, gu, _absdot(a_q, a_s, b_q, b_s, off), ue8m0=True)


@pytest.mark.parametrize("mg,N,K", [([3, 9, 0, 14, 1], 384, 256), ([100, 0, 129, 255, 7, 160], 384, 640),
                                    ([70, 90], 256, 128), ([161, 120, 150], 7168, 2048)])
def test_grouped_gemm_f32_ue8m0(mg, N, K):
    say(f"grouped GEMM f32 with UE8M0 scales (E8M0 MFMA scale operands) groups={mg} N={N} K={K}")
    a_q, a_s, b_q, b_s, off = _ue8m0_case(17 + N + K, mg, N, K)
    M = int(off[-1])
    out = moe.fp8_grouped_gemm_blockscaled(to_dev(a_q), to_dev(a_s), moe.moe_pack_weights(to_dev(b_q)), to_dev(b_s),
                                           to_dev(off), moe.MOE_EPI_STORE_F32, m_max=M, ue8m0=True)
    ref = gemm.grouped_gemm_blockscaled(a_q, a_s, None, b_q, b_s, off)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= FP8_MFMA_REL * _absdot(a_q, a_s, b_q, b_s, off) + 1e-30)


def _absdot(a_q, a_s, b_q, b_s, off):
    """sum_k |A[m,k] B[n,k]| in fp64, per group (the scale of the GEMMs' rounding)."""
    out = np.zeros((int(off[-1]), b_q.shape[1]))
    a = np.abs(quant.dequant_1x128(a_q, a_s))
    for g in range(b_q.shape[0]):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            out[lo:hi] = a[lo:hi] @ np.abs(quant.dequant_128x128(b_q[g], b_s[g])).T
    return out


# ---- layers ----

MID_A = synth.MoeShape("mid_a", 10, 200, 512, 256, 32, 4, 1, 256, 4, 2)
MID_B = synth.MoeShape("mid_b", 11, 1024, 384, 256, 16, 4, 1, 384, 4, 4)


@pytest.mark.parametrize("shape,ue8m0,with_norm", [(synth.TINY, True, True), (synth.TINY, False, True),
                                                    (MID_A, True, False), (MID_B, False, True)])
def test_layer_with_norm_and_ue8m0(shape, ue8m0, with_norm):
    say(f"forward {shape.name} ue8m0={ue8m0} rmsnorm={with_norm}, router on device")
    layer = Layer(shape, ue8m0=ue8m0, norm_gamma=_gamma_bits(shape.hidden, 5) if with_norm else None)
    xb = synth.gen_x(shape)
    compare_router_run(layer, xb, run_layer(layer, xb))


@pytest.mark.timeout(400)
def test_layer_v3_prefill_ue8m0_sampled():
    """The V3 prefill step (T = 4096) with power-of-two scales, as the benchmark times it: tokens at
    the first and last rows of the m tiles of one expert per tile shape (8 shapes, from a single
    tile to two split tiles), against the oracle with UE8M0 scales.  Few tokens: the oracle
    quantises every expert they touch again, with power-of-two scales."""
    s = synth.V3_PREFILL
    say("forward V3 prefill with UE8M0 scales, sampled tokens")
    layer = Layer(s, ue8m0=True)
    xb = synth.gen_x(s)
    got = run_layer(layer, xb)
    toks = pick_tokens(got["topk_idx"], s.n_experts, 16, s.cfg_id, max_shapes=8)
    compare_router_run(layer, xb, got, tokens=toks, chunks=8)


def test_layer_v3_decode_norm_ue8m0_sampled():
    s = synth.V3_DECODE
    say("forward V3 decode with RMSNorm + UE8M0, sampled tokens")
    layer = Layer(s, ue8m0=True, norm_gamma=_gamma_bits(s.hidden, 9))
    xb = synth.gen_x(s)
    compare_router_run(layer, xb, run_layer(layer, xb), tokens=np.arange(0, s.tokens, 8))
