"""GPU parity of each C-ABI call against the oracle (bit-exact where the method
fixes the result: FP8 codes and scales, expert sets and weights given the
scores, permutation and offsets)."""
import numpy as np
import pytest
import torch

import synth
from oracle import backward, e4m3, gemm, permute, quant, route

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_ffn_sigmoid_amd as moe
    from gpu_util import DEV, check_requant, say, to_dev


def _adversarial_rows(seed, rows, cols):
    r = np.random.default_rng(seed)
    v = r.standard_normal((rows, cols)).astype(np.float32)
    v[0] = 0.0                                                   # all-zero row
    v[1] *= np.float32(1e-30)                                    # tiny values (subnormal quotients)
    v[2] *= np.float32(1e30)
    v[3] = np.exp2(r.uniform(-40, 40, cols)).astype(np.float32)  # huge dynamic range inside tiles
    v[4, ::2] = np.float32(-0.0)
    v[5] *= np.float32(1e-44)                                    # subnormal values: scale clamped to 2^-126
    v[6] *= np.float32(1e-38)                                    # amax / 448 below the normal range
    return v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (512, 7168)])
def test_quant_1x128_bit_exact(dtype, rows, cols):
    say(f"quant_1x128 {dtype} {rows}x{cols}")
    v = _adversarial_rows(rows * 7 + cols, rows, cols) if rows > 4 else \
        np.random.default_rng(1).standard_normal((rows, cols)).astype(np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(v)
        v = synth.bf16_bits_to_f32(bits)
        xd = to_dev(bits)
    else:
        xd = to_dev(v)
    q, s = moe.fp8_quant_1x128(xd)
    want_q, want_s = quant.quant_1x128(v)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), want_q)


def test_e4m3_encoder_every_midpoint_and_random_fp32():
    """Tiles whose amax is exactly 448 have s = 1, so every other element is
    encoded as is: probe grid values, midpoints, their fp32 neighbours and
    random fp32 bit patterns of magnitude <= 448."""
    vals, _ = e4m3.finite_positive_grid()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    probe = np.concatenate([vals.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
                            np.nextafter(mids, np.float32(1000))])
    r = np.random.default_rng(5)
    bits = r.integers(0, 0x43E00000, size=400000, dtype=np.uint32)        # every fp32 pattern below 448
    probe = np.concatenate([probe, bits.view(np.float32)])
    probe = np.concatenate([probe, -probe])
    n = -(-probe.size // 127) * 127
    probe = np.concatenate([probe, np.zeros(n - probe.size, np.float32)])
    tiles = np.concatenate([np.full((n // 127, 1), 448.0, np.float32), probe.reshape(-1, 127)], axis=1)
    q, s = moe.fp8_quant_1x128(to_dev(np.ascontiguousarray(tiles)))
    assert np.all(s.cpu().numpy() == 1.0)
    assert np.array_equal(q.cpu().numpy(), e4m3.encode(tiles))


def _near_midpoint_values(amax: np.float32, count: int, seed: int) -> np.ndarray:
    """fp32 values v whose quotients fp32(v / s), s = fp32(amax / 448), fall on or within a few ulps
    of e4m3 rounding midpoints (the quantisers take a product with fp32(1 / s) instead of the
    division away from them; these probe the switch), with both signs."""
    s = np.float32(amax) / np.float32(448.0)
    vals, _ = e4m3.finite_positive_grid()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    mids = mids[mids < 440]
    t = [mids]
    lo, hi = mids.copy(), mids.copy()
    for _ in range(5):
        lo = np.nextafter(lo, np.float32(0))
        hi = np.nextafter(hi, np.float32(1000))
        t += [lo, hi]
    t = np.concatenate(t)
    v = (t * s).astype(np.float32)
    v = v[np.abs(v) < np.float32(amax)]
    r = np.random.default_rng(seed)
    v = r.choice(v, count) * r.choice(np.array([-1, 1], np.float32), count)
    return v.astype(np.float32)


@pytest.mark.parametrize("amax", [1.0, 3.7, 0.0031415926, 123.456, 7e-20, 1.3 * 2.0 ** -100, 448.0 * 1.1])
def test_quantisers_at_quotient_midpoints(amax):
    """Every quantiser (1x128 and 128x128 from fp32, the transposed 128x1) against the oracle on tiles
    whose quotients sit at and beside e4m3 rounding midpoints, for scales with many mantissa bits."""
    say(f"quantisers at quotient midpoints, amax {amax:g}")
    a = np.float32(amax)
    v = _near_midpoint_values(a, 256 * 1024, int(amax * 1000) % 97)
    # 1x128: 2048 rows, element 0 of each row is the amax
    t1 = v[: 2048 * 127].reshape(2048, 127)
    x1 = np.concatenate([np.full((2048, 1), a, np.float32), t1], axis=1)
    q, s = moe.fp8_quant_1x128(to_dev(x1))
    wq, ws = quant.quant_1x128(x1)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), wq)
    # 128x128: 2 x 8 blocks, each with the amax at its corner
    x2 = v[: 256 * 1024].reshape(256, 1024).copy()
    x2[::128, ::128] = a
    q, s = moe.fp8_quant_128x128(to_dev(x2))
    wq, ws = quant.quant_128x128(x2)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), wq)
    # 128x1 over two groups of 256 and 200 rows: the amax heads each column of each 128-row tile
    x3 = v[: 456 * 512].reshape(456, 512).copy()
    x3[[0, 128, 256, 384], :] = a
    off = np.array([0, 256, 456], np.int32)
    q, s, po = moe.fp8_quant_128x1_grouped(to_dev(x3), to_dev(off))
    wq, ws, wpo = backward.quant_128x1_grouped(x3, off)
    mp = int(wpo[-1])
    assert np.array_equal(q.cpu().numpy()[:, :mp], wq)
    assert np.array_equal(s.cpu().numpy()[:, :mp // 128].view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 256), (4096, 7168)])
def test_quant_128x128_bit_exact(rows, cols):
    say(f"quant_128x128 {rows}x{cols}")
    r = np.random.default_rng(rows + cols)
    w = (r.standard_normal((rows, cols)) * np.exp2(r.integers(-10, 10, (rows, 1)))).astype(np.float32)
    w[:128, :128] = 0.0
    if cols > 128:
        w[:128, 128:256] *= np.float32(1e-42)                     # a block of subnormal values
    q, s = moe.fp8_quant_128x128(to_dev(w))
    want_q, want_s = quant.quant_128x128(w)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), want_q)


ROUTE_CASES = [
    # (T, E, k, G, gk, ties, bias scale, rule)
    (64, 16, 2, 4, 2, False, 0.0, 0),
    (300, 16, 2, 4, 2, True, 0.0, 0),
    (4096, 256, 8, 8, 4, False, 0.0, 0),
    (4096, 256, 8, 8, 4, False, 0.3, 0),
    (1000, 256, 8, 8, 4, True, 0.0, 0),
    (777, 64, 6, 8, 8, False, 0.2, 0),
    (500, 96, 4, 3, 2, True, 0.1, 1),
    (129, 1024, 16, 32, 4, False, 0.05, 0),
    (1, 128, 64, 1, 1, False, 0.0, 0),        # the largest top_k, one group
    (5, 64, 64, 4, 4, True, 0.1, 0),          # every expert chosen
    (33, 1, 1, 1, 1, False, 0.0, 0),          # a single expert
]


@pytest.mark.parametrize("case", ROUTE_CASES)
def test_route_given_scores_bit_exact(case):
    T, E, k, G, gk, ties, bscale, rule = case
    say(f"moe_route scores given T={T} E={E} k={k} G={G} gk={gk} ties={ties} bias={bscale} rule={rule}")
    sc = synth.gen_scores(T, E, cfg_id=E + k, ties=ties)
    bias = synth.gen_bias(E, scale=bscale) if bscale else None
    cfg = moe.MoeConfig(128, 128, E, k, 0, 0, G, gk, rule, 1.0)
    _, idx, w = moe.moe_route(cfg, T, DEV, scores=to_dev(sc), bias=None if bias is None else to_dev(bias))
    want_idx, want_w = route.select(sc, bias, G, gk, k, 1.0, "max" if rule else "top2_sum")
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want_w.view(np.uint32))


@pytest.mark.parametrize("G,gk", [(1, 1), (4, 2)])
def test_route_signed_zero_ties(G, gk):
    """Biased scores of +0 (0.5 - 0.5) and -0 (-0 + -0) are equal: ties go to the lower expert id
    (a kernel ordering +0 above -0 would take the even experts instead)."""
    say(f"moe_route signed-zero ties G={G} gk={gk}")
    T, E, k = 8, 16, 4
    sc = np.where(np.arange(E) % 2 == 0, np.float32(0.5), np.float32(-0.0)).astype(np.float32)
    sc = np.tile(sc, (T, 1))
    bias = np.where(np.arange(E) % 2 == 0, np.float32(-0.5), np.float32(-0.0)).astype(np.float32)
    cfg = moe.MoeConfig(128, 128, E, k, 0, 0, G, gk, 0, 1.0)
    _, idx, w = moe.moe_route(cfg, T, DEV, scores=to_dev(sc), bias=to_dev(bias))
    want_idx, want_w = route.select(sc, bias, G, gk, k, 1.0, "top2_sum")
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want_w.view(np.uint32))
    assert np.array_equal(np.sort(want_idx[0]), np.arange(k))


@pytest.mark.parametrize("shape", [synth.TINY, synth.V3_DECODE, synth.with_tokens(synth.V3_PREFILL, 1000)])
def test_router_scores(shape):
    say(f"router scores {shape.name} T={shape.tokens}")
    xb = synth.gen_x(shape)
    wr = synth.gen_router_w(shape)
    cfg = moe.MoeConfig.of(shape)
    sc, idx, _ = moe.moe_route(cfg, shape.tokens, DEV, x=to_dev(xb), w_router=to_dev(wr))
    want = route.sigmoid_scores(route.router_logits(synth.bf16_bits_to_f32(xb), synth.bf16_bits_to_f32(wr)))
    got = sc.cpu().numpy()
    # fp32 accumulation of d products of bf16 values (|logit| ~ 1.7): a few 1e-6
    assert np.abs(got - want).max() <= 2e-5
    # expert sets: equal except where the oracle's own scores are within rounding of a tie
    want_idx, _ = route.select(want, None, shape.n_group, shape.topk_group, shape.top_k)
    gi = np.sort(idx.cpu().numpy(), 1)
    wi = np.sort(want_idx, 1)
    diff = np.flatnonzero((gi != wi).any(1))
    assert diff.size <= max(1, shape.tokens // 100)
    for t in diff:
        assert abs(float(want[t, gi[t]].astype(np.float64).sum() - want[t, wi[t]].astype(np.float64).sum())) < 1e-4


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (64, 2, 16), (64, 8, 256), (1000, 4, 7), (4096, 8, 256),
                                   (16384, 8, 256), (333, 3, 1024)])
def test_permute_bit_exact(T, k, E):
    say(f"moe_permute T={T} k={k} E={E}")
    r = np.random.default_rng(T + E)
    keys = r.random((T, E))
    keys[: T // 3, 0] = -1.0                                     # load skew: expert 0 first for a third of the tokens
    idx = np.argsort(keys, axis=1)[:, :k].astype(np.int32)
    rows = r.integers(0, 256, (T, 48), dtype=np.uint8)
    off, sa, ap, g = moe.moe_permute(to_dev(idx), E, rows=to_dev(rows))
    w_off, w_sa, w_ap = permute.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), w_off)
    assert np.array_equal(sa.cpu().numpy(), w_sa)
    assert np.array_equal(ap.cpu().numpy(), w_ap)
    assert np.array_equal(g.cpu().numpy(), permute.gather_rows(rows, w_sa, k))
    back = moe.moe_unpermute(g, ap, k)
    assert np.array_equal(back.cpu().numpy(), np.repeat(rows[:, None, :], k, axis=1))


def test_permute_empty_and_all_to_one():
    say("moe_permute T=0 and all tokens on one expert")
    off, sa, ap, _ = moe.moe_permute(torch.zeros((0, 4), dtype=torch.int32, device=DEV), 8)
    assert off.cpu().numpy().tolist() == [0] * 9
    idx = np.full((3000, 1), 5, np.int32)
    off, sa, ap, _ = moe.moe_permute(to_dev(idx), 8)
    assert off.cpu().numpy().tolist() == [0, 0, 0, 0, 0, 0, 3000, 3000, 3000]
    assert np.array_equal(sa.cpu().numpy(), np.arange(3000))


def test_unpermute_weighted_combine():
    say("moe_unpermute weighted combine")
    r = np.random.default_rng(9)
    T, k, E, d = 300, 4, 32, 512
    idx = np.argsort(r.random((T, E)), axis=1)[:, :k].astype(np.int32)
    _, _, ap = permute.permute(idx, E)
    y = r.standard_normal((T * k, d)).astype(np.float32)
    w = r.random((T, k)).astype(np.float32)
    sh = r.standard_normal((T, d)).astype(np.float32)
    out = moe.moe_unpermute(to_dev(y), to_dev(ap), k, topk_w=to_dev(w), shared_y=to_dev(sh))
    ref = np.asarray(permute.combine(y, ap, w, sh))
    got = out.float().cpu().numpy().astype(np.float64)
    # per element: the fp32 sum of k + 1 terms in slot order (each product and add rounded once) is
    # within (k + 2) 2^-24 sum |terms| of the exact sum, then rounded to bf16 (half an ulp of the result)
    terms = np.zeros((T, d))
    for j in range(k):
        terms += np.abs(w[:, j:j + 1].astype(np.float64) * y[ap.reshape(T, k)[:, j]])
    terms += np.abs(sh)
    _, e = np.frexp(np.maximum(np.abs(got), 2.0 ** -126))
    assert np.all(np.abs(got - ref) <= np.ldexp(1.0, e - 9) + (k + 2) * 2.0 ** -24 * terms)


# The gfx950 FP8 MFMA returns each 128-term block sum with a relative error up
# to ~1.4e-5 of the block's sum of |products| (measured on Gaussian-quantised
# tiles); allow 5e-5 of sum_k |a_k b_k| per output.
FP8_MFMA_REL = 5e-5


def _absdot(a_q, a_s, gat, b_q, b_s, off):
    """sum_k |A[m,k] B[n,k]| in fp64 (the scale of the FP8 MFMA's error)."""
    rows = np.arange(int(off[-1])) if gat is None else gat
    out = np.zeros((int(off[-1]), b_q.shape[1]))
    a = np.abs(quant.dequant_1x128(a_q, a_s))
    for g in range(b_q.shape[0]):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            out[lo:hi] = a[rows[lo:hi]] @ np.abs(quant.dequant_128x128(b_q[g], b_s[g])).T
    return out


def _packed(b_q):
    """Row-major codes [G, N, K] -> device tensor in the GEMMs' fragment order."""
    return moe.moe_pack_weights(to_dev(b_q))


def test_pack_weights_layout():
    say("moe_pack_weights layout")
    r = np.random.default_rng(12)
    G, N, K = 3, 48, 384
    src = r.integers(0, 256, (G, N, K), dtype=np.uint8)
    got = moe.moe_pack_weights(to_dev(src)).cpu().numpy().reshape(-1)
    # block (g, n16, kb) of 2048 bytes; byte h*1024 + (16 q + r)*16 + b = B[16 n16 + r][128 kb + 64 h + 16 q + b]
    want = src.reshape(G, N // 16, 16, K // 128, 2, 4, 16).transpose(0, 1, 3, 4, 5, 2, 6).reshape(-1)
    assert np.array_equal(got, want)


def _gemm_case(seed, M_groups, N, K, gather_rows=None):
    r = np.random.default_rng(seed)
    G = len(M_groups)
    M = int(sum(M_groups))
    src = gather_rows or M
    a = r.standard_normal((src, K)).astype(np.float32)
    a_q, a_s = quant.quant_1x128(a)
    bws = [(r.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32) for _ in range(G)]
    bq = [quant.quant_128x128(b) for b in bws]
    b_q = np.stack([x[0] for x in bq])
    b_s = np.stack([x[1] for x in bq])
    offsets = np.concatenate([[0], np.cumsum(M_groups)]).astype(np.int32)
    gather = r.integers(0, src, M).astype(np.int32) if gather_rows else None
    return a_q, a_s, b_q, b_s, offsets, gather


# Group sizes pick the kernel: <= 10 rows on average the weight-streaming kernel, else the LDS
# tile kernel with 64- or 128-row tiles; a group's partial last tile runs the kernel's
# partial-tile path (row blocks past the group's end skipped).
def _sizes(seed, G, lo, hi):
    return [int(v) for v in np.random.default_rng(seed).integers(lo, hi + 1, G)]


GEMM_CASES = [
    ([16], 128, 128, None),
    ([9], 128, 128, None),                           # weight-streaming path, one group
    ([1, 0, 37, 5, 130, 0, 64], 256, 384, None),
    ([300, 2, 0, 77], 512, 256, 120),
    ([2000], 384, 512, None),
    ([3] * 40, 256, 256, 50),
    ([100, 0, 129, 255, 7, 160], 384, 640, None),   # 128-row tiles: partial column tile, K tail of 2
    ([70, 90], 256, 128, 60),                        # 128-row tiles, one K block
    ([130, 0, 161, 95, 170, 224], 384, 640, None),   # partial second tiles of 2, 33, 42 and 96 rows
    ([150, 120, 118], 512, 256, 200),                # gathered rows, partial tiles of 22..120 rows, two K blocks
    ([3, 9, 0, 14, 1], 384, 256, 40),                # weight-streaming path: three 128-column workgroups
    ([17, 32, 0, 25, 9], 256, 384, None),            # 11-18 rows per group (the SwiGLU GEMM's 32-row streaming tiles)
    (_sizes(10, 48, 6, 30), 384, 256, 200),          # the same, gathered rows
]


# More than 64 groups: each lane of the tile lookup then scans several groups (G = 65 leaves the
# second lane one group), up to the largest G the call takes.
GEMM_CASES += [
    (_sizes(1, 200, 0, 20), 256, 256, 300),          # weight-streaming kernel (10 rows per group), 4 groups per lane
    (_sizes(2, 70, 0, 50), 384, 256, None),          # 64-row tiles, 27 rows per group on average
    (_sizes(3, 130, 10, 90), 256, 384, None),        # 64-row tiles
    (_sizes(4, 65, 60, 200), 256, 256, 500),         # 128-row tiles, partial second tiles
    (_sizes(5, 1024, 0, 6), 128, 128, None),         # G = 1024: 16 groups per lane
]


@pytest.mark.parametrize("case", GEMM_CASES)
def test_grouped_gemm_store_f32(case):
    mg, N, K, gr = case
    say(f"grouped GEMM f32 G={len(mg)} groups={mg[:8]} N={N} K={K} gather={gr}")
    a_q, a_s, b_q, b_s, off, gat = _gemm_case(len(mg) + N, mg, N, K, gr)
    out = moe.fp8_grouped_gemm_blockscaled(to_dev(a_q), to_dev(a_s), _packed(b_q), to_dev(b_s), to_dev(off),
                                           moe.MOE_EPI_STORE_F32, a_gather=None if gat is None else to_dev(gat),
                                           m_max=int(off[-1]))
    ref = gemm.grouped_gemm_blockscaled(a_q, a_s, gat, b_q, b_s, off)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= FP8_MFMA_REL * _absdot(a_q, a_s, gat, b_q, b_s, off) + 1e-30)


@pytest.mark.parametrize("mg", [[3, 0, 9, 14], [5, 0, 70, 33], [70, 100, 0, 90], [150, 0, 170, 200]])
def test_grouped_gemm_bf16_and_scatter(mg):
    say(f"grouped GEMM bf16 + weighted scatter-add groups={mg}")
    N, K = 256, 256
    a_q, a_s, b_q, b_s, off, _ = _gemm_case(77, mg, N, K)
    args = [to_dev(a_q), to_dev(a_s), _packed(b_q), to_dev(b_s), to_dev(off)]
    ref = gemm.grouped_gemm_blockscaled(a_q, a_s, None, b_q, b_s, off)
    out = moe.fp8_grouped_gemm_blockscaled(*args, moe.MOE_EPI_STORE_BF16, m_max=int(off[-1]))
    from oracle.ffn import round_bf16
    got = out.float().cpu().numpy()
    assert np.abs(got - round_bf16(ref)).max() <= np.abs(ref).max() * 2.0 ** -8
    r = np.random.default_rng(3)
    M = int(off[-1])
    dst = r.integers(0, 20, M).astype(np.int32)
    wt = r.random(M).astype(np.float32)
    acc = moe.fp8_grouped_gemm_blockscaled(*args, moe.MOE_EPI_WEIGHTED_SCATTER_ADD, m_max=M, dst_row=to_dev(dst),
                                           row_weight=to_dev(wt), out_rows=20)
    want = np.zeros((20, N))
    np.add.at(want, dst, wt[:, None].astype(np.float64) * ref)
    bound = np.zeros((20, N))
    np.add.at(bound, dst, wt[:, None].astype(np.float64) * _absdot(a_q, a_s, None, b_q, b_s, off))
    assert np.all(np.abs(acc.cpu().numpy() - want) <= FP8_MFMA_REL * bound + 1e-6 * np.abs(want).max())


@pytest.mark.parametrize("mg,W,K,wide", [([7, 0, 130], 128, 256, "tiny"), ([64] * 5, 256, 512, False),
                                         ([1000], 128, 384, False), ([40, 90], 128, 256, True),
                                         ([130, 0, 75, 200], 256, 768, False), ([66, 128], 128, 128, False),
                                         ([140, 0, 200, 161], 256, 768, False), ([120, 130], 128, 128, False),
                                         ([5, 0, 12, 16, 3], 384, 256, False), ([20, 0, 31, 12], 256, 384, False),
                                         (_sizes(11, 40, 4, 28), 128, 256, False),
                                         (_sizes(6, 80, 0, 60), 128, 256, False),
                                         (_sizes(7, 300, 0, 10), 256, 128, False)])
def test_grouped_gemm_swiglu_quant(mg, W, K, wide):
    say(f"grouped GEMM SwiGLU+quant G={len(mg)} groups={mg[:8]} W={W} K={K} full-range codes={wide}")
    a_q, a_s, b_q, b_s, off, _ = _gemm_case(W + K, mg, 2 * W, K)
    if wide == "tiny":                         # rows of activations ~1e-20: h ~1e-40 (subnormal fp32 tiles)
        a_s[::3] *= np.float32(1e-20)
    elif wide:                                 # every finite code, subnormals included, in A
        r = np.random.default_rng(8)
        a_q = r.integers(0, 256, a_q.shape).astype(np.uint8)
        a_q[(a_q & 0x7F) == 0x7F] = 0x01
    h_q, h_s = moe.fp8_grouped_gemm_blockscaled(to_dev(a_q), to_dev(a_s), _packed(b_q), to_dev(b_s), to_dev(off),
                                                moe.MOE_EPI_SWIGLU_QUANT, m_max=int(off[-1]))
    gu = gemm.grouped_gemm_blockscaled(a_q, a_s, None, b_q, b_s, off)
    from oracle.ffn import silu
    h = (silu(gu[:, :W]) * gu[:, W:]).astype(np.float32)
    got_q, got_s = h_q.cpu().numpy(), h_s.cpu().numpy()
    # exact products, fp32 accumulation (vs fp64): scales within a few ulps, codes equal
    # except at rounding midpoints (then one step apart)
    check_requant(got_q, got_s, gu, _absdot(a_q, a_s, None, b_q, b_s, off))
    deq_got = quant.dequant_1x128(got_q, got_s)
    srep = np.repeat(got_s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq_got - h) <= e4m3.half_ulp(np.abs(h) / srep) * srep * 1.01 + 1e-6 * np.abs(h) + 1e-30)


# The V3 layer's GEMM shapes element by element: gate/up (K = 7168, N = 2 x 2048, SwiGLU) and down
# (K = 2048, N = 7168), three experts of 120-161 rows gathered from a 4096-row activation pool as
# the layer gathers them: the 56-block K loop with its tail, and experts of more than 128 rows split
# into two partial tiles.
@pytest.mark.parametrize("epi", ["swiglu", "f32"])
def test_grouped_gemm_v3_shapes(epi):
    mg = [161, 120, 150]
    N, K = (4096, 7168) if epi == "swiglu" else (7168, 2048)
    say(f"grouped GEMM V3 shape {epi} groups={mg} N={N} K={K} gathered from 4096 rows")
    a_q, a_s, b_q, b_s, off, gat = _gemm_case(40 + N, mg, N, K, 4096)
    M = int(off[-1])
    args = [to_dev(a_q), to_dev(a_s), _packed(b_q), to_dev(b_s), to_dev(off)]
    ref = gemm.grouped_gemm_blockscaled(a_q, a_s, gat, b_q, b_s, off)
    if epi == "swiglu":
        h_q, h_s = moe.fp8_grouped_gemm_blockscaled(*args, moe.MOE_EPI_SWIGLU_QUANT, a_gather=to_dev(gat), m_max=M)
        check_requant(h_q.cpu().numpy(), h_s.cpu().numpy(), ref, _absdot(a_q, a_s, gat, b_q, b_s, off))
    else:
        out = moe.fp8_grouped_gemm_blockscaled(*args, moe.MOE_EPI_STORE_F32, a_gather=to_dev(gat), m_max=M)
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= FP8_MFMA_REL * _absdot(a_q, a_s, gat, b_q, b_s, off) + 1e-30)
