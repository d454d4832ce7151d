"""MOEFP8_VALIDATE on the GPU: with the switch on, valid data gives the same results as without
it, and data that breaks a call's contract is rejected with MOE_ERR_INVALID_DATA before any of the
call's own kernels runs (the message names the first bad element; output buffers stay as they
were).  The checks run first on calls whose bad data would be harmless anyway (non-finite given
scores, offsets that end early); the rest follow, so a checker that failed there stops the run
(pytest -x) before data that only the checks keep from the kernels is passed."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_ffn_sigmoid_amd as moe
    from sparse_moe_ffn_sigmoid_amd import _lib
    from gpu_util import Layer, say, to_dev


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("MOEFP8_VALIDATE", "1")
    assert moe.moe_validation_enabled()
    return monkeypatch


def _rejected(call, fn, *needles):
    with pytest.raises(moe.MoeError) as ei:
        fn()
    torch.cuda.synchronize()
    assert ei.value.status == _lib.MOE_ERR_INVALID_DATA, str(ei.value)
    msg = str(ei.value)
    assert msg.startswith(call) and "MOEFP8_VALIDATE" in msg, msg
    for n in needles:
        assert n in msg, (n, msg)
    say(f"  rejected: {msg}")


def _gemm_operands(sizes, N=256, K=256, seed=3):
    r = np.random.default_rng(seed)
    M = int(sum(sizes))
    G = len(sizes)
    a = r.standard_normal((M, K)).astype(np.float32)
    aq, as_ = moe.fp8_quant_1x128(to_dev(a))
    bq, bs = [], []
    for g in range(G):
        q, s = moe.quantize_pack_128x128(to_dev(r.standard_normal((N, K)).astype(np.float32)))
        bq.append(q)
        bs.append(s)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return aq, as_, torch.stack(bq), torch.stack(bs), off, M


def test_valid_data_gives_the_same_results(monkeypatch):
    say("MOEFP8_VALIDATE on valid data: route, permute, unpermute, GEMM, 128x1 quant, wgrad, forward")
    layer = Layer(synth.TINY)
    s = synth.TINY
    xb = synth.gen_x(s, 40)
    scores = synth.gen_scores(40, s.n_experts, cfg_id=9)
    aq, as_, bq, bs, off, M = _gemm_operands([70, 0, 130])
    gat = to_dev(np.random.default_rng(4).integers(0, M, M).astype(np.int32))
    xg = to_dev(np.random.default_rng(5).standard_normal((M, 256)).astype(np.float32))

    def run_all():
        x = to_dev(xb)
        sc = to_dev(scores)
        _, idx, w = moe.moe_route(layer.cfg, 40, x.device, scores=sc)
        offs, sa, ap, _ = moe.moe_permute(idx, s.n_experts)
        y = to_dev(np.random.default_rng(6).standard_normal((40 * s.top_k, 256)).astype(np.float32))
        comb = moe.moe_unpermute(y, ap, s.top_k, topk_w=w)
        c = moe.fp8_grouped_gemm_blockscaled(aq, as_, bq, bs, to_dev(off), moe.MOE_EPI_STORE_F32, a_gather=gat,
                                             m_max=M)
        qt, st, po = moe.fp8_quant_128x1_grouped(xg, to_dev(off))
        wg = moe.fp8_grouped_gemm_wgrad(qt, st, qt, st, po, M)
        out = moe.moe_ffn_forward(x, layer.cfg, layer.weights, scores=to_dev(scores), scores_given=True,
                                  topk_idx=torch.empty_like(idx), topk_w=torch.empty_like(w))
        torch.cuda.synchronize()
        mp = int(po[-1])                                   # columns past the padded rows are not written
        return [t.cpu() for t in (idx, w, offs, sa, ap, comb, c, qt[:, :mp], st[:, :mp // 128], po, wg, out)]

    monkeypatch.delenv("MOEFP8_VALIDATE", raising=False)
    plain = run_all()
    monkeypatch.setenv("MOEFP8_VALIDATE", "1")
    checked = run_all()
    for i, (p, c) in enumerate(zip(plain, checked)):
        assert torch.equal(p, c), i


def test_route_rejects_nonfinite_scores(validate):
    say("moe_route: NaN and infinite given scores, non-finite bias")
    s = synth.TINY
    cfg = moe.MoeConfig.of(s)
    sc = synth.gen_scores(8, s.n_experts, cfg_id=2)
    sc[5, 3] = np.nan
    _rejected("moe_route", lambda: moe.moe_route(cfg, 8, torch.device("cuda"), scores=to_dev(sc)), "scores[83]",
              "nan")
    sc[5, 3] = 0.5
    sc[7, 0] = np.inf
    _rejected("moe_route", lambda: moe.moe_route(cfg, 8, torch.device("cuda"), scores=to_dev(sc)), "scores[112]")
    sc[7, 0] = 0.5
    bias = np.zeros(s.n_experts, np.float32)
    bias[9] = -np.inf
    _rejected("moe_route",
              lambda: moe.moe_route(cfg, 8, torch.device("cuda"), scores=to_dev(sc), bias=to_dev(bias)), "bias[9]")
    moe.moe_route(cfg, 8, torch.device("cuda"), scores=to_dev(sc))      # the repaired data passes


def test_quant_128x1_rejects_offsets(validate):
    say("fp8_quant_128x1_grouped: offsets that end before M, decrease, or start above 0")
    x = to_dev(np.ones((200, 128), np.float32))
    cases = (([0, 50, 199], "offsets[2]"), ([0, 120, 100, 200], "offsets[2]"), ([10, 100, 200], "offsets[0]"))
    for off, bad in cases:
        _rejected("fp8_quant_128x1_grouped",
                  lambda: moe.fp8_quant_128x1_grouped(x, to_dev(np.array(off, np.int32))), bad)


def test_forward_rejects_nonfinite_scores(validate):
    say("moe_ffn_forward: NaN given score; the output buffer stays untouched")
    layer = Layer(synth.TINY)
    s = synth.TINY
    x = to_dev(synth.gen_x(s, 16))
    sc = synth.gen_scores(16, s.n_experts, cfg_id=3)
    sc[2, 1] = np.nan
    out = torch.full((16, s.hidden), 0x3F80, dtype=torch.int16, device=x.device).view(torch.bfloat16)
    _rejected("moe_ffn_forward", lambda: moe.moe_ffn_forward(x, layer.cfg, layer.weights, out=out,
                                                              scores=to_dev(sc), scores_given=True), "scores[33]")
    assert bool((out.view(torch.int16) == 0x3F80).all())


def test_permute_rejects_out_of_range_ids(validate):
    say("moe_permute: expert ids E and -1; offsets left as they were")
    E, T, k = 16, 10, 2
    idx = np.random.default_rng(1).integers(0, E, (T, k)).astype(np.int32)
    for bad_pos, bad_val in ((7, E), (12, -1)):
        idx2 = idx.copy()
        idx2.flat[bad_pos] = bad_val
        d = to_dev(idx2)
        offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=d.device)
        sa = torch.full((T * k,), -7, dtype=torch.int32, device=d.device)
        ap = torch.full((T * k,), -7, dtype=torch.int32, device=d.device)
        lib = _lib.load()
        nws = lib.moe_permute_workspace_size(T, k, E)
        ws = torch.empty(nws, dtype=torch.uint8, device=d.device)
        st = torch.cuda.current_stream().cuda_stream
        vp = ctypes.c_void_p
        rc = lib.moe_permute(vp(d.data_ptr()), T, k, E, vp(offsets.data_ptr()), vp(sa.data_ptr()),
                             vp(ap.data_ptr()), None, 0, None, vp(ws.data_ptr()), nws, vp(st))
        torch.cuda.synchronize()
        assert rc == _lib.MOE_ERR_INVALID_DATA, lib.moe_last_error()
        msg = lib.moe_last_error().decode()
        assert f"topk_idx[{bad_pos}] = {bad_val}" in msg, msg
        for t in (offsets, sa, ap):
            assert bool((t == -7).all())
    moe.moe_permute(to_dev(idx), E)


def test_unpermute_rejects_positions(validate):
    say("moe_unpermute: a position past T*k, a negative one")
    T, k, d = 6, 2, 16
    y = to_dev(np.ones((T * k, d), np.float32))
    for bad in (T * k, -3):
        ap = np.arange(T * k, dtype=np.int32)
        ap[4] = bad
        _rejected("moe_unpermute", lambda: moe.moe_unpermute(y, to_dev(ap), k), f"assign_pos[4] = {bad}")
        w = to_dev(np.full((T, k), 0.5, np.float32))
        _rejected("moe_unpermute", lambda: moe.moe_unpermute(y, to_dev(ap), k, topk_w=w), "assign_pos[4]")


def test_grouped_gemm_rejects_offsets_and_rows(validate):
    say("fp8_grouped_gemm_blockscaled: decreasing offsets, offsets past M_max, negative gather and dst rows")
    aq, as_, bq, bs, off, M = _gemm_operands([64, 32, 32])
    gat = to_dev(np.arange(M, dtype=np.int32))
    for o, needle in (([0, 64, 40, 128], "offsets[2]"), ([0, 64, 96, 129], "offsets[3]"), ([-1, 64, 96, 128],
                                                                                            "offsets[0]")):
        _rejected("fp8_grouped_gemm_blockscaled", lambda: moe.fp8_grouped_gemm_blockscaled(
            aq, as_, bq, bs, to_dev(np.array(o, np.int32)), moe.MOE_EPI_STORE_F32, m_max=M), needle)
    g = np.arange(M, dtype=np.int32)
    g[100] = -1
    _rejected("fp8_grouped_gemm_blockscaled", lambda: moe.fp8_grouped_gemm_blockscaled(
        aq, as_, bq, bs, to_dev(off), moe.MOE_EPI_STORE_F32, a_gather=to_dev(g), m_max=M), "a_gather[100] = -1")
    dst = np.arange(M, dtype=np.int32)
    dst[5] = -2
    _rejected("fp8_grouped_gemm_blockscaled", lambda: moe.fp8_grouped_gemm_blockscaled(
        aq, as_, bq, bs, to_dev(off), moe.MOE_EPI_WEIGHTED_SCATTER_ADD, a_gather=gat, m_max=M, dst_row=to_dev(dst),
        out_rows=M), "dst_row[5] = -2")


def test_wgrad_rejects_padded_offsets(validate):
    say("fp8_grouped_gemm_wgrad: padded offsets off the 128 grid, decreasing, past the padded bound")
    xg = to_dev(np.random.default_rng(8).standard_normal((200, 128)).astype(np.float32))
    qt, st, po = moe.fp8_quant_128x1_grouped(xg, to_dev(np.array([0, 100, 200], np.int32)))
    mp = moe.moe_padded_rows(200, 2)
    for p, needle in (([0, 100, 256], "padded_offsets[1]"), ([0, 256, 128], "padded_offsets[2]"),
                      ([0, 128, mp + 128], "padded_offsets[2]")):
        _rejected("fp8_grouped_gemm_wgrad",
                  lambda: moe.fp8_grouped_gemm_wgrad(qt, st, qt, st, to_dev(np.array(p, np.int32)), 200), needle)
    moe.fp8_grouped_gemm_wgrad(qt, st, qt, st, po, 200)
    torch.cuda.synchronize()
