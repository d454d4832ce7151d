"""Pins for the oracle's FP8 backward GEMMs (dgrad, wgrad) and the transposed 128x1 tile
quantisation: the adjoint identity of a GEMM and its two gradients, brute-force outer-product
sums, closed forms of the padding, and the quantisation's invariants and its reduction to the
(pinned) 1x128 quantiser."""
import numpy as np
import pytest

from oracle import backward, e4m3, gemm, quant


def _pow2_values(rng, shape, lo=-3, hi=3, p_zero=0.1):
    """Random signed powers of two (and zeros): every 128-long tile of them, in any orientation,
    is quantised losslessly with power-of-two scales, so the quantised operands equal the values."""
    v = np.exp2(rng.integers(lo, hi + 1, shape)).astype(np.float32)
    v *= rng.choice(np.array([-1.0, 1.0], np.float32), shape)
    v[rng.random(shape) < p_zero] = 0.0
    return v


def test_padded_offsets_closed_form():
    assert backward.padded_offsets(np.array([0, 130, 130, 200, 456])).tolist() == [0, 256, 256, 384, 640]
    assert backward.padded_offsets(np.array([0, 0])).tolist() == [0, 0]
    assert backward.padded_offsets(np.array([0, 128, 256])).tolist() == [0, 128, 256]


def test_quant_128x1_one_group_is_the_1x128_quantiser_of_the_transpose():
    r = np.random.default_rng(1)
    v = r.standard_normal((384, 256)).astype(np.float32)
    q, s, po = backward.quant_128x1_grouped(v, np.array([0, 384]))
    q1, s1 = quant.quant_1x128(np.ascontiguousarray(v.T))
    assert po.tolist() == [0, 384] and np.array_equal(q, q1) and np.array_equal(s, s1)


def test_quant_128x1_tiles_stay_inside_groups():
    r = np.random.default_rng(2)
    off = np.array([0, 130, 131, 131, 300])
    v = r.standard_normal((300, 128)).astype(np.float32)
    v[128:130] *= np.float32(1e-3)                # the 2-row tail of group 0: its own, small scale
    q, s, po = backward.quant_128x1_grouped(v, off)
    assert po.tolist() == [0, 256, 384, 384, 640]
    assert q.shape == (128, 640) and s.shape == (128, 5)
    # group 0's second tile holds rows 128, 129 and zeros
    assert np.all(s[:, 1] == (np.abs(v[128:130]).max(0) / np.float32(448)).astype(np.float32))
    assert not q[:, 130:256].any() and not q[:, 257:384].any() and not q[:, 553:640].any()
    # the element of largest magnitude in every tile encodes to +-448
    for g in range(4):
        for c0 in range(off[g], off[g + 1], 128):
            rows = v[c0:min(c0 + 128, off[g + 1])]
            if rows.size:
                col = po[g] + (c0 - off[g]) + np.argmax(np.abs(rows), 0)
                assert np.all(q[np.arange(128), col] & 0x7F == 0x7E)
    # changing another group's rows leaves a group's codes alone
    v2 = v.copy()
    v2[131:] *= np.float32(7.0)
    q2, _, _ = backward.quant_128x1_grouped(v2, off)
    assert np.array_equal(q2[:, :384], q[:, :384])


def test_quant_128x1_dequant_within_half_ulp():
    r = np.random.default_rng(3)
    off = np.array([0, 77, 300])
    v = (r.standard_normal((300, 256)) * np.exp2(r.integers(-8, 8, (300, 1)))).astype(np.float32)
    q, s, po = backward.quant_128x1_grouped(v, off)
    d = quant.dequant_1x128(q, s)
    for g in range(2):
        got = d[:, po[g]:po[g] + off[g + 1] - off[g]].T
        want = v[off[g]:off[g + 1]].astype(np.float64)
        srep = np.repeat(s[:, po[g] // 128:], 128, axis=1)[:, :off[g + 1] - off[g]].T.astype(np.float64)
        assert np.all(np.abs(got - want) <= e4m3.half_ulp(np.abs(want) / srep) * srep * (1 + 1e-12))


def test_wgrad_equals_brute_force_outer_products():
    r = np.random.default_rng(4)
    off = np.array([0, 3, 3, 9])
    dc = r.standard_normal((9, 128)).astype(np.float32)
    a = r.standard_normal((9, 256)).astype(np.float32)
    dq, ds, po = backward.quant_128x1_grouped(dc, off)
    aq, as_, _ = backward.quant_128x1_grouped(a, off)
    got = backward.wgrad_grouped(dq, ds, aq, as_, po)
    dcv = quant.dequant_1x128(dq, ds)
    av = quant.dequant_1x128(aq, as_)
    for g in range(3):
        want = np.zeros((128, 256))
        for m in range(off[g + 1] - off[g]):                # one outer product per row, in plain loops
            col = po[g] + m
            for i in range(0, 128, 31):
                for j in range(0, 256, 37):
                    want[i, j] += float(dcv[i, col]) * float(av[j, col])
        sub = got[g][::31, ::37]
        assert np.allclose(sub, want[::31, ::37], rtol=1e-13, atol=1e-300)
    assert not got[1].any()                                 # an empty group has no gradient


@pytest.mark.parametrize("sizes,N,K", [([0, 5, 130], 256, 384), ([256], 256, 256), ([1, 1, 200, 0], 384, 256)])
def test_adjoint_identity_of_the_gemm_and_its_gradients(sizes, N, K):
    """For C_g = A_g W_g^T: sum_g <dC_g, C_g> = <dA, A> = sum_g <dW_g, W_g>, with dA = dgrad and
    dW = wgrad.  Powers of two with power-of-two scales quantise losslessly in every tile
    orientation, so the three inner products are the same number (up to fp64 summation)."""
    r = np.random.default_rng(len(sizes) + sum(sizes))
    M = sum(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    G = len(sizes)
    A = _pow2_values(r, (M, K))
    W = _pow2_values(r, (G, N, K))
    dC = _pow2_values(r, (M, N))
    aq, as_ = quant.quant_1x128(A, ue8m0=True)
    wq = np.stack([quant.quant_128x128(W[g], ue8m0=True)[0] for g in range(G)])
    ws = np.stack([quant.quant_128x128(W[g], ue8m0=True)[1] for g in range(G)])
    dq, ds = quant.quant_1x128(dC, ue8m0=True)
    assert np.array_equal(quant.dequant_1x128(aq, as_), A) and np.array_equal(quant.dequant_1x128(dq, ds), dC)
    C = gemm.grouped_gemm_blockscaled(aq, as_, None, wq, ws, off)
    dA = backward.dgrad_grouped(dq, ds, wq, ws, off)
    dct, dcts, po = backward.quant_128x1_grouped(dC, off, ue8m0=True)
    at, ats, _ = backward.quant_128x1_grouped(A, off, ue8m0=True)
    dW = backward.wgrad_grouped(dct, dcts, at, ats, po)
    lhs = float(np.sum(dC.astype(np.float64) * C))
    mid = float(np.sum(dA * A))
    rhs = float(np.sum(dW * W))
    scale = 1.0 + sum(float(np.sum(np.abs(dC[off[g]:off[g + 1]].astype(np.float64)) *
                                   (np.abs(A[off[g]:off[g + 1]].astype(np.float64)) @ np.abs(W[g].astype(np.float64)).T)))
                      for g in range(G))
    assert abs(lhs - mid) <= 1e-12 * scale and abs(lhs - rhs) <= 1e-12 * scale
    # and each gradient equals its dense definition on the (exact) values
    for g in range(G):
        lo, hi = off[g], off[g + 1]
        assert np.allclose(dA[lo:hi], dC[lo:hi].astype(np.float64) @ W[g].astype(np.float64), rtol=0, atol=1e-9)
        assert np.allclose(dW[g], dC[lo:hi].T.astype(np.float64) @ A[lo:hi].astype(np.float64), rtol=0, atol=1e-9)


def test_transposed_weight_blocks():
    r = np.random.default_rng(6)
    w = r.standard_normal((256, 384)).astype(np.float32)
    q, s = quant.quant_128x128(w)
    qt, st = backward.transpose_weight(q, s)
    q2, s2 = quant.quant_128x128(np.ascontiguousarray(w.T))      # blocks of W^T quantised directly
    assert np.array_equal(qt, q2) and np.array_equal(st, s2)
