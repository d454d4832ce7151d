"""Pins for the oracle's permutation (a library stable sort, identities) and
block-scaled GEMM (exact integer products, a scalar brute force)."""
import numpy as np
import pytest

from oracle import e4m3, gemm, permute, quant


@pytest.mark.parametrize("t,k,e", [(0, 2, 4), (1, 1, 1), (64, 2, 16), (257, 8, 256), (100, 4, 7)])
def test_permute_is_stable_argsort(t, k, e):
    r = np.random.default_rng(t + e)
    idx = np.stack([r.permutation(e)[:k] for _ in range(t)]).astype(np.int32) if t else np.zeros((0, k), np.int32)
    off, sa, ap = permute.permute(idx, e)
    flat = idx.reshape(-1)
    assert np.array_equal(sa, np.argsort(flat, kind="stable"))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=e))]))
    assert np.array_equal(ap[sa], np.arange(t * k))
    assert np.array_equal(sa[ap], np.arange(t * k))


def test_permute_degenerate_loads():
    idx = np.full((50, 1), 3, np.int32)                 # every token on one expert
    off, sa, _ = permute.permute(idx, 8)
    assert off.tolist() == [0, 0, 0, 0, 50, 50, 50, 50, 50]
    assert np.array_equal(sa, np.arange(50))


def test_unpermute_inverts_permute_gather():
    r = np.random.default_rng(1)
    t, k, e = 40, 3, 9
    idx = np.stack([r.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
    rows = r.integers(0, 255, size=(t, 33)).astype(np.uint8)
    off, sa, ap = permute.permute(idx, e)
    g = permute.gather_rows(rows, sa, k)
    back = permute.unpermute(g, ap, k)
    assert np.array_equal(back, np.repeat(rows[:, None, :], k, axis=1))


def test_combine_one_hot_and_weights():
    r = np.random.default_rng(2)
    t, k, e, d = 10, 2, 5, 6
    idx = np.stack([r.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
    _, sa, ap = permute.permute(idx, e)
    y = r.standard_normal((t * k, d))
    w = np.zeros((t, k), np.float32)
    w[:, 1] = 1.0
    out = permute.combine(y, ap, w, None)
    assert np.array_equal(out, y[ap.reshape(t, k)[:, 1]])
    w = r.random((t, k)).astype(np.float32)
    sh = r.standard_normal((t, d))
    out = permute.combine(y, ap, w, sh)
    for ti in range(t):
        want = sh[ti].copy()
        for j in range(k):
            want += float(w[ti, j]) * y[ap[ti * k + j]]
        assert np.allclose(out[ti], want, rtol=1e-14, atol=1e-14)


def test_gemm_unit_scales_is_integer_matmul():
    r = np.random.default_rng(3)
    # codes of small integers 1..15 (exact e4m3 values), random signs
    ints = r.integers(-15, 16, size=(48, 256))
    intb = r.integers(-15, 16, size=(128, 256))
    a_q = e4m3.encode(ints.astype(np.float64))
    b_q = e4m3.encode(intb.astype(np.float64))
    out = gemm.gemm_blockscaled(a_q, np.ones((48, 2), np.float32), b_q, np.ones((1, 2), np.float32))
    assert np.array_equal(out, (ints @ intb.T).astype(np.float64))


def test_gemm_scalar_brute_force_with_block_scales():
    r = np.random.default_rng(4)
    m, n, k = 5, 256, 384
    a_q = r.integers(0, 256, size=(m, k)).astype(np.uint8)
    b_q = r.integers(0, 256, size=(n, k)).astype(np.uint8)
    a_q[(a_q & 0x7F) == 0x7F] = 0x11
    b_q[(b_q & 0x7F) == 0x7F] = 0x22
    a_s = r.uniform(0.01, 2, size=(m, 3)).astype(np.float32)
    b_s = r.uniform(0.01, 2, size=(2, 3)).astype(np.float32)
    out = gemm.gemm_blockscaled(a_q, a_s, b_q, b_s)
    for i in range(m):
        for j in range(0, n, 37):
            acc = 0.0
            for kb in range(3):      # per 128-wide K block: integer-exact partial, then the two scales
                part = sum(e4m3.decode_value(int(a_q[i, kk])) * e4m3.decode_value(int(b_q[j, kk]))
                           for kk in range(128 * kb, 128 * kb + 128))
                acc += part * float(a_s[i, kb]) * float(b_s[j // 128, kb])
            assert abs(out[i, j] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_gemm_power_of_two_scale_invariance():
    r = np.random.default_rng(5)
    a_q = e4m3.encode(r.standard_normal((16, 128)) * 10)
    b_q = e4m3.encode(r.standard_normal((128, 128)) * 10)
    base = gemm.gemm_blockscaled(a_q, np.ones((16, 1), np.float32), b_q, np.ones((1, 1), np.float32))
    out = gemm.gemm_blockscaled(a_q, np.full((16, 1), 0.25, np.float32), b_q, np.full((1, 1), 8.0, np.float32))
    assert np.array_equal(out, base * 2.0)


def test_grouped_gemm_slices_and_gather():
    r = np.random.default_rng(6)
    a = r.standard_normal((20, 256)).astype(np.float32)
    a_q, a_s = quant.quant_1x128(a)
    bs = [quant.quant_128x128(r.standard_normal((128, 256)).astype(np.float32)) for _ in range(3)]
    b_q = np.stack([b[0] for b in bs])
    b_s = np.stack([b[1] for b in bs])
    offsets = np.array([0, 7, 7, 12])                   # group 1 empty
    gather = r.integers(0, 20, size=12)
    out = gemm.grouped_gemm_blockscaled(a_q, a_s, gather, b_q, b_s, offsets)
    for g, (lo, hi) in enumerate(zip(offsets[:-1], offsets[1:])):
        for m in range(lo, hi):
            want = quant.dequant_1x128(a_q[gather[m]:gather[m] + 1], a_s[gather[m]:gather[m] + 1]) @ \
                quant.dequant_128x128(b_q[g], b_s[g]).T
            assert np.allclose(out[m], want[0], rtol=1e-13, atol=1e-13)
