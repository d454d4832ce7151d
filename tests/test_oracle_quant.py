"""Pins for the oracle's 1x128 / 128x128 quantisation (invariants, exact rationals)."""
from fractions import Fraction

import numpy as np

from oracle import e4m3, quant


def _nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational, by bracketing (positive normal range)."""
    f = np.float32(float(fr))                # within 1 ulp of the true value
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    errs = [abs(Fraction(float(c)) - fr) for c in cands]
    best = min(errs)
    ties = [c for c, e in zip(cands, errs) if e == best]
    if len(ties) == 1:
        return ties[0]
    return [c for c in ties if (np.array(c, np.float32).view(np.uint32) & 1) == 0][0]


def _tiles(seed=0, rows=24, cols=512):
    r = np.random.default_rng(seed)
    v = r.standard_normal((rows, cols)).astype(np.float32)
    v[1] *= np.float32(1e-4)
    v[2] *= np.float32(3e4)
    v[3, :128] = 0.0                                   # an all-zero tile
    v[4, 128:256] = np.float32(-2.5)                   # a constant tile
    v[5, :] = np.exp2(r.uniform(-20, 5, cols)).astype(np.float32) * np.sign(r.standard_normal(cols)).astype(np.float32)
    return v


def test_scale_is_correctly_rounded_amax_over_448():
    v = _tiles()
    _, s = quant.quant_1x128(v)
    tiles = v.reshape(v.shape[0], -1, 128)
    for i in range(tiles.shape[0]):
        for j in range(tiles.shape[1]):
            amax = np.max(np.abs(tiles[i, j]))
            want = np.float32(1.0) if amax == 0 else _nearest_f32(Fraction(float(amax)) / 448)
            assert s[i, j] == want


def test_quotients_are_correctly_rounded():
    v = _tiles(1, rows=6)
    q, s = quant.quant_1x128(v)
    r = np.random.default_rng(5)
    for _ in range(300):
        i, c = r.integers(v.shape[0]), r.integers(v.shape[1])
        if v[i, c] == 0:
            continue
        quot = Fraction(float(abs(v[i, c]))) / Fraction(float(s[i, c // 128]))
        if quot < Fraction(2.0 ** -126):
            continue
        code = e4m3.encode(np.array([float(_nearest_f32(quot))]))[0]
        assert q[i, c] & 0x7F == code


def test_amax_element_maps_to_448():
    v = _tiles()
    q, _ = quant.quant_1x128(v)
    tiles = v.reshape(v.shape[0], -1, 128)
    qt = q.reshape(tiles.shape)
    for i in range(tiles.shape[0]):
        for j in range(tiles.shape[1]):
            t = tiles[i, j]
            if np.max(np.abs(t)) == 0:
                continue
            k = int(np.argmax(np.abs(t)))
            assert qt[i, j, k] == (0xFE if t[k] < 0 else 0x7E)


def test_dequant_error_within_half_ulp_times_scale():
    v = _tiles()
    q, s = quant.quant_1x128(v)
    deq = quant.dequant_1x128(q, s)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    mag = np.abs(v.astype(np.float64)) / srep
    # |v/s| is first rounded to fp32 (relative 2^-24), then to the e4m3 grid
    bound = e4m3.half_ulp(np.minimum(mag, 448.0)) * srep * (1 + 2.0 ** -20) + np.abs(v) * 2.0 ** -23
    assert np.all(np.abs(deq - v) <= bound)


def test_zero_tile():
    v = np.zeros((2, 256), np.float32)
    v[1, 200] = np.float32(-0.0)
    q, s = quant.quant_1x128(v)
    assert np.all(s == 1.0)
    assert np.all((q & 0x7F) == 0)


def test_grid_values_times_power_of_two_roundtrip():
    r = np.random.default_rng(2)
    codes = r.integers(0, 0x7F, size=(8, 256)).astype(np.uint8)
    codes[:, ::128] = 0x7E                             # amax = 448 * 2^k exactly
    codes |= (r.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    for k in (-20, -3, 0, 5, 30):
        v = (e4m3.decode(codes) * 2.0 ** k).astype(np.float32)
        q, s = quant.quant_1x128(v)
        assert np.all(s == np.float32(2.0 ** k))
        nz = e4m3.decode(codes) != 0
        assert np.array_equal(q[nz], codes[nz])


def test_128x128_blocks_are_independent_tiles():
    r = np.random.default_rng(4)
    w = (r.standard_normal((256, 384)) * np.exp2(r.integers(-4, 4, size=(256, 1)))).astype(np.float32)
    q, s = quant.quant_128x128(w)
    assert s.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            # a 128x128 block is one tile of 16384 values: same rule as a 1x128 tile
            amax = np.max(np.abs(blk))
            assert s[bi, bj] == _nearest_f32(Fraction(float(amax)) / 448)
            quot = (blk / s[bi, bj]).astype(np.float32)
            assert np.array_equal(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128], e4m3.encode(quot))
    deq = quant.dequant_128x128(q, s)
    srep = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    bound = e4m3.half_ulp(np.abs(w) / srep) * srep * (1 + 2.0 ** -20) + np.abs(w) * 2.0 ** -23
    assert np.all(np.abs(deq - w) <= bound)


# ---- power-of-two (UE8M0) scales ----

def test_ue8m0_scale_is_the_smallest_power_of_two_covering_amax():
    v = _tiles(2)
    _, s = quant.quant_1x128(v, ue8m0=True)
    tiles = v.reshape(v.shape[0], -1, 128)
    for i in range(tiles.shape[0]):
        for j in range(tiles.shape[1]):
            amax = Fraction(float(np.max(np.abs(tiles[i, j]))))
            sc = Fraction(float(s[i, j]))
            if amax == 0:
                assert s[i, j] == 1.0
                continue
            m, _ = np.frexp(float(s[i, j]))
            assert m == 0.5                                   # a power of two
            assert amax <= 448 * sc < 2 * amax                # covers amax, and half of it would not


def test_ue8m0_codes_are_the_e4m3_rounding_of_the_exact_quotient():
    import torch
    v = _tiles(3)
    q, s = quant.quant_1x128(v, ue8m0=True)
    quot = v.reshape(v.shape[0], -1, 128) / s[..., None]       # exact: s is a power of two
    ref = torch.from_numpy(quot.reshape(v.shape).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(q, ref.numpy())


def test_ue8m0_exponent_clamp_and_dequant_bound():
    v = np.zeros((2, 256), np.float32)
    v[0, :128] = np.float32(1e-41)                            # amax / 448 below 2^-127: the scale clamps
    v[1] = np.random.default_rng(4).standard_normal(256).astype(np.float32) * 3
    q, s = quant.quant_1x128(v, ue8m0=True)
    assert s[0, 0] == np.float32(2.0 ** -127) and s[0, 1] == 1.0
    back = quant.dequant_1x128(q, s)
    half = e4m3.half_ulp(np.abs(v.astype(np.float64)) / np.repeat(s.astype(np.float64), 128, axis=1))
    assert np.all(np.abs(back[1] - v[1]) <= half[1] * np.repeat(s[1].astype(np.float64), 128) * (1 + 1e-12))


def test_ue8m0_weight_blocks():
    w = np.random.default_rng(6).standard_normal((256, 384)).astype(np.float32) * 0.05
    q, s = quant.quant_128x128(w, ue8m0=True)
    blocks = np.abs(w).reshape(2, 128, 3, 128).max(axis=(1, 3)).astype(np.float64)
    assert np.all(np.frexp(s)[0] == 0.5)
    assert np.all(blocks <= 448 * s) and np.all(448 * s < 2 * blocks)


def test_tiles_below_the_normal_range_take_the_smallest_normal_scale():
    """amax / 448 below the smallest normal fp32: s = 2^-126, and every quotient v / 2^-126 is
    exact (a power-of-two scaling), so the codes are the e4m3 rounding of v * 2^126 exactly;
    at amax = 448 * 2^-126 both readings meet; just above it the plain rule applies."""
    tiny = np.float32(2.0 ** -126)
    r = np.random.default_rng(11)
    rows = np.zeros((4, 128), np.float32)
    rows[0] = (r.standard_normal(128) * 1e-44).astype(np.float32)          # subnormal values
    rows[1] = (r.standard_normal(128) * 1e-38).astype(np.float32)          # amax / 448 subnormal
    rows[2] = (r.standard_normal(128) * 1e-40).astype(np.float32)
    rows[2, 7] = np.float32(448.0) * tiny                                   # amax exactly on the boundary
    rows[3] = rows[2]
    rows[3, 7] = np.nextafter(np.float32(448.0) * tiny, np.float32(1.0))    # one ulp above
    q, s = quant.quant_1x128(rows)
    assert s[0, 0] == tiny and s[1, 0] == tiny and s[2, 0] == tiny
    assert s[3, 0] == _nearest_f32(Fraction(float(rows[3, 7])) / 448) and s[3, 0] > tiny
    for i in range(3):
        exact = rows[i].astype(np.float64) * 2.0 ** 126          # exact in fp64, signed zeros kept
        assert np.all(np.abs(exact) <= 448.0)
        assert np.array_equal(q[i], e4m3.encode(exact))
