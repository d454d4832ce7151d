"""Pins for the oracle's E4M3FN codec (closed forms, brute force, a library cast)."""
import numpy as np
import pytest
import torch

from oracle import e4m3


def test_closed_form_table():
    d = e4m3.DECODE
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0          # largest finite
    assert d[0x08] == 2.0 ** -6                             # smallest normal
    assert d[0x01] == 2.0 ** -9                             # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert d[0x38] == 1.0 and d[0x40] == 2.0 and d[0x30] == 0.5
    assert d[0x3C] == 1.5 and d[0x77] == 240.0 and d[0x78] == 256.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])          # the only NaNs, no infinities
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d).sum() == 2 and np.isinf(d).sum() == 0
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                          # codes 0..126 ascend
    assert np.array_equal(d[0x80:0xFF], -pos)               # sign bit is a pure sign


def _brute_encode(a: float) -> int:
    """argmin over all finite non-negative codes, ties to the even code; saturating."""
    vals, codes = e4m3.finite_positive_grid()
    mag = abs(a)
    if mag >= 448.0:
        c = 0x7E
    else:
        dist = np.abs(vals - mag)
        best = np.flatnonzero(dist == dist.min())
        c = int(codes[best[0]]) if len(best) == 1 else int([x for x in codes[best] if x % 2 == 0][0])
    return c | (0x80 if np.signbit(a) else 0)


def _probe_values():
    vals, _ = e4m3.finite_positive_grid()
    mids = (vals[1:] + vals[:-1]) / 2
    r = np.random.default_rng(7)
    logu = np.exp2(r.uniform(-14, 10, 4000))
    probe = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), logu,
                            [448.0, 449.0, 463.99, 464.0, 465.0, 1e6, 2.0 ** -10, 2.0 ** -11, 1e-30]])
    return np.concatenate([probe, -probe])


def test_encode_matches_brute_force():
    p = _probe_values()
    got = e4m3.encode(p)
    want = np.array([_brute_encode(float(a)) for a in p], dtype=np.uint8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (p[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_encode_fp32_inputs_same_as_fp64():
    p = _probe_values().astype(np.float32)
    assert np.array_equal(e4m3.encode(p), e4m3.encode(p.astype(np.float64)))


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def test_against_torch_float8_cast():
    r = np.random.default_rng(3)
    v = np.concatenate([r.standard_normal(200000) * 50, r.uniform(-448, 448, 200000),
                        np.exp2(r.uniform(-12, 8.8, 100000))]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v), t)


def test_special_inputs():
    assert e4m3.encode(np.array([np.nan]))[0] == 0x7F
    assert e4m3.encode(np.array([np.inf, -np.inf])).tolist() == [0x7E, 0xFE]
    assert e4m3.encode(np.array([-0.0]))[0] == 0x80


@pytest.mark.parametrize("mag", [2.0 ** -9, 1e-3, 0.75, 3.3, 100.0, 447.0])
def test_half_ulp(mag):
    vals, _ = e4m3.finite_positive_grid()
    i = np.searchsorted(vals, mag, side="right") - 1
    assert e4m3.half_ulp(mag) == (vals[i + 1] - vals[i]) / 2
