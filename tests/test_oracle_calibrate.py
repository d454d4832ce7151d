"""Pins for the bias-adjustment rule and the stored skewed-workload bias."""
import numpy as np

import synth
from oracle import calibrate, route


def test_adjust_moves_toward_target():
    b = np.zeros(4, np.float32)
    out = calibrate.adjust(b, np.array([5, 1, 3, 0]), np.array([3, 3, 3, 3]), 0.5)
    assert out.tolist() == [-0.5, 0.5, 0.0, 0.5]          # overloaded down, underloaded up, on target unchanged


def test_calibration_reaches_small_targets():
    sc = synth.gen_scores(2000, 16, cfg_id=11)
    target = np.array([400, 300, 250, 200, 180, 160, 140, 120, 100, 80, 70, 0, 0, 0, 0, 0], np.float64)
    target = target * (2000 * 2 / target.sum())
    bias, ld = calibrate.calibrate(sc, target, 4, 4, 2, iters=300)
    assert np.all(ld[target == 0] == 0)
    assert np.abs(ld - target).max() <= 0.05 * 2000 * 2 / 16


def test_stored_skew_bias_reproduces_the_profile():
    s = synth.V3_SKEW
    bias = synth.skew_bias()
    assert bias.shape == (256,) and bias.dtype == np.float32
    assert (bias == np.float32(-10)).sum() == 16
    x = synth.bf16_bits_to_f32(synth.gen_x(s, tokens=2048))          # a different batch than the calibration one
    wr = synth.bf16_bits_to_f32(synth.gen_router_w(s))
    sc = route.sigmoid_scores(route.router_logits(x, wr))
    idx, _ = route.select(sc, bias, s.n_group, s.topk_group, s.top_k)
    ld = calibrate.loads(idx, 256)
    assert (ld == 0).sum() >= 16
    assert 12 <= ld.max() / ld.mean() <= 28


def test_balancing_update_by_hand():
    # E = 4, T = 2, k = 4: loads [3, 1, 2, 2], mean 2 -> expert 0 overloaded, 1 underloaded
    idx = np.array([[0, 0, 1, 2], [0, 2, 3, 3]])
    bias = np.array([0.5, -0.25, 0.0, 1e-3], np.float32)
    g = 0.01
    got = calibrate.update(bias, idx, 4, g)
    want = np.array([np.float32(0.5) - np.float32(g), np.float32(-0.25) + np.float32(g), 0.0, np.float32(1e-3)],
                    np.float32)
    assert np.array_equal(got, want)


def test_balancing_update_fractional_mean():
    # T*k = 6 over E = 4: mean 1.5, so every expert moves (none sits exactly at the mean)
    idx = np.array([[0, 1, 1], [2, 1, 0]])
    got = calibrate.update(np.zeros(4, np.float32), idx, 4, 0.5)
    assert np.array_equal(got, np.array([-0.5, -0.5, 0.5, 0.5], np.float32))   # loads 2, 3, 1, 0
