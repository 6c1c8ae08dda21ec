"""Pins for the oracle's calibrated codebooks and the TurboESM residual-sign codec (CPU only)."""

import math
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate

from oracle import calibrate, codec, estimate, quantize
from tests.conftest import golden


def test_calibration_follows_the_walkthrough_worked_example():
    # 7minutos.es, "Etapa 1": data 1.42, -0.85, 2.31, 0.97 with levels 0.5 and 1.5 move to the
    # printed 0.06 and 1.86 after one update (exact means 0.06 and 1.865)
    g = golden("lloyd_worked_example.json")
    one = calibrate.calibrate_codebook(g["data"], g["init_levels"], max_iter=1)
    assert one.iterations == 1
    assert np.allclose(one.centroids, g["first_update_printed"], atol=g["printed_precision"], rtol=0)
    assert np.allclose(one.centroids, [0.06, 1.865], atol=1e-6, rtol=0)
    # to the fixed point: one sample alone, the other three averaged
    fix = calibrate.calibrate_codebook(g["data"], g["init_levels"])
    assert np.allclose(fix.centroids, [-0.85, (0.97 + 1.42 + 2.31) / 3], atol=1e-6, rtol=0)
    assert fix.thresholds[0] == np.float32(0.5 * (-0.85 + 4.70 / 3))
    # mean residual magnitude at the fixed point, by hand
    want = (0.0 + abs(1.42 - 4.70 / 3) + abs(2.31 - 4.70 / 3) + abs(0.97 - 4.70 / 3)) / 4
    assert abs(fix.ebar - want) < 1e-12


def test_empty_cell_keeps_its_level_and_ties_go_up():
    cal = calibrate.calibrate_codebook([1.0, 1.0, 1.0], [-5.0, 0.0, 1.0], max_iter=1)
    assert cal.centroids[0] == -5.0  # no sample in cell 0
    # 0.5 is the midpoint of 0 and 1: a sample there belongs to the upper cell
    cal = calibrate.calibrate_codebook([0.5, 0.0], [0.0, 1.0], max_iter=1)
    assert np.array_equal(cal.centroids, np.float32([0.0, 0.5]))


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 2)])
def test_calibration_on_the_coordinate_law_finds_its_lloyd_max_levels(d, bits):
    # directions of uniform random vectors: the coordinate law of "Etapa 1"; started at an
    # offset codebook, the sample rule returns to the law's Lloyd-Max levels
    cb = codec.lloyd_max_beta(d, bits)
    g = np.random.default_rng(d + bits)
    x = g.standard_normal((20000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    cal = calibrate.calibrate_codebook(u, cb.centroids.astype(np.float64) * 1.3, max_iter=500, rel_tol=1e-10)
    assert np.max(np.abs(cal.centroids - cb.centroids)) < 2e-3 / math.sqrt(d) * 8
    # and e equals the law's mean |u - c(u)| (numerical integration of the density)
    f = codec.beta_coord_density(d)
    c = cb.centroids.astype(np.float64)
    t = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
    e = sum(integrate.quad(lambda v, cj=c[j]: abs(v - cj) * f(np.array([v]))[0], t[j], t[j + 1], limit=200)[0]
            for j in range(len(c)))
    assert abs(cal.ebar - e) < 0.01 * e


def test_mean_residual_magnitude_is_the_best_first_order_correction():
    # for u - c(u) = r, E (|r| - s)^2 over the scale s is smallest at s = E|r|, the calibrated e
    g = np.random.default_rng(5)
    u = g.standard_normal(50000) * 0.12
    cal = calibrate.calibrate_codebook(u, np.linspace(-0.3, 0.3, 8))
    lv = cal.centroids.astype(np.float64)
    r = u - lv[calibrate.cells(lv, u)]

    def mse(s):
        return np.mean((r - s * np.sign(r)) ** 2)
    assert mse(cal.ebar) < mse(0.9 * cal.ebar) and mse(cal.ebar) < mse(1.1 * cal.ebar)
    assert mse(cal.ebar) < np.mean(r ** 2)


def test_f16_exact_rounding():
    g = np.random.default_rng(6)
    v = np.exp(g.uniform(-12, 11, 2000))
    got = np.array([quantize.f16_rne_exact(Fraction(float(a))) for a in v])
    assert np.array_equal(got, v.astype(np.float16).view(np.uint16))
    # ties to even: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    assert quantize.f16_rne_exact(Fraction(1) + Fraction(1, 2 ** 11)) == 0x3C00
    assert quantize.f16_rne_exact(Fraction(1) + Fraction(3, 2 ** 11)) == 0x3C02
    assert quantize.f16_rne_exact(Fraction(65520)) == quantize.F16_INF_BITS


def test_turboesm_record_and_reconstruction():
    d, bits = 64, 3
    base = codec.make_codec(d, bits, 0, 1, 2)
    g = np.random.default_rng(7)
    xs = g.standard_normal((3000, d)) * np.where(g.random(d) < 0.05, 5.0, 1.0)
    cal = calibrate.calibrate_codebook(calibrate.rotated_directions(xs, base), base.centroids)
    tc = calibrate.turboesm_codec(base, cal)
    assert tc.m == d and np.array_equal(tc.sketch, np.eye(d, dtype=np.float32))
    assert tc.resid_scale == np.float32(cal.ebar * d / math.sqrt(math.pi / 2))
    x = (g.standard_normal((200, d)) * 3.0).astype(np.float32)
    codes = quantize.encode(x, tc, keep=True)
    # the sign bits are the signs of the rotated residual, coordinate by coordinate
    assert np.array_equal(codes.bits, (codes.resid >= 0).astype(codes.bits.dtype))
    # the high half of the norm word is fp16(nbar * resid_scale), exactly rounded
    n16 = (codes.norms & 0xFFFF).astype(np.uint16)
    nb = quantize.f16_value(n16)
    hi = (codes.norms >> 16).astype(np.uint16)
    assert np.array_equal(hi, np.float64(nb * np.float64(tc.resid_scale)).astype(np.float16).view(np.uint16))
    # reconstruction: Pi^T nbar (c[idx] + e sign), e up to that fp16 rounding
    xt = estimate.dequantize(codes, tc)
    index = codes.index
    sgn = 2.0 * codes.bits.astype(np.float64) - 1.0
    want = (nb[:, None] * (cal.centroids.astype(np.float64)[index] + cal.ebar * sgn)) @ tc.rot[0].astype(np.float64)
    err = np.abs(xt - want).max(axis=1)
    assert np.all(err <= 2.0 ** -10 * nb * cal.ebar * math.sqrt(d) + 1e-12)
    # the correction helps: reconstruction error below that of the index alone
    x_mse = (nb[:, None] * cal.centroids.astype(np.float64)[index]) @ tc.rot[0].astype(np.float64)
    assert np.mean((xt - x) ** 2) < np.mean((x_mse - x) ** 2)
