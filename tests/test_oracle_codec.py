"""Pins for the oracle's codec construction (rng, rotation, sketch, codebook).  CPU only."""

import math

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codec, rng
from tests.conftest import golden


# ----------------------------------------------------------------------------- rng


def test_splitmix64_reference_outputs():
    g = golden("splitmix64_reference.json")
    got = [rng.splitmix64(g["seed"], k) for k in range(len(g["outputs_hex"]))]
    assert got == [int(h, 16) for h in g["outputs_hex"]]


def test_box_muller_is_standard_normal():
    x = rng.gaussians(123, 200001)  # odd count exercises the unpaired tail
    assert x.shape == (200001,)
    assert abs(x.mean()) < 4 / math.sqrt(x.size)
    assert abs(x.var() - 1.0) < 4 * math.sqrt(2.0 / x.size)
    assert stats.kstest(x, "norm").pvalue > 1e-3
    # cos and sin halves are each N(0,1) and uncorrelated
    a, b = x[0:-1:2], x[1::2]
    assert abs(np.corrcoef(a, b)[0, 1]) < 4 / math.sqrt(a.size)
    assert stats.kstest(b, "norm").pvalue > 1e-3


def test_gaussians_prefix_stable():
    assert np.array_equal(rng.gaussians(7, 10)[:7], rng.gaussians(7, 7))


# ----------------------------------------------------------------------------- rotation


@pytest.mark.parametrize("d", [3, 64, 128, 200])
def test_rotation_orthogonal(d):
    p64 = codec.haar_rotation64(11, d)
    assert np.max(np.abs(p64.T @ p64 - np.eye(d))) < 1e-12
    p32 = codec.haar_rotation(11, d).astype(np.float64)
    assert np.max(np.abs(p32.T @ p32 - np.eye(d))) < 2e-6


def test_rotation_is_haar():
    # For Haar matrices E[tr P] = 0 and E[(tr P)^2] = 1; QR without the sign fix fails this.
    T = 400
    tr = np.array([np.trace(codec.haar_rotation64(1000 + s, 8)) for s in range(T)])
    assert abs(tr.mean()) < 4 / math.sqrt(T)
    assert abs((tr ** 2).mean() - 1.0) < 4 * math.sqrt(2.0 / T)


@pytest.mark.parametrize("d", [64, 128])
def test_rotated_coordinate_moments(d):
    # u = P x / ||x|| for Gaussian x is uniform on the sphere: E u^2 = 1/d, E u^4 = 3/(d(d+2)).
    p = codec.haar_rotation64(5, d)
    x = np.random.default_rng(0).standard_normal((4000, d))
    u = (x @ p.T) / np.linalg.norm(x, axis=1, keepdims=True)
    u2, u4 = u ** 2, u ** 4
    n = u.size
    assert abs(u2.mean() - 1 / d) < 4 * u2.std() / math.sqrt(n)
    assert abs(u4.mean() - 3 / (d * (d + 2))) < 4 * u4.std() / math.sqrt(n)


def test_rope_then_rotation_preserves_scores():
    # TurboESM summary 2.A: (Pi R_i q)^T (Pi R_j k) = q^T R_i^T R_j k.
    d = 64
    p = codec.haar_rotation64(3, d)
    g = np.random.default_rng(1)
    q, k = g.standard_normal(d), g.standard_normal(d)

    def rope(v, pos):
        half = d // 2
        theta = pos * 10000.0 ** (-2.0 * np.arange(half) / d)
        c, s = np.cos(theta), np.sin(theta)
        return np.concatenate([v[:half] * c - v[half:] * s, v[:half] * s + v[half:] * c])

    for i, j in [(0, 0), (5, 17), (1023, 3)]:
        lhs = (p @ rope(q, i)) @ (p @ rope(k, j))
        rhs = rope(q, i) @ rope(k, j)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


def test_head_rotations_compose():
    d = 16
    hr = codec.head_rotations(4, [9, 10], d).astype(np.float64)
    p = codec.haar_rotation64(4, d)
    for h, s in enumerate([9, 10]):
        want = p @ codec.haar_rotation64(s, d)
        assert np.max(np.abs(hr[h] - want)) < 1e-7
        assert np.max(np.abs(hr[h].T @ hr[h] - np.eye(d))) < 2e-6


def test_sketch_gaussian():
    s = codec.gaussian_sketch(2, 200, 200).astype(np.float64).ravel()
    assert abs(s.mean()) < 4 / math.sqrt(s.size)
    assert abs(s.var() - 1) < 4 * math.sqrt(2 / s.size)
    assert np.array_equal(codec.gaussian_sketch(2, 3, 4).ravel(), rng.gaussians(2, 12).astype(np.float32))


# ----------------------------------------------------------------------------- codebook


@pytest.mark.parametrize("d", [3, 4, 64, 200])
def test_density_normalised_with_sphere_moments(d):
    f = codec.beta_coord_density(d)
    one = integrate.quad(lambda x: float(f(x)), -1, 1, epsabs=1e-13)[0]
    m2 = integrate.quad(lambda x: x * x * float(f(x)), -1, 1, epsabs=1e-14)[0]
    m4 = integrate.quad(lambda x: x ** 4 * float(f(x)), -1, 1, epsabs=1e-15)[0]
    assert abs(one - 1) < 1e-10
    assert abs(m2 - 1 / d) < 1e-10
    assert abs(m4 - 3 / (d * (d + 2))) < 1e-10


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_d3_is_uniform_quantizer(bits):
    # d = 3: f_3 is uniform on [-1, 1]; the optimum is the uniform quantizer.
    L = 1 << bits
    cb = codec.lloyd_max_beta(3, bits)
    want = -1.0 + (2.0 * np.arange(L) + 1.0) / L
    assert np.max(np.abs(cb.centroids64 - want)) < 1e-12
    assert abs(cb.mse - 1.0 / (3 * L * L)) < 1e-12


@pytest.mark.parametrize("d", [4, 64, 128, 200])
def test_codebook_one_bit_closed_form(d):
    # One bit: levels +-E|u| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    cb = codec.lloyd_max_beta(d, 1)
    want = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert np.allclose(cb.centroids64, [-want, want], rtol=1e-13, atol=0)
    assert abs(cb.mse - (1.0 / d - want * want)) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_codebook_matches_max_1960(bits):
    g = golden("max1960_gaussian.json")
    c, t, mse = codec.lloyd_max_gauss(bits)
    L = 1 << bits
    assert np.allclose(c[L // 2:], g["levels"][str(bits)], atol=g["abs_tol"], rtol=0)
    assert abs(mse - g["mse"][str(bits)]) < 2e-4 * max(1.0, g["mse"][str(bits)] * 10)


@pytest.mark.parametrize("bits", [2, 3])
def test_beta_codebook_tends_to_gaussian(bits):
    c_g, _, mse_g = codec.lloyd_max_gauss(bits)
    d = 4000
    cb = codec.lloyd_max_beta(d, bits)
    assert np.max(np.abs(cb.centroids64 * math.sqrt(d) - c_g)) < 2e-3
    assert abs(cb.mse * d - mse_g) < 1e-3
    # and the gap shrinks with d (O(1/d))
    near = codec.lloyd_max_beta(400, bits)
    assert np.max(np.abs(near.centroids64 * math.sqrt(400) - c_g)) > np.max(np.abs(cb.centroids64 * math.sqrt(d) - c_g))


@pytest.mark.parametrize("d,bits", [(64, 2), (64, 3), (128, 2), (128, 3), (200, 2)])
def test_codebook_fixed_point_symmetric_sorted(d, bits):
    cb = codec.lloyd_max_beta(d, bits)
    c = cb.centroids64
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    assert np.array_equal(cb.thresholds64, 0.5 * (c[:-1] + c[1:]))
    mass, moment = codec._beta_cell_stats(d)
    again = codec.lloyd_step(c, mass, moment, -1.0, 1.0)
    assert np.max(np.abs(again - c)) < 1e-13 * np.max(np.abs(c))
    # MSE by quadrature is less than any perturbed codebook's (local optimality)
    f = codec.beta_coord_density(d)
    for eps in (1e-3, -1e-3):
        pert = c * (1 + eps)
        assert codec._cell_mse(f, pert, 0.5 * (pert[:-1] + pert[1:]), -1, 1) > cb.mse
    # the codebook depends only on (d, bits)
    assert np.array_equal(codec.lloyd_max_beta(d, bits).centroids, cb.centroids)


def test_lloyd_worked_example():
    g = golden("lloyd_worked_example.json")
    data, init = np.array(g["data"]), np.array(g["init_levels"])
    # assignment with the initial boundary
    t0 = 0.5 * (init[0] + init[1])
    assert abs(t0 - g["init_boundary_printed"]) <= g["printed_precision"]
    assign = np.where(data >= t0, init[1], init[0])
    assert np.array_equal(assign, g["first_assignment_printed"])
    first = codec.lloyd_step_samples(init, data)
    assert np.allclose(first, g["first_update_printed"], atol=g["printed_precision"], rtol=0)
    assert abs(0.5 * (first[0] + first[1]) - g["first_update_boundary_printed"]) <= g["printed_precision"]
    # continuing reaches a fixed point where MSE stops improving
    lv = first
    for _ in range(10):
        lv = codec.lloyd_step_samples(lv, data)
    assert np.allclose(codec.lloyd_step_samples(lv, data), lv)
    assert np.allclose(lv, [-0.85, (0.97 + 1.42 + 2.31) / 3])


def test_sample_and_density_lloyd_agree():
    # The density route and the sample route are the same rule: a large Gaussian sample's
    # one-step update matches the density update.
    x = np.random.default_rng(3).standard_normal(2_000_000)
    lv = np.array([-1.0, -0.3, 0.4, 1.2])
    mass, moment = codec._gauss_cell_stats()
    a = codec.lloyd_step(lv, mass, moment, -np.inf, np.inf)
    b = codec.lloyd_step_samples(lv, x)
    assert np.max(np.abs(a - b)) < 5e-3


def test_make_codec_shapes():
    c = codec.make_codec(64, 2, 32, 1, 2)
    assert c.rot.shape == (1, 64, 64) and c.sketch.shape == (32, 64)
    assert c.centroids.dtype == np.float32 and c.thresholds.shape == (3,)
    c0 = codec.make_codec(64, 3, 0, 1, 2)
    assert c0.sketch is None
