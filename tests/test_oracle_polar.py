"""Pins for the oracle's recursive polar stage 1 (CPU only)."""

import math

import numpy as np
import pytest
from scipy import special, stats

from oracle import polar, quantize


def _beta_cdf(k):
    return lambda p: special.betainc(k / 2.0, k / 2.0, np.sin(np.clip(p, 0, math.pi / 2)) ** 2)


def test_angle_law_of_each_level_is_the_stated_beta_law():
    # angles of the exact transform of Gaussian vectors (uniform directions) at every level
    y = np.random.default_rng(0).standard_normal((20000, 64))
    _, (_, _, psi1), ang = polar.exact_polar(y)
    assert stats.kstest(psi1.ravel()[:50000], _beta_cdf(1)).pvalue > 1e-3  # uniform on [0, pi/2]
    for lvl, a in enumerate(ang, start=2):
        k = 1 << (lvl - 1)
        assert stats.kstest(a.ravel()[:50000], _beta_cdf(k)).pvalue > 1e-3, lvl
        f = polar.angle_density(k)
        grid = np.linspace(0, math.pi / 2, 20001)
        assert abs(np.trapezoid(f(grid), grid) - 1.0) < 1e-6


@pytest.mark.parametrize("ab", [2, 3])
def test_level_tables(ab):
    L = 1 << ab
    # level 1 (uniform law): equal cells with centred levels
    t1 = polar.angle_table(1, ab)
    assert np.allclose(t1.centroids64, (np.arange(L) + 0.5) * (math.pi / 2) / L, rtol=0, atol=1e-15)
    for k in (2, 8, 64):
        t = polar.angle_table(k, ab)
        # symmetric about pi/4, thresholds at midpoints
        assert np.allclose(t.centroids64 + t.centroids64[::-1], math.pi / 2, rtol=0, atol=1e-12)
        assert np.allclose(t.thresholds64, 0.5 * (t.centroids64[:-1] + t.centroids64[1:]), rtol=0, atol=0)
        # Lloyd fixed point: each level is the mean of its cell (dense trapezoid rule, not quad)
        f = polar.angle_density(k)
        edges = np.concatenate(([0.0], t.thresholds64, [math.pi / 2]))
        for j in range(L):
            g = np.linspace(edges[j], edges[j + 1], 200001)
            w = f(g)
            assert abs(np.trapezoid(g * w, g) / np.trapezoid(w, g) - t.centroids64[j]) < 1e-8
        # the fp32 decision constants are cos^2 and sin^2 of the thresholds
        assert np.allclose(t.c2 + t.s2, 1.0, atol=1e-7)


def test_decisions_match_exact_angles_away_from_thresholds():
    pc = polar.make_polar_codec(64, 2, 1)
    y = (np.random.default_rng(1).standard_normal((3000, 64)) * 2.0).astype(np.float32)
    codes = polar.encode(y, pc, pre_rotated=True)
    _, (na, nb, psi1), ang = polar.exact_polar(y)
    pair, nodes = polar.decode_fields(codes, pc)
    assert np.array_equal(pair & 1, na.astype(np.uint32)) and np.array_equal((pair >> 1) & 1, nb.astype(np.uint32))
    for got, psi, lv in [(pair >> 2, psi1, pc.levels[0])] + [(nodes[i], ang[i], pc.levels[i + 1]) for i in range(len(ang))]:
        want = np.sum(psi[..., None] >= lv.thresholds64, axis=-1)
        near = np.min(np.abs(psi[..., None] - lv.thresholds64), axis=-1) < 1e-5
        assert np.all((got == want) | near)
        assert np.mean(got == want) > 0.999


def test_record_layout_by_hand():
    # d = 4, ab = 2: pair 0 at bits 0-3, pair 1 at bits 4-7 ([sign a, sign b, 2 angle bits]),
    # the root node's index at bits 8-9
    pc = polar.make_polar_codec(4, 2, 1)
    y = np.array([[-1.0, 0.1, 0.2, 3.0]], np.float32)  # pair 0: a < 0, angle small; pair 1: angle large
    c = polar.encode(y, pc, pre_rotated=True)
    pair, nodes = polar.decode_fields(c, pc)
    bits = int.from_bytes(c.bits[0].tobytes(), "little")
    assert bits & 0xF == pair[0, 0] and (bits >> 4) & 0xF == pair[0, 1] and (bits >> 8) & 0x3 == nodes[0][0, 0]
    assert pair[0, 0] & 3 == 1 and (pair[0, 0] >> 2) == 0       # a negative, b positive, psi ~ 0.1
    assert pair[0, 1] & 3 == 0 and (pair[0, 1] >> 2) == 3       # psi = atan(15) near pi/2
    assert nodes[0][0, 0] == 3                                  # |pair 1| >> |pair 0|
    assert bits >> 10 == 0                                      # pad bits zero
    assert pc.n_bits == 10 and c.bits.shape[1] == 4


def test_bits_per_value():
    # 2 angle bits per node: d/2 (2 + 2) + (d/2 - 1) 2 bits, about 3 per coordinate, inside
    # the "3 to 4 bits per value" of the pages
    pc = polar.make_polar_codec(128, 2, 1)
    assert pc.n_bits == 382 and 3.0 <= (pc.n_bits + 16) / 128 <= 4.0


def test_fine_tables_reconstruct_the_direction_and_scores():
    # with 6 angle bits the chain encode -> decode returns the rotated direction closely, and
    # the scores approach the exact inner products
    pc = polar.make_polar_codec(32, 6, 3)
    g = np.random.default_rng(2)
    x = (g.standard_normal((200, 32)) * 3.0).astype(np.float32)
    codes = polar.encode(x, pc)
    u = polar.unit_directions(codes, pc)
    y = x.astype(np.float64) @ pc.rot[0].astype(np.float64).T
    yn = y / np.linalg.norm(y, axis=1, keepdims=True)
    assert np.max(np.linalg.norm(u - yn, axis=1)) < 0.08
    assert np.allclose(np.linalg.norm(u, axis=1), 1.0, atol=1e-6)  # cos^2 + sin^2 at every node
    q = g.standard_normal((1, 2, 32))
    s = polar.scores(q, codes, pc, 100, 2)
    exact = np.stack([q[0, h] @ x[h * 100:(h + 1) * 100].T.astype(np.float64) for h in range(2)])
    assert np.max(np.abs(s[0] - exact)) < 0.08 * np.max(np.abs(exact))
    # the stored radius is the exact fp16 norm
    assert np.array_equal(codes.norms & 0xFFFF, quantize.f16_norm_bits(x))


def test_more_angle_bits_less_error():
    g = np.random.default_rng(4)
    y = g.standard_normal((2000, 64)).astype(np.float32)
    yn = y / np.linalg.norm(y, axis=1, keepdims=True)
    errs = []
    for ab in (1, 2, 3):
        pc = polar.make_polar_codec(64, ab, 1)
        u = polar.unit_directions(polar.encode(y, pc, pre_rotated=True), pc)
        errs.append(np.mean(np.sum((u - yn) ** 2, axis=1)))
    assert errs[0] > errs[1] > errs[2]


def test_each_level_table_fits_that_levels_angles():
    # a codec's table at level l is the Lloyd-Max table of the angles that level actually sees:
    # cell means of exact angles of Gaussian vectors sit on the table's levels (within 5 standard
    # errors), which a table built for another level's law would miss
    pc = polar.make_polar_codec(64, 2, 1)
    y = np.random.default_rng(7).standard_normal((40000, 64))
    _, (_, _, psi1), ang = polar.exact_polar(y)
    for lvl, psi in enumerate([psi1] + ang, start=1):
        lv = pc.levels[lvl - 1]
        assert lv.k == 1 << (lvl - 1)
        x = psi.ravel()
        cell = np.searchsorted(lv.thresholds64, x, side="right")
        for j in range(len(lv.centroids64)):
            s = x[cell == j]
            se = s.std() / math.sqrt(len(s))
            assert abs(s.mean() - lv.centroids64[j]) < 5 * se + 1e-12, (lvl, j, s.mean(), lv.centroids64[j], se)


def _two_stage_values(n, d, seed):
    from oracle import codec as oc

    vo = oc.make_codec(d, 3, 0, 3, 4)
    x = np.random.default_rng(seed).standard_normal((n, d)).astype(np.float32)
    return vo, quantize.encode(x, vo)


def test_attention_matches_textbook_route_over_reconstructed_keys():
    # second route: keys rebuilt in the original space (nbar Pi^T u^), logits q . k^ there, a
    # textbook softmax per (sequence, query head), grouped-query mapping h -> h // (hq / hkv)
    d, S, hq, hkv, n = 64, 2, 4, 2, 50
    pc = polar.make_polar_codec(d, 2, 1)
    g = np.random.default_rng(3)
    x = g.standard_normal((S * hkv * n, d)).astype(np.float32)
    kc = polar.encode(x, pc)
    vo, vc = _two_stage_values(S * hkv * n, d, 4)
    q = g.standard_normal((S, hq, d))
    scale = 0.125
    got = polar.attend(q, kc, vc, pc, vo, n, hkv, scale)
    from oracle import estimate as oe

    u = polar.unit_directions(kc, pc)
    nbar = quantize.f16_value((kc.norms & 0xFFFF).astype(np.uint16))
    khat = (u @ pc.rot[0].astype(np.float64)) * nbar[:, None]  # rows: nbar Pi^T u^
    vt = oe.dequantize(vc, vo)
    for s in range(S):
        for h in range(hq):
            blk = s * hkv + h // (hq // hkv)
            sl = slice(blk * n, (blk + 1) * n)
            lg = scale * (khat[sl] @ q[s, h])
            p = np.exp(lg - lg.max())
            p /= p.sum()
            want = p @ vt[sl]
            assert np.allclose(got[s, h], want, rtol=1e-10, atol=1e-12)


def test_attention_with_zero_scale_is_the_mean_value():
    d, n = 64, 33
    pc = polar.make_polar_codec(d, 2, 1)
    x = np.random.default_rng(5).standard_normal((n, d)).astype(np.float32)
    vo, vc = _two_stage_values(n, d, 6)
    from oracle import estimate as oe

    got = polar.attend(np.ones((1, 1, d)), polar.encode(x, pc), vc, pc, vo, n, 1, 0.0)
    assert np.allclose(got[0, 0], oe.dequantize(vc, vo).mean(axis=0), rtol=1e-12, atol=1e-14)
