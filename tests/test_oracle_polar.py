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


# ---------------------------------------------------------------------- QJL stage on the residual


def _with_sketch(pc, S):
    import dataclasses

    return dataclasses.replace(pc, m=S.shape[0], sketch=np.asarray(S, np.float32))


def test_qjl_on_polar_residual_is_unbiased_where_polar_alone_is_not():
    """hada.io TurboQuant page, "Etapa 2: eliminação do erro oculto": the 1-bit stage on the
    polar stage's error removes its bias.  Over many Gaussian sketches the two-stage estimate's
    mean is the exact <Pi q, y>, within its own sampling error (plus the fp16 rounding of the
    residual norm and fp32 reconstruction rounding), while the polar stage alone stays off by
    many of those errors."""
    d, ab, T = 64, 2, 600
    base = polar.make_polar_codec(d, ab, 1)
    g = np.random.default_rng(11)
    y = g.standard_normal((3, d)).astype(np.float32)
    q = g.standard_normal(d)
    y64 = y.astype(np.float64)
    exact = y64 @ q
    est = np.empty((T, 3))
    rel_rn = None
    for t in range(T):
        S = np.random.default_rng(1000 + t).standard_normal((d, d)).astype(np.float32)
        pc = _with_sketch(base, S)
        c = polar.encode(y, pc, pre_rotated=True)
        # scores in the rotated space: the rotation applied to q is the identity here
        pc_id = _with_sketch(polar.PolarCodec(d, ab, np.eye(d, dtype=np.float32)[None], base.levels), S)
        est[t] = polar.scores(q[None, None, :], c, pc_id, 3, 1)[0, 0]
        if rel_rn is None:
            r = c.extra["resid"].astype(np.float64)
            rn = quantize.f16_value((c.norms >> 16).astype(np.uint16))
            rel_rn = np.abs(rn / np.linalg.norm(r, axis=1) - 1.0) * np.abs(r @ q)
            polar_only = polar.scores(q[None, None, :], polar.PolarCodes(c.bits, c.norms & 0xFFFF), 
                                      polar.PolarCodec(d, ab, np.eye(d, dtype=np.float32)[None], base.levels),
                                      3, 1)[0, 0]
    mean, se = est.mean(axis=0), est.std(axis=0, ddof=1) / np.sqrt(T)
    assert np.all(np.abs(mean - exact) <= 4.0 * se + rel_rn + 1e-5 * np.abs(exact).max())
    # the polar stage alone: biased by far more than the two-stage estimate's sampling error
    assert np.max(np.abs(polar_only - exact) / se) > 10.0


def test_qjl_residual_is_the_stage_one_error_and_matches_explicit_dequantisation():
    d, ab, m = 128, 3, 128
    pc = polar.make_polar_codec(d, ab, 1, m=m, sketch_seed=2)
    g = np.random.default_rng(4)
    x = (g.standard_normal((40, d)) * np.where(g.random(d) < 0.05, 8.0, 1.0)).astype(np.float32)
    c = polar.encode(x, pc)
    y = c.extra["y"].astype(np.float64)
    nbar = quantize.f16_value((c.norms & 0xFFFF).astype(np.uint16))
    u32 = c.extra["u32"].astype(np.float64)
    rec = (nbar[:, None] * u32).astype(np.float32).astype(np.float64)
    r = c.extra["resid"].astype(np.float64)
    # r = fl32(y - fl32(nbar u^)): the residual is the stage-1 error up to one fp32 rounding
    assert np.all(np.abs(y - rec - r) <= 2.0 ** -24 * np.abs(y - rec))
    # the fp32 reconstruction is the fp64 one of the same record within the product chain's rounding
    u64 = polar.unit_directions(c, pc)
    assert np.max(np.abs(u32 - u64)) <= (pc.L + 1) * 2.0 ** -24
    # the residual norm word: fp16 of the exact norm; the signs: exact signs of S r
    assert np.array_equal(c.norms >> 16, quantize.f16_norm_bits(c.extra["resid"]).astype(np.uint32))
    want_bits = (r @ pc.sketch.astype(np.float64).T >= 0).astype(np.uint32)
    got_bits = quantize.unpack_bits(c.sign, 1, m)
    z = r @ pc.sketch.astype(np.float64).T
    clear = np.abs(z) > 1e-9 * (np.abs(r) @ np.abs(pc.sketch.astype(np.float64)).T)
    assert np.array_equal(got_bits[clear], want_bits[clear])
    # scores equal the inner products with the explicitly dequantised keys
    q = g.standard_normal((1, 2, d))
    sc = polar.scores(q, c, pc, 40, 1)[0]
    xt = polar.dequantize(c, pc)
    assert np.max(np.abs(sc - q[0] @ xt.T)) <= 1e-12 * np.max(np.abs(sc))


def test_qjl_on_polar_zero_residual():
    """A vector that is exactly its own stage-1 reconstruction: residual 0, every sign bit 1
    (a zero dot product counts as +), rn16 = 0, and the QJL term vanishes."""
    d, ab, m = 64, 2, 64
    pc = polar.make_polar_codec(d, ab, 1, m=m, sketch_seed=5)
    g = np.random.default_rng(9)
    c0 = polar.encode(g.standard_normal((8, d)).astype(np.float32), pc, pre_rotated=True)
    nbar = quantize.f16_value((c0.norms & 0xFFFF).astype(np.uint16)).astype(np.float32)
    y = (nbar[:, None] * c0.extra["u32"]).astype(np.float32)  # on the grid
    c = polar.encode(y, pc, pre_rotated=True)
    same = np.all(c.bits == c0.bits, axis=1) & ((c.norms & 0xFFFF) == (c0.norms & 0xFFFF))
    assert same.sum() >= 6  # re-encoding a grid point gives back its record (norm rounding aside)
    assert np.all(c.extra["resid"][same] == 0.0)
    assert np.all((c.norms[same] >> 16) == 0)
    assert np.all(quantize.unpack_bits(c.sign[same], 1, m) == 1)
    q = g.standard_normal((1, 1, d))
    plain = polar.PolarCodec(d, ab, pc.rot, pc.levels)
    a = polar.scores(q, c, pc, 8, 1)[0, 0]
    b = polar.scores(q, polar.PolarCodes(c.bits, c.norms & 0xFFFF), plain, 8, 1)[0, 0]
    assert np.array_equal(a[same], b[same])


# ------------------------------------------------------------------ append into a growing cache


@pytest.mark.parametrize("m", [0, 32])
def test_polar_append_reduces_to_encode(m):
    # no RoPE, or RoPE at position 0 (the identity): append is the encoder with the slots' rotations
    pc = polar.make_polar_codec(32, 3, 4, m=m, sketch_seed=6 if m else None)
    x = np.random.default_rng(1).standard_normal((40, 32)).astype(np.float32)
    want = polar.encode(x, pc)
    for base, pos in ((0.0, np.arange(40) * 7), (10000.0, np.zeros(40, np.int64))):
        got = polar.append(x, pc, np.arange(40), pos, base)
        assert np.array_equal(got.bits, want.bits) and np.array_equal(got.norms, want.norms)
        if m:
            assert np.array_equal(got.sign, want.sign)


def test_polar_append_slot_selects_the_rotation_block():
    # per-block rotations: a row appended at slot t is the encoder's record of that row at offset t
    pc = polar.make_polar_codec(32, 2, 4, basis_seeds=[10, 11, 12], vecs_per_rot=8)
    x = np.random.default_rng(2).standard_normal((6, 32)).astype(np.float32)
    slots = np.array([0, 7, 8, 15, 16, 40])  # blocks 0, 0, 1, 1, 2, 2 (past the last block: the last)
    got = polar.append(x, pc, slots, np.zeros(6, np.int64), 0.0)
    for i, t in enumerate(slots):
        one = polar.encode(x[i:i + 1], pc, first=int(t))
        assert np.array_equal(got.bits[i], one.bits[0])
    # and the rotation matters: block 0's record of the row at slot 40 differs
    assert not np.array_equal(got.bits[5], polar.encode(x[5:6], pc).bits[0])


def test_polar_append_keeps_the_norm_and_encodes_the_turned_vector():
    # RoPE keeps the norm, so the radius is fp16(||x||); the record is the direction of RoPE(x, p):
    # its reconstruction is as close to RoPE(x, p) as an encoding of RoPE(x, p) itself is, and far
    # from x (the turn is large at these positions)
    d, base = 64, 10000.0
    pc = polar.make_polar_codec(d, 4, 4)
    g = np.random.default_rng(3)
    x = g.standard_normal((400, d)).astype(np.float32)
    pos = g.integers(50, 5000, 400)
    got = polar.append(x, pc, np.arange(400), pos, base)
    assert np.array_equal(got.norms, quantize.f16_norm_bits(x))
    xr = quantize.rope(x, pos, base)
    rec = polar.dequantize(got, pc)
    direct = polar.dequantize(polar.encode(xr.astype(np.float32), pc), pc)

    def rel(a, b):
        return float(np.mean(np.sum((a - b) ** 2, 1) / np.sum(b * b, 1)))

    assert rel(rec, xr) < 1.1 * rel(direct, xr) + 1e-6
    assert rel(rec, xr) < 0.01
    assert rel(rec, x.astype(np.float64)) > 0.5


# ------------------------------------------------------------------ search


@pytest.mark.parametrize("m", [0, 64])
def test_polar_search_ranks_the_explicit_reconstructions(m):
    # the estimated score is the inner product with the dequantised record (the polar stage's
    # reconstruction plus the QJL term), so the top-k by score is the top-k of q . x^ computed
    # from the explicit reconstruction
    d = 64
    pc = polar.make_polar_codec(d, 3, 7, m=m, sketch_seed=8 if m else None)
    g = np.random.default_rng(4)
    db = polar.encode(g.standard_normal((3000, d)).astype(np.float32), pc)
    q = g.standard_normal((7, d))
    idx, sc = polar.search_topk(q, db, pc, 10)
    xhat = polar.dequantize(db, pc)
    ip = q @ xhat.T
    for i in range(7):
        order = np.argsort(-ip[i], kind="stable")[:10]
        assert np.array_equal(idx[i], order)
        assert np.allclose(sc[i], ip[i][order], rtol=1e-10, atol=1e-10)


def test_polar_search_ties_take_the_smaller_row_and_k_n_is_a_sorted_permutation():
    d = 32
    pc = polar.make_polar_codec(d, 2, 9)
    x = np.random.default_rng(5).standard_normal((50, d)).astype(np.float32)
    x[30] = x[3]  # identical records score identically
    x[41] = x[3]
    db = polar.encode(x, pc)
    q = x[3:4].astype(np.float64)
    idx, sc = polar.search_topk(q, db, pc, 3)
    assert list(idx[0]) == [3, 30, 41] and sc[0, 0] == sc[0, 1] == sc[0, 2]
    idx, sc = polar.search_topk(np.random.default_rng(6).standard_normal((2, d)), db, pc, 50)
    for i in range(2):
        assert sorted(idx[i]) == list(range(50))
        assert np.all(np.diff(sc[i]) <= 0)


def test_polar_search_recall_against_exact_top_k():
    # the codec serves search: with 4 angle bits most of the exact top 10 is found in the top 10
    from oracle import estimate

    d = 64
    pc = polar.make_polar_codec(d, 4, 11)
    g = np.random.default_rng(7)
    x = g.standard_normal((4000, d)).astype(np.float32)
    q = g.standard_normal((20, d))
    found, _ = polar.search_topk(q, polar.encode(x, pc), pc, 10)
    truth, _ = estimate.exact_topk(q, x, 10)
    assert estimate.recall_at_k(found, truth) > 0.8


# ------------------------------------------------------------------ decode step over growing caches


def _polar_caches(S, hkv, cap, d, pc, vc, seed):
    g = np.random.default_rng(seed)
    kx = g.standard_normal((S * hkv * cap, d)).astype(np.float32)
    vx = g.standard_normal((S * hkv * cap, d)).astype(np.float32)
    return polar.encode(kx, pc), quantize.encode(vx, vc)


def test_polar_attend_lens_reduces_to_attend_and_to_one_token():
    from oracle import codec as oc
    from oracle import estimate

    S, hkv, hq, cap, d = 2, 2, 4, 24, 32
    pc = polar.make_polar_codec(d, 3, 1, m=d, sketch_seed=2)
    vc = oc.make_codec(d, 3, 0, 3, 4)
    kc, vcodes = _polar_caches(S, hkv, cap, d, pc, vc, 5)
    q = np.random.default_rng(6).standard_normal((S, hq, d))
    full = polar.attend_lens(q, kc, vcodes, pc, vc, cap, [cap, cap], hkv, 0.3)
    assert np.allclose(full, polar.attend(q, kc, vcodes, pc, vc, cap, hkv, 0.3), rtol=0, atol=1e-12)
    # one token: the softmax of one logit is 1, so the output is that token's dequantised value
    one = polar.attend_lens(q, kc, vcodes, pc, vc, cap, [1, 0], hkv, 0.3)
    v = estimate.dequantize(vcodes, vc)
    for h in range(hq):
        assert np.allclose(one[0, h], v[(h // 2) * cap], rtol=0, atol=1e-12)
    assert not one[1].any()  # no token: zero output


def test_polar_decode_step_appends_then_attends_over_the_prefix():
    from oracle import codec as oc

    S, hkv, hq, cap, d = 3, 2, 4, 16, 32
    pc = polar.make_polar_codec(d, 2, 1, basis_seeds=[7, 8, 9, 10, 11, 12], vecs_per_rot=cap, m=d, sketch_seed=2)
    vc = oc.make_codec(d, 3, d, 3, 4)
    kc, vcodes = _polar_caches(S, hkv, cap, d, pc, vc, 9)
    g = np.random.default_rng(10)
    kn, vn = g.standard_normal((S, hkv, d)), g.standard_normal((S, hkv, d))
    q = g.standard_normal((S, hq, d))
    pos = np.array([5, cap, cap - 1])  # the second sequence is past its capacity
    out, k2, v2 = polar.decode_step(q, kn, vn, kc, vcodes, pc, vc, cap, pos, 10000.0, hkv, 0.25)
    # sequence 1: nothing appended, zero output
    assert not out[1].any()
    for h in range(hkv):
        a = (1 * hkv + h) * cap
        assert np.array_equal(k2.bits[a:a + cap], kc.bits[a:a + cap])
        assert np.array_equal(v2.idx[a:a + cap], vcodes.idx[a:a + cap])
    # the appended records are the append of the same rows, every other record unchanged
    for s_ in (0, 2):
        for h in range(hkv):
            slot = (s_ * hkv + h) * cap + pos[s_]
            want = polar.append(kn[s_, h][None].astype(np.float32), pc, [slot], [pos[s_]], 10000.0)
            assert np.array_equal(k2.bits[slot], want.bits[0]) and k2.norms[slot] == want.norms[0]
            assert np.array_equal(k2.sign[slot], want.sign[0])
    changed = np.nonzero(np.any(k2.bits != kc.bits, axis=1))[0]
    assert set(changed) <= {(s_ * hkv + h) * cap + pos[s_] for s_ in (0, 2) for h in range(hkv)}
    # attention over the prefix: tokens past pos[s] do not matter (scramble them)
    k3 = polar.PolarCodes(k2.bits.copy(), k2.norms.copy(), sign=k2.sign.copy())
    for h in range(hkv):
        a = (0 * hkv + h) * cap
        k3.bits[a + pos[0] + 1:a + cap] ^= 0x5A
    qr = quantize.rope(q.reshape(S * hq, d), np.repeat(pos, hq), 10000.0).reshape(S, hq, d)
    again = polar.attend_lens(qr, k3, v2, pc, vc, cap, [pos[0] + 1, 0, pos[2] + 1], hkv, 0.25)
    assert np.allclose(again, out, rtol=0, atol=1e-12)
