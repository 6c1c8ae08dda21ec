"""Pins for the oracle's estimator, attention and search.  CPU only."""

import math

import numpy as np
import pytest

from oracle import codec, estimate, quantize


def test_qjl_estimator_unbiased_over_sketch_seeds():
    # E_S[ sqrt(pi/2)/m ||r|| <S q, sign(S r)> ] = <q, r>; variance (pi/2 |q|^2 |r|^2 - <q,r>^2)/m.
    d, m, T = 64, 32, 3000  # m != d catches a 1/d constant
    g = np.random.default_rng(0)
    q = g.standard_normal(d)
    r = g.standard_normal(d).astype(np.float32).astype(np.float64)
    est = np.empty(T)
    for t in range(T):
        S = g.standard_normal((m, d)).astype(np.float32)
        bits = quantize.exact_sign_bits(S, r[None].astype(np.float32))[0]
        est[t] = estimate.qjl_scale(m) * np.linalg.norm(r) * ((2.0 * bits - 1.0) @ (S.astype(np.float64) @ q))
    V = (math.pi / 2 * (q @ q) * (r @ r) - (q @ r) ** 2) / m
    assert abs(est.mean() - q @ r) < 4 * math.sqrt(V / T)
    assert abs(est.var() / V - 1) < 0.15


@pytest.fixture(scope="module")
def codecs():
    kc = codec.make_codec(32, 2, 24, 1, 2)
    vc = codec.make_codec(32, 3, 16, 3, 4)
    vc0 = codec.make_codec(32, 3, 0, 3, 4)
    return kc, vc, vc0


def test_estimator_equals_explicit_dequantisation(codecs):
    kc, _, _ = codecs
    g = np.random.default_rng(1)
    x = g.standard_normal((70, 32)).astype(np.float32)
    q = g.standard_normal(32)
    k = quantize.encode(x, kc)
    s = estimate.scores_one(q, k, kc)
    kt = estimate.dequantize(k, kc)
    assert np.allclose(s, kt @ q, rtol=0, atol=1e-12 * np.abs(s).max())


def test_estimator_special_cases(codecs):
    kc, _, _ = codecs
    q = np.random.default_rng(2).standard_normal(32)
    # zero vector scores exactly 0
    z = quantize.encode(np.zeros((1, 32), np.float32), kc)
    assert estimate.scores_one(q, z, kc)[0] == 0.0
    # a zero residual norm removes the QJL term: flipping every sign bit changes nothing
    g = np.random.default_rng(12)
    enc = quantize.encode(g.standard_normal((6, 32)).astype(np.float32), kc)
    enc.norms = enc.norms & 0xFFFF
    flipped = quantize.Codes(enc.idx, (~enc.sign) & 0xFF, enc.norms)
    flipped.sign[:, quantize.sign_bytes(kc.m):] = 0
    assert np.array_equal(estimate.scores_one(q, enc, kc), estimate.scores_one(q, flipped, kc))
    qt, _ = estimate.prepare_query(q, kc)
    index, _, nbar, _ = quantize.unpack(enc, kc)
    assert np.allclose(estimate.scores_one(q, enc, kc), nbar * (kc.centroids.astype(np.float64)[index] @ qt),
                       rtol=1e-15, atol=0)


def test_gqa_mapping_and_rotation_blocks(codecs):
    kc, _, _ = codecs
    g = np.random.default_rng(3)
    S, hq, hkv, N = 2, 4, 2, 9
    x = g.standard_normal((S * hkv * N, 32)).astype(np.float32)
    q = g.standard_normal((S, hq, 32))
    k = quantize.encode(x, kc)
    got = estimate.scores(q, k, kc, N, hkv)
    for s in range(S):
        for h in range(hq):
            blk = s * hkv + h // 2
            kt = estimate.dequantize(estimate._slice(k, blk * N, (blk + 1) * N), kc)
            assert np.allclose(got[s, h], kt @ q[s, h], atol=1e-12 * np.abs(got).max())


def test_per_block_rotations():
    d = 16
    kc = codec.make_codec(d, 2, 16, 5, 6, basis_seeds=[7, 8, 9, 10], vecs_per_rot=5)
    g = np.random.default_rng(4)
    x = g.standard_normal((20, d)).astype(np.float32)
    enc = quantize.encode(x, kc, keep=True)
    for i in range(20):
        y = (kc.rot[i // 5].astype(np.float64) @ x[i].astype(np.float64)).astype(np.float32)
        assert np.array_equal(enc.y[i], y)
    q = g.standard_normal(d)
    kt = estimate.dequantize(enc, kc)
    for blk in range(4):
        s = estimate.scores_one(q, estimate._slice(enc, 5 * blk, 5 * blk + 5), kc, rot=blk)
        assert np.allclose(s, kt[5 * blk:5 * blk + 5] @ q, atol=1e-12 * np.abs(s).max())


@pytest.mark.parametrize("vidx", [1, 2])
def test_attention_equals_materialised_route(codecs, vidx):
    kc = codecs[0]
    vc = codecs[vidx]
    g = np.random.default_rng(5)
    S, hq, hkv, N = 2, 4, 2, 33
    k = quantize.encode(g.standard_normal((S * hkv * N, 32)).astype(np.float32), kc)
    v = quantize.encode(g.standard_normal((S * hkv * N, 32)).astype(np.float32), vc)
    q = g.standard_normal((S, hq, 32))
    scale = 1 / math.sqrt(32)
    a = estimate.attend(q, k, v, kc, vc, N, hkv, scale)
    b = estimate.attend_materialised(q, k, v, kc, vc, N, hkv, scale)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b))


def test_attention_special_cases(codecs):
    kc, vc, _ = codecs
    g = np.random.default_rng(6)
    v = quantize.encode(g.standard_normal((5, 32)).astype(np.float32), vc)
    vt = estimate.dequantize(v, vc)
    # N = 1: the output is the single dequantised value
    k1 = quantize.encode(g.standard_normal((1, 32)).astype(np.float32), kc)
    v1 = estimate._slice(v, 0, 1)
    o = estimate.attend(g.standard_normal((1, 1, 32)), k1, v1, kc, vc, 1, 1, 0.1)
    assert np.allclose(o[0, 0], vt[0], atol=1e-14)
    # identical keys: equal scores -> the mean of the values
    kx = np.repeat(g.standard_normal((1, 32)).astype(np.float32), 5, axis=0)
    k5 = quantize.encode(kx, kc)
    o = estimate.attend(g.standard_normal((1, 1, 32)), k5, v, kc, vc, 5, 1, 0.3)
    assert np.allclose(o[0, 0], vt.mean(axis=0), atol=1e-13)


def test_score_error_matches_qjl_variance_and_attention_tracks_exact():
    # With m = d the estimate's error variance relative to the exact score spread is about
    # (pi/2) d MSE(d, b) for random directions: ~0.18 at d = 128, b = 2 (std ~0.43).
    d, N = 128, 4096
    kc = codec.make_codec(d, 2, 128, 1, 2)
    vc = codec.make_codec(d, 3, 0, 3, 4)
    g = np.random.default_rng(7)
    K = g.standard_normal((N, d)).astype(np.float32)
    V = g.standard_normal((N, d)).astype(np.float32)
    kk, vv = quantize.encode(K, kc), quantize.encode(V, vc)
    ratios = []
    for _ in range(4):
        q = g.standard_normal(d)
        s_est = estimate.scores_one(q, kk, kc)
        s_ex = K.astype(np.float64) @ q
        ratios.append(np.var(s_est - s_ex) / np.var(s_ex))
    want = math.pi / 2 * d * codec.lloyd_max_beta(d, 2).mse
    assert abs(np.mean(ratios) - want) < 0.2 * want
    # informational: attention with unit-variance logits tracks exact attention
    q = g.standard_normal((1, 1, d))
    scale = 1 / math.sqrt(d)
    o = estimate.attend(q, kk, vv, kc, vc, N, 1, scale)[0, 0]
    exact = estimate.softmax(scale * (K.astype(np.float64) @ q[0, 0])) @ V.astype(np.float64)
    assert o @ exact / np.linalg.norm(o) / np.linalg.norm(exact) > 0.8


def test_topk_rows_order_and_ties():
    rows = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5]])
    idx, sc = estimate.topk_rows(rows, 4)
    want = sorted(range(6), key=lambda n: (-rows[0, n], n))[:4]
    assert idx[0].tolist() == want == [1, 2, 4, 0]
    assert sc[0].tolist() == [2.0, 2.0, 2.0, 0.5]
    g = np.random.default_rng(8)
    r = np.round(g.standard_normal((5, 50)), 1)
    idx, _ = estimate.topk_rows(r, 10)
    for i in range(5):
        assert idx[i].tolist() == sorted(range(50), key=lambda n: (-r[i, n], n))[:10]


def test_search_recall_sane():
    d = 64
    c = codec.make_codec(d, 2, d, 1, 2)
    g = np.random.default_rng(9)
    means = g.standard_normal((20, d))
    db = means[g.integers(0, 20, 2000)] + g.standard_normal((2000, d))
    db /= np.linalg.norm(db, axis=1, keepdims=True)
    qs = means[g.integers(0, 20, 20)] + g.standard_normal((20, d))
    codes = quantize.encode(db.astype(np.float32), c)
    a, _ = estimate.search_topk(qs, codes, c, 10)
    e, _ = estimate.exact_topk(qs, db.astype(np.float32), 10)
    assert estimate.recall_at_k(e, e) == 1.0
    assert estimate.recall_at_k(a, e) > 0.4
    assert estimate.one_at_k(a, e) > 0.6


def test_search_scores_equal_per_query_estimates():
    d = 64
    c = codec.make_codec(d, 2, 32, 1, 2)
    g = np.random.default_rng(10)
    codes = quantize.encode(g.standard_normal((300, d)).astype(np.float32), c)
    qs = g.standard_normal((4, d))
    got = estimate.search_scores(qs, codes, c, chunk=77)
    want = np.stack([estimate.scores_one(q, codes, c) for q in qs])
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
