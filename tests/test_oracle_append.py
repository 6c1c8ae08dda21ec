"""Pins for the oracle's decode-step additions: RoPE, append into a growing cache, attention over
per-sequence lengths, and the composed decode step.  CPU only."""

import numpy as np
import pytest

from oracle import codec, estimate, quantize


def test_rope_is_a_rotation_group_turning_like_complex_multiplication():
    d, base = 16, 10000.0
    g = np.random.default_rng(0)
    x = g.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 131071])
    r = quantize.rope(x, pos, base)
    # orthogonal: norms kept; position 0 is the identity
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.array_equal(r[0], x[0])
    # composition: turning by a then by b is turning by a + b
    a, b = np.array([3, 11, 250, 9, 40]), np.array([5, 2, 17, 1000, 7])
    assert np.allclose(quantize.rope(quantize.rope(x, a, base), b, base), quantize.rope(x, a + b, base),
                       rtol=0, atol=1e-11)
    # direction and frequencies: pair (i, i + d/2) as the complex number x_i + 1j x_{i+d/2}
    # multiplied by exp(1j * pos * base^(-2i/d))
    half = d // 2
    z = (x[:, :half] + 1j * x[:, half:]) * np.exp(1j * pos[:, None] * base ** (-2.0 * np.arange(half) / d))
    assert np.allclose(r[:, :half], z.real, atol=1e-9) and np.allclose(r[:, half:], z.imag, atol=1e-9)


def test_rope_scores_depend_on_relative_position_only():
    # TurboESM summary, "Metodologia" A: (Pi R_i q)^T (Pi R_j k) = q^T R_{j-i} k
    d, base = 32, 10000.0
    g = np.random.default_rng(1)
    q, k = g.standard_normal((1, d)), g.standard_normal((1, d))
    P = codec.haar_rotation64(5, d)
    for i, j in ((0, 0), (3, 10), (1000, 1007), (5, 2)):
        lhs = (quantize.rope(q, [i], base) @ P.T) @ (quantize.rope(k, [j], base) @ P.T).T
        rhs = q @ quantize.rope(k, [j - i], base).T
        assert abs(lhs - rhs) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)


@pytest.fixture(scope="module")
def codecs():
    kc = codec.make_codec(32, 2, 32, 1, 2)
    vc = codec.make_codec(32, 3, 0, 3, 4)
    return kc, vc


def test_append_reduces_to_encode(codecs):
    kc, _ = codecs
    g = np.random.default_rng(2)
    x = g.standard_normal((40, 32)).astype(np.float32)
    # at position 0 RoPE is the identity; without RoPE the position does not matter
    for pos, base in ((np.zeros(40, int), 10000.0), (g.integers(0, 5000, 40), 0.0)):
        a = quantize.append(x, kc, np.arange(40), pos, base)
        e = quantize.encode(x, kc)
        assert np.array_equal(a.idx, e.idx) and np.array_equal(a.sign, e.sign) and np.array_equal(a.norms, e.norms)


def test_append_keeps_the_norm_of_x_and_rotates_rope_x(codecs):
    kc, _ = codecs
    g = np.random.default_rng(3)
    x = g.standard_normal((30, 32)).astype(np.float32)
    pos = g.integers(1, 100000, 30)
    a = quantize.append(x, kc, np.arange(30), pos, 10000.0, keep=True)
    assert np.array_equal(a.norms & 0xFFFF, quantize.f16_norm_bits(x))
    y = quantize.rope(x, pos, 10000.0) @ kc.rot[0].astype(np.float64).T
    assert np.allclose(a.y, y, rtol=0, atol=1e-6 * np.abs(y).max())
    # the estimator sees the rotated key: its score against a RoPE'd query at the same position
    # tracks the plain inner product q.x (RoPE turns both by the same angles)
    q = g.standard_normal(32)
    qr = quantize.rope(np.repeat(q[None], 30, 0), pos, 10000.0)
    est = np.array([estimate.scores_one(qr[i], estimate._slice(a, i, i + 1), kc)[0] for i in range(30)])
    exact = x.astype(np.float64) @ q
    assert np.corrcoef(est, exact)[0, 1] > 0.9


def _cache(kc, vc, S, hkv, cap, seed):
    g = np.random.default_rng(seed)
    K = g.standard_normal((S * hkv * cap, 32)).astype(np.float32)
    V = g.standard_normal((S * hkv * cap, 32)).astype(np.float32)
    return quantize.encode(K, kc), quantize.encode(V, vc)


def test_attend_lens_full_and_truncated(codecs):
    kc, vc = codecs
    S, hq, hkv, cap = 2, 4, 2, 50
    kcodes, vcodes = _cache(kc, vc, S, hkv, cap, 4)
    q = np.random.default_rng(5).standard_normal((S, hq, 32))
    full = estimate.attend_lens(q, kcodes, vcodes, kc, vc, cap, [cap, cap], hkv, 0.3)
    assert np.allclose(full, estimate.attend(q, kcodes, vcodes, kc, vc, cap, hkv, 0.3), rtol=0, atol=1e-12)
    # sequence 1 holding only its first 17 tokens: the same as a cache of capacity 17
    lens = [cap, 17]
    got = estimate.attend_lens(q, kcodes, vcodes, kc, vc, cap, lens, hkv, 0.3)
    for kvh in range(hkv):
        a = (1 * hkv + kvh) * cap
        k1 = estimate._slice(kcodes, a, a + 17)
        v1 = estimate._slice(vcodes, a, a + 17)
        ref = estimate.attend(q[1:2, 2 * kvh:2 * kvh + 2], k1, v1, kc, vc, 17, 1, 0.3)
        assert np.allclose(got[1, 2 * kvh:2 * kvh + 2], ref[0], rtol=0, atol=1e-12)
    # slots past a sequence's length do not matter
    k2 = quantize.Codes(kcodes.idx.copy(), kcodes.sign.copy(), kcodes.norms.copy())
    a = (1 * hkv + 1) * cap
    k2.idx[a + 17:a + cap] = 0xFF
    k2.norms[a + 17:a + cap] = 0x7BFF7BFF
    assert np.array_equal(estimate.attend_lens(q, k2, vcodes, kc, vc, cap, lens, hkv, 0.3), got)


def test_decode_step_composes_append_and_attention(codecs):
    kc, vc = codecs
    S, hq, hkv, cap = 2, 4, 2, 40
    kcodes, vcodes = _cache(kc, vc, S, hkv, cap, 6)
    g = np.random.default_rng(7)
    q = g.standard_normal((S, hq, 32))
    kn = g.standard_normal((S, hkv, 32)).astype(np.float32)
    vn = g.standard_normal((S, hkv, 32)).astype(np.float32)
    pos = np.array([25, 3])
    out, k2, v2 = estimate.decode_step(q, kn, vn, kcodes, vcodes, kc, vc, cap, pos, 10000.0, hkv, 0.25)
    # the new codes sit at slot pos[s]; everything else is untouched
    for s in range(S):
        for h in range(hkv):
            slot = (s * hkv + h) * cap + pos[s]
            a = quantize.append(kn[s, h][None], kc, [slot], [pos[s]], 10000.0)
            assert np.array_equal(k2.idx[slot], a.idx[0]) and k2.norms[slot] == a.norms[0]
    mask = np.ones(len(kcodes.norms), bool)
    mask[[(s * hkv + h) * cap + pos[s] for s in range(S) for h in range(hkv)]] = False
    assert np.array_equal(k2.norms[mask], kcodes.norms[mask]) and np.array_equal(v2.idx[mask], vcodes.idx[mask])
    # the attention of the RoPE'd query over tokens 0..pos[s]
    qr = quantize.rope(q.reshape(S * hq, 32), np.repeat(pos, hq), 10000.0).reshape(S, hq, 32)
    ref = estimate.attend_lens(qr, k2, v2, kc, vc, cap, pos + 1, hkv, 0.25)
    assert np.array_equal(out, ref)
    # a sequence at position 0 attends to its new token alone: the output is that value
    out0, _, v0 = estimate.decode_step(q, kn, vn, kcodes, vcodes, kc, vc, cap, np.array([0, 0]), 10000.0, hkv, 0.25)
    for s in range(S):
        for h in range(hq):
            slot = (s * hkv + h // 2) * cap
            assert np.allclose(out0[s, h], estimate.dequantize(estimate._slice(v0, slot, slot + 1), vc, slot)[0],
                               rtol=0, atol=1e-12)
