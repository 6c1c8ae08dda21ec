"""Pins for the oracle's encoder: exact norms, exact signs, packing, special cases.  CPU only."""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, quantize
from tests.conftest import golden


def _brute_f16_sqrt(vals):
    """Independent route: exact sum of squares, then scan every fp16 value."""
    s = sum((Fraction(float(v)) ** 2 for v in vals), Fraction(0))
    best, bestd = None, None
    for bits in range(0, 0x7C00):
        h = Fraction(float(np.uint16(bits).view(np.float16)))
        # |h - sqrt(s)| compared via squares is not monotone-safe; compare (h^2 - s) signs
        # on both sides of the root by distance of h to sqrt(s) using exact rationals:
        d = abs(h * h - s) / (h + _sqrt_upper(s)) if (h + _sqrt_upper(s)) > 0 else abs(h)
        if bestd is None or d < bestd or (d == bestd and bits % 2 == 0):
            best, bestd = bits, d
    return best


def _sqrt_upper(s):
    return Fraction(math.sqrt(float(s)))


def test_f16_sqrt_exact_against_scan():
    g = np.random.default_rng(0)
    for _ in range(6):
        v = g.standard_normal(5).astype(np.float32) * np.float32(g.uniform(0.01, 30))
        s = sum((Fraction(float(t)) ** 2 for t in v), Fraction(0))
        got = quantize.f16_rne_sqrt_exact(s)
        # away from ties the nearest fp16 by the scan is unique
        assert got == _brute_f16_sqrt(v)


def test_f16_sqrt_ties_to_even_and_overflow():
    # value exactly midway between two fp16 numbers -> even significand
    a = float(np.float16(1.0))
    b = float(np.nextafter(np.float16(1.0), np.float16(2.0)))  # 1 + 2^-10, odd
    mid = Fraction(a + b) / 2
    assert quantize.f16_rne_sqrt_exact(mid * mid) == np.float16(1.0).view(np.uint16)
    c = float(np.nextafter(np.float16(b), np.float16(2.0)))  # 1 + 2^-9, even
    mid2 = (Fraction(b) + Fraction(c)) / 2
    assert quantize.f16_rne_sqrt_exact(mid2 * mid2) == np.float16(c).view(np.uint16)
    # just above / below a midpoint
    tiny = Fraction(1, 2 ** 60)
    assert quantize.f16_rne_sqrt_exact(mid * mid + tiny) == np.float16(b).view(np.uint16)
    assert quantize.f16_rne_sqrt_exact(mid2 * mid2 - tiny) == np.float16(b).view(np.uint16)
    # overflow: >= 65520 rounds to inf; just below stays 65504
    assert quantize.f16_rne_sqrt_exact(Fraction(65520) ** 2) == 0x7C00
    assert quantize.f16_rne_sqrt_exact(Fraction(65519) ** 2) == 0x7BFF
    # zero and subnormals
    assert quantize.f16_rne_sqrt_exact(Fraction(0)) == 0
    assert quantize.f16_rne_sqrt_exact(Fraction(2 ** -24) ** 2) == 1


def test_f16_norm_bits_fast_path_equals_exact():
    g = np.random.default_rng(1)
    v = (g.standard_normal((300, 64)) * g.uniform(1e-3, 50, (300, 1))).astype(np.float32)
    # rows built to sit exactly on a midpoint (tie) and a hair off it
    b = float(np.nextafter(np.float16(1.0), np.float16(2.0)))
    mid = np.float32(0.5 * (1.0 + b))  # exactly representable: 12 significant bits
    v[0] = 0
    v[0, 5] = mid
    v[1] = 0
    v[1, 5] = mid
    v[1, 9] = np.float32(2.0 ** -20)
    v[2] = 0
    got = quantize.f16_norm_bits(v)
    for i in range(v.shape[0]):
        s = sum((Fraction(float(t)) ** 2 for t in v[i]), Fraction(0))
        assert got[i] == quantize.f16_rne_sqrt_exact(s), i
    assert got[0] == np.float16(1.0).view(np.uint16)
    assert got[1] == np.float16(b).view(np.uint16)
    assert got[2] == 0


def test_exact_sign_bits_against_rationals():
    g = np.random.default_rng(2)
    S = g.standard_normal((16, 12)).astype(np.float32)
    r = g.standard_normal((40, 12)).astype(np.float32)
    # rows with exact cancellation and with a hard case for fp64 summation
    r[0] = 0
    r[1] = 0
    r[1, 0] = 1
    r[1, 1] = -1
    S[3, 0], S[3, 1] = 2.5, 2.5  # row 3 . r[1] = 0 exactly
    bits = quantize.exact_sign_bits(S, r)
    for i in range(r.shape[0]):
        for j in range(S.shape[0]):
            z = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(S[j], r[i])), Fraction(0))
            assert bits[i, j] == (1 if z >= 0 else 0)
    assert bits[0].all() and bits[1, 3] == 1


def test_exact_sign_beats_fp64_cancellation():
    # products 2^60, -1, -2^60: exact sum -1 (bit 0); naive fp64 left-to-right gives 0 (bit 1).
    S = np.array([[2.0 ** 30, 1.0, -(2.0 ** 30)]], dtype=np.float32)
    r = np.array([[2.0 ** 30, -1.0, 2.0 ** 30]], dtype=np.float32)
    assert quantize.exact_sign_bits(S, r)[0, 0] == 0
    r2 = np.array([[2.0 ** 30, 1.0, 2.0 ** 30]], dtype=np.float32)
    assert quantize.exact_sign_bits(S, r2)[0, 0] == 1


def test_pack_bits_layout():
    # index i at bit bits*i, LSB first: [1, 2, 3, 0] with 2 bits -> 0b00_11_10_01 = 0x39
    packed = quantize.pack_bits(np.array([[1, 2, 3, 0, 3]]), 2, stride=4)
    assert packed.tolist() == [[0x39, 0x03, 0x00, 0x00]]
    # 3-bit fields straddle bytes: [5, 6, 7] -> bits 101 011 111 (LSB first) = 0b1_1111_0101
    p3 = quantize.pack_bits(np.array([[5, 6, 7]]), 3)
    assert p3.tolist() == [[0xF5, 0x01]]
    g = np.random.default_rng(3)
    for w in (1, 2, 3, 4):
        vals = g.integers(0, 1 << w, (7, 37))
        assert np.array_equal(quantize.unpack_bits(quantize.pack_bits(vals, w), w, 37), vals)


@pytest.fixture(scope="module")
def small_codec():
    return codec.make_codec(64, 2, 48, 1, 2)


def test_encode_zero_vector(small_codec):
    out = quantize.encode(np.zeros((2, 64), np.float32), small_codec, keep=True)
    L = 1 << small_codec.bits
    assert np.all(out.index == L - 1)
    assert np.all(out.norms == 0)
    assert np.all(out.bits == 1)
    assert np.all(out.resid == 0)


def test_encode_index_is_nearest_level(small_codec):
    g = np.random.default_rng(4)
    x = g.standard_normal((200, 64)).astype(np.float32)
    out = quantize.encode(x, small_codec, keep=True)
    nbar = quantize.f16_value(out.norms & 0xFFFF)
    u = out.y.astype(np.float64) / nbar[:, None]
    c = small_codec.centroids.astype(np.float64)
    nearest = np.argmin(np.abs(u[:, :, None] - c[None, None, :]), axis=2)
    t = small_codec.thresholds.astype(np.float64)
    far = np.min(np.abs(u[:, :, None] - t[None, None, :]), axis=2) > 1e-6
    assert np.array_equal(out.index[far], nearest[far])
    # norm is of the input, rounded once to fp16
    assert np.allclose(nbar, np.linalg.norm(x.astype(np.float64), axis=1), rtol=2.0 ** -11)


def test_residual_matches_original_space_residual(small_codec):
    # <Pi q, r> = <q, eps> with eps = x - Pi^T (nbar c[idx]) the walkthrough's residual.
    g = np.random.default_rng(5)
    x = g.standard_normal((50, 64)).astype(np.float32)
    q = g.standard_normal(64)
    out = quantize.encode(x, small_codec, keep=True)
    P = small_codec.rot[0].astype(np.float64)
    nbar = quantize.f16_value(out.norms & 0xFFFF)
    khat = (nbar[:, None] * small_codec.centroids.astype(np.float64)[out.index]) @ P
    eps = x.astype(np.float64) - khat
    lhs = out.resid.astype(np.float64) @ (P @ q)
    # r is y - khat_rot with y rounded to fp32: agreement to fp32 rounding of y
    assert np.allclose(lhs, eps @ q, atol=1e-5 * np.abs(eps @ q).max())
    rn = quantize.f16_value(out.norms >> 16)
    assert np.allclose(rn, np.linalg.norm(eps, axis=1), rtol=3e-3)


def test_pre_rotated_mode_equals_full_mode_given_same_y(small_codec):
    g = np.random.default_rng(6)
    x = g.standard_normal((64, 64)).astype(np.float32)
    full = quantize.encode(x, small_codec, keep=True)
    pre = quantize.encode(full.y, small_codec, pre_rotated=True, keep=True)
    same_norm = (pre.norms & 0xFFFF) == (full.norms & 0xFFFF)
    assert same_norm.mean() > 0.9
    assert np.array_equal(pre.idx[same_norm], full.idx[same_norm])
    assert np.array_equal(pre.sign[same_norm], full.sign[same_norm])


def test_mse_stage_distortion_matches_codebook():
    # E ||u - u^||^2 = d * MSE(d, b) for u uniform on the sphere (the codebook's own MSE).
    d, bits = 128, 2
    cdc = codec.make_codec(d, bits, 0, 9, 0)
    cb = codec.lloyd_max_beta(d, bits)
    g = np.random.default_rng(7)
    x = g.standard_normal((3000, d)).astype(np.float32)
    out = quantize.encode(x, cdc, keep=True)
    nbar = quantize.f16_value(out.norms & 0xFFFF)
    u = out.y.astype(np.float64) / nbar[:, None]
    err = np.sum((u - cdc.centroids.astype(np.float64)[out.index]) ** 2, axis=1)
    assert abs(err.mean() - d * cb.mse) < 4 * err.std() / math.sqrt(err.size)


def test_record_sizes_reproduce_esm2_footprint():
    g = golden("esm2_bit_accounting.json")
    d, bits, m = g["head_dim"], 3, 64
    rec = quantize.idx_bytes(d, bits) + quantize.sign_bytes(m) + 4
    assert rec == 36
    vectors = g["layers"] * g["heads"] * g["tokens"] * 2  # K and V
    comp = vectors * rec
    base = vectors * d * g["baseline_bytes_per_value"]
    mib = 2.0 ** 20
    assert round(base / mib) == g["printed_baseline_mb"]
    assert abs(comp / mib - g["printed_compressed_mb"]) < 1.0
    assert round(base / comp, 1) == g["printed_ratio"]
