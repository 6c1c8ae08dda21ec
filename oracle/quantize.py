"""Two-stage encode of K/V vectors.  Test infrastructure only.

Stage 1 (7minutos.es TurboQuant walkthrough, "Etapa 1 (PolarQuant)"; sudonull.com
"Cómo funciona PolarQuant": the radius is stored, the direction is quantised):
  * n16  = fp16 (round to nearest even) of the exact Euclidean norm of the input;
  * y    = Pi x (rotation), or y given directly in pre-rotated mode;
  * idx_i = number of thresholds t_j with y_i >= fl32(nbar * t_j), nbar = float(n16):
    the nearest Lloyd-Max level of the direction y / nbar, measured with the stored norm;
  * the index of each coordinate is stored, not the float ("Los valores cuantificados no
    se almacenan en flotante").
Stage 2 ("Etapa 2 (Corrección Residual)"):
  * residual r_i = fl32(y_i - fl32(nbar * c[idx_i])) -- the residual is formed in the
    rotated space; <Pi q, r> = <q, Pi^T r> and ||r|| = ||Pi^T r||, so this equals the
    walkthrough's original-space residual seen through the rotation;
  * rn16 = fp16 of the exact norm of r ("la norma L2 del residual ... como un único escalar");
  * sign bit j = [ (S r)_j >= 0 ], the exact sign of the real dot product (zero counts
    as +1).

Stored record per vector: the idx bitstream (bits*d bits, index i at bit bits*i, least
significant bit first, bytes little-endian, pad bits zero), the sign bitstream (bit j =
sign j, same order) and one 32-bit word (low half: n16, high half: rn16).

The fp32 steps use NumPy float32 arithmetic (each operation rounded to nearest even, no
fused multiply-add).  The two norms and the signs are exact: fp64 sums whose error bound
decides the result when it can, exact rational arithmetic (``fractions.Fraction``) or
``math.fsum`` when it cannot.
"""

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import Optional

import numpy as np

from .codec import Codec

_U64 = 2.0 ** -53
F16_INF_BITS = 0x7C00


# ------------------------------------------------------------------ fp16 rounding helpers


def f16_value(bits) -> np.ndarray:
    """fp16 bit patterns -> their values as fp64 (0x7C00 -> inf)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _f16_value_ext(bits: int) -> float:
    """Value of a non-negative fp16 pattern, with 0x7C00 standing for 65536 (the overflow step)."""
    if bits >= F16_INF_BITS:
        return 65536.0
    return float(np.uint16(bits).view(np.float16))


def f16_rne_sqrt_exact(sumsq: Fraction) -> int:
    """fp16 bits of sqrt(sumsq) rounded to nearest, ties to even, by exact comparisons.

    Finds the largest fp16 value h with h^2 <= sumsq, then compares sumsq with the square
    of the midpoint between h and its successor.  Overflow (>= 65520) gives +inf.
    """
    lo, hi = 0, F16_INF_BITS  # invariant: value(lo)^2 <= sumsq
    if Fraction(_f16_value_ext(hi)) ** 2 <= sumsq:
        return F16_INF_BITS
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if Fraction(_f16_value_ext(mid)) ** 2 <= sumsq:
            lo = mid
        else:
            hi = mid
    a = Fraction(_f16_value_ext(lo))
    b = Fraction(_f16_value_ext(lo + 1))
    m2 = ((a + b) / 2) ** 2
    if sumsq < m2:
        return lo
    if sumsq > m2:
        return lo + 1
    return lo if lo % 2 == 0 else lo + 1


def f16_rne_exact(v: Fraction) -> int:
    """fp16 bits of the non-negative rational v rounded to nearest, ties to even (>= 65520 -> inf)."""
    lo, hi = 0, F16_INF_BITS  # invariant: value(lo) <= v
    if Fraction(_f16_value_ext(hi)) <= v:
        return F16_INF_BITS
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if Fraction(_f16_value_ext(mid)) <= v:
            lo = mid
        else:
            hi = mid
    mid = (Fraction(_f16_value_ext(lo)) + Fraction(_f16_value_ext(lo + 1))) / 2
    if v < mid:
        return lo
    if v > mid:
        return lo + 1
    return lo if lo % 2 == 0 else lo + 1


def f16_scaled_norm_bits(n16: np.ndarray, scale: float) -> np.ndarray:
    """fp16 bits of nbar * scale (nbar the value of n16, scale an fp32 value), exactly rounded."""
    s = Fraction(float(np.float32(scale)))
    out = np.empty(len(n16), dtype=np.uint16)
    for i, b in enumerate(np.asarray(n16, dtype=np.uint16)):
        out[i] = f16_rne_exact(Fraction(float(f16_value(b))) * s)
    return out


def f16_norm_bits(v: np.ndarray) -> np.ndarray:
    """fp16 bits of the exactly rounded Euclidean norm of each row of ``v``.

    ``v`` holds values exactly representable in fp64 (fp32/fp16/bf16 inputs).  Squares of
    such values are exact in fp64; their fp64 sum has error at most (n-1) u sum.  The
    candidate from the fp64 root is accepted when the sum is farther than that bound from
    the squares of both neighbouring midpoints; otherwise the exact routine decides.
    """
    v64 = np.asarray(v, dtype=np.float64)
    n, d = v64.shape
    s = np.sum(v64 * v64, axis=1)
    with np.errstate(over="ignore"):
        cand = np.sqrt(s).astype(np.float16).view(np.uint16).astype(np.int64)
    slack = 4.0 * (d + 2) * _U64
    finite = cand < F16_INF_BITS
    c = np.where(finite, cand, 0)
    vh = f16_value(c)
    nxt = np.where(c + 1 >= F16_INF_BITS, 65536.0, f16_value(np.minimum(c + 1, 0x7BFF)))
    prv = f16_value(np.maximum(c - 1, 0))
    up = 0.5 * (vh + nxt)
    dn = 0.5 * (vh + prv)
    ok = finite & (s < up * up * (1.0 - slack)) & ((c == 0) | (s > dn * dn * (1.0 + slack)))
    out = c.astype(np.uint16)
    for i in np.flatnonzero(~ok):
        exact = sum((Fraction(float(t)) ** 2 for t in v64[i]), Fraction(0))
        out[i] = f16_rne_sqrt_exact(exact)
    return out


# ------------------------------------------------------------------ exact signs


def exact_sign_bits(sketch: np.ndarray, r: np.ndarray) -> np.ndarray:
    """bits[i, j] = 1 iff sum_k sketch[j, k] * r[i, k] >= 0 in exact arithmetic.

    Products of fp32 values are exact in fp64.  The fp64 matrix product has error at most
    d u sum_k |products|; entries whose fp64 value is not farther than twice that from
    zero are recomputed with ``math.fsum`` (correctly rounded, hence sign-exact).
    """
    s64 = np.asarray(sketch, dtype=np.float64)
    r64 = np.asarray(r, dtype=np.float64)
    d = s64.shape[1]
    z = r64 @ s64.T
    bound = 2.0 * (d + 2) * _U64 * (np.abs(r64) @ np.abs(s64).T)
    bits = (z >= 0).astype(np.uint8)
    amb = np.argwhere(np.abs(z) <= bound)
    for i, j in amb:
        exact = math.fsum(float(a) * float(b) for a, b in zip(s64[j], r64[i]))
        bits[i, j] = 1 if exact >= 0 else 0
    return bits


# ------------------------------------------------------------------ packing


def pack_bits(values: np.ndarray, width: int, stride: Optional[int] = None) -> np.ndarray:
    """Pack ``width``-bit unsigned fields per row, field i at bit width*i, LSB first."""
    values = np.asarray(values, dtype=np.uint32)
    n, cnt = values.shape
    bits = ((values[:, :, None] >> np.arange(width, dtype=np.uint32)) & 1).astype(np.uint8)
    packed = np.packbits(bits.reshape(n, cnt * width), axis=1, bitorder="little")
    need = packed.shape[1]
    stride = need if stride is None else stride
    if stride < need:
        raise ValueError("stride too small")
    out = np.zeros((n, stride), dtype=np.uint8)
    out[:, :need] = packed
    return out


def unpack_bits(packed: np.ndarray, width: int, count: int) -> np.ndarray:
    """Inverse of ``pack_bits``: [n, count] fields of ``width`` bits."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    bits = np.unpackbits(packed, axis=1, bitorder="little")[:, : count * width]
    bits = bits.reshape(n, count, width).astype(np.uint32)
    return np.sum(bits << np.arange(width, dtype=np.uint32), axis=2)


# ------------------------------------------------------------------ encode


@dataclass
class Codes:
    idx: np.ndarray  # [n, idx_stride] uint8
    sign: Optional[np.ndarray]  # [n, sign_stride] uint8 or None (m == 0)
    norms: np.ndarray  # [n] uint32: low 16 bits fp16 ||x||, high 16 bits fp16 ||r||
    # intermediate values kept for tests
    y: Optional[np.ndarray] = None
    index: Optional[np.ndarray] = None
    resid: Optional[np.ndarray] = None
    bits: Optional[np.ndarray] = None


def idx_bytes(d: int, bits: int) -> int:
    return (d * bits + 7) // 8


def sign_bytes(m: int) -> int:
    return (m + 7) // 8


def rotate(x: np.ndarray, codec: Codec, first: int = 0) -> np.ndarray:
    """y = Pi x per vector (fp64 product of the stored fp32 rotation), rounded to fp32."""
    x64 = np.asarray(x, dtype=np.float64)
    rid = codec.rot_index(x64.shape[0], first)
    y = np.empty(x64.shape, dtype=np.float32)
    for r in np.unique(rid):
        sel = rid == r
        y[sel] = (x64[sel] @ codec.rot[r].astype(np.float64).T).astype(np.float32)
    return y


def encode(x: np.ndarray, codec: Codec, pre_rotated: bool = False, first: int = 0,
           idx_stride: Optional[int] = None, sign_stride: Optional[int] = None,
           keep: bool = False) -> Codes:
    """Encode rows of ``x`` ([n, d]; fp32, fp16 or bf16 values given as fp32/fp64).

    ``pre_rotated``: x already is y = Pi x in fp32; the norm is then taken of y.
    ``first``: index of x[0] in the whole cache (selects the per-block rotation).
    """
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != codec.d:
        raise ValueError("x must be [n, d]")
    if pre_rotated:
        y = np.asarray(x, dtype=np.float32)
        norm_src = y
    else:
        y = rotate(x, codec, first)
        norm_src = x
    return encode_rotated(y, f16_norm_bits(norm_src), codec, idx_stride, sign_stride, keep)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding in fp64 (TurboESM summary, "Metodología" A: applied to the keys
    (and queries) before the orthogonal rotation).  The pages do not spell out the pairing; the
    reading taken is the half-split one: coordinate i < d/2 turns with coordinate i + d/2 by the
    angle pos * base^(-2i/d)."""
    x64 = np.asarray(x, dtype=np.float64)
    d = x64.shape[-1]
    half = d // 2
    inv = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x64[:, :half], x64[:, half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def append(x: np.ndarray, codec: Codec, slots: np.ndarray, pos: np.ndarray, rope_base: float,
           idx_stride: Optional[int] = None, sign_stride: Optional[int] = None, keep: bool = False) -> Codes:
    """Codes of new vectors appended to a growing cache (7minutos.es walkthrough, "Etapa 1": the
    indices stay in the cache until the token is evicted; TurboESM summary, "Metodología" A:
    RoPE first, then the rotation).  Row k goes to cache slot ``slots[k]`` (which selects the
    per-block rotation) at position ``pos[k]``; with rope_base > 0 the rotation sees
    RoPE(x, pos) in fp64: y = fl32(Pi RoPE(x)).  The stored norm is that of x itself -- RoPE is
    orthogonal, so this is the norm of the rotated input as well."""
    x = np.asarray(x)
    x64 = np.asarray(x, dtype=np.float64)
    xr = rope(x64, pos, rope_base) if rope_base > 0 else x64
    rid = np.array([codec.rot_index(1, int(sl))[0] for sl in slots], dtype=np.int64)
    y = np.empty(x64.shape, dtype=np.float32)
    for r in np.unique(rid):
        sel = rid == r
        y[sel] = (xr[sel] @ codec.rot[r].astype(np.float64).T).astype(np.float32)
    return encode_rotated(y, f16_norm_bits(x), codec, idx_stride, sign_stride, keep)


def encode_rotated(y: np.ndarray, n16: np.ndarray, codec: Codec, idx_stride: Optional[int] = None,
                   sign_stride: Optional[int] = None, keep: bool = False) -> Codes:
    """The steps after the rotation: indices against the thresholds scaled by the stored norm,
    residual, its norm and the exact signs of S r; y is fp32, n16 the fp16 bits of the norm."""
    y = np.asarray(y, dtype=np.float32)
    nbar = f16_value(n16).astype(np.float32)  # exact: fp16 values are fp32 values

    thr = nbar[:, None] * codec.thresholds[None, :].astype(np.float32)  # fp32 products
    index = np.sum(y[:, :, None] >= thr[:, None, :], axis=2).astype(np.uint32)
    cval = nbar[:, None] * codec.centroids.astype(np.float32)[index]  # fp32 products
    resid = (y - cval).astype(np.float32)  # fp32 differences
    if codec.resid_scale > 0:
        # TurboESM residual-sign correction: the decoder adds nbar * ebar * sign per coordinate;
        # the word carries nbar * ebar * m / sqrt(pi/2) so the QJL formula reads it unchanged
        rn16 = f16_scaled_norm_bits(n16, codec.resid_scale)
    else:
        rn16 = f16_norm_bits(resid)

    idx = pack_bits(index, codec.bits, idx_stride)
    if codec.m > 0:
        bits = exact_sign_bits(codec.sketch, resid)
        sign = pack_bits(bits, 1, sign_stride)
    else:
        bits, sign = None, None
    norms = (rn16.astype(np.uint32) << 16) | n16.astype(np.uint32)
    out = Codes(idx, sign, norms)
    if keep:
        out.y, out.index, out.resid, out.bits = y, index, resid, bits
    return out


def unpack(codes: Codes, codec: Codec):
    """Codes -> (index [n, d], signs in {-1, +1} [n, m] or None, nbar, rnbar) as fp64."""
    index = unpack_bits(codes.idx, codec.bits, codec.d)
    signs = None
    if codec.m > 0:
        signs = 2.0 * unpack_bits(codes.sign, 1, codec.m).astype(np.float64) - 1.0
    nbar = f16_value((codes.norms & 0xFFFF).astype(np.uint16))
    rnbar = f16_value((codes.norms >> 16).astype(np.uint16))
    return index, signs, nbar, rnbar
