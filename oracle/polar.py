"""Recursive polar stage 1 ("PolarQuant" proper): radius + angle tree.  Test infrastructure
only: the tests, __graft_entry__.smoke() and bench.py's cpu_baseline use it; the library does
not.

Sources: hada.io TurboQuant page, "PolarQuant: um novo 'ângulo' para compressão": pairs of
coordinates go to polar form, the radii are paired and turned to polar form again,
recursively, until one radius and a set of angles remain; the angles' law is known and
concentrated, so they are quantised on a fixed grid with known boundaries, with no
per-vector normalisation.  sudonull.com, "Cómo funciona PolarQuant": a random rotation
first; the radius carries the magnitude, the angles the direction; 3 to 4 bits per value.

Readings (the pages leave these open):
  * d = 2^L.  Level 1 pairs coordinates (2j, 2j+1) of y = Pi x; level l + 1 pairs the level-l
    radii (2i, 2i+1).  A node's angle is psi = atan2(r_b, r_a) in [0, pi/2]; at level 1 the
    pair (a, b) keeps its two signs (2 bits) and psi = atan2(|b|, |a|).
  * Law of psi at level l, whose children hold k = 2^(l-1) coordinates each (direction uniform
    on the sphere): density 2 / B(k/2, k/2) sin^(k-1) psi cos^(k-1) psi on [0, pi/2] (uniform
    at level 1).  Each level's table: Lloyd-Max on that law with 2^ab levels, midpoint
    thresholds, symmetrised about pi/4.  ab is one number for all levels.
  * Decisions without angles: psi >= tau  <=>  r_b^2 cos^2 tau >= r_a^2 sin^2 tau, taken as
    fl32(B * C) >= fl32(A * S) with A, B the children's sums of squares in fp32 (leaves
    fl32(y^2), a node fl32(A + B)) and C = fl32(cos^2 tau), S = fl32(sin^2 tau).  The index is
    the number of thresholds passed (a tie goes up).
  * Radius: n16 = fp16(||x||), exactly rounded, as in the standard stage 1.
  * Reconstruction: from the root (value 1) down, child a = parent cos psi^, child b =
    parent sin psi^ (psi^ the level's level for the node's index, as fp32 cos and sin); a
    level-1 pair gives (sign a * r cos psi^, sign b * r sin psi^); y^ = nbar u^.  Scores:
    nbar <Pi q, u^>.
  * Record: one bitstream, LSB first: pair j at bit (2 + ab) j as [sign of a (1 = negative),
    sign of b, angle index]; then the node indices of levels 2, 3, ..., L in order, ab bits
    each; pad bits zero.  Norm word: n16 in the low half, 0 in the high half.

Stage 2 on the polar residual (hada.io TurboQuant page, "Estrutura de compressão em 2 etapas"
and "Etapa 2: eliminação do erro oculto": the polar stage first, then the 1-bit QJL correction
of the error it leaves), when the codec carries a sketch S (m x d):
  * the stage-1 reconstruction in fp32, from the root down: the root is 1; a node's children
    are fl32(parent * cos psi^) and fl32(parent * sin psi^) with the level's fp32 table values;
    a pair gives +-fl32(r * cos psi^), +-fl32(r * sin psi^) (the recorded signs);
  * residual in the rotated space r_i = fl32(y_i - fl32(nbar * u^_i)), rn16 = fp16 of the exact
    norm of r, sign bit j = [ (S r)_j >= 0 ] exact -- the two-stage codec's stage 2 with the
    polar reconstruction in place of the codebook levels;
  * norm word: n16 low, rn16 high; scores nbar <Pi q, u^> + rnbar sqrt(pi/2)/m <S Pi q, 2 b - 1>.
"""

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
from scipy import special

from . import codec as oc
from .quantize import f16_norm_bits, f16_value, pack_bits, unpack_bits


def angle_density(k: int):
    """Density of psi at a level whose children hold k coordinates each."""
    c = 2.0 / special.beta(k / 2.0, k / 2.0)
    return lambda p: c * np.sin(p) ** (k - 1) * np.cos(p) ** (k - 1)


@dataclass
class PolarLevel:
    k: int
    centroids64: np.ndarray   # psi^ (2^ab, ascending in [0, pi/2])
    thresholds64: np.ndarray  # tau (2^ab - 1)
    cos: np.ndarray           # fp32 cos psi^
    sin: np.ndarray           # fp32 sin psi^
    c2: np.ndarray            # fp32 cos^2 tau
    s2: np.ndarray            # fp32 sin^2 tau


def angle_table(k: int, ab: int) -> PolarLevel:
    """Lloyd-Max levels of the level law with children of k coordinates."""
    L = 1 << ab
    half = math.pi / 2.0
    f = angle_density(k)

    def mass(a, b):
        return special.betainc(k / 2.0, k / 2.0, np.sin(b) ** 2) - special.betainc(k / 2.0, k / 2.0, np.sin(a) ** 2)

    gx, gw = np.polynomial.legendre.leggauss(64)

    def moment(a, b):
        # 64-point Gauss-Legendre per cell (the density is smooth on [0, pi/2])
        a = np.atleast_1d(a)[:, None]
        b = np.atleast_1d(b)[:, None]
        p = 0.5 * (b - a) * gx[None, :] + 0.5 * (a + b)
        return 0.5 * (b - a)[:, 0] * np.sum(gw[None, :] * p * f(p), axis=1)

    if k == 1:
        c64 = (np.arange(L) + 0.5) * half / L  # uniform law: equal cells, centred levels
    else:
        # start from the law's quantiles (every cell holds mass, however concentrated the law)
        init = np.arcsin(np.sqrt(special.betaincinv(k / 2.0, k / 2.0, (np.arange(L) + 0.5) / L)))
        c64, _ = oc.lloyd_max(mass, moment, 0.0, half, init, rel_tol=1e-13, floor_tol=1e-11)
    c64 = 0.5 * (c64 + (half - c64[::-1]))  # symmetric about pi/4
    t64 = 0.5 * (c64[:-1] + c64[1:])
    return PolarLevel(k, c64, t64, np.cos(c64).astype(np.float32), np.sin(c64).astype(np.float32),
                      (np.cos(t64) ** 2).astype(np.float32), (np.sin(t64) ** 2).astype(np.float32))


@dataclass
class PolarCodec:
    d: int
    ab: int
    rot: np.ndarray                  # [n_rot, d, d] fp32
    levels: List[PolarLevel]         # levels[l - 1] for l = 1..L
    vecs_per_rot: int = 0
    m: int = 0                       # > 0: QJL stage on the polar residual
    sketch: Optional[np.ndarray] = None  # [m, d] fp32

    @property
    def L(self) -> int:
        return int(round(math.log2(self.d)))

    @property
    def n_bits(self) -> int:
        return (self.d // 2) * (2 + self.ab) + (self.d // 2 - 1) * self.ab

    def rot_index(self, n_vec: int, first: int = 0) -> np.ndarray:
        ids = np.arange(first, first + n_vec, dtype=np.int64)
        if self.rot.shape[0] == 1 or self.vecs_per_rot <= 0:
            return np.zeros(n_vec, dtype=np.int64)
        return np.minimum(ids // self.vecs_per_rot, self.rot.shape[0] - 1)


def make_polar_codec(d: int, ab: int, rot_seed: int, basis_seeds=None, vecs_per_rot: int = 0, m: int = 0,
                     sketch_seed: Optional[int] = None) -> PolarCodec:
    L = int(round(math.log2(d)))
    assert 1 << L == d, "d must be a power of two"
    rot = oc.haar_rotation(rot_seed, d)[None] if basis_seeds is None else oc.head_rotations(rot_seed, basis_seeds, d)
    sk = oc.gaussian_sketch(sketch_seed, m, d) if m > 0 else None
    return PolarCodec(d, ab, rot, [angle_table(1 << (l - 1), ab) for l in range(1, L + 1)], vecs_per_rot, m, sk)


@dataclass
class PolarCodes:
    bits: np.ndarray   # [n][stride] u8
    norms: np.ndarray  # [n] u32
    extra: dict = field(default_factory=dict)
    sign: Optional[np.ndarray] = None  # [n][sign_stride] u8 (QJL stage), else None


def _decide(A, B, lv: PolarLevel):
    """Index per node: thresholds passed, fl32(B C_j) >= fl32(A S_j)."""
    A = A.astype(np.float32)
    B = B.astype(np.float32)
    return np.sum((B[..., None] * lv.c2) >= (A[..., None] * lv.s2), axis=-1).astype(np.uint32)


def encode_rotated(y: np.ndarray, n16: np.ndarray, pc: PolarCodec, stride: Optional[int] = None,
                   sign_stride: Optional[int] = None) -> PolarCodes:
    y = np.asarray(y, dtype=np.float32)
    n, d = y.shape
    a, b = y[:, 0::2], y[:, 1::2]
    A = (a * a).astype(np.float32)
    B = (b * b).astype(np.float32)
    sa = (a < 0).astype(np.uint32)
    sb = (b < 0).astype(np.uint32)
    k1 = _decide(A, B, pc.levels[0])
    pair = sa | (sb << 1) | (k1 << 2)                         # [n, d/2], 2 + ab bits each
    s = (A + B).astype(np.float32)                              # level-1 radii squared
    nodes = []
    for lvl in range(2, pc.L + 1):
        A, B = s[:, 0::2], s[:, 1::2]
        nodes.append(_decide(A, B, pc.levels[lvl - 1]))
        s = (A + B).astype(np.float32)
    # one bitstream: pairs, then nodes of levels 2..L
    fields = [(pair, 2 + pc.ab)] + [(c, pc.ab) for c in nodes]
    nb = pc.n_bits
    stride = stride or 4 * ((nb + 31) // 32)
    out = np.zeros((n, stride), dtype=np.uint8)
    bitpos = 0
    words = np.zeros((n, (stride + 3) // 4 * 32), dtype=np.uint8)  # one byte per bit
    for vals, w in fields:
        for j in range(vals.shape[1]):
            for t in range(w):
                words[:, bitpos + t] = (vals[:, j] >> t) & 1
            bitpos += w
    assert bitpos == nb
    packed = np.packbits(words[:, :stride * 8].reshape(n, stride, 8)[:, :, ::-1], axis=-1).reshape(n, stride)
    out[:] = packed
    norms = n16.astype(np.uint32)
    codes = PolarCodes(out, norms, {"pair": pair, "nodes": nodes, "y": y})
    if pc.m > 0:
        _residual_stage(codes, y, n16, pc, sign_stride)
    return codes


def unit_directions32(pair: np.ndarray, nodes, pc: PolarCodec) -> np.ndarray:
    """The stage-1 reconstruction u^ [n, d] in fp32, one rounding per product, from the root down
    (the order the residual of the QJL stage is defined in)."""
    n = pair.shape[0]
    r = np.ones((n, 1), dtype=np.float32)
    for lvl in range(pc.L, 1, -1):
        lv = pc.levels[lvl - 1]
        idx = nodes[lvl - 2]
        r = np.stack([r * lv.cos[idx], r * lv.sin[idx]], axis=-1).reshape(n, -1).astype(np.float32)
    lv = pc.levels[0]
    k = pair >> 2
    ua = (r * lv.cos[k]).astype(np.float32)
    ub = (r * lv.sin[k]).astype(np.float32)
    ua = np.where(pair & 1, -ua, ua)
    ub = np.where(pair & 2, -ub, ub)
    return np.stack([ua, ub], axis=-1).reshape(n, pc.d).astype(np.float32)


def _residual_stage(codes: PolarCodes, y: np.ndarray, n16: np.ndarray, pc: PolarCodec, sign_stride):
    """QJL on the polar residual: r = fl32(y - fl32(nbar u^)), rn16, exact signs of S r."""
    from .quantize import exact_sign_bits

    u32 = unit_directions32(codes.extra["pair"], codes.extra["nodes"], pc)
    nbar = f16_value(n16).astype(np.float32)
    resid = (y - (nbar[:, None] * u32).astype(np.float32)).astype(np.float32)
    rn16 = f16_norm_bits(resid)
    bits = exact_sign_bits(pc.sketch, resid)
    codes.sign = pack_bits(bits, 1, sign_stride)
    codes.norms = (rn16.astype(np.uint32) << 16) | n16.astype(np.uint32)
    codes.extra.update({"u32": u32, "resid": resid, "sign_bits": bits})


def encode(x: np.ndarray, pc: PolarCodec, pre_rotated: bool = False, first: int = 0,
           stride: Optional[int] = None, sign_stride: Optional[int] = None) -> PolarCodes:
    x32 = np.asarray(x, dtype=np.float32)
    n16 = f16_norm_bits(x32)
    if pre_rotated:
        y = x32
    else:
        rid = pc.rot_index(x32.shape[0], first)
        y = np.empty_like(x32)
        for r in np.unique(rid):
            sel = rid == r
            y[sel] = (x32[sel].astype(np.float64) @ pc.rot[r].astype(np.float64).T).astype(np.float32)
    return encode_rotated(y, n16, pc, stride, sign_stride)


def decode_fields(codes: PolarCodes, pc: PolarCodec):
    """Record -> (pair fields [n, d/2], node indices per level 2..L)."""
    n = codes.bits.shape[0]
    bits = np.unpackbits(codes.bits, axis=-1, bitorder="little")
    pos = 0

    def take(cnt, w):
        nonlocal pos
        v = np.zeros((n, cnt), dtype=np.uint32)
        for j in range(cnt):
            for t in range(w):
                v[:, j] |= bits[:, pos + t].astype(np.uint32) << t
            pos += w
        return v
    pair = take(pc.d // 2, 2 + pc.ab)
    nodes = [take(pc.d >> lvl, pc.ab) for lvl in range(2, pc.L + 1)]
    return pair, nodes


def unit_directions(codes: PolarCodes, pc: PolarCodec) -> np.ndarray:
    """u^ [n, d] in the rotated space (fp64), from the root down."""
    pair, nodes = decode_fields(codes, pc)
    n = pair.shape[0]
    r = np.ones((n, 1))
    for lvl in range(pc.L, 1, -1):          # nodes of level lvl: children radii
        lv = pc.levels[lvl - 1]
        idx = nodes[lvl - 2]
        c = lv.cos.astype(np.float64)[idx]
        s = lv.sin.astype(np.float64)[idx]
        r = np.stack([r * c, r * s], axis=-1).reshape(n, -1)
    lv = pc.levels[0]
    k = pair >> 2
    sa = np.where(pair & 1, -1.0, 1.0)
    sb = np.where(pair & 2, -1.0, 1.0)
    u = np.stack([r * sa * lv.cos.astype(np.float64)[k], r * sb * lv.sin.astype(np.float64)[k]], axis=-1)
    return u.reshape(n, pc.d)


def scores(q: np.ndarray, codes: PolarCodes, pc: PolarCodec, n_keys: int, hkv: int) -> np.ndarray:
    """Logits [S, hq, n_keys] = nbar <Pi_b q, u^> (+ rnbar sqrt(pi/2)/m <S Pi_b q, 2 b - 1> with the
    QJL stage) for queries [S, hq, d] (fp64)."""
    from .estimate import qjl_scale

    S, hq, d = q.shape
    G = hq // hkv
    u = unit_directions(codes, pc)
    nbar = f16_value((codes.norms & 0xFFFF).astype(np.uint16))
    if pc.m > 0:
        signs = 2.0 * unpack_bits(codes.sign, 1, pc.m).astype(np.float64) - 1.0
        rnbar = f16_value((codes.norms >> 16).astype(np.uint16))
    out = np.empty((S, hq, n_keys))
    for s_ in range(S):
        for h in range(hkv):
            blk = s_ * hkv + h
            sl = slice(blk * n_keys, (blk + 1) * n_keys)
            rid = pc.rot_index(1, blk * n_keys)[0]
            qt = q[s_, h * G:(h + 1) * G].astype(np.float64) @ pc.rot[rid].astype(np.float64).T
            out[s_, h * G:(h + 1) * G] = (qt @ u[sl].T) * nbar[sl][None, :]
            if pc.m > 0:
                qh = qt @ pc.sketch.astype(np.float64).T
                out[s_, h * G:(h + 1) * G] += (qh @ signs[sl].T) * (rnbar[sl] * qjl_scale(pc.m))[None, :]
    return out


def dequantize(codes: PolarCodes, pc: PolarCodec, first: int = 0) -> np.ndarray:
    """Explicit reconstruction in the original space (fp64): Pi^T (nbar u^ + [m > 0]
    rnbar sqrt(pi/2)/m S^T (2 b - 1))."""
    from .estimate import qjl_scale

    u = unit_directions(codes, pc)
    nbar = f16_value((codes.norms & 0xFFFF).astype(np.uint16))
    rot_space = nbar[:, None] * u
    if pc.m > 0:
        signs = 2.0 * unpack_bits(codes.sign, 1, pc.m).astype(np.float64) - 1.0
        rnbar = f16_value((codes.norms >> 16).astype(np.uint16))
        rot_space = rot_space + (rnbar * qjl_scale(pc.m))[:, None] * (signs @ pc.sketch.astype(np.float64))
    rid = pc.rot_index(u.shape[0], first)
    out = np.empty_like(rot_space)
    for r in np.unique(rid):
        sel = rid == r
        out[sel] = rot_space[sel] @ pc.rot[r].astype(np.float64)
    return out


def append(x: np.ndarray, pc: PolarCodec, slots, pos, rope_base: float, stride: Optional[int] = None,
           sign_stride: Optional[int] = None) -> PolarCodes:
    """Polar codes of new vectors appended to a growing cache, the two-stage append's steps with
    the polar stage (TurboESM summary, "Metodologia" A: RoPE first, then the orthogonal rotation;
    7minutos.es walkthrough, "Etapa 1": the codes stay in the cache): row k goes to cache slot
    slots[k], whose block selects the rotation, at position pos[k]; with rope_base > 0 the
    rotation sees RoPE(x, pos) in fp64, y = fl32(Pi_b RoPE(x)); the stored radius is fp16(||x||)
    (RoPE keeps norms)."""
    from .quantize import rope

    x32 = np.asarray(x, dtype=np.float32)
    x64 = x32.astype(np.float64)
    xr = rope(x64, np.asarray(pos), rope_base) if rope_base > 0 else x64
    rid = np.array([pc.rot_index(1, int(sl))[0] for sl in slots], dtype=np.int64)
    y = np.empty(x64.shape, dtype=np.float32)
    for r in np.unique(rid):
        sel = rid == r
        y[sel] = (xr[sel] @ pc.rot[r].astype(np.float64).T).astype(np.float32)
    return encode_rotated(y, f16_norm_bits(x32), pc, stride, sign_stride)


def _slice(codes: PolarCodes, a: int, b: int) -> PolarCodes:
    return PolarCodes(codes.bits[a:b], codes.norms[a:b], sign=None if codes.sign is None else codes.sign[a:b])


def attend_lens(q: np.ndarray, kcodes: PolarCodes, vcodes, pc: PolarCodec, vcodec, cap: int, lens, hkv: int,
                scale: float) -> np.ndarray:
    """Decode attention [S, Hq, d] over caches of capacity ``cap`` per (sequence, kv head) in which
    sequence s holds its first lens[s] tokens (none: a zero output): softmax over those tokens of
    scale times the polar estimate (with the rotation of the block's first record), times their
    values dequantised as the two-stage decoder does (fp64)."""
    from . import estimate as oe

    S, hq, d = q.shape
    g = hq // hkv
    out = np.zeros((S, hq, vcodec.d))
    for s_ in range(S):
        n = int(lens[s_])
        if n <= 0:
            continue
        for h in range(hkv):
            a = (s_ * hkv + h) * cap
            kc = _slice(kcodes, a, a + n)
            rid = pc.rot_index(1, a)[0]
            qt = q[s_, h * g:(h + 1) * g].astype(np.float64) @ pc.rot[rid].astype(np.float64).T
            lg = (qt @ unit_directions(kc, pc).T) * f16_value((kc.norms & 0xFFFF).astype(np.uint16))[None, :]
            if pc.m > 0:
                from .estimate import qjl_scale

                signs = 2.0 * unpack_bits(kc.sign, 1, pc.m).astype(np.float64) - 1.0
                rn = f16_value((kc.norms >> 16).astype(np.uint16))
                lg = lg + ((qt @ pc.sketch.astype(np.float64).T) @ signs.T) * (rn * qjl_scale(pc.m))[None, :]
            v = oe.dequantize(oe.Codes(vcodes.idx[a:a + n], None if vcodes.sign is None else vcodes.sign[a:a + n],
                                       vcodes.norms[a:a + n]), vcodec, a)
            out[s_, h * g:(h + 1) * g] = oe.softmax(scale * lg) @ v
    return out


def decode_step(q, k_new, v_new, kcodes: PolarCodes, vcodes, pc: PolarCodec, vcodec, cap: int, pos, rope_base: float,
                hkv: int, scale: float):
    """One decode step over growing caches [S][Hkv][cap] with polar keys and two-stage values:
    sequence s appends its new key (RoPE at pos[s], then the slot block's rotation) and value at
    slot pos[s], then its queries, turned by RoPE at pos[s], attend over tokens 0 .. pos[s]; a
    sequence whose position is outside [0, cap) appends nothing and gets a zero output.  Returns
    (outputs [S, Hq, d], updated key codes, updated value codes); the inputs are not modified."""
    from . import quantize as oq

    S, hq, d = q.shape
    pos = np.asarray(pos, dtype=np.int64)
    ok = (pos >= 0) & (pos < cap)
    slots = ((np.arange(S)[:, None] * hkv + np.arange(hkv)[None, :]) * cap + np.where(ok, pos, 0)[:, None]).reshape(-1)
    rows = np.repeat(ok, hkv)
    kpos = np.repeat(pos, hkv)
    k2 = PolarCodes(kcodes.bits.copy(), kcodes.norms.copy(), sign=None if kcodes.sign is None else kcodes.sign.copy())
    v2 = oq.Codes(vcodes.idx.copy(), None if vcodes.sign is None else vcodes.sign.copy(), vcodes.norms.copy())
    if rows.any():
        kn = np.asarray(k_new, dtype=np.float32).reshape(S * hkv, d)[rows]
        vn = np.asarray(v_new, dtype=np.float32).reshape(S * hkv, vcodec.d)[rows]
        nk = append(kn, pc, slots[rows], kpos[rows], rope_base, stride=k2.bits.shape[1],
                    sign_stride=None if k2.sign is None else k2.sign.shape[1])
        k2.bits[slots[rows]] = nk.bits
        k2.norms[slots[rows]] = nk.norms
        if k2.sign is not None:
            k2.sign[slots[rows]] = nk.sign
        nv = oq.append(vn, vcodec, slots[rows], kpos[rows], 0.0, idx_stride=v2.idx.shape[1],
                       sign_stride=None if v2.sign is None else v2.sign.shape[1])
        v2.idx[slots[rows]] = nv.idx
        v2.norms[slots[rows]] = nv.norms
        if v2.sign is not None:
            v2.sign[slots[rows]] = nv.sign
    qr = np.asarray(q, dtype=np.float64)
    if rope_base > 0:
        qr = oq.rope(qr.reshape(S * hq, d), np.repeat(pos, hq), rope_base).reshape(S, hq, d)
    out = attend_lens(qr, k2, v2, pc, vcodec, cap, np.where(ok, pos + 1, 0), hkv, scale)
    return out, k2, v2


def search_scores(queries: np.ndarray, db: PolarCodes, pc: PolarCodec, chunk: int = 65536) -> np.ndarray:
    """Estimated <q, x_n> [Q, n_db] of every query against every database record (one shared
    rotation): the logits of scores() with the database as one block of keys."""
    qs = np.asarray(queries, dtype=np.float64)
    n = db.norms.shape[0]
    out = np.empty((qs.shape[0], n))
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        part = PolarCodes(db.bits[a:b], db.norms[a:b], sign=None if db.sign is None else db.sign[a:b])
        out[:, a:b] = scores(qs[None], part, pc, b - a, 1)[0]
    return out


def search_topk(queries: np.ndarray, db: PolarCodes, pc: PolarCodec, k: int):
    """Top-k database records per query by estimated inner product (hada.io TurboQuant page,
    "Desempenho em busca vetorial"): score descending, then row ascending."""
    from .estimate import topk_rows

    return topk_rows(search_scores(queries, db, pc), k)


def exact_polar(y: np.ndarray):
    """The unquantised transform of y (fp64): (radius, level-1 signs and angles, node angles)."""
    y = np.asarray(y, dtype=np.float64)
    a, b = y[:, 0::2], y[:, 1::2]
    psi1 = np.arctan2(np.abs(b), np.abs(a))
    r = np.hypot(a, b)
    ang = []
    while r.shape[1] > 1:
        ra, rb = r[:, 0::2], r[:, 1::2]
        ang.append(np.arctan2(rb, ra))
        r = np.hypot(ra, rb)
    return r[:, 0], (a < 0, b < 0, psi1), ang


def attend(q: np.ndarray, kcodes: PolarCodes, vcodes, pc: PolarCodec, vcodec, n_ctx: int, hkv: int,
           scale: float) -> np.ndarray:
    """Decode attention [S, Hq, d] with polar keys and two-stage values (fp64): softmax over the
    keys of scale * nbar <Pi q, u^>, times the values dequantised as the two-stage decoder does
    (TurboESM summary, section 2.E: scores, softmax, weighted sum of the values)."""
    from . import estimate as oe

    S, hq, d = q.shape
    g = hq // hkv
    p = oe.softmax(scale * scores(q, kcodes, pc, n_ctx, hkv))
    out = np.empty((S, hq, vcodec.d))
    for s_ in range(S):
        for h in range(hkv):
            blk = s_ * hkv + h
            sl = slice(blk * n_ctx, (blk + 1) * n_ctx)
            v = oe.dequantize(oe.Codes(vcodes.idx[sl], None if vcodes.sign is None else vcodes.sign[sl],
                                       vcodes.norms[sl]), vcodec, blk * n_ctx)
            out[s_, h * g:(h + 1) * g] = p[s_, h * g:(h + 1) * g] @ v
    return out
