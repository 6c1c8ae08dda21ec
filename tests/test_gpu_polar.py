"""GPU parity of the recursive polar stage (tq_polar_encode, tq_polar_scores) against the oracle.

Encode, pre-rotated: from identical fp32 rotated inputs the bitstream and the norm word must be
bit-identical (every decision is a single-rounding fp32 comparison on both sides, and the
norm is the exactly rounded fp16 of the exact norm).  Full mode: the device rotation is
checked against the exact rotation within ROT_BOUND through the y tap; the records are
compared with the oracle's own encoding, the norm words exactly, every other difference
explained by the rotation bound (see _check_full).  Scores: records written by the oracle's encoder (or uniform random bits), logits
within score_tol(d) of the oracle's fp64 nbar <Pi q, u^>.  The tables are the oracle's, uploaded.
"""

import numpy as np
import pytest

import synth
from oracle import polar as op
from oracle import quantize as oq
from tests._util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

# Rotation error relative to sum_k |Pi_ik x_k|: the MFMA encoder (d = 64, 128, aligned rows) splits
# each operand into bf16 hi + lo (3 * 2^-16 missed) and accumulates 3d products in fp32
# (3d 2^-24); the FMA kernel (d = 256, or unaligned rows) (d + 2) 2^-24.  All below 2^-13.
ROT_BOUND = 2.0 ** -13
# Logit error bound relative to nbar ||q||.  The rotated query in fp32 is off by at most
# d 2^-24 ||q|| per coordinate (the rows of Pi are unit vectors), which moves <Pi q, u^> by at
# most sqrt(d) times that (||u^||_1 <= sqrt(d)); the radii (products of at most L fp32
# factors), the leaf terms and the fp32 sum of d/2 terms add at most (L + 4 + d/2) 2^-24
# sqrt(d) more.  With L + 4 <= 12 <= 16: (1.5 d + 16) sqrt(d) 2^-24.
def score_tol(d):
    return (1.5 * d + 16) * np.sqrt(d) * 2.0 ** -24


def _tables(pc):
    n = 1 << pc.ab
    t = np.zeros((pc.L, 4, n), np.float32)
    for l, lv in enumerate(pc.levels):
        t[l, 0], t[l, 1] = lv.cos, lv.sin
        t[l, 2, :n - 1], t[l, 3, :n - 1] = lv.c2, lv.s2
    return t


def _codecs(d, ab, rot_seed=1, basis=None, vpr=0, m=0, sketch_seed=5):
    ora = op.make_polar_codec(d, ab, rot_seed, basis_seeds=basis, vecs_per_rot=vpr, m=m,
                              sketch_seed=sketch_seed if m else None)
    lib = tq.polar_codec_from_arrays(d, ab, ora.rot, _tables(ora), vecs_per_rot=vpr, sketch=ora.sketch)
    return lib, ora


def _edge_rows(d):
    rows = np.zeros((8, d), np.float32)
    rows[1, 0] = 1.0                       # one coordinate: every other pair and node is 0 / 0
    rows[2, :] = np.float32(0.25)          # a == b everywhere: psi = pi/4 at every node
    rows[3, 1::2] = np.float32(-2.0)       # even coordinates zero, odd negative
    rows[4, ::2] = np.float32(-0.0)        # negative zeros keep a clear sign bit
    rows[4, 1::2] = np.float32(3.0)
    rows[5, :d // 2] = np.float32(1e-20)   # squares and sums in the fp32 subnormal range
    rows[6, :] = np.float32(2000.0)        # large norm, below 65520
    rows[7, ::4] = np.float32(1.5)
    rows[7, 1::4] = np.float32(-1.5)
    return rows


def _gpu_encode(lib, x_np, pre, dtype=None, first=0, tap=False, stride=None):
    x = torch.from_numpy(x_np).to("cuda")
    if dtype is not None:
        x = x.to(dtype)
    ytap = torch.empty((x.shape[0], lib.d), dtype=torch.float32, device="cuda") if tap else None
    out = tq.alloc_polar_codes(lib, x.shape[0], stride=stride)
    tq.polar_encode(lib, x, pre_rotated=pre, first=first, out=out, y_tap=ytap)
    torch.cuda.synchronize()
    got = out.numpy()
    res = (got[0], got[1], None if ytap is None else ytap.cpu().numpy())
    return res if lib.m == 0 else res + (got[2],)


@pytest.mark.parametrize("d,ab", [(64, 2), (64, 3), (128, 2), (128, 3), (128, 4), (256, 2), (256, 4)])
def test_pre_rotated_bit_exact(d, ab):
    say("polar encode pre-rotated", d, ab)
    lib, ora = _codecs(d, ab)
    y = np.concatenate([_edge_rows(d), synth.pre_rotated(2053, d, seed=d * 10 + ab)])
    y[100:200] *= np.float32(1e-3)
    y[200:300] *= np.float32(300.0)
    bits, norms, _ = _gpu_encode(lib, y, pre=True)
    want = op.encode(y, ora, pre_rotated=True, stride=lib.stride)
    assert np.array_equal(norms, want.norms)
    assert np.array_equal(bits, want.bits)
    assert norms[0] == 0
    # the pi/4 row: the level-1 index passes every threshold below pi/4 and the tie at pi/4
    pair, nodes = op.decode_fields(want, ora)
    assert np.all(pair[2] >> 2 == (1 << ab) // 2)


def test_pre_rotated_padded_stride():
    d, ab = 128, 2
    lib, ora = _codecs(d, ab)
    y = synth.pre_rotated(515, d, seed=3)
    stride = lib.stride + 32
    bits, norms, _ = _gpu_encode(lib, y, pre=True, stride=stride)
    want = op.encode(y, ora, pre_rotated=True, stride=stride)
    assert np.array_equal(bits, want.bits) and np.array_equal(norms, want.norms)
    assert not bits[:, lib.stride:].any()


def _near_nodes(A, B, dA, dB, lv):
    """Nodes whose index the y perturbation could change: for some threshold j,
    |B c2_j - A s2_j| is within what dA, dB and the fp32 roundings of the two products move."""
    c2 = lv.c2.astype(np.float64)
    s2 = lv.s2.astype(np.float64)
    margin = np.abs(B[..., None] * c2 - A[..., None] * s2)
    slack = dB[..., None] * c2 + dA[..., None] * s2 + 2.0 ** -22 * (B[..., None] * c2 + A[..., None] * s2)
    return np.any(margin <= 2.0 * slack + 1e-300, axis=-1)


def _check_full(x_seen, lib, ora, gpu, first=0, max_rows=0.02, low_norms_only=False):
    """Full-mode records against the oracle's own encoding (its fp64 rotation rounded to fp32):
    the rotation within ROT_BOUND of the exact one (through the y tap, where the call wrote one),
    the norm words exact, and every other difference explained by that bound (_explain_fields)."""
    bits, norms, ytap = gpu
    n, d = x_seen.shape
    y_ex, bound = _exact_rotation(x_seen.astype(np.float64), ora, ora.rot_index(n, first))
    if ytap is not None:
        assert np.all(np.abs(ytap.astype(np.float64) - y_ex) <= bound)
    want = op.encode(x_seen, ora, first=first, stride=lib.stride)
    assert np.array_equal(norms, want.norms & 0xFFFF if low_norms_only else want.norms)
    _explain_fields(bits, norms, want, bound + np.abs(want.extra["y"].astype(np.float64) - y_ex), ora, max_rows)


def _exact_rotation(x64, ora, rid):
    """The exact fp64 rotation of each row by its block's Pi, and ROT_BOUND carried to each y_i."""
    y_ex = np.empty_like(x64)
    bound = np.empty_like(x64)
    for r in np.unique(rid):
        sel = rid == r
        P = ora.rot[r].astype(np.float64)
        y_ex[sel] = x64[sel] @ P.T
        bound[sel] = ROT_BOUND * (np.abs(x64[sel]) @ np.abs(P).T) + 1e-45
    return y_ex, bound


def _explain_fields(bits, norms, want, dy, ora, max_rows):
    """Device records against the oracle's, given dy >= |y_device - y_oracle| per coordinate: a
    sign differs only where |y| is within dy, a node index only where dy, carried into the node's
    sums of squares, reaches one of its thresholds (each node's index depends on its own subtree's
    sums alone).  Returns the rows whose fields all agree."""
    n, d = dy.shape
    y_o = want.extra["y"].astype(np.float64)
    gp, gn = op.decode_fields(op.PolarCodes(bits, norms), ora)
    wp, wn = op.decode_fields(want, ora)
    # signs
    a, b = y_o[:, 0::2], y_o[:, 1::2]
    ok_sa = ((gp & 1) == (wp & 1)) | (np.abs(a) <= dy[:, 0::2])
    ok_sb = (((gp >> 1) & 1) == ((wp >> 1) & 1)) | (np.abs(b) <= dy[:, 1::2])
    assert ok_sa.all() and ok_sb.all()
    bad_rows = ((gp & 3) != (wp & 3)).any(axis=1)
    # node indices, level by level: sums of squares of each child's coordinates and their bounds
    sq = y_o * y_o
    dsq = 2.0 * np.abs(y_o) * dy + dy * dy
    for lvl in range(1, ora.L + 1):
        half = 1 << (lvl - 1)
        S = sq.reshape(n, d >> lvl, 2, half).sum(-1)
        dS = dsq.reshape(n, d >> lvl, 2, half).sum(-1) + 2.0 * (half + 1) * 2.0 ** -24 * S
        near = _near_nodes(S[..., 0], S[..., 1], dS[..., 0], dS[..., 1], ora.levels[lvl - 1])
        got = (gp >> 2) if lvl == 1 else gn[lvl - 2]
        exp = (wp >> 2) if lvl == 1 else wn[lvl - 2]
        diff = got != exp
        assert not (diff & ~near).any(), (lvl, np.argwhere(diff & ~near)[:5])
        bad_rows |= diff.any(axis=1)
    assert np.mean(bad_rows) <= max_rows, np.mean(bad_rows)
    return ~bad_rows


def _explain_qjl(norms, sign, want, dy, same, ora):
    """The QJL half of device records whose polar fields agree with the oracle's (rows `same`):
    the residual then differs by at most dr = dy (1 + 2^-23) + 2^-22 |r| per coordinate, which
    bounds fp16 ||r|| (within ||dr|| plus half an fp16 ulp) and any sign flip (only where
    |(S r)_j| <= sum_i |S_ji| dr_i)."""
    d = dy.shape[1]
    r_o = want.extra["resid"].astype(np.float64)
    dr = dy * (1.0 + 2.0 ** -23) + 2.0 ** -22 * np.abs(r_o) + 1e-45
    rn_gpu = oq.f16_value((norms >> 16).astype(np.uint16))
    rn_o = np.linalg.norm(r_o, axis=1)
    half_ulp = np.abs(np.spacing(rn_o.astype(np.float16)).astype(np.float64)) / 2
    slack = np.linalg.norm(dr, axis=1) + half_ulp
    assert np.all(np.abs(rn_gpu - rn_o)[same] <= slack[same])
    Sk = ora.sketch.astype(np.float64)
    z = r_o @ Sk.T
    zb = dr @ np.abs(Sk).T
    gb = np.unpackbits(sign, axis=1, bitorder="little")[:, :ora.m].astype(bool)
    wb = want.extra["sign_bits"].astype(bool)
    flip = (gb != wb) & same[:, None]
    assert not (flip & (np.abs(z) > zb)).any()
    return int(flip.sum())


@pytest.mark.parametrize("d,ab,dtype", [(64, 3, "float32"), (128, 2, "bfloat16"), (128, 4, "float16"),
                                        (256, 3, "float32")])
def test_full_mode_codes_of_the_tap(d, ab, dtype):
    say("polar encode full", d, ab, dtype)
    lib, ora = _codecs(d, ab)
    g = np.random.default_rng(d + ab)
    x = (g.standard_normal((1501, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    tdt = getattr(torch, dtype)
    x_seen = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    _check_full(x_seen, lib, ora, _gpu_encode(lib, x, pre=False, dtype=tdt, tap=True))


@pytest.mark.parametrize("d,dtype,first", [(128, "float32", 64), (128, "bfloat16", 64), (64, "float32", 64),
                                           (64, "float16", 64), (64, "float16", 40)])
def test_full_mode_rotation_blocks(d, dtype, first):
    # 40 blocks of 32 vectors from an offset, 40 vectors past the last block (they take the last
    # rotation); bf16 at d = 128 and every type at d = 64 run the MFMA encoder's block loop when
    # the offset is a multiple of 32, the FMA kernel otherwise (and for fp32 at d = 128)
    ab, n_rot, vpr = 2, 40, 32
    lib, ora = _codecs(d, ab, basis=[500 + i for i in range(n_rot)], vpr=vpr)
    n = n_rot * vpr - first + 40
    x = (np.random.default_rng(9).standard_normal((n, d)) * 3.0).astype(np.float32)
    tdt = getattr(torch, dtype)
    x_seen = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    _check_full(x_seen, lib, ora, _gpu_encode(lib, x, pre=False, dtype=tdt, first=first, tap=True), first=first)


@pytest.mark.parametrize("d,ab", [(64, 3), (128, 2)])
def test_full_mode_unaligned_rows(d, ab):
    # rows d + 1 floats apart: not 16-byte aligned, so the FMA kernel encodes them
    lib, ora = _codecs(d, ab)
    x = (np.random.default_rng(d).standard_normal((777, d + 1)) * 2.0).astype(np.float32)
    xt = torch.from_numpy(x).cuda()[:, :d]
    ytap = torch.empty((x.shape[0], d), dtype=torch.float32, device="cuda")
    out = tq.polar_encode(lib, xt, y_tap=ytap)
    torch.cuda.synchronize()
    bits, norms = out.numpy()
    _check_full(np.ascontiguousarray(x[:, :d]), lib, ora, (bits, norms, ytap.cpu().numpy()))


def _score_case(lib, ora, q, codes_bits, norms, n_keys, hkv):
    n_seq, hq, d = q.shape
    k = tq.PolarCodes(torch.from_numpy(np.ascontiguousarray(codes_bits)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(norms).view(np.int32)).cuda())
    got = tq.polar_scores(lib, torch.from_numpy(q).cuda(), k, n_keys, hkv).cpu().numpy()
    want = op.scores(q, op.PolarCodes(codes_bits, norms), ora, n_keys, hkv)
    nbar = oq.f16_value((norms & 0xFFFF).astype(np.uint16)).reshape(n_seq, hkv, 1, n_keys)
    qn = np.linalg.norm(q.astype(np.float64), axis=-1).reshape(n_seq, hkv, hq // hkv, 1)
    tol = (score_tol(d) * nbar * qn).reshape(n_seq, hq, n_keys) + 1e-30
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= tol), float(np.max(err / tol))
    return float(np.max(err / tol))


@pytest.mark.parametrize("d,ab,n_seq,hq,hkv,n_keys", [
    (128, 2, 2, 8, 2, 1000),    # 4 heads per table
    (128, 3, 1, 3, 3, 777),     # one head per table
    (64, 3, 2, 6, 3, 515),      # two
    (64, 2, 1, 16, 2, 300),     # eight
    (256, 4, 1, 4, 2, 400),     # two (the table limit)
    (128, 2, 1, 4, 1, 1),       # a single key
])
def test_scores_match_oracle(d, ab, n_seq, hq, hkv, n_keys):
    say("polar scores", d, ab, n_seq, hq, hkv, n_keys)
    lib, ora = _codecs(d, ab)
    g = np.random.default_rng(d * ab + n_keys)
    x = (g.standard_normal((n_seq * hkv * n_keys, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    enc = op.encode(x, ora, stride=lib.stride)
    q = g.standard_normal((n_seq, hq, d)).astype(np.float32)
    r = _score_case(lib, ora, q, enc.bits, enc.norms, n_keys, hkv)
    say("  max err / tol", r)


def _random_records(n, d, ab, stride, seed):
    g = np.random.default_rng(seed)
    nb = (d // 2) * (2 + ab) + (d // 2 - 1) * ab
    bitsarr = g.integers(0, 2, (n, stride * 8), dtype=np.uint8)
    bitsarr[:, nb:] = 0
    rec = np.packbits(bitsarr, axis=-1, bitorder="little")
    norms = np.abs(g.standard_normal(n) * np.sqrt(d)).astype(np.float16).view(np.uint16).astype(np.uint32)
    return rec, norms


@pytest.mark.parametrize("d,ab", [(64, 4), (128, 2), (256, 3)])
def test_scores_random_records(d, ab):
    # uniform bits reach every field value of every pair and node
    lib, ora = _codecs(d, ab)
    n_seq, hq, hkv, n_keys = 1, 4, 2, 600
    rec, norms = _random_records(n_seq * hkv * n_keys, d, ab, lib.stride, seed=d + ab)
    q = np.random.default_rng(1).standard_normal((n_seq, hq, d)).astype(np.float32)
    _score_case(lib, ora, q, rec, norms, n_keys, hkv)


def test_scores_per_block_rotations():
    d, ab, n_seq, hq, hkv, n_keys = 64, 2, 2, 6, 3, 200
    seeds = [700 + i for i in range(n_seq * hkv)]
    lib, ora = _codecs(d, ab, basis=seeds, vpr=n_keys)
    x = np.random.default_rng(4).standard_normal((n_seq * hkv * n_keys, d)).astype(np.float32)
    enc = op.encode(x, ora, stride=lib.stride)
    q = np.random.default_rng(5).standard_normal((n_seq, hq, d)).astype(np.float32)
    _score_case(lib, ora, q, enc.bits, enc.norms, n_keys, hkv)


def test_full_size_sampled():
    # the 8B decode shape of one layer's batch at full context (8 sequences x 8 kv heads x 32768
    # keys, 32 query heads), in the launch configuration of the bench.  Scores: seeded random
    # records (uniform bits, fp16 norms) scored on the device, the oracle's logits on 512
    # sampled keys.  Encode: the device encodes the 2.1M bf16 keys in one call (the MFMA
    # encoder's multi-pass grid-stride loop); the norm words must equal the exact fp16 norms of
    # the inputs (65536 sampled), and the records of 4096 sampled keys of that same call must
    # match the oracle's encoding up to differences the rotation bound explains (no y tap: the
    # bound is taken from the exact fp64 rotation).  A y-tapped re-encode of 1024 of them is
    # checked against the tap as well.
    w = synth.GQA_DECODE
    d, ab, n_seq = w.d, 2, w.batch
    lib, ora = _codecs(d, ab)
    n = n_seq * w.hkv * w.n_ctx
    rec, norms = _random_records(n, d, ab, lib.stride, seed=21)
    g = np.random.default_rng(22)
    q = g.standard_normal((n_seq, w.hq, d)).astype(np.float32)
    kd = tq.PolarCodes(torch.from_numpy(rec).cuda(), torch.from_numpy(norms.view(np.int32)).cuda())
    logits = tq.polar_scores(lib, torch.from_numpy(q).cuda(), kd, w.n_ctx, w.hkv).cpu().numpy()
    keys = np.sort(g.choice(n, 512, replace=False))
    u = op.unit_directions(op.PolarCodes(rec[keys], norms[keys]), ora)
    nbar = oq.f16_value((norms[keys] & 0xFFFF).astype(np.uint16))
    blk = keys // w.n_ctx
    s_idx, h_idx, t_idx = blk // w.hkv, blk % w.hkv, keys % w.n_ctx
    G = w.hq // w.hkv
    P = ora.rot[0].astype(np.float64)
    for i in range(len(keys)):
        heads = np.arange(h_idx[i] * G, (h_idx[i] + 1) * G)
        qh = q[s_idx[i], heads].astype(np.float64)
        want = (qh @ P.T) @ u[i] * nbar[i]
        tol = score_tol(d) * nbar[i] * np.linalg.norm(qh, axis=-1)
        assert np.all(np.abs(logits[s_idx[i], heads, t_idx[i]] - want) <= tol)

    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    K = torch.randn((n, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    codes = tq.polar_encode(lib, K)
    torch.cuda.synchronize()
    x_seen = K.float().cpu().numpy()
    rows = np.sort(g.choice(n, 65536, replace=False))
    assert np.array_equal(codes.norms.cpu().numpy().view(np.uint32)[rows], oq.f16_norm_bits(x_seen[rows]))
    sub = np.sort(g.choice(n, 4096, replace=False))
    full = (codes.bits.cpu().numpy()[sub], codes.norms.cpu().numpy().view(np.uint32)[sub], None)
    _check_full(x_seen[sub], lib, ora, full)
    sub = sub[:1024]
    _check_full(x_seen[sub], lib, ora, _gpu_encode(lib, x_seen[sub], pre=False, dtype=torch.bfloat16, tap=True))


def test_attention_with_polar_keys_full_size_sampled():
    # the same shape, seeded random polar key records and random 3-bit value planes; attention
    # outputs of 6 sampled (sequence, query head) pairs against the oracle's
    from oracle import codec as oc

    w = synth.GQA_DECODE
    d, ab, n_seq = w.d, 2, w.batch
    lib, ora = _codecs(d, ab)
    vl = tq.make_codec(d, w.v_bits, w.v_m, 3, 4)
    vo = oc.make_codec(d, w.v_bits, w.v_m, 3, 4)
    n = n_seq * w.hkv * w.n_ctx
    rec, norms = _random_records(n, d, ab, lib.stride, seed=31)
    vidx, vsign, vnorms = synth.random_codes(n, d, w.v_bits, w.v_m, vl.idx_stride, vl.sign_stride, seed=32)
    g = np.random.default_rng(33)
    q = g.standard_normal((n_seq, w.hq, d)).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    kd = tq.PolarCodes(torch.from_numpy(rec).cuda(), torch.from_numpy(norms.view(np.int32)).cuda())
    vd = tq.Codes(torch.from_numpy(vidx).cuda(), None, torch.from_numpy(vnorms.view(np.int32)).cuda())
    out = tq.polar_attend_decode(lib, vl, torch.from_numpy(q).cuda(), kd, vd, w.n_ctx, w.hkv, scale).cpu().numpy()
    G = w.hq // w.hkv
    for s, h in [(0, 0), (0, 31), (3, 9), (5, 17), (7, 4), (7, 30)]:
        blk = s * w.hkv + h // G
        sl = slice(blk * w.n_ctx, (blk + 1) * w.n_ctx)
        kc = op.PolarCodes(rec[sl], norms[sl])
        vc = oq.Codes(vidx[sl], None, vnorms[sl])
        # one block: its rotation is the shared one, so the block can be scored on its own
        want = op.attend(q[s:s + 1, h:h + 1].astype(np.float64), kc, vc, ora, vo, w.n_ctx, 1, scale)[0, 0]
        err = np.max(np.abs(out[s, h] - want)) / np.max(np.abs(want))
        assert err <= 1e-3, (s, h, err)


def test_zero_sizes_and_errors():
    lib, _ = _codecs(64, 2)
    empty = tq.alloc_polar_codes(lib, 0)
    x = torch.zeros((0, 64), device="cuda")
    tq.polar_encode(lib, x, out=empty)
    q = torch.zeros((1, 2, 64), device="cuda")
    tq.polar_scores(lib, q, empty, 0, 1, logits=torch.zeros((1, 2, 0), device="cuda"))
    bad = tq.alloc_polar_codes(lib, 4, stride=lib.stride - 4)
    x4 = torch.zeros((4, 64), device="cuda")
    with pytest.raises(ValueError):  # the binding's check
        tq.polar_encode(lib, x4, out=bad)
    cc = lib.c()  # the library's own check of the same call, before any launch
    assert tq.lib.tq_polar_encode(tq.ctypes.byref(cc), tq._ptr(x4), 0, 4, 64, 0, 0, bad.c(), None,
                                  tq._stream()) == -1


@pytest.mark.parametrize("d,ab,vbits,vm,n_seq,hq,hkv,n_ctx", [
    (128, 2, 3, 0, 2, 8, 2, 1000),     # 4 heads per kv head, 3-bit values (the 8B value codec)
    (128, 2, 3, 0, 1, 16, 2, 3000),    # 8 heads per kv head: two groups of four
    (64, 3, 3, 64, 1, 6, 3, 515),      # 2 heads, values with QJL
    (128, 2, 2, 128, 1, 2, 2, 2000),   # 1 head; several context chunks
])
def test_attention_with_polar_keys(d, ab, vbits, vm, n_seq, hq, hkv, n_ctx):
    from oracle import codec as oc

    say("polar attention", d, ab, vbits, vm, n_seq, hq, hkv, n_ctx)
    lib, ora = _codecs(d, ab)
    vl = tq.make_codec(d, vbits, vm, 3, 4)
    vo = oc.make_codec(d, vbits, vm, 3, 4)
    g = np.random.default_rng(d + n_ctx)
    n = n_seq * hkv * n_ctx
    x = (g.standard_normal((n, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    kc = op.encode(x, ora, stride=lib.stride)
    vc = oq.encode(g.standard_normal((n, d)).astype(np.float32), vo, idx_stride=vl.idx_stride,
                   sign_stride=vl.sign_stride)
    q = g.standard_normal((n_seq, hq, d)).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    kd = tq.PolarCodes(torch.from_numpy(kc.bits).cuda(), torch.from_numpy(kc.norms.view(np.int32)).cuda())
    vd = tq.Codes(torch.from_numpy(vc.idx).cuda(), None if vc.sign is None else torch.from_numpy(vc.sign).cuda(),
                  torch.from_numpy(vc.norms.view(np.int32)).cuda())
    got = tq.polar_attend_decode(lib, vl, torch.from_numpy(q).cuda(), kd, vd, n_ctx, hkv, scale).cpu().numpy()
    want = op.attend(q.astype(np.float64), kc, vc, ora, vo, n_ctx, hkv, scale)
    err = np.max(np.abs(got - want), axis=-1) / np.max(np.abs(want), axis=-1)
    say("  max rel err", float(err.max()))
    assert np.all(err <= 1e-3)


def test_attention_with_polar_keys_argument_errors():
    lib, _ = _codecs(64, 2)
    vl = tq.make_codec(128, 3, 0, 3, 4)  # another d
    k = tq.alloc_polar_codes(lib, 8)
    v = tq.alloc_codes(vl, 8)
    q = torch.zeros((1, 2, 64), device="cuda")
    with pytest.raises(ValueError):  # the binding's check
        tq.polar_attend_decode(lib, vl, q, k, v, 4, 2, 1.0)
    cc0, vc0 = lib.c(), vl.c()  # the library's own check: d differs
    assert tq.lib.tq_polar_attend_decode(tq.ctypes.byref(cc0), tq.ctypes.byref(vc0), tq._ptr(q), 1, 2, 2, 4, k.c(),
                                         v.c(), 1.0, tq._ptr(q), None, 0, tq._stream()) == -1
    vl64 = tq.make_codec(64, 3, 0, 3, 4)
    cc, vc = lib.c(), vl64.c()
    need = tq.lib.tq_polar_attend_workspace_bytes(tq.ctypes.byref(cc), tq.ctypes.byref(vc), 1, 2, 2, 4)
    assert need >= 2 * 4 * 4
    rc = tq.lib.tq_polar_attend_decode(tq.ctypes.byref(cc), tq.ctypes.byref(vc), tq._ptr(q), 1, 2, 2, 4, k.c(),
                                       tq.alloc_codes(vl64, 8).c(), 1.0, tq._ptr(q), None, 0, tq._stream())
    assert rc == -4


# ------------------------------------------------------------------ the QJL stage on the polar residual


def _qjl_score_tol(lib, ora, q, norms, n_keys, hkv):
    """Bound on the QJL term's error, per logit: the sketched query S q~ in fp32 is off by at most
    2^-24 (d + 1) sum_k |S_jk| (|q~_k| + sum_i |Pi_ki| |q_i|) per row (its own fp32 sum plus the
    rotated query's), each table entry sums 4 of them and each logit m/4 entries (m/4 + 3 more
    roundings of sum_j |S q~|_j, taken as m/4 + 8), and the fma with rnbar sqrt(pi/2)/m rounds
    once more."""
    n_seq, hq, d = q.shape
    G = hq // hkv
    S = np.abs(ora.sketch.astype(np.float64))
    tol = np.empty((n_seq, hq, n_keys))
    rq = oq.f16_value((norms >> 16).astype(np.uint16)) * np.sqrt(np.pi / 2) / ora.m
    for s_ in range(n_seq):
        for h in range(hkv):
            blk = s_ * hkv + h
            P = ora.rot[ora.rot_index(1, blk * n_keys)[0]].astype(np.float64)
            qq = q[s_, h * G:(h + 1) * G].astype(np.float64)
            qt = qq @ P.T
            base = (np.abs(qt) + np.abs(qq) @ np.abs(P).T) @ S.T  # [G, m]
            e = 2.0 ** -24 * ((d + 1) * base.sum(-1) + (ora.m // 4 + 8) * np.abs(qt @ ora.sketch.astype(np.float64).T).sum(-1))
            tol[s_, h * G:(h + 1) * G] = e[:, None] * rq[blk * n_keys:(blk + 1) * n_keys][None, :]
    return tol


def _qjl_score_case(lib, ora, q, codes, n_keys, hkv):
    n_seq, hq, d = q.shape
    k = tq.PolarCodes(torch.from_numpy(np.ascontiguousarray(codes.bits)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(codes.norms).view(np.int32)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(codes.sign)).cuda())
    got = tq.polar_scores(lib, torch.from_numpy(q).cuda(), k, n_keys, hkv).cpu().numpy()
    want = op.scores(q, codes, ora, n_keys, hkv)
    nbar = oq.f16_value((codes.norms & 0xFFFF).astype(np.uint16)).reshape(n_seq, hkv, 1, n_keys)
    qn = np.linalg.norm(q.astype(np.float64), axis=-1).reshape(n_seq, hkv, hq // hkv, 1)
    tol = (score_tol(d) * nbar * qn).reshape(n_seq, hq, n_keys)
    tol = tol + _qjl_score_tol(lib, ora, q, codes.norms, n_keys, hkv) + 2.0 ** -24 * np.abs(want) + 1e-30
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= tol), float(np.max(err / tol))
    return float(np.max(err / tol))


@pytest.mark.parametrize("d,ab", [(64, 2), (64, 4), (128, 2), (128, 3)])
def test_qjl_pre_rotated_bit_exact(d, ab):
    # from identical rotated inputs the whole record is bit-identical: the polar fields, fp16 ||x||,
    # the fp32 reconstruction from the root down and its residual, fp16 ||r|| and the exact signs
    say("polar+qjl encode pre-rotated", d, ab)
    lib, ora = _codecs(d, ab, m=d)
    y = np.concatenate([_edge_rows(d), synth.pre_rotated(1027, d, seed=d * 10 + ab + 1)])
    y[100:200] *= np.float32(1e-3)
    y[200:300] *= np.float32(300.0)
    bits, norms, _, sign = _gpu_encode(lib, y, pre=True)
    want = op.encode(y, ora, pre_rotated=True, stride=lib.stride, sign_stride=lib.sign_stride)
    assert np.array_equal(bits, want.bits)
    assert np.array_equal(norms, want.norms)
    assert np.array_equal(sign, want.sign)
    assert norms[0] == 0 and np.all(sign[0] == 0xFF)  # zero vector: zero residual, (S 0)_j = 0 >= 0
    assert np.any(norms[8:] >> 16)


def test_qjl_pre_rotated_padded_sign_stride():
    d, ab = 64, 3
    lib, ora = _codecs(d, ab, m=d)
    y = synth.pre_rotated(300, d, seed=8)
    out = tq.alloc_polar_codes(lib, y.shape[0])
    out.sign = torch.full((y.shape[0], lib.sign_stride + 16), 0xAB, dtype=torch.uint8, device="cuda")
    tq.polar_encode(lib, torch.from_numpy(y).cuda(), pre_rotated=True, out=out)
    bits, norms, sign = out.numpy()
    want = op.encode(y, ora, pre_rotated=True, stride=lib.stride, sign_stride=lib.sign_stride)
    assert np.array_equal(bits, want.bits) and np.array_equal(norms, want.norms)
    assert np.array_equal(sign[:, :lib.sign_stride], want.sign)
    assert not sign[:, lib.sign_stride:].any()  # the whole row is written, pad bytes zero


@pytest.mark.parametrize("d,ab,dtype", [(64, 3, "float32"), (128, 2, "bfloat16"), (128, 3, "float16")])
def test_qjl_full_mode_explained(d, ab, dtype):
    # full mode: the rotation is the FMA kernel's (the MFMA encoder has no residual stage); the
    # polar fields as _check_full, and on rows whose fields agree the residual differs from the
    # oracle's by at most dr = dy (1 + 2^-23) + 2^-22 |r|, which bounds fp16 ||r|| and any sign flip
    say("polar+qjl encode full", d, ab, dtype)
    lib, ora = _codecs(d, ab, m=d)
    g = np.random.default_rng(d + ab + 7)
    x = (g.standard_normal((1201, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    tdt = getattr(torch, dtype)
    x_seen = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    bits, norms, ytap, sign = _gpu_encode(lib, x, pre=False, dtype=tdt, tap=True)
    y_ex, bound = _exact_rotation(x_seen.astype(np.float64), ora, ora.rot_index(x.shape[0]))
    assert np.all(np.abs(ytap.astype(np.float64) - y_ex) <= bound)
    want = op.encode(x_seen, ora, stride=lib.stride, sign_stride=lib.sign_stride)
    assert np.array_equal(norms & 0xFFFF, want.norms & 0xFFFF)
    # the device's y (the tap) against the oracle's
    dy = np.abs(ytap.astype(np.float64) - want.extra["y"].astype(np.float64))
    same = _explain_fields(bits, norms, want, dy, ora, 0.02)
    flips = _explain_qjl(norms, sign, want, dy, same, ora)
    assert flips <= max(1, int(0.02 * x.shape[0]))


@pytest.mark.parametrize("d,ab,n_seq,hq,hkv,n_keys", [
    (128, 2, 2, 8, 2, 700),   # 4 heads per kv head: two heads per table (the table limit)
    (128, 3, 1, 3, 3, 333),   # one head per table
    (64, 2, 1, 16, 2, 300),   # eight heads per kv head: four per table
    (64, 4, 2, 6, 3, 257),    # two
    (128, 2, 1, 4, 1, 1),     # a single key
])
def test_qjl_scores_match_oracle(d, ab, n_seq, hq, hkv, n_keys):
    say("polar+qjl scores", d, ab, n_seq, hq, hkv, n_keys)
    lib, ora = _codecs(d, ab, m=d)
    g = np.random.default_rng(d * ab + n_keys + 1)
    x = (g.standard_normal((n_seq * hkv * n_keys, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    enc = op.encode(x, ora, stride=lib.stride, sign_stride=lib.sign_stride)
    q = g.standard_normal((n_seq, hq, d)).astype(np.float32)
    say("  max err / tol", _qjl_score_case(lib, ora, q, enc, n_keys, hkv))


def test_qjl_scores_random_records_and_rotations():
    # uniform bits reach every polar field value and every sign group value of every position;
    # per-block rotations
    d, ab, n_seq, hq, hkv, n_keys = 64, 3, 2, 4, 2, 400
    lib, ora = _codecs(d, ab, basis=[900 + i for i in range(n_seq * hkv)], vpr=n_keys, m=d)
    rec, norms = _random_records(n_seq * hkv * n_keys, d, ab, lib.stride, seed=77)
    g = np.random.default_rng(78)
    rn = np.abs(g.standard_normal(norms.shape[0]) * 2.0).astype(np.float16).view(np.uint16).astype(np.uint32)
    sign = g.integers(0, 256, (norms.shape[0], lib.sign_stride), dtype=np.uint8)
    codes = op.PolarCodes(rec, norms | (rn << 16), sign=sign)
    q = g.standard_normal((n_seq, hq, d)).astype(np.float32)
    _qjl_score_case(lib, ora, q, codes, n_keys, hkv)


@pytest.mark.parametrize("d,ab,vbits,vm,n_seq,hq,hkv,n_ctx", [
    (128, 2, 3, 0, 2, 8, 2, 1000),
    (64, 3, 3, 64, 1, 6, 3, 515),
])
def test_qjl_attention_with_polar_keys(d, ab, vbits, vm, n_seq, hq, hkv, n_ctx):
    from oracle import codec as oc

    say("polar+qjl attention", d, ab, vbits, vm, n_seq, hq, hkv, n_ctx)
    lib, ora = _codecs(d, ab, m=d)
    vl = tq.make_codec(d, vbits, vm, 3, 4)
    vo = oc.make_codec(d, vbits, vm, 3, 4)
    g = np.random.default_rng(d + n_ctx + 5)
    n = n_seq * hkv * n_ctx
    x = (g.standard_normal((n, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    kc = op.encode(x, ora, stride=lib.stride, sign_stride=lib.sign_stride)
    vc = oq.encode(g.standard_normal((n, d)).astype(np.float32), vo, idx_stride=vl.idx_stride,
                   sign_stride=vl.sign_stride)
    q = g.standard_normal((n_seq, hq, d)).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    kd = tq.PolarCodes(torch.from_numpy(kc.bits).cuda(), torch.from_numpy(kc.norms.view(np.int32)).cuda(),
                       torch.from_numpy(kc.sign).cuda())
    vd = tq.Codes(torch.from_numpy(vc.idx).cuda(), None if vc.sign is None else torch.from_numpy(vc.sign).cuda(),
                  torch.from_numpy(vc.norms.view(np.int32)).cuda())
    got = tq.polar_attend_decode(lib, vl, torch.from_numpy(q).cuda(), kd, vd, n_ctx, hkv, scale).cpu().numpy()
    want = op.attend(q.astype(np.float64), kc, vc, ora, vo, n_ctx, hkv, scale)
    err = np.max(np.abs(got - want), axis=-1) / np.max(np.abs(want), axis=-1)
    say("  max rel err", float(err.max()))
    assert np.all(err <= 1e-3)


def test_qjl_codec_errors():
    lib, _ = _codecs(64, 2, m=64)
    x = torch.zeros((4, 64), device="cuda")
    nosign = tq.alloc_polar_codes(lib, 4)
    nosign.sign = None
    with pytest.raises(ValueError):  # the binding's check
        tq.polar_encode(lib, x, out=nosign)
    cc = lib.c()  # the library's own check: m > 0 needs a sign plane
    assert tq.lib.tq_polar_encode(tq.ctypes.byref(cc), tq._ptr(x), 0, 4, 64, 0, 0, nosign.c(), None,
                                  tq._stream()) == -1
    bad = tq._PolarCodec(64, 2, 1, 0, lib.rot.data_ptr(), lib.tables.data_ptr(), 32, lib.sketch.data_ptr())
    ok = tq.alloc_polar_codes(lib, 4)
    assert tq.lib.tq_polar_encode(tq.ctypes.byref(bad), tq._ptr(x), 0, 4, 64, 0, 0, ok.c(), None,
                                  tq._stream()) == -2  # m other than 0 or d


# ------------------------------------------------------------------ append


@pytest.mark.parametrize("d,ab,m,dtype,rope_base,per_block", [
    (128, 2, 0, "bfloat16", 10000.0, False),  # the 8B key shape, RoPE
    (64, 3, 64, "float32", 10000.0, True),    # QJL stage, a rotation per cache block
    (128, 3, 128, "float16", 0.0, False),     # values: no RoPE
    (256, 2, 0, "float32", 500000.0, False),
])
def test_polar_append_matches_oracle(d, ab, m, dtype, rope_base, per_block):
    # ragged positions over a [n_seq][hkv][cap] cache, one below 0 and one at cap (skipped); the
    # appended records against the oracle's append (RoPE in fp64, then the slot block's rotation):
    # the radius word exact, every other difference explained by the rotation bound (the device
    # rounds RoPE(x) to fp32 before its fp32 rotation: (d + 3) 2^-24, within ROT_BOUND); every
    # other record untouched
    n_seq, hkv, cap = 6, 3, 40
    basis = [300 + i for i in range(n_seq * hkv)] if per_block else None
    lib, ora = _codecs(d, ab, basis=basis, vpr=cap if per_block else 0, m=m)
    say("polar append", d, ab, m, dtype, rope_base, per_block)
    g = np.random.default_rng(d + ab + m)
    x = (g.standard_normal((n_seq, hkv, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    pos = np.array([0, 17, cap - 1, -1, cap, 5], np.int32)
    tdt = getattr(torch, dtype)
    xt = torch.from_numpy(x).cuda().to(tdt)
    x_seen = xt.float().cpu().numpy().reshape(-1, d)
    n_rec = n_seq * hkv * cap
    cache = tq.alloc_polar_codes(lib, n_rec)
    cache.bits.fill_(0xAB)
    cache.norms.fill_(0x1234567)
    if m:
        cache.sign.fill_(0xCD)
    tq.polar_append(lib, xt, torch.from_numpy(pos).cuda(), cap, rope_base, cache)
    torch.cuda.synchronize()
    got = cache.numpy()
    rows = np.array([r for r in range(n_seq * hkv) if 0 <= pos[r // hkv] < cap])
    slots = rows * cap + pos[rows // hkv]
    want = op.append(x_seen[rows], ora, slots, pos[rows // hkv], rope_base, stride=lib.stride,
                     sign_stride=lib.sign_stride if m else None)
    assert np.array_equal(got[1][slots] & 0xFFFF, oq.f16_norm_bits(x_seen[rows]))  # the radius of x itself
    if not m:
        assert np.array_equal(got[1][slots], want.norms)
    xr = oq.rope(x_seen[rows], pos[rows // hkv], rope_base) if rope_base > 0 else x_seen[rows].astype(np.float64)
    rid = np.array([ora.rot_index(1, int(t))[0] for t in slots])
    y_ex, bound = _exact_rotation(xr, ora, rid)
    dy = bound + np.abs(want.extra["y"].astype(np.float64) - y_ex)
    same = _explain_fields(got[0][slots], got[1][slots], want, dy, ora, 0.1)
    if m:
        flips = _explain_qjl(got[1][slots], got[2][slots], want, dy, same, ora)
        assert flips <= 2
    other = np.setdiff1d(np.arange(n_rec), slots)
    assert np.all(got[0][other] == 0xAB) and np.all(got[1][other] == 0x1234567)
    if m:
        assert np.all(got[2][other] == 0xCD)


def test_polar_append_then_scores_see_the_turned_keys():
    # keys appended with RoPE at their positions score against a query turned by RoPE at the
    # query's position like the unturned pair at the relative offset (RoPE then the rotation keeps
    # inner products): the logits of the appended cache within the codec's error of q . k
    d, ab, cap, base = 128, 4, 64, 10000.0
    lib, ora = _codecs(d, ab)
    g = np.random.default_rng(41)
    keys = g.standard_normal((cap, d)).astype(np.float32)
    cache = tq.alloc_polar_codes(lib, cap)
    for t in range(cap):
        tq.polar_append(lib, torch.from_numpy(keys[t][None, None]).cuda(), torch.tensor([t], dtype=torch.int32,
                        device="cuda"), cap, base, cache)
    q = g.standard_normal((1, 1, d)).astype(np.float32)
    qpos = cap - 1
    qr = oq.rope(q[0], np.array([qpos]), base).astype(np.float32)[None]
    got = tq.polar_scores(lib, torch.from_numpy(qr).cuda(), cache, cap, 1).cpu().numpy()[0, 0]
    exact = np.array([(oq.rope(q[0], [qpos], base) @ oq.rope(keys[t:t + 1], [t], base).T).item() for t in range(cap)])
    bits, norms = cache.numpy()
    want = op.scores(qr.astype(np.float64), op.PolarCodes(bits, norms), ora, cap, 1)[0, 0]
    nbar = oq.f16_value((norms & 0xFFFF).astype(np.uint16))
    assert np.all(np.abs(got - want) <= score_tol(d) * np.linalg.norm(qr) * nbar + 1e-30)
    # and the estimate tracks the exact RoPE'd inner product (4 angle bits: about 1% of |q||k|)
    rel = np.abs(got - exact) / (np.linalg.norm(q) * np.linalg.norm(keys, axis=1))
    assert np.mean(rel) < 0.02


# ------------------------------------------------------------------ search


def _check_polar_topk(gi, gs, osc, tol, k):
    """gi/gs the device's lists [Q, k]; osc the oracle's estimates [Q, n_db] (fp64), tol the
    bound on the device's score error per entry [Q, n_db].  Every returned score within its bound
    of the oracle's, the list in the device's score order, and a row in one top-k but not the
    other only where its score is within the bounds of the oracle's k-th."""
    oi, os_ = topk_rows_np(osc, k)
    for q in range(gi.shape[0]):
        assert len(set(gi[q].tolist())) == k
        assert np.all(np.abs(gs[q] - osc[q, gi[q]]) <= tol[q, gi[q]])
        assert np.all(np.diff(gs[q]) <= 0)  # ordered by the device's own scores
        kth = os_[q, -1]
        tk = tol[q].max()
        for r in set(gi[q].tolist()) ^ set(oi[q].tolist()):
            assert abs(osc[q, r] - kth) <= 2 * tk, (q, r, osc[q, r], kth)


def topk_rows_np(rows, k):
    from oracle import estimate as oe

    return oe.topk_rows(rows, k)


def _search_tol(lib, ora, qs, codes):
    """Per-entry bound on the device's search scores: score_tol on the polar term, the QJL term's
    bound as for tq_polar_scores."""
    nbar = oq.f16_value((codes.norms & 0xFFFF).astype(np.uint16))
    qn = np.linalg.norm(qs.astype(np.float64), axis=1)
    tol = score_tol(lib.d) * qn[:, None] * nbar[None, :]
    if ora.m:
        tol = tol + _qjl_score_tol(lib, ora, qs[None], codes.norms, codes.norms.shape[0], 1)[0]
    return tol + 1e-30


@pytest.mark.parametrize("d,ab,m,n_db,n_q,k", [
    (128, 2, 0, 5000, 7, 10),       # one query group of 4 and a ragged one
    (64, 3, 64, 40000, 3, 32),      # several slices and the merge, k = 32
    (256, 4, 0, 3000, 5, 1),        # one query per group (the table limit)
    (128, 3, 128, 9000, 9, 16),     # QJL: two queries per group
    (64, 2, 0, 20, 2, 20),          # tiny database: k = n_db
])
def test_polar_search_matches_oracle(d, ab, m, n_db, n_q, k):
    say("polar search", d, ab, m, n_db, n_q, k)
    lib, ora = _codecs(d, ab, m=m)
    db, qs = synth.search_data(n_db=n_db, n_q=n_q, d=d, clusters=50)
    codes = op.encode(db, ora, stride=lib.stride, sign_stride=lib.sign_stride if m else None)
    dcodes = tq.PolarCodes(torch.from_numpy(codes.bits).cuda(), torch.from_numpy(codes.norms.view(np.int32)).cuda(),
                           None if codes.sign is None else torch.from_numpy(codes.sign).cuda())
    gi, gs = tq.polar_search_topk(lib, torch.from_numpy(qs).cuda(), dcodes, n_db, k)
    torch.cuda.synchronize()
    osc = op.search_scores(qs, codes, ora)
    _check_polar_topk(gi.cpu().numpy(), gs.cpu().numpy(), osc, _search_tol(lib, ora, qs, codes), k)


def test_polar_search_ties_take_the_smaller_row():
    # duplicated records score identically on the device too; the earlier row comes first
    d, ab = 64, 2
    lib, ora = _codecs(d, ab)
    x = np.random.default_rng(51).standard_normal((5000, d)).astype(np.float32)
    x[4000] = x[123]
    x[2500] = x[123]
    codes = op.encode(x, ora, stride=lib.stride)
    dcodes = tq.PolarCodes(torch.from_numpy(codes.bits).cuda(), torch.from_numpy(codes.norms.view(np.int32)).cuda())
    gi, gs = tq.polar_search_topk(lib, torch.from_numpy(x[123:124] * 3.0).cuda(), dcodes, 5000, 3)
    gi, gs = gi.cpu().numpy()[0], gs.cpu().numpy()[0]
    assert list(gi) == [123, 2500, 4000] and gs[0] == gs[1] == gs[2]


def test_polar_search_errors():
    lib, _ = _codecs(64, 2, basis=[1, 2], vpr=10)  # two rotations: search takes one
    db = tq.alloc_polar_codes(lib, 20)
    q = torch.zeros((2, 64), device="cuda")
    cc = lib.c()
    i = torch.empty((2, 4), dtype=torch.int64, device="cuda")
    s = torch.empty((2, 4), device="cuda")
    assert tq.lib.tq_polar_search_topk(tq.ctypes.byref(cc), tq._ptr(q), 2, db.c(), 20, 4, tq._ptr(i), tq._ptr(s),
                                       None, 0, tq._stream()) == -1
    lib1, _ = _codecs(64, 2)
    cc1 = lib1.c()
    with pytest.raises(ValueError):
        tq.polar_search_topk(lib1, q, db, 20, 21)  # k > n_db
    assert tq.lib.tq_polar_search_topk(tq.ctypes.byref(cc1), tq._ptr(q), 2, db.c(), 20, 33, tq._ptr(i), tq._ptr(s),
                                       None, 0, tq._stream()) == -1  # k > 32


@pytest.mark.parametrize("d,dtype,first", [(128, "bfloat16", 64), (64, "float32", 64), (64, "float16", 40)])
def test_qjl_full_mode_rotation_blocks(d, dtype, first):
    # per-block rotations with the QJL stage: the MFMA encoder's block loop (offsets that are
    # multiples of 32; bf16 at d = 128) and the FMA kernel (offset 40); fields, rn16 and signs
    # explained by the rotation bound as in the single-rotation case
    ab, n_rot, vpr = 2, 24, 32
    lib, ora = _codecs(d, ab, basis=[800 + i for i in range(n_rot)], vpr=vpr, m=d)
    n = n_rot * vpr - first + 40
    x = (np.random.default_rng(d + first).standard_normal((n, d)) * 3.0).astype(np.float32)
    tdt = getattr(torch, dtype)
    x_seen = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    bits, norms, ytap, sign = _gpu_encode(lib, x, pre=False, dtype=tdt, first=first, tap=True)
    y_ex, bound = _exact_rotation(x_seen.astype(np.float64), ora, ora.rot_index(n, first))
    assert np.all(np.abs(ytap.astype(np.float64) - y_ex) <= bound)
    want = op.encode(x_seen, ora, first=first, stride=lib.stride, sign_stride=lib.sign_stride)
    assert np.array_equal(norms & 0xFFFF, want.norms & 0xFFFF)
    dy = np.abs(ytap.astype(np.float64) - want.extra["y"].astype(np.float64))
    same = _explain_fields(bits, norms, want, dy, ora, 0.02)
    assert _explain_qjl(norms, sign, want, dy, same, ora) <= max(1, int(0.02 * n))


def test_qjl_full_size_sampled():
    # the 8B decode shape's 2.1M bf16 keys (one layer) encoded with the QJL stage in one call (the
    # MFMA encoder's multi-pass loop): norm words' low halves on 65536 sampled keys, and the
    # records, rn16 and signs of 2048 sampled keys explained against the oracle with the bound
    # taken from the exact fp64 rotation (no y tap)
    w = synth.GQA_DECODE
    d, ab = w.d, 2
    lib, ora = _codecs(d, ab, m=d)
    n = w.batch * w.hkv * w.n_ctx
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    K = torch.randn((n, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    codes = tq.polar_encode(lib, K)
    torch.cuda.synchronize()
    x_seen = K.float().cpu().numpy()
    g = np.random.default_rng(14)
    rows = np.sort(g.choice(n, 65536, replace=False))
    nw = codes.norms.cpu().numpy().view(np.uint32)
    assert np.array_equal(nw[rows] & 0xFFFF, oq.f16_norm_bits(x_seen[rows]))
    sub = np.sort(g.choice(n, 2048, replace=False))
    y_ex, bound = _exact_rotation(x_seen[sub].astype(np.float64), ora, ora.rot_index(len(sub)))
    want = op.encode(x_seen[sub], ora, stride=lib.stride, sign_stride=lib.sign_stride)
    dy = bound + np.abs(want.extra["y"].astype(np.float64) - y_ex)
    bits = codes.bits.cpu().numpy()[sub]
    sign = codes.sign.cpu().numpy()[sub]
    same = _explain_fields(bits, nw[sub], want, dy, ora, 0.02)
    assert _explain_qjl(nw[sub], sign, want, dy, same, ora) <= max(1, int(0.02 * len(sub)))


# ------------------------------------------------------------------ decode step


def _polar_appended(lib, ora, x, pos, cap, hkv, rope_base, before, after):
    """Device records at the appended slots against the oracle's append (explained by the rotation
    bound, as test_polar_append_matches_oracle); every other record unchanged.  Returns the
    oracle's cache after the append (its own records at the slots)."""
    S, _, d = x.shape
    valid = [(s, h) for s in range(S) for h in range(hkv) if 0 <= pos[s] < cap]
    slots = np.array([(s * hkv + h) * cap + pos[s] for s, h in valid], dtype=np.int64)
    rows = np.array([x[s, h] for s, h in valid], dtype=np.float32)
    p = np.array([pos[s] for s, _ in valid], dtype=np.int64)
    want = op.append(rows, ora, slots, p, rope_base, stride=lib.stride,
                     sign_stride=lib.sign_stride if ora.m else None)
    bits, norms = after[0], after[1]
    assert np.array_equal(norms[slots] & 0xFFFF, oq.f16_norm_bits(rows))
    xr = oq.rope(rows, p, rope_base) if rope_base > 0 else rows.astype(np.float64)
    rid = np.array([ora.rot_index(1, int(t))[0] for t in slots])
    y_ex, bound = _exact_rotation(xr, ora, rid)
    dy = bound + np.abs(want.extra["y"].astype(np.float64) - y_ex)
    same = _explain_fields(bits[slots], norms[slots], want, dy, ora, 0.2)
    if ora.m:
        assert _explain_qjl(norms[slots], after[2][slots], want, dy, same, ora) <= 2
    other = np.setdiff1d(np.arange(bits.shape[0]), slots)
    assert np.array_equal(bits[other], before.bits[other]) and np.array_equal(norms[other], before.norms[other])
    cache = op.PolarCodes(before.bits.copy(), before.norms.copy(),
                          sign=None if before.sign is None else before.sign.copy())
    cache.bits[slots], cache.norms[slots] = want.bits, want.norms
    if ora.m:
        cache.sign[slots] = want.sign
    return cache


@pytest.mark.parametrize("m,hq,hkv,S,cap,pos", [
    (0, 8, 2, 3, 5000, [4999, 1234, -1]),     # several chunks; ragged lengths; one sequence appends nothing
    (128, 4, 4, 2, 700, [699, 350]),          # the QJL stage; one head per kv head
    (128, 16, 4, 2, 20000, [17000, 20000]),   # four heads per kv head, long; one past its capacity
])
def test_polar_decode_step_matches_oracle(m, hq, hkv, S, cap, pos):
    from oracle import codec as oc

    say("polar decode step", m, hq, hkv, S, cap, pos)
    d, ab, base = 128, 2, 10000.0
    lib, ora = _codecs(d, ab, m=m)
    vl = tq.make_codec(d, 3, 0, 3, 4)
    vo = oc.make_codec(d, 3, 0, 3, 4)
    g = np.random.default_rng(cap + hq + m)
    n = S * hkv * cap
    kx = (g.standard_normal((n, d)) * np.where(g.random(d) < 0.03, 8.0, 1.0)).astype(np.float32)
    kb = op.encode(kx, ora, stride=lib.stride, sign_stride=lib.sign_stride if m else None)
    vb = oq.encode(g.standard_normal((n, d)).astype(np.float32), vo, idx_stride=vl.idx_stride,
                   sign_stride=vl.sign_stride)
    kc = tq.PolarCodes(torch.from_numpy(kb.bits.copy()).cuda(), torch.from_numpy(kb.norms.view(np.int32).copy()).cuda(),
                       None if kb.sign is None else torch.from_numpy(kb.sign.copy()).cuda())
    vc = tq.Codes(torch.from_numpy(vb.idx.copy()).cuda(), None, torch.from_numpy(vb.norms.view(np.int32).copy()).cuda())
    q = g.standard_normal((S, hq, d)).astype(np.float32)
    kn = g.standard_normal((S, hkv, d)).astype(np.float32)
    vn = g.standard_normal((S, hkv, d)).astype(np.float32)
    p = np.array(pos, dtype=np.int32)
    scale = 1.0 / np.sqrt(d)
    out = tq.polar_decode_step(lib, vl, torch.from_numpy(q).cuda(), torch.from_numpy(kn).cuda(),
                               torch.from_numpy(vn).cuda(), torch.from_numpy(p).cuda(), cap, base, kc, vc,
                               scale).cpu().numpy()
    ka = _polar_appended(lib, ora, kn, p, cap, hkv, base, kb, kc.numpy())
    # values: the two-stage append (tested on its own); the reference reads the oracle's records
    _, _, va = op.decode_step(q, kn, vn, kb, vb, ora, vo, cap, p, base, hkv, scale)
    vidx = vc.idx.cpu().numpy()
    ok = (p >= 0) & (p < cap)
    vslots = {(s * hkv + h) * cap + p[s] for s in range(S) for h in range(hkv) if ok[s]}
    other = np.array(sorted(set(range(n)) - vslots))
    assert np.array_equal(vidx[other], vb.idx[other])
    qr = oq.rope(q.reshape(S * hq, d), np.repeat(p, hq), base).reshape(S, hq, d)
    want = op.attend_lens(qr, ka, va, ora, vo, cap, np.where(ok, p + 1, 0), hkv, scale)
    for s in range(S):
        if not ok[s]:
            assert not out[s].any()
    rows = [s for s in range(S) if ok[s]]
    err = np.max(np.abs(out[rows] - want[rows]), axis=-1) / np.max(np.abs(want[rows]), axis=-1)
    say("  max rel err", float(err.max()))
    assert np.all(err <= 1e-3)


def test_polar_decode_step_unsupported_changes_nothing():
    # 4-bit values are not a value codec of the logits-in attention: refused before any launch
    from oracle import codec as oc  # noqa: F401

    d, hq, hkv, S, cap = 64, 2, 1, 1, 16
    lib, _ = _codecs(d, 2)
    vl = tq.make_codec(d, 4, 0, 3, 4)
    kc = tq.alloc_polar_codes(lib, S * hkv * cap)
    vc = tq.alloc_codes(vl, S * hkv * cap)
    kc.bits.fill_(7)
    vc.idx.fill_(9)
    q = torch.zeros((S, hq, d), device="cuda")
    kn = torch.ones((S, hkv, d), device="cuda")
    p = torch.zeros((S,), dtype=torch.int32, device="cuda")
    with pytest.raises(tq.TQError):
        tq.polar_decode_step(lib, vl, q, kn, kn, p, cap, 0.0, kc, vc, 1.0)
    torch.cuda.synchronize()
    assert bool((kc.bits == 7).all()) and bool((vc.idx == 9).all())
