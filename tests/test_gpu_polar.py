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


def _codecs(d, ab, rot_seed=1, basis=None, vpr=0):
    ora = op.make_polar_codec(d, ab, rot_seed, basis_seeds=basis, vecs_per_rot=vpr)
    lib = tq.polar_codec_from_arrays(d, ab, ora.rot, _tables(ora), vecs_per_rot=vpr)
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
    bits, norms = out.numpy()
    return bits, norms, (None if ytap is None else ytap.cpu().numpy())


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


def _check_full(x_seen, lib, ora, gpu, first=0, max_rows=0.02):
    """Full-mode records against the oracle's own encoding (its fp64 rotation rounded to fp32):
    the rotation within ROT_BOUND of the exact one (through the y tap), the norm words exact,
    and every other difference explained by that bound: a sign only where |y| is within it, a
    node index only where the bound, carried into the node's sums of squares, reaches one of
    its thresholds (each node's index depends on its own subtree's sums alone)."""
    bits, norms, ytap = gpu
    n, d = x_seen.shape
    x64 = x_seen.astype(np.float64)
    rid = ora.rot_index(n, first)
    y_ex = np.empty_like(x64)
    bound = np.empty_like(x64)
    for r in np.unique(rid):
        sel = rid == r
        P = ora.rot[r].astype(np.float64)
        y_ex[sel] = x64[sel] @ P.T
        bound[sel] = ROT_BOUND * (np.abs(x64[sel]) @ np.abs(P).T) + 1e-45
    assert np.all(np.abs(ytap.astype(np.float64) - y_ex) <= bound)
    want = op.encode(x_seen, ora, first=first, stride=lib.stride)
    assert np.array_equal(norms, want.norms)
    y_o = want.extra["y"].astype(np.float64)
    dy = bound + np.abs(y_o - y_ex)  # |y_gpu - y_oracle|
    gp, gn = op.decode_fields(op.PolarCodes(bits, norms), ora)
    wp, wn = op.decode_fields(want, ora)
    # signs
    a, b = y_o[:, 0::2], y_o[:, 1::2]
    ok_sa = ((gp & 1) == (wp & 1)) | (np.abs(a) <= dy[:, 0::2])
    ok_sb = (((gp >> 1) & 1) == ((wp >> 1) & 1)) | (np.abs(b) <= dy[:, 1::2])
    assert ok_sa.all() and ok_sb.all()
    # node indices, level by level: sums of squares of each child's coordinates and their bounds
    sq = y_o * y_o
    dsq = 2.0 * np.abs(y_o) * dy + dy * dy
    bad_rows = np.zeros(n, bool)
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
    # sampled keys.  Encode: the device encodes the bf16 keys; the norm words must equal the
    # exact fp16 norms of the inputs (65536 sampled), and a y-tapped re-encode of 4096 of them must be bit-exact
    # against the oracle's encoding of the tap.
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
    with pytest.raises(tq.TQError):
        tq.polar_encode(lib, torch.zeros((4, 64), device="cuda"), out=bad)


@pytest.mark.parametrize("d,ab,vbits,vm,n_seq,hq,hkv,n_ctx", [
    (128, 2, 3, 0, 2, 8, 2, 1000),     # 4 heads per kv head, 3-bit values (the 8B value codec)
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
    with pytest.raises(tq.TQError):
        tq.polar_attend_decode(lib, vl, q, k, v, 4, 2, 1.0)
    vl64 = tq.make_codec(64, 3, 0, 3, 4)
    cc, vc = lib.c(), vl64.c()
    need = tq.lib.tq_polar_attend_workspace_bytes(tq.ctypes.byref(cc), tq.ctypes.byref(vc), 1, 2, 2, 4)
    assert need >= 2 * 4 * 4
    rc = tq.lib.tq_polar_attend_decode(tq.ctypes.byref(cc), tq.ctypes.byref(vc), tq._ptr(q), 1, 2, 2, 4, k.c(),
                                       tq.alloc_codes(vl64, 8).c(), 1.0, tq._ptr(q), None, 0, tq._stream())
    assert rc == -4
