"""GPU encode parity against the oracle.

Pre-rotated mode: given identical fp32 rotated inputs, the packed index stream, the sign
stream and the norm words must be bit-identical (the norms and signs are defined by exact
real quantities on both sides).  Full mode: the rotation is a contraction on the GPU (bf16
hi/lo split MFMA with fp32 accumulation for d = 64, 128; fp32 FMA otherwise), so y differs
from the oracle's correctly rounded y within ROT_BOUND; the norm word's low half (the input's
norm) must still match exactly, and every other mismatch must be explained by that bound.
"""

import math

import numpy as np
import pytest

import synth
from oracle import codec as oc
from oracle import quantize as oq
from tests._util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

# Error bound of the encoder's rotation relative to sum_k |Pi_ik x_k|.  MFMA path (d = 64, 128):
# each operand's bf16 hi/lo split misses at most 2^-16 of it, so hi*hi + hi*lo + lo*hi misses
# at most 3 * 2^-16, and the fp32 accumulation of 3d products adds at most 3d * 2^-24 -- together
# 6.9e-5 at d = 128.  FMA path (d = 200): (d + 2) * 2^-24.  Both are below 2^-13.
ROT_BOUND = 2.0 ** -13

CASES = [(64, 2, 64), (64, 3, 64), (128, 2, 128), (128, 3, 0), (128, 3, 128), (200, 2, 200), (64, 4, 0),
         (200, 3, 0)]


def _codecs(d, bits, m, rot_seed=1, sketch_seed=2, basis=None, vpr=0):
    lib = tq.make_codec(d, bits, m, rot_seed, sketch_seed, basis_seeds=basis, vecs_per_rot=vpr)
    ora = oc.make_codec(d, bits, m, rot_seed, sketch_seed, basis_seeds=basis, vecs_per_rot=vpr)
    return lib, ora


def _edge_rows(d):
    b = float(np.nextafter(np.float16(1.0), np.float16(2.0)))
    mid = np.float32(0.5 * (1.0 + b))  # an fp16 midpoint: the norm ties, rounds to even (1.0)
    rows = np.zeros((6, d), np.float32)
    rows[1, 3] = mid
    rows[2, 3] = mid
    rows[2, 7] = np.float32(2.0 ** -20)  # just above the midpoint
    rows[3] = np.float32(1e-30)  # tiny (squares far below fp32 range, fine in fp64)
    rows[4, :] = np.float32(3000.0)  # large norm, still below 65520
    rows[5, ::2] = np.float32(-0.5)
    return rows


def _gpu_encode(lib_codec, x_np, pre, dtype=None, first=0, tap=False):
    x = torch.from_numpy(x_np).to("cuda")
    if dtype is not None:
        x = x.to(dtype)
    ytap = torch.empty((x.shape[0], lib_codec.d), dtype=torch.float32, device="cuda") if tap else None
    codes = tq.encode(lib_codec, x, pre_rotated=pre, first=first, y_tap=ytap)
    torch.cuda.synchronize()
    idx, sign, norms = codes.numpy()
    return idx, sign, norms, (None if ytap is None else ytap.cpu().numpy())


@pytest.mark.parametrize("d,bits,m", CASES)
def test_pre_rotated_bit_exact(d, bits, m):
    say("encode pre-rotated", d, bits, m)
    lib, ora = _codecs(d, bits, m)
    y = np.concatenate([_edge_rows(d), synth.pre_rotated(4099, d, seed=d * 10 + bits)])
    y[200:300] *= np.float32(1e-3)
    y[300:400] *= np.float32(300.0)
    idx, sign, norms, _ = _gpu_encode(lib, y, pre=True)
    want = oq.encode(y, ora, pre_rotated=True, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    assert np.array_equal(norms, want.norms)
    assert np.array_equal(idx, want.idx)
    if m > 0:
        assert np.array_equal(sign, want.sign)
    # the tie row rounds to even
    assert norms[1] & 0xFFFF == np.float16(1.0).view(np.uint16)
    assert norms[0] == 0


@pytest.mark.parametrize("d,blocks", [(64, False), (200, False), (200, True)])
def test_exact_sign_fallback_with_crafted_sketch(d, blocks):
    # rows of S whose dot product with r is exactly zero force the exact expansion path (d = 64:
    # the MFMA encoder's band; d = 200: the several-vectors-per-wavefront encoder's fp32 band,
    # 509 rows there, so that its last group of 8 vectors is a partial one; d = 200 with two
    # rotation blocks: the one-wavefront-per-vector encoder's fp32 band, then its fp64 sum)
    bits, m = 2, d
    g = np.random.default_rng(5)
    S = g.standard_normal((m, d)).astype(np.float32)
    S[0] = 0
    S[1] = 0
    S[1, 0], S[1, 1] = 1.0, -1.0
    S[2] = 0
    S[2, 2], S[2, 3] = 3.0, 3.0
    S[3] = 0
    S[3, 4], S[3, 5], S[3, 6] = 2.0 ** 30, 1.0, -(2.0 ** 30)
    rot = np.eye(d, dtype=np.float32)
    cb = oc.lloyd_max_beta(d, bits)
    lib = tq.codec_from_arrays(d, bits, m, np.stack([rot, rot]) if blocks else rot, S, cb.centroids,
                               cb.thresholds, vecs_per_rot=256 if blocks else 0)
    ora = oc.Codec(d, bits, m, rot[None], S, cb.centroids, cb.thresholds)
    y = synth.pre_rotated(512 if d == 64 else 509, d, seed=77)
    y[:, 1] = y[:, 0]  # r_0 == r_1: row 1 sums to exactly 0
    y[:, 3] = -y[:, 2]  # r_3 == -r_2: row 2 sums to exactly 0
    y[:, 6] = y[:, 4]  # row 3: 2^30 r_4 + r_5 - 2^30 r_4 == r_5
    idx, sign, norms, _ = _gpu_encode(lib, y, pre=True)
    want = oq.encode(y, ora, pre_rotated=True, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
    assert np.array_equal(norms, want.norms)
    assert np.array_equal(idx, want.idx)
    assert np.array_equal(sign, want.sign)
    bits0 = oq.unpack_bits(sign, 1, m)
    assert np.all(bits0[:, 0] == 1) and np.all(bits0[:, 1] == 1) and np.all(bits0[:, 2] == 1)
    assert np.array_equal(bits0[:, 3], (want.resid[:, 5] >= 0).astype(np.uint32))


def _f16_half_ulp(v):
    """Half the fp16 spacing at the non-negative values v (fp64): 2^-11 of the binade's base for
    normal values, 2^-25 in the subnormal range."""
    v = np.asarray(v, np.float64)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -14)))
    return np.ldexp(1.0, (e - 11).astype(np.int64))


def _explained_mismatches(x, lib, ora, gpu, want, first=0, rates=True, rid=None):
    """Check full-mode GPU codes against the oracle's, allowing only bound-explained differences.

    ``rid`` gives each row's rotation (default: rows first, first + 1, ... of the cache).  On rows
    whose indices agree, the residual norm's fp16 word must be the exactly rounded norm of a
    residual within the propagated y bound of the oracle's: r_i = fl32(y_i - fl32(nbar c[idx_i]))
    on both sides with the same subtrahend, so |r_gpu,i - r_ora,i| <= |dy_i| (1 + 2^-23) +
    2^-22 |r_ora,i|, and | ||r_gpu|| - ||r_ora|| | <= the norm of that bound (triangle inequality);
    the stored fp16 adds at most half an fp16 spacing.  With rates=True the index-flip rate is
    capped as well; the counts (rows with an index flip, rows whose residual-norm word differs,
    rows) are returned either way."""
    d, bits, m = ora.d, ora.bits, ora.m
    idx_g, sign_g, norms_g, ytap = gpu
    x64 = np.asarray(x, np.float64)
    if rid is None:
        rid = ora.rot_index(x64.shape[0], first)
    rid = np.asarray(rid, np.int64)
    y_ex = np.empty_like(x64)
    bound = np.empty_like(x64)
    for r in np.unique(rid):
        sel = rid == r
        P = ora.rot[r].astype(np.float64)
        y_ex[sel] = x64[sel] @ P.T
        bound[sel] = ROT_BOUND * (np.abs(x64[sel]) @ np.abs(P).T) + 1e-45
    # (1) rotation within the contraction bound (checked where the call wrote a y tap)
    if ytap is not None:
        assert np.all(np.abs(ytap.astype(np.float64) - y_ex) <= bound)
    # (2) the input's norm is exact
    assert np.array_equal(norms_g & 0xFFFF, want.norms & 0xFFFF)
    # (3) index mismatches only where y is within the bound of a scaled threshold
    ig = oq.unpack_bits(idx_g, bits, d).astype(np.int64)
    iw = want.index.astype(np.int64)
    nbar = oq.f16_value(want.norms & 0xFFFF).astype(np.float32)
    thr = (nbar[:, None] * ora.thresholds[None, :]).astype(np.float64)
    near = np.min(np.abs(y_ex[:, :, None] - thr[:, None, :]), axis=2) <= 2 * bound + np.abs(y_ex) * 2.0 ** -23
    bad = (ig != iw) & ~near
    assert not bad.any(), np.argwhere(bad)[:5]
    same_rows = np.all(ig == iw, axis=1)
    if rates:
        assert np.mean(~same_rows) < 0.02
    # |y_gpu - y_oracle| per coordinate: the tap, else |y_gpu - y_exact| + |y_exact - y_oracle|
    if ytap is not None:
        dy = np.abs(ytap.astype(np.float64) - want.y.astype(np.float64))
    else:
        dy = bound + np.abs(y_ex - want.y.astype(np.float64))
    r = want.resid.astype(np.float64)
    dr = dy * (1.0 + 2.0 ** -23) + 2.0 ** -22 * np.abs(r) + 1e-45
    # (4) on rows with equal indices the residuals differ by the y difference only
    if m > 0:
        sg = oq.unpack_bits(sign_g, 1, m)
        sw = want.bits
        zb = dr @ np.abs(ora.sketch.astype(np.float64)).T
        z = r @ ora.sketch.astype(np.float64).T
        diff = (sg != sw) & same_rows[:, None]
        assert np.all(np.abs(z[diff]) <= 2 * zb[diff] + 1e-30)
    # (5) the residual-norm half of the word on rows with equal indices
    rn_g, rn_w = norms_g >> 16, want.norms >> 16
    rn_diff = (rn_g != rn_w) & same_rows
    if m > 0 and ora.resid_scale > 0:
        # residual-sign records: fp16(nbar resid_scale), a function of the exact low half
        assert np.array_equal(rn_g, rn_w)
    else:
        R = np.sqrt(np.sum(r * r, axis=1))  # the oracle's exact-input residual norm (fp64)
        delta = np.sqrt(np.sum(dr * dr, axis=1)) * (1.0 + 1e-12)
        got = oq.f16_value(rn_g.astype(np.uint16))
        lim = delta + _f16_half_ulp(R + delta) * (1.0 + 1e-12) + 1e-300
        off = same_rows & ~(np.abs(got - R) <= lim)
        assert not off.any(), (np.argwhere(off)[:5].ravel(), got[off][:5], R[off][:5], lim[off][:5])
    flips, rns, rows = int(np.sum(~same_rows)), int(np.sum(rn_diff)), len(same_rows)
    if rates:
        return flips / rows
    return flips, rns, rows


@pytest.mark.parametrize("d,bits,m,dtype", [(64, 2, 64, "float32"), (64, 3, 64, "float16"), (128, 2, 128, "bfloat16"),
                                            (128, 3, 0, "bfloat16"), (200, 2, 200, "float32")])
def test_full_mode_matches_within_rotation_bound(d, bits, m, dtype):
    say("encode full", d, bits, m, dtype)
    lib, ora = _codecs(d, bits, m)
    g = np.random.default_rng(d + bits)
    x = (g.standard_normal((3001, d)) * np.where(g.random(d) < 0.05, 10.0, 1.0)).astype(np.float32)
    tdt = getattr(torch, dtype)
    x_rounded = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()  # the values the GPU sees
    gpu = _gpu_encode(lib, x, pre=False, dtype=tdt, tap=True)
    want = oq.encode(x_rounded, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
    frac = _explained_mismatches(x_rounded, lib, ora, gpu, want)
    say("  rows with an index flip:", frac)


def test_full_mode_per_head_rotations():
    # ESM-2-shaped slice: per-(layer, head) rotation Pi @ B_h, 3-bit + QJL, fp16 input
    d, bits, m, N = 64, 3, 64, 256
    seeds = [synth.esm2_basis_seed(l, h) for l in range(2) for h in range(3)]
    lib, ora = _codecs(d, bits, m, basis=seeds, vpr=N)
    K, V, q = synth.esm2(layers=2, heads=3, seq=N)
    x = K.reshape(-1, d).astype(np.float32)
    gpu = _gpu_encode(lib, x, pre=False, dtype=torch.float16, tap=True)
    want = oq.encode(x, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
    _explained_mismatches(x, lib, ora, gpu, want)


@pytest.mark.parametrize("d,bits,m,dtype", [(128, 2, 128, "bfloat16"), (128, 3, 0, "bfloat16"), (64, 3, 64, "float32")])
def test_full_mode_rotation_blocks(d, bits, m, dtype):
    # per-block rotations on the MFMA path: 300 blocks of 32 vectors (more blocks than
    # workgroups), an offset first that skips two blocks, and 40 vectors past the last block
    # (they take the last rotation)
    n_rot, vpr, first = 300, 32, 64
    seeds = [1000 + i for i in range(n_rot)]
    lib, ora = _codecs(d, bits, m, basis=seeds, vpr=vpr)
    n = n_rot * vpr - first + 40
    x = (np.random.default_rng(d + bits).standard_normal((n, d)) * 3.0).astype(np.float32)
    x = torch.from_numpy(x).to(getattr(torch, dtype)).float().numpy()  # exactly representable input
    gpu = _gpu_encode(lib, x, pre=False, dtype=getattr(torch, dtype), first=first, tap=True)
    want = oq.encode(x, ora, first=first, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
    _explained_mismatches(x, lib, ora, gpu, want, first=first)


def test_encode_offset_first_selects_rotation_block():
    d, bits, m, N = 64, 2, 64, 100
    seeds = [11, 12, 13, 14]
    lib, ora = _codecs(d, bits, m, basis=seeds, vpr=N)
    x = synth.pre_rotated(150, d, seed=3)  # rows 250..399 of a cache: blocks 2 and 3
    gpu = _gpu_encode(lib, x, pre=False, first=250, tap=True)
    want = oq.encode(x, ora, first=250, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
    _explained_mismatches(x, lib, ora, gpu, want, first=250)


def test_encode_deterministic_and_pads_zero():
    lib, ora = _codecs(200, 2, 200)
    y = synth.pre_rotated(777, 200, seed=9)
    a = _gpu_encode(lib, y, pre=True)
    b = _gpu_encode(lib, y, pre=True)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u, v)
    assert np.all(a[0][:, 50:] == 0)  # 400 index bits -> bytes 50, 51 are padding
    assert np.all(a[1][:, 25:] == 0)


def _sampled_runs(n, runs, length, seed):
    """Starts of `runs` runs of `length` consecutive vectors spread over [0, n), ends included."""
    g = np.random.default_rng(seed)
    starts = np.unique(np.concatenate([[0, n - length], g.integers(0, n - length, runs - 2)]))
    return [int(s0) for s0 in starts]


def _check_runs(lib, ora, X, codes, starts, length):
    idx_d, sign_d, norms_d = codes.idx, codes.sign, codes.norms
    flips = rn = rows = 0
    for s0 in starts:
        sl = slice(s0, s0 + length)
        x = X[sl].float().cpu().numpy()
        gpu = (idx_d[sl].cpu().numpy(), None if sign_d is None else sign_d[sl].cpu().numpy(),
               norms_d[sl].cpu().numpy().view(np.uint32), None)
        want = oq.encode(x, ora, first=s0, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
        f, r, nr = _explained_mismatches(x, lib, ora, gpu, want, first=s0, rates=False)
        flips, rn, rows = flips + f, rn + r, rows + nr
    # the index-flip rate over all sampled rows, as in the small full-mode tests (the residual
    # norms of rows without a flip are bound-checked row by row)
    assert flips / rows < 0.02, (flips, rn, rows)
    return flips / rows


def test_full_size_8b_decode_sampled_vectors():
    """The whole 8B-class decode cache (2 x 67.1M bf16 vectors) encoded by the bench's calls;
    runs of vectors spread over every layer and sequence checked against the oracle."""
    w = synth.GQA_DECODE
    say("encode full size", w.name)
    K, V, _ = synth.gqa_decode(w, seed=2, device="cuda")
    for X, bits, m, rs, ss in ((K, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K),
                               (V, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)):
        lib, ora = _codecs(w.d, bits, m, rs, ss)
        Xf = X.reshape(-1, w.d)
        out = tq.alloc_codes(lib, Xf.shape[0])
        tq.encode(lib, Xf, out=out)
        torch.cuda.synchronize()
        starts = _sampled_runs(Xf.shape[0], 24, 16, seed=bits + m)
        frac = _check_runs(lib, ora, Xf, out, starts, 16)
        say("  bits", bits, "m", m, "rows with an index flip:", frac)
        del out
    del K, V
    torch.cuda.empty_cache()


def test_full_size_esm2_sampled_vectors():
    """The whole ESM-2-shaped cache (33 layers x 20 heads x 1024 tokens, fp16, one rotation per
    (layer, head)) encoded by the bench's calls; runs of vectors from many rotation blocks."""
    w = synth.ESM2
    say("encode full size", w.name)
    K, V, _ = synth.esm2(layers=w.layers, heads=w.hkv, seq=w.n_ctx, d=w.d)
    seeds = [synth.esm2_basis_seed(l, h) for l in range(w.layers) for h in range(w.hkv)]
    for X, bits, m, rs, ss in ((K, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K),
                               (V, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)):
        lib, ora = _codecs(w.d, bits, m, rs, ss, basis=seeds, vpr=w.n_ctx)
        Xd = torch.from_numpy(X.reshape(-1, w.d)).cuda()
        out = tq.alloc_codes(lib, Xd.shape[0])
        tq.encode(lib, Xd, out=out)
        torch.cuda.synchronize()
        starts = _sampled_runs(Xd.shape[0], 24, 32, seed=7)
        frac = _check_runs(lib, ora, Xd, out, starts, 32)
        say("  rows with an index flip:", frac)
