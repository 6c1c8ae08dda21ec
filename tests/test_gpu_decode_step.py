"""GPU decode step (append into a growing cache + attention over each sequence's length) against
the oracle.  Appended records: the norm word's low half exact, every other difference explained
by the rotation bound (the rotation sees RoPE(x), computed in fp64 on both sides).  Outputs:
within 1e-3 relative per (sequence, head), the oracle reading the GPU's own updated caches."""

import dataclasses
import math

import numpy as np
import pytest

import synth
from oracle import codec as oc
from oracle import estimate as oe
from oracle import quantize as oq
from tests._util import oracle_codes, rel_err_rows, say, to_device_codes
from tests.test_gpu_encode import _explained_mismatches

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

TOL = 1e-3
BASE = 10000.0


def _codecs(d, bits, m, rs, ss, basis=None, vpr=0):
    return (tq.make_codec(d, bits, m, rs, ss, basis_seeds=basis, vecs_per_rot=vpr),
            oc.make_codec(d, bits, m, rs, ss, basis_seeds=basis, vecs_per_rot=vpr))


def _host_codes(c, sl=slice(None)):
    return oracle_codes(c.idx[sl].cpu().numpy(), None if c.sign is None else c.sign[sl].cpu().numpy(),
                        c.norms[sl].cpu().numpy().view(np.uint32))


def _check_appended(lib, ora, x, pos, cap, hkv, rope_base, before, after):
    """The records at the appended slots against the oracle; every other record unchanged.
    Returns the oracle's cache after the append: ``before`` with the oracle's own records at the
    appended slots (the attention reference reads it, never the device's records)."""
    S = x.shape[0]
    valid = [(s, h) for s in range(S) for h in range(hkv) if 0 <= pos[s] < cap]
    slots = np.array([(s * hkv + h) * cap + pos[s] for s, h in valid], dtype=np.int64)
    rows = np.array([x[s, h] for s, h in valid], dtype=np.float32)
    p = np.array([pos[s] for s, _ in valid])
    want = oq.append(rows, ora, slots, p, rope_base, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride,
                     keep=True)
    got = (after.idx[slots], None if after.sign is None else after.sign[slots], after.norms[slots], None)
    xr = oq.rope(rows, p, rope_base) if rope_base > 0 else rows.astype(np.float64)
    # each appended record's rotation is the one of its cache slot
    rid = np.array([ora.rot_index(1, int(sl))[0] for sl in slots], dtype=np.int64)
    flips, rns, n_rows = _explained_mismatches(xr, lib, ora, got, want, rates=False, rid=rid)
    # every difference is bound-explained (checked above); index flips stay rare: at most one
    # row, or 2% of the rows, as in the full-mode encode tests
    assert flips <= max(1, int(0.02 * n_rows)), (flips, rns, n_rows)
    keep = np.ones(len(before.norms), bool)
    keep[slots] = False
    assert np.array_equal(after.norms[keep], before.norms[keep])
    assert np.array_equal(after.idx[keep], before.idx[keep])
    if after.sign is not None:
        assert np.array_equal(after.sign[keep], before.sign[keep])
    return _with_records(before, slots, want)


def _with_records(base, slots, recs):
    """A host copy of the codes ``base`` with the records ``recs`` written at ``slots``."""
    idx = base.idx.copy()
    idx[slots] = recs.idx
    sign = None
    if base.sign is not None:
        sign = base.sign.copy()
        sign[slots] = recs.sign
    norms = base.norms.copy()
    norms[slots] = recs.norms
    return oracle_codes(idx, sign, norms)


@pytest.mark.parametrize("d,bits,m,rope,dtype", [(128, 2, 128, True, "bfloat16"), (128, 3, 0, False, "float32"),
                                                  (64, 3, 64, True, "float16"), (200, 2, 200, True, "float32")])
def test_append_matches_oracle(d, bits, m, rope, dtype):
    say("append", d, bits, m, rope, dtype)
    lib, ora = _codecs(d, bits, m, 1, 2)
    S, hkv, cap = 5, 4, 300
    pos = np.array([0, 57, 299, -1, 300], dtype=np.int32)  # the last two are outside the cache
    g = np.random.default_rng(d + bits)
    x = (g.standard_normal((S, hkv, d)) * 3.0).astype(np.float32)
    x = torch.from_numpy(x).to(getattr(torch, dtype)).float().numpy()  # the values the GPU sees
    cache = tq.alloc_codes(lib, S * hkv * cap)
    cache.idx.fill_(0xA5)
    if cache.sign is not None:
        cache.sign.fill_(0x5A)
    cache.norms.fill_(0x12345678)
    before = _host_codes(cache)
    tq.append(lib, torch.from_numpy(x).to(getattr(torch, dtype)).cuda(), torch.from_numpy(pos).cuda(), cap,
              BASE if rope else 0.0, cache)
    torch.cuda.synchronize()
    _check_appended(lib, ora, x, pos, cap, hkv, BASE if rope else 0.0, before, _host_codes(cache))


@pytest.mark.parametrize("d,bits,m,dtype", [(128, 2, 128, "bfloat16"), (64, 3, 64, "float32"),
                                            (128, 3, 0, "float16")])
def test_append_per_block_rotations(d, bits, m, dtype):
    """One rotation per (sequence, kv head) block (vecs_per_rot = cap): each appended record must
    use its slot's rotation, on the MFMA-free append kernel and in the oracle alike."""
    say("append per-block rotations", d, bits, m, dtype)
    S, hkv, cap = 3, 4, 40
    seeds = [500 + i for i in range(S * hkv)]
    lib, ora = _codecs(d, bits, m, 1, 2, basis=seeds, vpr=cap)
    pos = np.array([0, 17, 39], dtype=np.int32)
    g = np.random.default_rng(3 * d + bits)
    x = (g.standard_normal((S, hkv, d)) * 2.0).astype(np.float32)
    x = torch.from_numpy(x).to(getattr(torch, dtype)).float().numpy()
    cache = tq.alloc_codes(lib, S * hkv * cap)
    cache.idx.fill_(0x3C)
    if cache.sign is not None:
        cache.sign.fill_(0xC3)
    cache.norms.fill_(0x0BADBEEF)
    before = _host_codes(cache)
    tq.append(lib, torch.from_numpy(x).to(getattr(torch, dtype)).cuda(), torch.from_numpy(pos).cuda(), cap,
              BASE, cache)
    torch.cuda.synchronize()
    _check_appended(lib, ora, x, pos, cap, hkv, BASE, before, _host_codes(cache))
    # the rotation used is the block's own: encoding with the first block's rotation instead would
    # give other indices for the other blocks
    slots = np.array([(s * hkv + h) * cap + pos[s] for s in range(S) for h in range(hkv)])
    wrong = oq.append(x.reshape(-1, d), dataclasses.replace(ora, rot=ora.rot[:1], vecs_per_rot=0), slots,
                      np.repeat(pos, hkv), BASE, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    assert not np.array_equal(wrong.idx[hkv:], _host_codes(cache).idx[slots][hkv:])


def _prefix_cache(lib, ora, S, hkv, cap, seed):
    """A cache whose every slot holds a random vector encoded by the oracle (slots past a
    sequence's length must not matter): (device codes, the same codes on the host)."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((S * hkv * cap, lib.d)) * np.where(g.random(lib.d) < 0.03, 8.0, 1.0)).astype(np.float32)
    host = oq.encode(x, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    return to_device_codes(tq, host.idx, host.sign, host.norms), oracle_codes(host.idx, host.sign, host.norms)


@pytest.mark.parametrize("hq,hkv,S,cap,pos", [
    (8, 2, 3, 5000, [4999, 1234, 0]),       # several chunks; ragged lengths cut chunks, some empty
    (4, 4, 2, 700, [699, 350]),             # one head per kv head
    (16, 4, 1, 20000, [17000]),             # four heads per kv head, long
])
def test_decode_step_matches_oracle(hq, hkv, S, cap, pos):
    say("decode step", hq, hkv, S, cap, pos)
    d = 128
    kl, ko = _codecs(d, 2, 128, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vl, vo = _codecs(d, 3, 0, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    kc, kb = _prefix_cache(kl, ko, S, hkv, cap, 1)
    vc, vb = _prefix_cache(vl, vo, S, hkv, cap, 2)
    g = np.random.default_rng(cap + hq)
    q = g.standard_normal((S, hq, d)).astype(np.float32)
    kn = g.standard_normal((S, hkv, d)).astype(np.float32)
    vn = g.standard_normal((S, hkv, d)).astype(np.float32)
    p = np.array(pos, dtype=np.int32)
    scale = 1.0 / math.sqrt(d)
    out = tq.decode_step(kl, vl, torch.from_numpy(q).cuda(), torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                         torch.from_numpy(p).cuda(), cap, BASE, kc, vc, scale)
    torch.cuda.synchronize()
    ka = _check_appended(kl, ko, kn, p, cap, hkv, BASE, kb, _host_codes(kc))
    va = _check_appended(vl, vo, vn, p, cap, hkv, 0.0, vb, _host_codes(vc))
    qr = oq.rope(q.reshape(S * hq, d), np.repeat(p, hq), BASE).reshape(S, hq, d)
    want = oe.attend_lens(qr, ka, va, ko, vo, cap, p.astype(np.int64) + 1, hkv, scale)
    err = rel_err_rows(out.cpu().numpy(), want)
    say("  max rel err", err.max())
    assert err.max() <= TOL


def test_decode_loop_and_out_of_range_sequence():
    """Three steps in a row on one cache; a sequence whose position is past the cache gets a
    zero output and leaves its records alone."""
    d, hq, hkv, S, cap = 64, 4, 1, 3, 600
    kl, ko = _codecs(d, 3, 64, 1, 2)
    vl, vo = _codecs(d, 3, 64, 3, 4)
    kc, ko_cache = _prefix_cache(kl, ko, S, hkv, cap, 3)
    vc, vo_cache = _prefix_cache(vl, vo, S, hkv, cap, 4)
    g = np.random.default_rng(9)
    start = np.array([100, 599 - 2, cap], dtype=np.int32)  # the third is outside the cache
    for step in range(3):
        p = start + np.array([step, step, 0], dtype=np.int32)
        q = g.standard_normal((S, hq, d)).astype(np.float32)
        kn = g.standard_normal((S, hkv, d)).astype(np.float16)
        vn = g.standard_normal((S, hkv, d)).astype(np.float16)
        out = tq.decode_step(kl, vl, torch.from_numpy(q).cuda(), torch.from_numpy(kn).cuda(),
                             torch.from_numpy(vn).cuda(), torch.from_numpy(p).cuda(), cap, BASE, kc, vc, 0.125)
        torch.cuda.synchronize()
        # the device's records against the oracle's; the oracle's caches advance with its own
        ko_cache = _check_appended(kl, ko, kn.astype(np.float32), p, cap, hkv, BASE, ko_cache, _host_codes(kc))
        vo_cache = _check_appended(vl, vo, vn.astype(np.float32), p, cap, hkv, 0.0, vo_cache, _host_codes(vc))
        o = out.cpu().numpy()
        assert np.all(o[2] == 0.0)
        qr = oq.rope(q[:2].reshape(2 * hq, d), np.repeat(p[:2], hq), BASE).reshape(2, hq, d)
        want = oe.attend_lens(qr, ko_cache, vo_cache, ko, vo, cap, p[:2].astype(np.int64) + 1, hkv, 0.125)
        err = rel_err_rows(o[:2], want)
        say("  step", step, "max rel err", err.max())
        assert err.max() <= TOL


def test_full_size_decode_step_sampled_heads():
    """The 8B-class decode shape (256 sequences x 8 kv heads, capacity 32768) with ragged
    positions, in the bench's launch configuration; sampled heads checked by the oracle."""
    w = synth.GQA_DECODE
    say("decode step full size", w.name)
    kl, ko = _codecs(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vl, vo = _codecs(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    cap = w.n_ctx
    n_vec = w.n_seq * w.hkv * cap
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)

    def fill(codes):
        codes.idx.copy_(torch.randint(0, 256, codes.idx.shape, generator=gen, device="cuda", dtype=torch.uint8))
        if codes.sign is not None:
            codes.sign.copy_(torch.randint(0, 256, codes.sign.shape, generator=gen, device="cuda", dtype=torch.uint8))
        nrm = torch.randn(n_vec, generator=gen, device="cuda").abs() * math.sqrt(w.d)
        rn = torch.randn(n_vec, generator=gen, device="cuda").abs() * (0.35 * math.sqrt(w.d))
        lo = nrm.half().view(torch.int16).to(torch.int32) & 0xFFFF
        hi = rn.half().view(torch.int16).to(torch.int32) & 0xFFFF
        codes.norms.copy_(lo | (hi << 16))

    kc, vc = tq.alloc_codes(kl, n_vec), tq.alloc_codes(vl, n_vec)
    fill(kc)
    fill(vc)
    pos = torch.randint(cap // 2, cap, (w.n_seq,), generator=gen, device="cuda", dtype=torch.int32)
    pos[0], pos[-1] = cap - 1, 0
    q = torch.randn((w.n_seq, w.hq, w.d), generator=gen, device="cuda")
    kn = torch.randn((w.n_seq, w.hkv, w.d), generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn((w.n_seq, w.hkv, w.d), generator=gen, device="cuda").to(torch.bfloat16)
    scale = 1.0 / math.sqrt(w.d)
    heads = [(0, 0), (w.n_seq - 1, w.hq - 1), (w.n_seq // 2, 9), (77, 30)]
    # the sampled blocks as they are before the step (inputs of the oracle)
    before = {}
    for s, h in heads:
        blk = s * w.hkv + h // w.group
        sl = slice(blk * cap, (blk + 1) * cap)
        before[(s, h)] = (_host_codes(kc, sl), _host_codes(vc, sl))
    out = tq.decode_step(kl, vl, q, kn, vn, pos, cap, BASE, kc, vc, scale)
    torch.cuda.synchronize()
    p = pos.cpu().numpy().astype(np.int64)
    qn = q.cpu().numpy().astype(np.float64)
    kn_h, vn_h = kn.float().cpu().numpy(), vn.float().cpu().numpy()
    for s, h in heads:
        blk = s * w.hkv + h // w.group
        kvh = h // w.group
        kb1, vb1 = before[(s, h)]
        slot = np.array([blk * cap + p[s]])
        # the oracle's own records of the new key and value at slot pos[s] of this block
        kr = oq.append(kn_h[s, kvh][None], ko, slot, np.array([p[s]]), BASE, idx_stride=kl.idx_stride,
                       sign_stride=kl.sign_stride)
        vr = oq.append(vn_h[s, kvh][None], vo, slot, np.array([p[s]]), 0.0, idx_stride=vl.idx_stride,
                       sign_stride=vl.sign_stride)
        k1 = _with_records(kb1, np.array([p[s]]), kr)
        v1 = _with_records(vb1, np.array([p[s]]), vr)
        qr = oq.rope(qn[s, h][None], [p[s]], BASE)
        want = oe.attend_lens(qr[None], k1, v1, ko, vo, cap, [p[s] + 1], 1, scale)[0, 0]
        err = rel_err_rows(out[s, h].cpu().numpy()[None], want[None])[0]
        say("  head", s, h, "pos", p[s], "rel err", err)
        assert err <= TOL
