"""GPU score stream against the oracle: same codes in, logits within 1e-3 relative per row
(max_n |gpu - oracle| / max_n |oracle| for each (sequence, query head)).

Small cases take codes from the oracle's encoder; the full-size cases (the 8B-class decode
step and the 131k-token decode in the bench's launch configuration) take seeded synthetic
code planes and compare sampled rows."""

import math

import numpy as np
import pytest

import synth
from oracle import codec as oc
from oracle import estimate as oe
from oracle import quantize as oq
from tests._util import oracle_codes, rel_err_rows, sampled_heads, say, to_device_codes

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

TOL = 1e-3


def _run(lib, ora, K, q, n_keys, hkv, first_rot_blocks=True):
    """Oracle-encode K ([S*hkv*N, d] fp32), score on GPU and in the oracle."""
    codes = oq.encode(K, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    dc = to_device_codes(tq, codes.idx, codes.sign, codes.norms)
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    got = tq.scores(lib, qd, dc, n_keys, hkv).cpu().numpy()
    want = oe.scores(q.astype(np.float64), codes, ora, n_keys, hkv)
    return got, want


def test_tiny_workload():
    say("scores tiny")
    K, V, q = synth.tiny()
    w = synth.TINY
    lib = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    ora = oc.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    got, want = _run(lib, ora, K, q.reshape(1, 1, -1), 256, 1)
    err = rel_err_rows(got, want)
    say("  rel err", err.max())
    assert err.max() <= TOL


@pytest.mark.parametrize("d,bits,m,hq,hkv,S,N", [
    (64, 3, 64, 20, 20, 2, 1024),      # ESM-2 shape (per-head rotations below)
    (128, 2, 128, 32, 8, 1, 40000),    # 8B GQA shape, 3 chunks + ragged tail
    (128, 2, 128, 16, 8, 2, 777),      # two heads per kv head
    (128, 3, 0, 8, 8, 2, 513),         # MSE only
    (200, 2, 200, 1, 1, 3, 3001),      # search shape
    (64, 4, 64, 8, 2, 1, 300),
    (128, 3, 128, 8, 2, 1, 1500),      # four heads per lookup, 512-thread workgroups
    (128, 2, 0, 4, 1, 2, 900),         # four heads per lookup without a sketch, 512 threads
    # from 32 query heads per kv head on: bit-plane products on the matrix cores
    (64, 3, 64, 64, 2, 2, 300),        # 32 heads per kv head, ragged last tile
    (128, 2, 128, 96, 1, 1, 1001),     # 64 + 32 heads, key count not a multiple of 4
    (200, 3, 0, 40, 1, 2, 515),        # a partly filled wavefront of heads, no sketch
    (128, 3, 128, 33, 1, 1, 4100),     # several key chunks
    (64, 2, 0, 64, 4, 1, 2048),
    (200, 2, 200, 32, 1, 1, 700),
])
def test_scores_match_oracle(d, bits, m, hq, hkv, S, N):
    say("scores", d, bits, m, hq, hkv, S, N)
    lib = tq.make_codec(d, bits, m, 1, 2)
    ora = oc.make_codec(d, bits, m, 1, 2)
    g = np.random.default_rng(d + bits + hq)
    K = (g.standard_normal((S * hkv * N, d)) * np.where(g.random(d) < 0.03, 10.0, 1.0)).astype(np.float32)
    q = g.standard_normal((S, hq, d)).astype(np.float32)
    got, want = _run(lib, ora, K, q, N, hkv)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max())
    assert err.max() <= TOL


def test_scores_per_head_rotations_esm2_slice():
    say("scores esm2 slice")
    d, bits, m, N, layers, heads = 64, 3, 64, 1024, 2, 20
    seeds = [synth.esm2_basis_seed(l, h) for l in range(layers) for h in range(heads)]
    lib = tq.make_codec(d, bits, m, 1, 2, basis_seeds=seeds, vecs_per_rot=N)
    ora = oc.make_codec(d, bits, m, 1, 2, basis_seeds=seeds, vecs_per_rot=N)
    K, V, q = synth.esm2(layers=layers, heads=heads, seq=N)
    got, want = _run(lib, ora, K.reshape(-1, d).astype(np.float32), q, N, heads)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max())
    assert err.max() <= TOL


@pytest.mark.parametrize("wname", ["gqa", "long"])
def test_full_size_sampled_rows(wname):
    """All layers x batch x heads at full context, in the bench's launch configuration."""
    w = synth.GQA_DECODE if wname == "gqa" else synth.LONG_CTX
    say("scores full size", w.name)
    lib = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    ora = oc.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    n_vec = w.n_seq * w.hkv * w.n_ctx
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    codes = tq.alloc_codes(lib, n_vec)
    codes.idx.copy_(torch.randint(0, 256, codes.idx.shape, generator=gen, device="cuda", dtype=torch.uint8))
    codes.sign.copy_(torch.randint(0, 256, codes.sign.shape, generator=gen, device="cuda", dtype=torch.uint8))
    nrm = torch.randn(n_vec, generator=gen, device="cuda").abs() * math.sqrt(w.d)
    rn = torch.randn(n_vec, generator=gen, device="cuda").abs() * (0.35 * math.sqrt(w.d))
    lo = nrm.half().view(torch.int16).to(torch.int32) & 0xFFFF
    hi = rn.half().view(torch.int16).to(torch.int32) & 0xFFFF
    codes.norms.copy_(lo | (hi << 16))
    q = torch.randn((w.n_seq, w.hq, w.d), generator=gen, device="cuda")
    logits = tq.scores(lib, q, codes, w.n_ctx, w.hkv)
    torch.cuda.synchronize()
    qn = q.cpu().numpy().astype(np.float64)
    worst = 0.0
    rows = sampled_heads(w, 64 if wname == "gqa" else 32, seed=5)
    for blk, heads in rows:
        sl = slice(blk * w.n_ctx, (blk + 1) * w.n_ctx)
        oc_codes = oracle_codes(codes.idx[sl].cpu().numpy(), codes.sign[sl].cpu().numpy(),
                                codes.norms[sl].cpu().numpy().view(np.uint32))
        s = blk // w.hkv
        want = oe.scores(qn[s:s + 1, heads], oc_codes, ora, w.n_ctx, 1)[0]
        got = logits[s, heads].cpu().numpy()
        err = rel_err_rows(got, want)
        worst = max(worst, err.max())
        assert err.max() <= TOL, (s, heads, err)
    say("  rows", sum(len(h) for _, h in rows), "max rel err", worst)


def test_scores_empty_and_tiny_n():
    lib = tq.make_codec(64, 2, 64, 1, 2)
    q = torch.randn((1, 1, 64), device="cuda")
    codes = tq.alloc_codes(lib, 1)
    y = torch.randn((1, 64), device="cuda")
    tq.encode(lib, y, pre_rotated=True, out=codes)
    out = tq.scores(lib, q, codes, 1, 1)
    torch.cuda.synchronize()
    assert out.shape == (1, 1, 1) and torch.isfinite(out).all()
    e = tq.scores(lib, torch.empty((0, 1, 64), device="cuda"), codes, 1, 1)
    assert e.shape == (0, 1, 1)


def _orthogonal_queries(K, q, n_keys, hkv, frac, g):
    """Replace a fraction of the queries by ones nearly orthogonal to every key of their kv block
    (the component in the keys' span removed, 1e-4 of noise added back)."""
    S, hq, d = q.shape
    G = hq // hkv
    q = q.copy()
    Kb = K.reshape(S, hkv, n_keys, d).astype(np.float64)
    for s in range(S):
        for h in range(hq):
            if g.random() < frac:
                B = Kb[s, h // G]
                Q, _ = np.linalg.qr(B.T)  # orthonormal basis of the keys' span
                v = q[s, h].astype(np.float64)
                v = v - Q @ (Q.T @ v)
                v += 1e-4 * np.linalg.norm(v) * g.standard_normal(d)
                q[s, h] = v.astype(np.float32)
    return q


@pytest.mark.parametrize("d,bits,m,N", [(128, 2, 128, 1), (128, 2, 128, 2), (128, 2, 128, 3), (128, 2, 128, 17),
                                        (128, 3, 0, 1), (128, 3, 0, 17), (64, 3, 64, 3)])
def test_four_heads_per_kv_head_tiny_n(d, bits, m, N):
    """Four query heads per kv head share 16-bit fixed-point table entries; with a handful of keys
    (or a query nearly orthogonal to them) the row's largest |logit| can be small next to the
    tables' rounding, and the kernel must fall back to fp32 tables for that row: every row within
    1e-3 of the oracle."""
    say("scores G=4 tiny N", d, bits, m, N)
    lib = tq.make_codec(d, bits, m, 1, 2)
    ora = oc.make_codec(d, bits, m, 1, 2)
    S, hkv, hq = 128, 2, 8
    g = np.random.default_rng(1000 * N + d + bits)
    K = (g.standard_normal((S * hkv * N, d)) * np.where(g.random(d) < 0.03, 10.0, 1.0)).astype(np.float32)
    q = g.standard_normal((S, hq, d)).astype(np.float32)
    q = _orthogonal_queries(K, q, N, hkv, 0.5, g)
    got, want = _run(lib, ora, K, q, N, hkv)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max(), "rows", err.size)
    assert err.max() <= TOL


def test_scores_many_heads_per_head_rotations():
    """Every token of a short protein-like sequence querying every cached key, per (layer, head)
    rotations: 64 queries per kv head on the bit-plane path."""
    say("scores esm2-shaped all pairs")
    d, bits, m, N, layers, heads = 64, 3, 64, 256, 1, 4
    seeds = [synth.esm2_basis_seed(l, h) for l in range(layers) for h in range(heads)]
    lib = tq.make_codec(d, bits, m, 1, 2, basis_seeds=seeds, vecs_per_rot=N)
    ora = oc.make_codec(d, bits, m, 1, 2, basis_seeds=seeds, vecs_per_rot=N)
    K, V, q = synth.esm2(layers=layers, heads=heads, seq=N)
    g = np.random.default_rng(7)
    qa = (K.reshape(layers, heads, N, d)[:, :, :64] + 0.1 * g.standard_normal((layers, heads, 64, d)))
    qa = qa.reshape(layers, heads * 64, d).astype(np.float32)
    got, want = _run(lib, ora, K.reshape(-1, d).astype(np.float32), qa, N, heads)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max())
    assert err.max() <= TOL


def test_scores_many_heads_asymmetric_codebook():
    """A codebook not symmetric about zero on the bit-plane path (its even Walsh planes)."""
    import dataclasses
    say("scores many heads, asymmetric codebook")
    for d, bits, m in ((128, 2, 128), (64, 3, 0)):
        ora0 = oc.make_codec(d, bits, m, 1, 2)
        c = ora0.centroids.astype(np.float64)
        c2 = (c + np.linspace(0.05, 0.3, len(c)) * (c.max() - c.min())).astype(np.float32)
        t2 = (0.5 * (c2[:-1].astype(np.float64) + c2[1:])).astype(np.float32)
        ora = dataclasses.replace(ora0, centroids=c2, thresholds=t2)
        lib = tq.codec_from_arrays(d, bits, m, ora.rot, ora.sketch, c2, t2)
        g = np.random.default_rng(d + bits)
        K = g.standard_normal((2 * 600, d)).astype(np.float32)
        q = g.standard_normal((1, 2 * 48, d)).astype(np.float32)
        got, want = _run(lib, ora, K, q, 600, 2)
        err = rel_err_rows(got, want)
        say("  ", d, bits, m, "max rel err", err.max())
        assert err.max() <= TOL


def test_full_size_esm2_all_pairs_sampled():
    """The all-pairs scoring of the ESM-2-shaped cache in the bench's launch configuration: 33
    layers x 20 heads, every one of the 1024 tokens a query head of its (layer, head), one rotation
    per (layer, head) -- the query prep with 64 heads per workgroup (from 65536 query heads on) and
    the bit-plane scan.  Seeded random code planes; 48 sampled (kv block, query) rows and the whole
    last block against the oracle."""
    w = synth.ESM2
    say("scores full size all pairs", w.name)
    seeds = [synth.esm2_basis_seed(l, h) for l in range(w.layers) for h in range(w.hkv)]
    lib = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K, basis_seeds=seeds,
                        vecs_per_rot=w.n_ctx)
    ora = oc.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K, basis_seeds=seeds,
                        vecs_per_rot=w.n_ctx)
    n_blk = w.layers * w.hkv
    n_vec = n_blk * w.n_ctx
    idx, sign, norms = synth.random_codes(n_vec, w.d, w.k_bits, w.k_m, lib.idx_stride, lib.sign_stride, seed=43)
    codes = to_device_codes(tq, idx, sign, norms)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(44)
    q = torch.randn((w.layers, w.hkv * w.n_ctx, w.d), generator=gen, device="cuda")
    assert q.shape[0] * q.shape[1] >= 65536  # the 64-heads-per-workgroup query prep
    logits = tq.scores(lib, q, codes, w.n_ctx, w.hkv)
    torch.cuda.synchronize()
    g = np.random.default_rng(45)
    picks = [(int(b), int(t)) for b, t in zip(g.integers(0, n_blk, 48), g.integers(0, w.n_ctx, 48))]
    picks += [(n_blk - 1, t) for t in (0, 511, w.n_ctx - 1)]
    worst = 0.0
    for blk, t in picks:
        l, h = divmod(blk, w.hkv)
        sl = slice(blk * w.n_ctx, (blk + 1) * w.n_ctx)
        qv = q[l, h * w.n_ctx + t].cpu().numpy().astype(np.float64)
        want = oe.scores_one(qv, oracle_codes(idx[sl], sign[sl], norms[sl]), ora, blk)
        got = logits[l, h * w.n_ctx + t].cpu().numpy()
        err = rel_err_rows(got, want)
        worst = max(worst, float(err))
        assert err <= TOL, (blk, t, err)
    say("  rows", len(picks), "max rel err", worst)
