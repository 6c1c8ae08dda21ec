"""GPU decode attention against the oracle: identical (oracle-encoded) codes in, outputs within
1e-3 relative per (sequence, query head): max_k |gpu - oracle| / max_k |oracle|."""

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


def _case(d, kb, km, vb, vm, hq, hkv, S, N, seed, K=None, V=None, q=None, basis=None, scale=None):
    kl = tq.make_codec(d, kb, km, synth.SEED_ROT_K, synth.SEED_SKETCH_K, basis_seeds=basis, vecs_per_rot=N if basis else 0)
    vl = tq.make_codec(d, vb, vm, synth.SEED_ROT_V, synth.SEED_SKETCH_V, basis_seeds=basis, vecs_per_rot=N if basis else 0)
    ko = oc.make_codec(d, kb, km, synth.SEED_ROT_K, synth.SEED_SKETCH_K, basis_seeds=basis, vecs_per_rot=N if basis else 0)
    vo = oc.make_codec(d, vb, vm, synth.SEED_ROT_V, synth.SEED_SKETCH_V, basis_seeds=basis, vecs_per_rot=N if basis else 0)
    g = np.random.default_rng(seed)
    if K is None:
        K = (g.standard_normal((S * hkv * N, d)) * np.where(g.random(d) < 0.03, 10.0, 1.0)).astype(np.float32)
        V = g.standard_normal((S * hkv * N, d)).astype(np.float32)
        q = g.standard_normal((S, hq, d)).astype(np.float32)
    kcodes = oq.encode(K, ko, idx_stride=kl.idx_stride, sign_stride=kl.sign_stride)
    vcodes = oq.encode(V, vo, idx_stride=vl.idx_stride, sign_stride=vl.sign_stride)
    scale = scale or 1.0 / math.sqrt(d)
    got = tq.attend_decode(kl, vl, torch.from_numpy(q).cuda(), to_device_codes(tq, kcodes.idx, kcodes.sign, kcodes.norms),
                           to_device_codes(tq, vcodes.idx, vcodes.sign, vcodes.norms), N, hkv, scale)
    torch.cuda.synchronize()
    want = oe.attend(q.astype(np.float64), kcodes, vcodes, ko, vo, N, hkv, scale)
    return got.cpu().numpy(), want


def test_tiny_workload():
    say("attend tiny")
    K, V, q = synth.tiny()
    got, want = _case(64, 2, 64, 2, 64, 1, 1, 1, 256, 0, K=K, V=V, q=q.reshape(1, 1, -1))
    err = rel_err_rows(got, want)
    say("  rel err", err.max())
    assert err.max() <= TOL


@pytest.mark.parametrize("d,kb,km,vb,vm,hq,hkv,S,N", [
    (128, 2, 128, 3, 0, 32, 8, 2, 5000),    # 8B GQA decode shape, ragged last tile, several chunks
    (128, 2, 128, 3, 0, 8, 8, 1, 20000),    # one head per kv head, many chunks
    (128, 2, 128, 3, 0, 16, 8, 1, 3000),    # two heads per kv head
    (128, 2, 128, 3, 0, 16, 2, 2, 2500),    # eight heads per kv head: two groups of four
    (64, 3, 64, 3, 64, 20, 20, 1, 1024),    # ESM-2 shape with V QJL
    (64, 2, 64, 2, 64, 4, 1, 2, 700),
    (128, 3, 128, 3, 128, 4, 2, 1, 1000),
    (128, 3, 0, 3, 0, 4, 4, 1, 1),          # a single cached token
])
def test_attend_matches_oracle(d, kb, km, vb, vm, hq, hkv, S, N):
    say("attend", d, kb, km, vb, vm, hq, hkv, S, N)
    got, want = _case(d, kb, km, vb, vm, hq, hkv, S, N, seed=d + N)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max())
    assert err.max() <= TOL


def test_attend_peaked_softmax_and_equal_keys():
    # large logit scale: softmax nearly one-hot; identical keys: uniform weights (mean of values)
    d, N = 128, 2048
    g = np.random.default_rng(3)
    K = g.standard_normal((N, d)).astype(np.float32)
    V = g.standard_normal((N, d)).astype(np.float32)
    q = (4 * g.standard_normal((1, 4, d))).astype(np.float32)
    got, want = _case(d, 2, 128, 3, 0, 4, 1, 1, N, 0, K=K, V=V, q=q, scale=1.0)
    assert rel_err_rows(got, want).max() <= TOL
    K2 = np.repeat(K[:1], N, axis=0)
    got, want = _case(d, 2, 128, 3, 0, 4, 1, 1, N, 0, K=K2, V=V, q=q)
    assert rel_err_rows(got, want).max() <= TOL


def test_attend_esm2_per_head_rotations():
    say("attend esm2 slice")
    d, N, layers, heads = 64, 1024, 2, 20
    seeds = [synth.esm2_basis_seed(l, h) for l in range(layers) for h in range(heads)]
    K, V, q = synth.esm2(layers=layers, heads=heads, seq=N)
    got, want = _case(d, 3, 64, 3, 64, heads, heads, layers, N, 0, K=K.reshape(-1, d).astype(np.float32),
                      V=V.reshape(-1, d).astype(np.float32), q=q, basis=seeds)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max())
    assert err.max() <= TOL


def test_running_max_moves_in_most_tiles():
    """Key norms growing along the context, so that the running maxima move in most tiles, at a
    size where every wavefront takes several tiles of its chunk (the accumulators are rescaled
    between tiles); four query heads per kv head; sampled heads against the oracle."""
    d, S, hkv, hq, N = 128, 2, 8, 32, 65536
    say("attend growing key norms", S, hkv, hq, N)
    kl = tq.make_codec(d, 2, 128, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vl = tq.make_codec(d, 3, 0, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    ko = oc.make_codec(d, 2, 128, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vo = oc.make_codec(d, 3, 0, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    n_vec = S * hkv * N
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    ramp = (1.0 + 4.0 * torch.arange(N, device="cuda", dtype=torch.float32) / N).repeat(S * hkv)

    def fill(codes, grow):
        codes.idx.copy_(torch.randint(0, 256, codes.idx.shape, generator=gen, device="cuda", dtype=torch.uint8))
        if codes.sign is not None:
            codes.sign.copy_(torch.randint(0, 256, codes.sign.shape, generator=gen, device="cuda", dtype=torch.uint8))
        nrm = torch.randn(n_vec, generator=gen, device="cuda").abs() * math.sqrt(d)
        if grow:
            nrm = nrm * ramp
        rn = torch.randn(n_vec, generator=gen, device="cuda").abs() * (0.35 * math.sqrt(d))
        lo = nrm.half().view(torch.int16).to(torch.int32) & 0xFFFF
        hi = rn.half().view(torch.int16).to(torch.int32) & 0xFFFF
        codes.norms.copy_(lo | (hi << 16))

    kcodes, vcodes = tq.alloc_codes(kl, n_vec), tq.alloc_codes(vl, n_vec)
    fill(kcodes, True)
    fill(vcodes, False)
    q = torch.randn((S, hq, d), generator=gen, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = tq.attend_decode(kl, vl, q, kcodes, vcodes, N, hkv, scale)
    torch.cuda.synchronize()
    qn = q.cpu().numpy().astype(np.float64)
    g = hq // hkv
    worst = 0.0
    for blk in (0, 5, 11, 15):
        s, kvh = blk // hkv, blk % hkv
        heads = list(range(kvh * g, (kvh + 1) * g))
        sl = slice(blk * N, (blk + 1) * N)
        kc = oracle_codes(kcodes.idx[sl].cpu().numpy(), kcodes.sign[sl].cpu().numpy(),
                          kcodes.norms[sl].cpu().numpy().view(np.uint32))
        vc = oracle_codes(vcodes.idx[sl].cpu().numpy(), None, vcodes.norms[sl].cpu().numpy().view(np.uint32))
        want = oe.attend(qn[s:s + 1, heads], kc, vc, ko, vo, N, 1, scale)[0]
        err = rel_err_rows(out[s, heads].cpu().numpy(), want)
        worst = max(worst, err.max())
        assert err.max() <= TOL, (blk, err)
    say("  max rel err", worst)


@pytest.mark.parametrize("wname", ["gqa", "long"])
def test_full_size_sampled_heads(wname):
    """Full decode step in the bench's launch configuration; sampled query heads recomputed by
    the oracle from the same (seeded synthetic) code planes."""
    w = synth.GQA_DECODE if wname == "gqa" else synth.LONG_CTX
    say("attend full size", w.name)
    kl = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vl = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    ko = oc.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vo = oc.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    n_vec = w.n_seq * w.hkv * w.n_ctx
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)

    def fill(codes, bits_d, m):
        codes.idx.copy_(torch.randint(0, 256, codes.idx.shape, generator=gen, device="cuda", dtype=torch.uint8))
        if bits_d % 32:
            raise AssertionError("record padding not handled here")
        if codes.sign is not None:
            codes.sign.copy_(torch.randint(0, 256, codes.sign.shape, generator=gen, device="cuda", dtype=torch.uint8))
        nrm = torch.randn(n_vec, generator=gen, device="cuda").abs() * math.sqrt(w.d)
        rn = torch.randn(n_vec, generator=gen, device="cuda").abs() * (0.35 * math.sqrt(w.d))
        lo = nrm.half().view(torch.int16).to(torch.int32) & 0xFFFF
        hi = rn.half().view(torch.int16).to(torch.int32) & 0xFFFF
        codes.norms.copy_(lo | (hi << 16))

    kcodes, vcodes = tq.alloc_codes(kl, n_vec), tq.alloc_codes(vl, n_vec)
    fill(kcodes, w.d * w.k_bits, w.k_m)
    fill(vcodes, w.d * w.v_bits, w.v_m)
    q = torch.randn((w.n_seq, w.hq, w.d), generator=gen, device="cuda")
    scale = 1.0 / math.sqrt(w.d)
    out = tq.attend_decode(kl, vl, q, kcodes, vcodes, w.n_ctx, w.hkv, scale)
    torch.cuda.synchronize()
    qn = q.cpu().numpy().astype(np.float64)
    worst, n_heads = 0.0, 0
    for blk, heads in sampled_heads(w, 64 if wname == "gqa" else 32, seed=6):
        s = blk // w.hkv
        sl = slice(blk * w.n_ctx, (blk + 1) * w.n_ctx)
        kc = oracle_codes(kcodes.idx[sl].cpu().numpy(), kcodes.sign[sl].cpu().numpy(),
                          kcodes.norms[sl].cpu().numpy().view(np.uint32))
        vc = oracle_codes(vcodes.idx[sl].cpu().numpy(), None, vcodes.norms[sl].cpu().numpy().view(np.uint32))
        want = oe.attend(qn[s:s + 1, heads], kc, vc, ko, vo, w.n_ctx, 1, scale)[0]
        err = rel_err_rows(out[s, heads].cpu().numpy(), want)
        worst, n_heads = max(worst, err.max()), n_heads + len(heads)
        assert err.max() <= TOL, (s, heads, err)
    say("  heads", n_heads, "max rel err", worst)


@pytest.mark.parametrize("kb,km,vb,vm,N", [(2, 128, 3, 0, 1), (2, 128, 3, 0, 2), (2, 128, 3, 0, 3),
                                           (2, 128, 3, 0, 17), (3, 128, 3, 128, 3), (3, 0, 3, 0, 17)])
def test_four_heads_per_kv_head_tiny_n(kb, km, vb, vm, N):
    """Four query heads per kv head (16-bit fixed-point key tables) over a handful of tokens, half
    the queries nearly orthogonal to every key of their block (logits near zero, weights near
    uniform)."""
    from tests.test_gpu_scores import _orthogonal_queries

    say("attend G=4 tiny N", kb, km, vb, vm, N)
    d, S, hkv, hq = 128, 64, 2, 8
    g = np.random.default_rng(77 * N + kb + vb)
    K = (g.standard_normal((S * hkv * N, d)) * np.where(g.random(d) < 0.03, 10.0, 1.0)).astype(np.float32)
    V = g.standard_normal((S * hkv * N, d)).astype(np.float32)
    q = _orthogonal_queries(K, g.standard_normal((S, hq, d)).astype(np.float32), N, hkv, 0.5, g)
    got, want = _case(d, kb, km, vb, vm, hq, hkv, S, N, 0, K=K, V=V, q=q)
    err = rel_err_rows(got, want)
    say("  max rel err", err.max())
    assert err.max() <= TOL
