"""tq_decode_step_noalloc (workspace in the library's static scratch array) against tq_decode_step
(workspace given by the caller), through the C ABI: two calls in a row, the second smaller, with
identical appended records (bit-exact) and identical outputs; a call larger than the array is
refused before any launch."""

import ctypes
import math

import numpy as np
import pytest

import synth
from tests._util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")


def _cache(codec, n, gen):
    c = tq.alloc_codes(codec, n)
    c.idx.copy_(torch.randint(0, 256, c.idx.shape, generator=gen, device="cuda", dtype=torch.uint8))
    if c.sign is not None:
        c.sign.copy_(torch.randint(0, 256, c.sign.shape, generator=gen, device="cuda", dtype=torch.uint8))
    nrm = (torch.rand(n, generator=gen, device="cuda") * 20 + 1).half().view(torch.int16).to(torch.int32) & 0xFFFF
    rn = (torch.rand(n, generator=gen, device="cuda") * 5).half().view(torch.int16).to(torch.int32) & 0xFFFF
    c.norms.copy_(nrm | (rn << 16))
    return c


def _clone(c):
    return tq.Codes(c.idx.clone(), None if c.sign is None else c.sign.clone(), c.norms.clone())


def _step_pair(kl, vl, n_seq, hq, hkv, cap, gen, first_call):
    kc, vc = _cache(kl, n_seq * hkv * cap, gen), _cache(vl, n_seq * hkv * cap, gen)
    kc2, vc2 = _clone(kc), _clone(vc)
    q = torch.randn((n_seq, hq, kl.d), generator=gen, device="cuda")
    kn = torch.randn((n_seq, hkv, kl.d), generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn((n_seq, hkv, kl.d), generator=gen, device="cuda").to(torch.bfloat16)
    pos = torch.randint(0, cap, (n_seq,), generator=gen, device="cuda", dtype=torch.int32)
    pos[0] = cap - 1
    scale = 1.0 / math.sqrt(kl.d)
    ref = tq.decode_step(kl, vl, q, kn, vn, pos, cap, 10000.0, kc, vc, scale)
    out = torch.full((n_seq, hq, kl.d), float("nan"), device="cuda")
    kcc, vcc = kl.c(), vl.c()
    rc = tq.lib.tq_decode_step_noalloc(ctypes.byref(kcc), ctypes.byref(vcc), tq._ptr(q), tq._ptr(kn), tq._ptr(vn),
                                       tq.TQ_BF16, n_seq, hq, hkv, cap, tq._ptr(pos), ctypes.c_float(10000.0),
                                       kc2.c(), vc2.c(), ctypes.c_float(scale), tq._ptr(out), tq._stream())
    assert rc == 0, tq.lib.tq_status_str(rc).decode()
    torch.cuda.synchronize()
    for a, b in ((kc.idx, kc2.idx), (kc.sign, kc2.sign), (kc.norms, kc2.norms), (vc.idx, vc2.idx),
                 (vc.norms, vc2.norms)):
        assert torch.equal(a, b)
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref)  # the same kernels on the same inputs
    say("  no-alloc decode step", n_seq, hq, hkv, cap, "identical to tq_decode_step")


def test_noalloc_matches_decode_step_twice_then_smaller():
    w = synth.GQA_DECODE
    kl = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vl = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    # a large call (about 4 MiB of scratch), then a smaller one: the second must not see the first's
    # leftovers
    _step_pair(kl, vl, 64, 32, 8, 4096, gen, True)
    _step_pair(kl, vl, 3, 8, 2, 700, gen, False)


def test_noalloc_refuses_a_call_beyond_the_array():
    w = synth.GQA_DECODE
    kl = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vl = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    n_seq, hq, hkv, cap = 4096, 32, 8, 32768
    kcc, vcc = kl.c(), vl.c()
    need = tq.lib.tq_workspace_bytes(tq.TQ_OP_DECODE_STEP, ctypes.byref(kcc), ctypes.byref(vcc), n_seq, hq, hkv, cap)
    assert need > (32 << 20)
    # small real buffers: the call must return before any launch touches them
    kc, vc = tq.alloc_codes(kl, 8), tq.alloc_codes(vl, 8)
    kc.norms.fill_(7)
    q = torch.zeros((1, 1, w.d), device="cuda")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = tq.lib.tq_decode_step_noalloc(ctypes.byref(kcc), ctypes.byref(vcc), tq._ptr(q), tq._ptr(q), tq._ptr(q),
                                       tq.TQ_F32, n_seq, hq, hkv, cap, tq._ptr(pos), ctypes.c_float(0.0), kc.c(),
                                       vc.c(), ctypes.c_float(1.0), tq._ptr(q), tq._stream())
    assert rc == -6
    torch.cuda.synchronize()
    assert torch.all(kc.norms == 7)
