"""The TurboESM variant on the GPU against the oracle: codebooks calibrated separately for K
and V (the oracle's calibration, uploaded to the library; the library's own calibration is
checked against it on the CPU), per-coordinate residual signs (S = I,
m = d) and the norm word's high half fp16(nbar * resid_scale).  Encode: bit-exact in
pre-rotated mode, every difference explained by the rotation bound in full mode.  Scores and
attention: within 1e-3 relative per row from identical codes, on the table path and on the
many-heads (bit-plane) path, whose calibrated tables are not symmetric about zero."""

import math

import numpy as np
import pytest

import synth
from oracle import calibrate
from oracle import codec as oc
from oracle import estimate as oe
from oracle import quantize as oq
from tests._util import rel_err_rows, say, to_device_codes
from tests.test_gpu_encode import _explained_mismatches, _gpu_encode

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

TOL = 1e-3


def _turbo(d, bits, samples, rot_seed, basis=None, vpr=0):
    """The oracle's calibrated table for these sample vectors (its Lloyd rule from its own
    codebook), uploaded to the library: (library, oracle) codecs of the same table."""
    ora0 = oc.make_codec(d, bits, 0, rot_seed, 2, basis_seeds=basis, vecs_per_rot=vpr)
    u = calibrate.rotated_directions(samples, ora0)
    cal = calibrate.calibrate_codebook(u, oc.lloyd_max_beta(d, bits).centroids64)
    ora = calibrate.turboesm_codec(ora0, cal)
    lib = tq.codec_from_arrays(d, bits, d, ora.rot, ora.sketch, ora.centroids, ora.thresholds, vecs_per_rot=vpr,
                               resid_scale=ora.resid_scale)
    return lib, ora


def _esm(layers, heads, n):
    K, V, q = synth.esm2(layers=layers, heads=heads, seq=n)
    return K, V, q


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 2)])
def test_encode_pre_rotated_bit_exact(d, bits):
    say("turboesm encode pre-rotated", d, bits)
    g = np.random.default_rng(d)
    lib, ora = _turbo(d, bits, g.standard_normal((2000, d)) * np.where(g.random(d) < 0.05, 8.0, 1.0), 1)
    y = synth.pre_rotated(1500, d, seed=5)
    idx, sign, norms, _ = _gpu_encode(lib, y, pre=True)
    want = oq.encode(y, ora, pre_rotated=True, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    assert np.array_equal(idx, want.idx)
    assert np.array_equal(sign, want.sign)
    assert np.array_equal(norms, want.norms)


def test_encode_full_mode_esm_slice():
    say("turboesm encode full, per-head rotations")
    d, bits, N = 64, 3, 256
    seeds = [synth.esm2_basis_seed(l, h) for l in range(2) for h in range(3)]
    K, V, q = _esm(2, 3, N)
    x = K.reshape(-1, d).astype(np.float32)
    lib, ora = _turbo(d, bits, x, 1, basis=seeds, vpr=N)
    gpu = _gpu_encode(lib, x, pre=False, dtype=torch.float16, tap=True)
    want = oq.encode(x, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride, keep=True)
    _explained_mismatches(x, lib, ora, gpu, want)
    assert np.array_equal(gpu[2] >> 16, want.norms >> 16)  # fp16(nbar * resid_scale) from the exact nbar


@pytest.mark.parametrize("G", [1, 4, 32])
def test_scores_and_attention_dual_tables(G):
    """K and V calibrated on their own samples; the cache encoded by the oracle; queries per kv
    head G (32: the bit-plane path, whose planes include the even ones of these tables)."""
    say("turboesm scores/attend, heads per kv head", G)
    d, bits, N, layers, heads = 64, 3, 300, 2, 2
    seeds = [synth.esm2_basis_seed(l, h) for l in range(layers) for h in range(heads)]
    K, V, q = _esm(layers, heads, N)
    Kx, Vx = K.reshape(-1, d).astype(np.float32), V.reshape(-1, d).astype(np.float32)
    kl, ko = _turbo(d, bits, Kx, 1, basis=seeds, vpr=N)
    vl, vo = _turbo(d, bits, Vx, 3, basis=seeds, vpr=N)
    assert not np.array_equal(ko.centroids, vo.centroids)  # two tables
    kc = oq.encode(Kx, ko, idx_stride=kl.idx_stride, sign_stride=kl.sign_stride)
    vc = oq.encode(Vx, vo, idx_stride=vl.idx_stride, sign_stride=vl.sign_stride)
    kd = to_device_codes(tq, kc.idx, kc.sign, kc.norms)
    vd = to_device_codes(tq, vc.idx, vc.sign, vc.norms)
    g = np.random.default_rng(G)
    qq = g.standard_normal((layers, heads * G, d)).astype(np.float32)
    qd = torch.from_numpy(qq).cuda()
    got = tq.scores(kl, qd, kd, N, heads).cpu().numpy()
    want = oe.scores(qq.astype(np.float64), kc, ko, N, heads)
    err = rel_err_rows(got, want)
    say("  scores max rel err", err.max())
    assert err.max() <= TOL
    if G <= 4:
        scale = 1.0 / math.sqrt(d)
        out = tq.attend_decode(kl, vl, qd, kd, vd, N, heads, scale).cpu().numpy()
        ref = oe.attend(qq.astype(np.float64), kc, vc, ko, vo, N, heads, scale)
        err = rel_err_rows(out, ref)
        say("  attend max rel err", err.max())
        assert err.max() <= TOL
