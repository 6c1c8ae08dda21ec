"""GPU top-k search against the oracle.  Several top-k sets are correct when estimates tie or
nearly tie, so the check is: every returned score equals the oracle's estimate for that row
within 1e-3 of the query's score scale; the returned list is ordered; and any row that is in
one list but not the other has an oracle score within that tolerance of the oracle's k-th."""

import math

import numpy as np
import pytest

import synth
from oracle import codec as oc
from oracle import estimate as oe
from oracle import quantize as oq
from tests._util import oracle_codes, say, to_device_codes

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

TOL = 1e-3


def check_topk(gi, gs, oscores, k):
    """gi/gs: GPU result [Q, k]; oscores: oracle estimates [Q, n_db] (fp64)."""
    oi, os_ = oe.topk_rows(oscores, k)
    for q in range(gi.shape[0]):
        scale = np.max(np.abs(oscores[q]))
        tol = TOL * scale
        assert len(set(gi[q].tolist())) == k
        assert np.all(np.abs(gs[q] - oscores[q, gi[q]]) <= tol)
        assert np.all(np.diff(gs[q]) <= tol)  # descending within tolerance
        kth = os_[q, -1]
        for r in set(gi[q].tolist()) ^ set(oi[q].tolist()):
            assert abs(oscores[q, r] - kth) <= 2 * tol, (q, r, oscores[q, r], kth)


@pytest.mark.parametrize("d,bits,m,n_db,n_q,k", [
    (200, 2, 200, 20000, 37, 10),     # search shape, several slices, ragged query group
    (128, 2, 128, 9000, 8, 32),
    (64, 3, 64, 5000, 5, 1),
    (200, 2, 200, 40, 3, 10),         # tiny database, one slice
    # from 32 queries on: the matrix-core scan (16 queries per workgroup)
    (128, 3, 0, 9000, 40, 32),        # no sign term, k = 32, ragged query group
    (64, 2, 64, 5000, 33, 7),
    (64, 3, 64, 3000, 64, 1),
    (200, 3, 0, 70000, 48, 16),       # several slices, the last one short
    (128, 2, 128, 50, 35, 20),        # tiny database: one short slice, a ragged row tile
])
def test_search_matches_oracle(d, bits, m, n_db, n_q, k):
    say("search", d, bits, m, n_db, n_q, k)
    lib = tq.make_codec(d, bits, m, 1, 2)
    ora = oc.make_codec(d, bits, m, 1, 2)
    db, qs = synth.search_data(n_db=n_db, n_q=n_q, d=d, clusters=50)
    codes = oq.encode(db, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    gi, gs = tq.search_topk(lib, torch.from_numpy(qs).cuda(), to_device_codes(tq, codes.idx, codes.sign, codes.norms),
                            n_db, k)
    torch.cuda.synchronize()
    check_topk(gi.cpu().numpy(), gs.cpu().numpy(), oe.search_scores(qs, codes, ora), k)


def test_search_full_size_sampled_queries():
    """1M-row database and 10,000 queries in the bench's launch configuration (synthetic code
    planes); 24 sampled queries recomputed by the oracle."""
    d, bits, m = synth.SEARCH_D, synth.SEARCH_BITS, synth.SEARCH_M
    n_db, n_q = synth.SEARCH_N_DB, synth.SEARCH_N_Q
    say("search full size")
    lib = tq.make_codec(d, bits, m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    ora = oc.make_codec(d, bits, m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    idx, sign, norms = synth.random_codes(n_db, d, bits, m, lib.idx_stride, lib.sign_stride, seed=21)
    qs = np.random.default_rng(22).standard_normal((n_q, d)).astype(np.float32)
    gi, gs = tq.search_topk(lib, torch.from_numpy(qs).cuda(), to_device_codes(tq, idx, sign, norms), n_db, 10)
    torch.cuda.synchronize()
    sample = np.random.default_rng(23).choice(n_q, 24, replace=False)
    osc = oe.search_scores(qs[sample], oracle_codes(idx, sign, norms), ora)
    check_topk(gi.cpu().numpy()[sample], gs.cpu().numpy()[sample], osc, 10)


@pytest.mark.parametrize("d,bits,m,n_db,n_q,k", [
    (128, 2, 128, 6000, 40, 10),      # matrix-core scan: the even Walsh planes come in
    (64, 3, 64, 4000, 33, 5),
    (200, 3, 0, 3000, 64, 8),
    (128, 2, 128, 6000, 6, 10),       # table scan
])
def test_search_asymmetric_codebook(d, bits, m, n_db, n_q, k):
    """A codebook that is not symmetric about zero (levels shifted by an increasing offset) is
    still searched exactly: the estimate uses the codec's own levels."""
    import dataclasses
    say("search, asymmetric codebook", d, bits, m, n_db, n_q, k)
    ora0 = oc.make_codec(d, bits, m, 1, 2)
    c = ora0.centroids.astype(np.float64)
    c2 = (c + np.linspace(0.05, 0.3, len(c)) * (c.max() - c.min())).astype(np.float32)
    t2 = (0.5 * (c2[:-1].astype(np.float64) + c2[1:])).astype(np.float32)
    ora = dataclasses.replace(ora0, centroids=c2, thresholds=t2)
    lib = tq.codec_from_arrays(d, bits, m, ora.rot, ora.sketch, c2, t2)
    db, qs = synth.search_data(n_db=n_db, n_q=n_q, d=d, clusters=20)
    codes = oq.encode(db, ora, idx_stride=lib.idx_stride, sign_stride=lib.sign_stride)
    gi, gs = tq.search_topk(lib, torch.from_numpy(qs).cuda(), to_device_codes(tq, codes.idx, codes.sign, codes.norms),
                            n_db, k)
    torch.cuda.synchronize()
    check_topk(gi.cpu().numpy(), gs.cpu().numpy(), oe.search_scores(qs, codes, ora), k)
