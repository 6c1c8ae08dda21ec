"""Helpers shared by the GPU parity tests (no method arithmetic: marshalling and comparisons)."""

import numpy as np

from oracle import quantize as oq


def to_device_codes(tq, idx, sign, norms, device="cuda"):
    import torch

    return tq.Codes(torch.from_numpy(np.ascontiguousarray(idx)).to(device),
                    None if sign is None else torch.from_numpy(np.ascontiguousarray(sign)).to(device),
                    torch.from_numpy(np.ascontiguousarray(norms).view(np.int32)).to(device))


def oracle_codes(idx, sign, norms):
    return oq.Codes(idx, sign, np.asarray(norms, np.uint32))


def rel_err_rows(got, want):
    """max_n |got - want| / max_n |want| per row of the last axis (want in fp64)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.max(np.abs(got - want), axis=-1)
    den = np.maximum(np.max(np.abs(want), axis=-1), 1e-30)
    return num / den


def say(*a):
    print("[gpu-test]", *a, flush=True)


def sampled_heads(w, n_rows, seed):
    """About n_rows (sequence, query head) rows of a workload, spread over its layers, batches and
    kv heads: [(kv block, [query heads of that block])], two heads per sampled block, the first and
    last blocks always included."""
    g = np.random.default_rng(seed)
    n_blk = w.n_seq * w.hkv
    k = max(2, (n_rows + 1) // 2)
    blks = np.unique(np.concatenate([[0, n_blk - 1], g.choice(n_blk, size=min(n_blk, k) - 2, replace=False)]))
    out = []
    for b in blks:
        kvh = int(b % w.hkv)
        hs = sorted(set(int(kvh * w.group + x) for x in g.choice(w.group, size=min(2, w.group), replace=False)))
        out.append((int(b), hs))
    return out
