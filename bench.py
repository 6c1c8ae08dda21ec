"""Benchmark of the compressed-KV decode path on one MI355X.

Workload (default): 8B-class GQA decode step -- 32 layers, 32 query / 8 KV heads, d = 128,
batch 8, 32768 cached tokens; keys 2-bit index + 1-bit QJL (m = 128), values 3-bit index.
The cache is encoded once from seeded bf16 K/V (bulk encode, timed on its own); a timed step
is one decode step over the resident compressed cache for all layers: the score stream
(tq_scores, the headline) followed by attention (tq_attend_decode).

Prints one JSON line.  value = decode-scoring GB/s: algorithmic bytes of one tq_scores call
(the key code planes, unpadded, + the fp32 logits written + the queries read) divided by the
call's median duration measured with HIP events on the launch stream.  The same line carries the
other workloads under "configs" (the tiny case, the ESM-2-shaped cache, the 131072-token
sequence and the 1M-vector search), each timed by its own medians in the same run.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
SCORE_SOURCES = ("vector_quantization_amd/csrc/tq_scores.hip", "vector_quantization_amd/csrc/tq_lut.h",
                 "vector_quantization_amd/csrc/tq_qprep.h", "vector_quantization_amd/csrc/tq_planes.h",
                 "vector_quantization_amd/csrc/tq_device.h", "vector_quantization_amd/csrc/tq_internal.h",
                 "include/tq.h")
SCORE_KERNELS = ("tq::score_kernel<128, 2, 128, 4, 1024>",)
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "score_kernel_gqa8b_decode_b8_32k_traffic.txt")
METRIC = "compressed-KV decode scoring GB/s (% HBM peak) + keys/s; encode vectors/s"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["gqa", "long", "search", "esm2", "decode_step", "polar"], default="gqa",
                    help="gqa (default, the headline line), long (single 131072-token sequence), "
                         "search (1M x d=200 database, 10k queries: pairs/s and recall), "
                         "esm2 (33 layers x 20 heads x 1024 tokens, d=64, per-head rotations), "
                         "decode_step (the gqa cache growing: append one token per sequence, then attend), "
                         "polar (the gqa keys under the recursive polar stage, 2 angle bits: 52 B per key)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attend", action="store_true")
    ap.add_argument("--encode-reps", type=int, default=3)
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for hardware byte counters)")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload only: skip the other workloads' sub-objects (profiling runs)")
    return ap.parse_args()


def score_source_hash():
    """sha256 over the sources the score stream is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in SCORE_SOURCES:
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel_names):
    """HBM bytes per tq_scores call from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by the copy calibration), or None when the kernels have changed since
    the counters were taken."""
    try:
        lines = open(TRAFFIC_PROFILE).read().splitlines()
    except OSError:
        return None
    vals, src = {}, None
    for ln in lines:
        if ln.startswith("source_sha256:"):
            src = ln.split(":", 1)[1].strip()
        elif ln.startswith("traffic_bytes_per_launch["):
            k, v = ln[len("traffic_bytes_per_launch["):].split("]:", 1)
            vals[k] = float(v)
    if src != score_source_hash() or not all(k in vals for k in kernel_names):
        return None
    return sum(vals[k] for k in kernel_names)


ENCODE_SOURCES = ("vector_quantization_amd/csrc/tq_encode.hip", "vector_quantization_amd/csrc/tq_device.h")
ENCODE_PROFILE = os.path.join(ROOT, "profiles", "encode_mfma_gqa8b_decode_b8_32k_counters.txt")
BF16_PEAK_TFLOPS = 2500.0


def source_hash(names):
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def encode_counters():
    """MFMA busy fractions of the two encode launches of the decode workload from the committed
    counter summary (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs), or None when
    the encoder's sources have changed since the counters were taken."""
    try:
        lines = open(ENCODE_PROFILE).read().splitlines()
    except OSError:
        return None
    vals, src = {}, None
    for ln in lines:
        if ln.startswith("source_sha256:"):
            src = ln.split(":", 1)[1].strip()
        elif ln.startswith("mfma_busy_frac["):
            k, v = ln[len("mfma_busy_frac["):].split("]:", 1)
            vals[k] = float(v)
    if src != source_hash(ENCODE_SOURCES) or not vals:
        return None
    return vals


def gpu_clocks():
    """Current clocks as rocm-smi reports them (sclk, mclk, fclk ...) for GPU 0, or None."""
    import subprocess

    # under a profiler every child process is instrumented too; rocm-smi (a script that starts
    # its interpreter through env) is then better left out
    if any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
        card = next(iter(sorted(k for k in data if k.startswith("card"))))
        return {k: v for k, v in data[card].items() if "clock" in k.lower() or "clk" in k.lower()}
    except Exception:
        return None


def hbm_ceiling(dev):
    """Practical HBM ceilings on this part, measured in the same run with plain torch kernels
    (no code of this library): a read-only stream (row sums over 4 GiB) and a device copy (2 GiB
    read + 2 GiB written), best of three each."""
    import torch

    x = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    t_read = best(lambda: x.view(-1, 4096).sum(1))  # row sums: the fastest torch read stream here
    t_copy = best(lambda: y.copy_(x[: 1 << 29]))
    # three read streams and one write stream of 768 MiB each: the 3.3 : 1 read : write mix of the
    # score stream (52 B of codes read and 16 B of logits written per key) is closest to this
    n = 3 << 26
    a3, b3, c3 = x[:n], x[n:2 * n], x[2 * n:3 * n]
    d3 = torch.empty(n, dtype=torch.float32, device=dev)
    t_mix = best(lambda: torch.addcmul(a3, b3, c3, out=d3))
    res = {"read_stream_GBps": round(x.numel() * 4 / (t_read * 1e-3) / 1e9, 1),
           "copy_GBps": round(2 * y.numel() * 4 / (t_copy * 1e-3) / 1e9, 1),
           "mixed_3r1w_GBps": round(4 * n * 4 / (t_mix * 1e-3) / 1e9, 1),
           "kernels": "torch row sums over 4 GiB fp32 (rows of 4096); torch copy of 2 GiB; torch addcmul "
                      "(3 x 768 MiB read, 768 MiB written)"}
    del x, y, d3
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, K, q, seed_rot, seed_sk, V=None):
    """Time the oracle's encode and scoring of four (layer, batch) slices -- layers {0, L-1} x
    batches {0, B-1}, all kv heads, full context -- on the host cores; with V, also the oracle's
    attention over the first slice (its values encoded by the oracle as well)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import codec as oc
    from oracle import estimate as oe
    from oracle import quantize as oq

    ora = oc.make_codec(w.d, w.k_bits, w.k_m, seed_rot, seed_sk)
    slices = sorted({(0, 0), (0, w.batch - 1), (w.layers - 1, 0), (w.layers - 1, w.batch - 1)})
    t_enc = t_sc = 0.0
    for l, b in slices:
        kx = K[l, b].float().cpu().numpy().reshape(-1, w.d)  # [hkv * n_ctx, d]
        qx = q[l, b].cpu().numpy().astype(np.float64)  # [hq, d]
        t0 = time.perf_counter()
        codes = oq.encode(kx, ora)
        t_enc += time.perf_counter() - t0
        t0 = time.perf_counter()
        for h in range(w.hq):
            kvh = h // w.group
            sl = slice(kvh * w.n_ctx, (kvh + 1) * w.n_ctx)
            oe.scores_one(qx[h], oq.Codes(codes.idx[sl], codes.sign[sl], codes.norms[sl]), ora)
        t_sc += time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    keys = len(slices) * w.hkv * w.n_ctx
    code_b = (w.d * w.k_bits + 7) // 8 + (w.k_m + 7) // 8 + 4
    res = {
        "value": keys / t_sc, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"(layer, batch) in {slices}: {w.hkv} kv heads x {w.n_ctx} keys each, scored for {w.hq} query "
                   f"heads ({t_sc:.1f} s); oracle encode of the same {keys} keys took {t_enc:.1f} s "
                   f"({keys / t_enc:.3g} vectors/s)"),
        "GBps": keys * (code_b + 4 * w.group) / t_sc / 1e9,
        "encode_vectors_per_s": keys / t_enc,
        "affinity_cores": len(os.sched_getaffinity(0)),
    }
    if V is not None:
        import synth

        vora = oc.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
        kx = K[0, 0].float().cpu().numpy().reshape(-1, w.d)
        vx = V[0, 0].float().cpu().numpy().reshape(-1, w.d)
        kcodes, vcodes = oq.encode(kx, ora), oq.encode(vx, vora)
        qx = q[0, 0].cpu().numpy().astype(np.float64)[None]  # [1, hq, d]
        t0 = time.perf_counter()
        oe.attend(qx, kcodes, vcodes, ora, vora, w.n_ctx, w.hkv, 1.0 / math.sqrt(w.d))
        t_at = time.perf_counter() - t0
        res["attend_tokens_per_s"] = w.hkv * w.n_ctx / t_at
        res["attend_sample"] = (f"(layer, batch) (0, 0): {w.hq} query heads over {w.hkv} kv heads x {w.n_ctx} "
                                f"tokens ({t_at:.1f} s)")
    return res


INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix peak
CLOCK_HZ = 2.4e9
N_CU = 256


def search_main(a):
    """Top-10 inner-product search over 1M encoded d=200 vectors for 10k queries."""
    print(json.dumps(search_line(a)), flush=True)


def search_line(a, cpu=None):
    """The search workload's line (dict); cpu: run the oracle leg (default: unless
    --no-cpu-baseline)."""
    import numpy as np
    import torch

    import synth
    import vector_quantization_amd as tq

    k = 10
    log("search data (1M x 200 mixture, 10k queries)")
    db_np, q_np = synth.search_data()
    db = torch.from_numpy(db_np).cuda()
    qs = torch.from_numpy(q_np).cuda()
    c = tq.make_codec(synth.SEARCH_D, synth.SEARCH_BITS, synth.SEARCH_M, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    codes = tq.encode(c, db)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    tq.encode(c, db, out=codes)
    ev[1].record()
    torch.cuda.synchronize()
    t_enc = ev[0].elapsed_time(ev[1])
    # exact fp32 top-k (ground truth), chunked over queries
    truth = torch.empty((qs.shape[0], k), dtype=torch.int64, device="cuda")
    for q0 in range(0, qs.shape[0], 512):
        truth[q0:q0 + 512] = torch.topk(qs[q0:q0 + 512] @ db.T, k, dim=1).indices
    for _ in range(a.warmup):
        idx, _ = tq.search_topk(c, qs, codes, db.shape[0], k)
    torch.cuda.synchronize()
    # each timed call starts with the database out of the 256 MB MALL: a 512 MB buffer is written
    # before it (outside the timed region)
    flush = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    times = []
    for _ in range(a.steps):
        flush.fill_(1.0)
        ev[0].record()
        idx, _ = tq.search_topk(c, qs, codes, db.shape[0], k)
        ev[1].record()
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_time(ev[1]))
    t = float(np.median(times))
    found = idx.cpu().numpy()
    tr = truth.cpu().numpy()
    recall = float(np.mean([len(set(f) & set(g)) / k for f, g in zip(found, tr)]))
    one_at = float(np.mean([g[0] in set(f) for f, g in zip(found, tr)]))
    pairs = qs.shape[0] * db.shape[0]
    pairs_s = pairs / (t * 1e-3)
    # from 32 queries on the scan runs on the matrix cores as int8 products over bit planes; its
    # algorithmic work is the estimator's d + m multiply-adds per pair (2 ops each), priced
    # against the int8 dense peak; the time is the whole search (query prep, scan, merge)
    ops_s = pairs * 2 * (synth.SEARCH_D + synth.SEARCH_M) / (t * 1e-3)
    res = {
        "metric": "compressed search: query-vector pairs/s (top-10 by estimated inner product); recall@10",
        "value": pairs_s, "unit": "pairs/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(t, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic (1000-component Gaussian mixture, unit-normalised, d=200)",
        "config": {"workload": f"search: {db.shape[0]} x d={synth.SEARCH_D} database, {qs.shape[0]} queries, "
                               f"{synth.SEARCH_BITS}-bit + QJL m={synth.SEARCH_M}, top-{k}",
                   "n_db": db.shape[0], "n_q": qs.shape[0], "k": k},
        "recall_at_10": recall, "one_at_10": one_at,
        "encode_ms": round(t_enc, 3), "encode_vectors_per_s": db.shape[0] / (t_enc * 1e-3),
        "roofline": {"bound": "mfma", "achieved": round(ops_s / 1e12, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(ops_s / 1e12 / INT8_PEAK_TOPS, 4), "traffic": None,
                     "kernel": "tq::search_planes (v_mfma_i32_16x16x64_i8 over index/sign bit planes, "
                               "two int8 query limbs, 64 queries per workgroup)"},
        "gpu": torch.cuda.get_device_name(0), "clocks": gpu_clocks(),
    }
    if cpu if cpu is not None else not a.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import codec as oc
        from oracle import estimate as oe
        from oracle import quantize as oq
        nq = 4
        ora = oc.make_codec(synth.SEARCH_D, synth.SEARCH_BITS, synth.SEARCH_M, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
        ocodes = oq.encode(db_np, ora)
        t0 = time.perf_counter()
        oe.search_topk(q_np[:nq], ocodes, ora, k)
        tc = time.perf_counter() - t0
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": nq * db.shape[0] / tc, "unit": "pairs/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"{nq} queries against the full {db.shape[0]}-row database ({tc:.1f} s)"}
    del db, qs, codes, truth, flush
    torch.cuda.empty_cache()
    return res


def decode_step_main(a):
    """The 8B-class decode cache (capacity 32768 per sequence and kv head) growing by one token
    per step: tq_decode_step appends each sequence's new K (RoPE) and V at the next position and
    attends over the cache up to it.  The prefix is encoded once; the steps fill the last slots."""
    import numpy as np
    import torch

    import synth
    import vector_quantization_amd as tq

    w = synth.GQA_DECODE
    dev = "cuda"
    torch.cuda.init()
    log("decode step", w)
    K, V, _ = synth.gqa_decode(w, seed=2, device=dev)
    kc = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vc = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    cap = w.n_ctx
    kcodes = tq.encode(kc, K.reshape(-1, w.d))
    vcodes = tq.encode(vc, V.reshape(-1, w.d))
    del K, V
    torch.cuda.empty_cache()
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    n = a.warmup + a.steps
    qs = torch.randn((n, w.n_seq, w.hq, w.d), generator=gen, device=dev)
    kn = torch.randn((n, w.n_seq, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((n, w.n_seq, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    pos = [torch.full((w.n_seq,), cap - n + i, dtype=torch.int32, device=dev) for i in range(n)]
    out = torch.empty((w.n_seq, w.hq, w.d), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(w.d)
    base = 10000.0
    step = lambda i: tq.decode_step(kc, vc, qs[i], kn[i], vn[i], pos[i], cap, base, kcodes, vcodes, scale, out=out)
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for j in range(a.steps):
        ev[j][0].record()
        step(a.warmup + j)
        ev[j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    # the appends alone (the same two encode launches the step makes), over the last slots again
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record()
    for j in range(a.steps):
        i = a.warmup + j
        tq.append(kc, kn[i], pos[i], cap, base, kcodes)
        tq.append(vc, vn[i], pos[i], cap, 0.0, vcodes)
    eb.record()
    torch.cuda.synchronize()
    t_app = ea.elapsed_time(eb) / a.steps
    mid = cap - n + a.warmup + a.steps // 2  # tokens attended at the middle step: 0 .. mid
    code_b_k = (w.d * w.k_bits + 7) // 8 + (w.k_m + 7) // 8 + 4
    code_b_v = (w.d * w.v_bits + 7) // 8 + (w.v_m + 7) // 8 + 4
    step_bytes = (w.n_seq * w.hkv * (mid + 1) * (code_b_k + code_b_v) + 2 * w.n_seq * w.hq * w.d * 4
                  + 2 * w.n_seq * w.hkv * w.d * 2)
    res = {
        "metric": "decode step over a growing compressed cache: tokens/s (append K/V with RoPE + attention)",
        "value": w.n_seq / (t_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(wall * 1e3 / a.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (the gqa cache encoded from seeded bf16 K/V; new K/V bf16 N(0,1); fp32 queries)",
        "config": {"workload": f"decode_step_{w.name}: {w.n_seq} sequences (32 layers x batch 8) x {w.hkv} kv heads, "
                               f"{w.hq} q heads, d={w.d}, capacity {cap}, positions {cap - n}..{cap - 1}, "
                               f"RoPE base {base:g}",
                   "layers": w.layers, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "head_dim": w.d, "capacity": cap},
        "step_ms": round(t_step, 4), "append_us": round(t_app * 1e3, 2),
        "step_GBps": round(step_bytes / (t_step * 1e-3) / 1e9, 1), "step_algorithmic_bytes": step_bytes,
        "gpu": torch.cuda.get_device_name(0), "clocks": gpu_clocks(),
    }
    print(json.dumps(res), flush=True)


def esm2_main(a):
    """ESM-2-650M-shaped cache: encode of all K/V (fp16, per-(layer, head) rotations), one decode
    query per (layer, head) scored and attended over the 1024 cached tokens, and all-pairs scoring
    (every token against every cached key of its (layer, head))."""
    print(json.dumps(esm2_line(a)), flush=True)


def esm2_line(a):
    import numpy as np
    import torch

    import synth
    import vector_quantization_amd as tq

    w = synth.ESM2
    log("esm2 data", w)
    K, V, q = synth.esm2(layers=w.layers, heads=w.hkv, seq=w.n_ctx, d=w.d)
    seeds = [synth.esm2_basis_seed(l, h) for l in range(w.layers) for h in range(w.hkv)]
    kc = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K, basis_seeds=seeds,
                       vecs_per_rot=w.n_ctx)
    vc = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V, basis_seeds=seeds,
                       vecs_per_rot=w.n_ctx)
    Kd = torch.from_numpy(K.reshape(-1, w.d)).cuda()
    Vd = torch.from_numpy(V.reshape(-1, w.d)).cuda()
    qd = torch.from_numpy(q.reshape(w.n_seq, w.hq, w.d).astype(np.float32)).cuda()
    n_vec = Kd.shape[0]
    kcodes, vcodes = tq.alloc_codes(kc, n_vec), tq.alloc_codes(vc, n_vec)
    logits = torch.empty((w.n_seq, w.hq, w.n_ctx), dtype=torch.float32, device="cuda")
    out = torch.empty((w.n_seq, w.hq, w.d), dtype=torch.float32, device="cuda")
    flush = torch.empty(1 << 27, dtype=torch.float32, device="cuda")  # 512 MB: evicts the 256 MB MALL
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            flush.fill_(1.0)
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ts))

    enc = lambda: (tq.encode(kc, Kd, out=kcodes), tq.encode(vc, Vd, out=vcodes))
    sco = lambda: tq.scores(kc, qd, kcodes, w.n_ctx, w.hkv, logits=logits)
    att = lambda: tq.attend_decode(kc, vc, qd, kcodes, vcodes, w.n_ctx, w.hkv, 1.0 / math.sqrt(w.d), out=out)
    # all pairs: every token of the sequence queries every cached key of its (layer, head) -- 1024
    # query heads per kv head, the matrix-core path of tq_scores (queries: the keys plus noise)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(41)
    qa = (Kd.view(w.layers, w.hkv, w.n_ctx, w.d).float()
          + 0.1 * torch.randn((w.layers, w.hkv, w.n_ctx, w.d), generator=gq, device="cuda"))
    qa = qa.reshape(w.layers, w.hkv * w.n_ctx, w.d).contiguous()
    logits_all = torch.empty((w.layers, w.hkv * w.n_ctx, w.n_ctx), dtype=torch.float32, device="cuda")
    allp = lambda: tq.scores(kc, qa, kcodes, w.n_ctx, w.hkv, logits=logits_all)
    for _ in range(a.warmup):
        enc(); sco(); att(); allp()
    torch.cuda.synchronize()
    t_enc = timed(enc, a.steps)
    t_sc = timed(sco, a.steps)
    t_at = timed(att, a.steps)
    t_all = timed(allp, a.steps)
    pairs_all = w.layers * w.hkv * w.n_ctx * w.n_ctx

    # TurboESM variant (TurboESM summary, sections 2.C and 2.D): K and V tables calibrated by the
    # library on the cache's own rotated directions (every 16th vector), one residual sign per
    # coordinate (S = I, m = d) and x~ = x^ + sign * e; same bits per vector as the codec above
    def turbo(base, X, codes):
        ytap = torch.empty((X.shape[0], w.d), dtype=torch.float32, device="cuda")
        tq.encode(base, X, out=codes, y_tap=ytap)
        u = (ytap / X.float().norm(dim=1, keepdim=True))[::16].cpu().numpy()
        c, t, _, rs = tq.calibrate_codebook(u, base.centroids.cpu().numpy(), m=w.d)
        return tq.codec_from_arrays(w.d, base.bits, w.d, base.rot.cpu().numpy(), np.eye(w.d, dtype=np.float32), c, t,
                                    vecs_per_rot=w.n_ctx, resid_scale=rs)
    tkc, tvc = turbo(kc, Kd, kcodes), turbo(vc, Vd, vcodes)
    tkcodes, tvcodes = tq.alloc_codes(tkc, n_vec), tq.alloc_codes(tvc, n_vec)
    tout = torch.empty_like(out)
    t_enc_t = timed(lambda: (tq.encode(tkc, Kd, out=tkcodes), tq.encode(tvc, Vd, out=tvcodes)), a.steps)
    t_at_t = timed(lambda: tq.attend_decode(tkc, tvc, qd, tkcodes, tvcodes, w.n_ctx, w.hkv, 1.0 / math.sqrt(w.d),
                                            out=tout), a.steps)
    enc(); att()
    torch.cuda.synchronize()
    # decode-step attention against the exact fp32 attention over the uncompressed cache
    Kf = Kd.float().view(w.layers, w.hkv, w.n_ctx, w.d)
    Vf = Vd.float().view(w.layers, w.hkv, w.n_ctx, w.d)
    qf = qd.view(w.layers, w.hkv, w.d, 1)
    p_ex = torch.softmax(torch.matmul(Kf, qf).squeeze(-1) / math.sqrt(w.d), dim=-1)
    o_ex = torch.matmul(p_ex.unsqueeze(-2), Vf).squeeze(-2)
    cos = lambda o: float(torch.nn.functional.cosine_similarity(o.view(w.layers, w.hkv, w.d), o_ex, dim=-1).mean())
    code_b = (w.d * w.k_bits + 7) // 8 + (w.k_m + 7) // 8 + 4
    sc_bytes = n_vec * code_b + w.n_seq * w.hq * w.n_ctx * 4 + w.n_seq * w.hq * w.d * 4
    res = {
        "metric": "ESM-2-shaped cache: encode vectors/s; full-prefix scoring and attention time (cold MALL)",
        "value": 2 * n_vec / (t_enc * 1e-3), "unit": "vectors/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(t_enc + t_sc + t_at, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (20-prototype vocabulary + noise, 4 spiked channels per head, RoPE on K; fp16)",
        "config": {"workload": f"{w.name}: {w.layers} layers x {w.hkv} heads x {w.n_ctx} tokens, d={w.d}, "
                               f"{w.k_bits}-bit + QJL m={w.k_m} for K and V, per-(layer, head) rotations",
                   "layers": w.layers, "heads": w.hkv, "n_ctx": w.n_ctx, "head_dim": w.d},
        "encode_ms": round(t_enc, 4), "scores_us": round(t_sc * 1e3, 2), "attend_us": round(t_at * 1e3, 2),
        "scores_GBps": round(sc_bytes / (t_sc * 1e-3) / 1e9, 1),
        "allpairs_ms": round(t_all, 4), "allpairs_pairs_per_s": pairs_all / (t_all * 1e-3),
        "allpairs_logits_GBps": round(pairs_all * 4 / (t_all * 1e-3) / 1e9, 1),
        "attend_cos_vs_exact": round(cos(out), 5),
        "turboesm": {"encode_ms": round(t_enc_t, 4), "attend_us": round(t_at_t * 1e3, 2),
                     "attend_cos_vs_exact": round(cos(tout), 5),
                     "codec": "K and V tables calibrated on the cache (library Lloyd on rotated directions), "
                              "3-bit index + one residual sign per coordinate"},
        "cache_bytes": 2 * n_vec * code_b,
        "gpu": torch.cuda.get_device_name(0), "clocks": gpu_clocks(),
    }
    del Kd, Vd, kcodes, vcodes, tkcodes, tvcodes, logits_all, qa, flush
    torch.cuda.empty_cache()
    return res


def polar_main(a):
    """The 8B-class key cache (32 layers x batch 8 x 8 kv heads x 32768 tokens, d = 128) under the
    recursive polar stage with 2 angle bits per node: 48 B of bitstream + 4 B norm per key, the
    size of the 2-bit + QJL record.  Timed: tq_polar_scores over every layer (the score stream);
    the bulk encode on its own.  Quality on layer 0, batch 0 against exact fp32 logits, beside
    the two-stage codec at the same record size (and both at 68 B: 3 angle bits / 3-bit + QJL)."""
    import numpy as np
    import torch

    import synth
    import vector_quantization_amd as tq

    w = synth.GQA_DECODE
    ab = 2
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    log("workload", w, "polar ab", ab)
    K, V, q = synth.gqa_decode(w, seed=2, device="cuda")
    # values: the decode workload's 3-bit two-stage codec, for attention with polar keys
    vc = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    vcodes = tq.encode(vc, V.reshape(-1, w.d))
    v0 = V[0, 0].float()  # layer 0, batch 0 for the quality comparison
    del V
    pc = tq.make_polar_codec(w.d, ab, synth.SEED_ROT_K)
    n_vec = w.n_seq * w.hkv * w.n_ctx
    codes = tq.alloc_polar_codes(pc, n_vec)
    Kf = K.reshape(-1, w.d)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    tq.polar_encode(pc, Kf, out=codes)
    torch.cuda.synchronize()
    enc = []
    for _ in range(a.encode_reps):
        ev[0].record(stream)
        tq.polar_encode(pc, Kf, out=codes)
        ev[1].record(stream)
        torch.cuda.synchronize()
        enc.append(ev[0].elapsed_time(ev[1]))
    t_enc = float(np.median(enc))
    log(f"polar encode {t_enc:.2f} ms")
    qf = q.reshape(w.n_seq, w.hq, w.d).contiguous()
    logits = torch.empty((w.n_seq, w.hq, w.n_ctx), dtype=torch.float32, device="cuda")
    for _ in range(a.warmup):
        tq.polar_scores(pc, qf, codes, w.n_ctx, w.hkv, logits=logits)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        tq.polar_scores(pc, qf, codes, w.n_ctx, w.hkv, logits=logits)
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_sc = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    # attention: polar-key logits, then the online softmax and value pass over the 3-bit values
    scale = 1.0 / math.sqrt(w.d)
    aout = torch.empty((w.n_seq, w.hq, w.d), dtype=torch.float32, device="cuda")
    for _ in range(a.warmup):
        tq.polar_attend_decode(pc, vc, qf, codes, vcodes, w.n_ctx, w.hkv, scale, out=aout)
    torch.cuda.synchronize()
    aev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
    for e in aev:
        e[0].record(stream)
        tq.polar_attend_decode(pc, vc, qf, codes, vcodes, w.n_ctx, w.hkv, scale, out=aout)
        e[1].record(stream)
    torch.cuda.synchronize()
    t_att = float(np.mean([e[0].elapsed_time(e[1]) for e in aev]))
    rec_b = tq.polar_record_bytes(w.d, ab) + 4
    keys = n_vec
    q_bytes = w.n_seq * w.hq * w.d * 4
    score_bytes = keys * rec_b + w.n_seq * w.hq * w.n_ctx * 4 + q_bytes
    gbps = score_bytes / (t_sc * 1e-3) / 1e9

    # quality on layer 0, batch 0 (8 kv heads x 32768 keys, 32 query heads) vs exact fp32 logits
    k0 = K[0, 0].float()                                   # [hkv, n_ctx, d]
    q0 = q[0, 0].float()                                   # [hq, d]
    exact = torch.matmul(q0.view(w.hkv, w.group, w.d), k0.transpose(1, 2).contiguous()).reshape(1, w.hq, w.n_ctx)
    qs0 = q0.view(1, w.hq, w.d).contiguous()

    def quality(est):
        est = est.reshape(w.hq, w.n_ctx).double()
        ex = exact.reshape(w.hq, w.n_ctx).double()
        cos = torch.nn.functional.cosine_similarity(est, ex, dim=1).mean().item()
        rel = (torch.linalg.norm(est - ex, dim=1) / torch.linalg.norm(ex, dim=1)).mean().item()
        return {"logit_cos_vs_exact": round(cos, 5), "logit_rel_l2_err": round(rel, 5)}

    # exact fp32 attention on the slice, against which both key codecs' outputs are compared (the
    # values through the same 3-bit codec in both)
    p_ex = torch.softmax(exact.view(w.hkv, w.group, w.n_ctx) * scale, dim=-1)
    o_ex = torch.matmul(p_ex, v0).reshape(w.hq, w.d)
    vslice = vcodes.slice(0, w.hkv * w.n_ctx)

    def out_cos(o):
        return round(torch.nn.functional.cosine_similarity(o.reshape(w.hq, w.d).double(), o_ex.double(),
                                                           dim=1).mean().item(), 5)

    comp = {}
    for bits_, abits in ((2, 2), (3, 3)):
        pcb = tq.make_polar_codec(w.d, abits, synth.SEED_ROT_K)
        pcodes = tq.polar_encode(pcb, k0.reshape(-1, w.d))
        pq = quality(tq.polar_scores(pcb, qs0, pcodes, w.n_ctx, w.hkv))
        kc = tq.make_codec(w.d, bits_, w.d, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
        tcodes = tq.encode(kc, k0.reshape(-1, w.d))
        tqq = quality(tq.scores(kc, qs0, tcodes, w.n_ctx, w.hkv))
        if bits_ == w.k_bits:  # attention at the workload's own key size (52 B), 3-bit values for both
            pq["attention_cos_vs_exact"] = out_cos(tq.polar_attend_decode(pcb, vc, qs0, pcodes, vslice, w.n_ctx,
                                                                          w.hkv, scale))
            tqq["attention_cos_vs_exact"] = out_cos(tq.attend_decode(kc, vc, qs0, tcodes, vslice, w.n_ctx, w.hkv,
                                                                     scale))
        comp[f"{tq.polar_record_bytes(w.d, abits) + 4}B_per_key"] = {
            f"polar_ab{abits}": pq, f"two_stage_{bits_}bit_qjl{w.d}": tqq}
    # the QJL stage on the polar residual (m = d, 48 + 16 + 4 = 68 B per key) over every layer:
    # the residual stage runs in the one-wavefront-per-vector encoder (timed once)
    pcq = tq.make_polar_codec(w.d, ab, synth.SEED_ROT_K, m=w.d, sketch_seed=synth.SEED_SKETCH_K)
    n0 = w.batch * w.hkv * w.n_ctx
    k_l0 = K[0].reshape(-1, w.d)
    qcodes = tq.alloc_polar_codes(pcq, n_vec)
    tq.polar_encode(pcq, k_l0, out=qcodes.slice(0, n0))
    torch.cuda.synchronize()
    ev[0].record(stream)
    tq.polar_encode(pcq, Kf, out=qcodes)
    ev[1].record(stream)
    torch.cuda.synchronize()
    t_qenc = ev[0].elapsed_time(ev[1])
    qt = []
    for i in range(a.warmup + a.steps):
        ev[0].record(stream)
        tq.polar_scores(pcq, qf, qcodes, w.n_ctx, w.hkv, logits=logits)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= a.warmup:
            qt.append(ev[0].elapsed_time(ev[1]))
    t_qsc = float(np.median(qt))
    qrec_b = tq.polar_record_bytes(w.d, ab) + w.d // 8 + 4
    q_score_bytes = keys * qrec_b + w.n_seq * w.hq * w.n_ctx * 4 + q_bytes
    qjl_line = {"record_bytes": qrec_b, "encode_ms": round(t_qenc, 2),
                "encode_vectors_per_s": round(n_vec / (t_qenc * 1e-3)),
                "scores_ms": round(t_qsc, 4), "scores_GBps": round(q_score_bytes / (t_qsc * 1e-3) / 1e9, 1),
                "scores_hbm_frac": round(q_score_bytes / (t_qsc * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "keys_per_s": keys / (t_qsc * 1e-3)}
    # search over polar records: the layer-0 keys (2.1M, d = 128) as a database, 1024 queries,
    # top-10, recall@10 against exact fp32 search
    n_qs = 1024
    gq = torch.Generator(device="cuda")
    gq.manual_seed(41)
    qs = torch.randn((n_qs, w.d), generator=gq, device="cuda")
    db = codes.slice(0, n0)
    tq.polar_search_topk(pc, qs, db, n0, 10)
    torch.cuda.synchronize()
    st_ = []
    for _ in range(3):
        ev[0].record(stream)
        idx, _sc = tq.polar_search_topk(pc, qs, db, n0, 10)
        ev[1].record(stream)
        torch.cuda.synchronize()
        st_.append(ev[0].elapsed_time(ev[1]))
    t_srch = float(np.median(st_))
    exact_top = torch.topk(qs @ k_l0.float().T, 10, dim=1).indices
    rec10 = float(np.mean([len(set(a_.tolist()) & set(b_.tolist())) / 10.0
                           for a_, b_ in zip(idx.cpu(), exact_top.cpu())]))
    search_line_p = {"database": f"layer-0 keys, {n0} x {w.d}, polar ab = {ab} ({rec_b} B per record)",
                     "queries": n_qs, "k": 10, "ms": round(t_srch, 3),
                     "pairs_per_s": n_qs * n0 / (t_srch * 1e-3), "recall_at_10_vs_exact_fp32": round(rec10, 4)}
    # one decode step over the whole cache: every sequence appends its token at the last slot
    # (polar key with RoPE, 3-bit value), then attends over all 32768 tokens
    gs = torch.Generator(device="cuda")
    gs.manual_seed(31)
    k_new = torch.randn((w.n_seq, w.hkv, w.d), generator=gs, device="cuda", dtype=torch.bfloat16)
    v_new = torch.randn((w.n_seq, w.hkv, w.d), generator=gs, device="cuda", dtype=torch.bfloat16)
    pos_t = torch.full((w.n_seq,), w.n_ctx - 1, dtype=torch.int32, device="cuda")
    st_out = torch.empty((w.n_seq, w.hq, w.d), dtype=torch.float32, device="cuda")
    dsteps = []
    for i in range(a.warmup + a.steps):
        ev[0].record(stream)
        tq.polar_decode_step(pc, vc, qf, k_new, v_new, pos_t, w.n_ctx, 10000.0, codes, vcodes, scale, out=st_out)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= a.warmup:
            dsteps.append(ev[0].elapsed_time(ev[1]))
    t_step = float(np.median(dsteps))
    step_line = {"ms": round(t_step, 4), "tokens_per_s": round(w.n_seq / (t_step * 1e-3)),
                 "note": f"{w.n_seq} sequences x {w.hkv} kv heads append one token at position {w.n_ctx - 1} "
                         f"(polar keys with RoPE, 3-bit values), then attention over {w.n_ctx} tokens"}
    comp.setdefault(f"{qrec_b}B_per_key", {})[f"polar_ab{ab}_qjl{w.d}"] = quality(
        tq.polar_scores(pcq, qs0, qcodes.slice(0, w.hkv * w.n_ctx), w.n_ctx, w.hkv))
    torch.cuda.synchronize()
    res = {
        "metric": "recursive-polar decode scoring GB/s (% HBM peak) + keys/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(wall * 1e3 / a.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded bf16 K, N(0,1) with 2% channels x10; fp32 queries)",
        "config": {"workload": f"polar_{w.name}: {w.layers} layers x batch {w.batch}, {w.hq} q / {w.hkv} kv heads, "
                               f"d={w.d}, {w.n_ctx} cached tokens; K recursive polar, {ab} angle bits per node, "
                               f"{rec_b} B per key",
                   "layers": w.layers, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "head_dim": w.d,
                   "n_ctx": w.n_ctx, "angle_bits": ab},
        "scores_ms": round(t_sc, 4), "keys_per_s": keys / (t_sc * 1e-3),
        "qk_pairs_per_s": keys * w.group / (t_sc * 1e-3), "scores_algorithmic_bytes": score_bytes,
        "encode_ms": round(t_enc, 3), "encode_vectors_per_s": round(n_vec / (t_enc * 1e-3)),
        "attend_ms": round(t_att, 4),
        "attend_note": f"polar keys + {w.v_bits}-bit values: tq_polar_scores into the workspace, then the value pass",
        "quality_layer0_batch0": comp,
        "polar_qjl": qjl_line,
        "polar_search": search_line_p,
        "polar_decode_step": step_line,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": f"tq::polar_score_kernel<{w.d}, {ab}, 4, 256> (one tq_polar_scores call)"},
        "gpu": torch.cuda.get_device_name(0), "clocks": gpu_clocks(),
    }
    if not a.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import polar as op
        ora = op.make_polar_codec(w.d, ab, synth.SEED_ROT_K)
        slices = sorted({(0, 0), (0, w.batch - 1), (w.layers - 1, 0), (w.layers - 1, w.batch - 1)})
        t_oe = tc = 0.0
        for l, b in slices:
            kx = K[l, b].float().reshape(-1, w.d).cpu().numpy()
            t0 = time.perf_counter()
            ocodes = op.encode(kx, ora)
            t_oe += time.perf_counter() - t0
            t0 = time.perf_counter()
            op.scores(q[l, b].float().cpu().numpy()[None], ocodes, ora, w.n_ctx, w.hkv)
            tc += time.perf_counter() - t0
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        nk = len(slices) * w.hkv * w.n_ctx
        res["cpu_baseline"] = {"value": nk / tc, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
                               "sample": (f"(layer, batch) in {slices}: {w.hkv} kv heads x {w.n_ctx} keys each, "
                                          f"scored for {w.hq} query heads ({tc:.1f} s); oracle encode of the same "
                                          f"{nk} keys took {t_oe:.1f} s")}
    print(json.dumps(res), flush=True)


def tiny_line(a):
    """The tiny case (1 head, d = 64, 256 keys and values, 2-bit + QJL m = 64 for both): encode of
    K and V, scores and attention of one query, each the median of a.steps calls (launch-bound)."""
    import numpy as np
    import torch

    import synth
    import vector_quantization_amd as tq

    w = synth.TINY
    K, V, q = synth.tiny()
    kc = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vc = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    Kd, Vd = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    qd = torch.from_numpy(q.reshape(1, 1, -1)).cuda()
    kcodes, vcodes = tq.alloc_codes(kc, w.n_ctx), tq.alloc_codes(vc, w.n_ctx)
    logits = torch.empty((1, 1, w.n_ctx), dtype=torch.float32, device="cuda")
    out = torch.empty((1, 1, w.d), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(w.d)
    calls = {
        "encode_kv": lambda: (tq.encode(kc, Kd, out=kcodes), tq.encode(vc, Vd, out=vcodes)),
        "scores": lambda: tq.scores(kc, qd, kcodes, w.n_ctx, 1, logits=logits),
        "attend": lambda: tq.attend_decode(kc, vc, qd, kcodes, vcodes, w.n_ctx, 1, scale, out=out),
    }
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    res = {"workload": f"tiny: 1 head, d={w.d}, {w.n_ctx} keys and values, 2-bit + QJL m={w.k_m} (K and V), "
                       "1 query", "unit": "us (median per call, HIP events)"}
    for name, fn in calls.items():
        for _ in range(a.warmup):
            fn()
        ts = []
        for _ in range(max(a.steps, 20)):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
        res[f"{name}_us"] = round(float(np.median(ts)), 2)
    res["step_us"] = round(res["encode_kv_us"] + res["scores_us"] + res["attend_us"], 2)
    return res


def kv_line(a, w, seed, cpu):
    """The decode workload w (8B-class GQA, or the 131072-token sequence): bulk encode of the whole
    K/V prefix (timed on its own), then a.steps decode steps over the resident compressed cache --
    tq_scores then tq_attend_decode, each timed by HIP events on the launch stream; medians."""
    import numpy as np
    import torch

    import synth
    import vector_quantization_amd as tq

    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    log("workload", w)
    K, V, q = synth.gqa_decode(w, seed=seed, device=dev)
    kc = tq.make_codec(w.d, w.k_bits, w.k_m, synth.SEED_ROT_K, synth.SEED_SKETCH_K)
    vc = tq.make_codec(w.d, w.v_bits, w.v_m, synth.SEED_ROT_V, synth.SEED_SKETCH_V)
    n_vec = w.n_seq * w.hkv * w.n_ctx
    kcodes = tq.alloc_codes(kc, n_vec)
    vcodes = tq.alloc_codes(vc, n_vec)

    # ---- bulk encode of the whole prefix (K and V), timed on its own
    Kf, Vf = K.reshape(-1, w.d), V.reshape(-1, w.d)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    tq.encode(kc, Kf, out=kcodes)
    tq.encode(vc, Vf, out=vcodes)
    torch.cuda.synchronize()
    enc_k, enc_v = [], []
    for _ in range(a.encode_reps):
        ev[0].record(stream)
        tq.encode(kc, Kf, out=kcodes)
        ev[1].record(stream)
        tq.encode(vc, Vf, out=vcodes)
        ev[2].record(stream)
        torch.cuda.synchronize()
        enc_k.append(ev[0].elapsed_time(ev[1]))
        enc_v.append(ev[1].elapsed_time(ev[2]))
    t_enc_k, t_enc_v = float(np.median(enc_k)), float(np.median(enc_v))
    log(f"encode K {t_enc_k:.2f} ms, V {t_enc_v:.2f} ms")
    qf = q.reshape(w.n_seq, w.hq, w.d).contiguous()
    logits = torch.empty((w.n_seq, w.hq, w.n_ctx), dtype=torch.float32, device=dev)
    out = torch.empty((w.n_seq, w.hq, w.d), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(w.d)
    do_attend = not a.no_attend

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        tq.scores(kc, qf, kcodes, w.n_ctx, w.hkv, logits=logits)
        if evs:
            evs[1].record(stream)
        if do_attend:
            tq.attend_decode(kc, vc, qf, kcodes, vcodes, w.n_ctx, w.hkv, scale, out=out)
        if evs:
            evs[2].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sc_ms = [e[0].elapsed_time(e[1]) for e in evs]
    at_ms = [e[1].elapsed_time(e[2]) for e in evs]
    t_sc = float(np.median(sc_ms))
    t_at = float(np.median(at_ms)) if do_attend else None
    ms_step = wall * 1e3 / a.steps
    twin = score_traffic_twin(w, kc, kcodes, logits, stream, lambda: tq.scores(kc, qf, kcodes, w.n_ctx, w.hkv,
                                                                                 logits=logits))

    keys = w.n_seq * w.hkv * w.n_ctx
    code_b_k = (w.d * w.k_bits + 7) // 8 + (w.k_m + 7) // 8 + 4
    code_b_v = (w.d * w.v_bits + 7) // 8 + (w.v_m + 7) // 8 + 4
    q_bytes = w.n_seq * w.hq * w.d * 4
    score_bytes = keys * code_b_k + w.n_seq * w.hq * w.n_ctx * 4 + q_bytes
    attend_bytes = keys * (code_b_k + code_b_v) + q_bytes + w.n_seq * w.hq * w.d * 4
    gbps = score_bytes / (t_sc * 1e-3) / 1e9
    enc_in = n_vec * w.d * 2
    enc_out_k = n_vec * code_b_k
    enc_out_v = n_vec * code_b_v
    # the encoder's matrix products, algorithmic: y = Pi x (2 d^2 flop per vector) and, for keys,
    # z = S r (2 m d)
    fl_k, fl_v = n_vec * (2 * w.d * w.d + 2 * w.k_m * w.d), n_vec * (2 * w.d * w.d + 2 * w.v_m * w.d)
    res = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": ("fp32 queries and accumulation; with 4 query heads per kv head the lookup entries are "
                       "16-bit fixed point, and a chunk whose error bound is not below 8e-4 of its largest "
                       "|logit| is scored again with fp32 entries"),
        "data": "synthetic (seeded bf16 K/V, N(0,1) with 2% channels x10; fp32 queries)",
        "config": {
            "workload": f"{w.name}: {w.layers} layers x batch {w.batch}, {w.hq} q / {w.hkv} kv heads, d={w.d}, "
                        f"{w.n_ctx} cached tokens; K {w.k_bits}-bit + QJL m={w.k_m}, V {w.v_bits}-bit",
            "layers": w.layers, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "head_dim": w.d, "n_ctx": w.n_ctx,
            "k_bits": w.k_bits, "k_qjl_m": w.k_m, "v_bits": w.v_bits, "v_qjl_m": w.v_m,
        },
        "timing": "medians of the timed steps (HIP events on the launch stream); ms_per_step is wall time",
        "scores_ms": round(t_sc, 4),
        "scores_ms_min_max": [round(min(sc_ms), 4), round(max(sc_ms), 4)],
        "scores_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "keys_per_s": keys / (t_sc * 1e-3),
        "qk_pairs_per_s": keys * w.group / (t_sc * 1e-3),
        "scores_algorithmic_bytes": score_bytes,
        "attend_ms": None if t_at is None else round(t_at, 4),
        "attend_GBps": None if t_at is None else round(attend_bytes / (t_at * 1e-3) / 1e9, 1),
        "attend_hbm_frac": None if t_at is None else round(attend_bytes / (t_at * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "attend_algorithmic_bytes": attend_bytes,
        "encode_ms": {"K": round(t_enc_k, 3), "V": round(t_enc_v, 3)},
        "encode_vectors_per_s": round(2 * n_vec / ((t_enc_k + t_enc_v) * 1e-3)),
        "encode_GBps": round((2 * enc_in + enc_out_k + enc_out_v) / ((t_enc_k + t_enc_v) * 1e-3) / 1e9, 1),
        "encode_mfma": {"K_algorithmic_TFLOPs": round(fl_k / (t_enc_k * 1e-3) / 1e12, 1),
                        "V_algorithmic_TFLOPs": round(fl_v / (t_enc_v * 1e-3) / 1e12, 1),
                        "peak_TFLOPs": BF16_PEAK_TFLOPS,
                        "K_frac_of_bf16_peak": round(fl_k / (t_enc_k * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "busy_frac_counters": encode_counters() if w.name == "gqa8b_decode_b8_32k" else None,
                        "note": "algorithmic flops: y = Pi x (2 d^2) and z = S r (2 m d) per vector; the "
                                "kernel issues them as bf16 hi/lo split products (2 for bf16 input, 3 for "
                                "the sketch).  busy_frac: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x "
                                "1024 SIMDs) from the committed counter summary (null when the encoder "
                                "changed since)"},
        "score_traffic_twin": None if twin is None else {
            "ms": round(twin[0], 4), "scores_ms_same_run": round(twin[1], 4),
            "GBps": round(score_bytes / (twin[0] * 1e-3) / 1e9, 1),
            "scores_frac_of_twin": round(twin[0] / twin[1], 4),
            "kernel": "score_traffic (lib/libtq_traffic.so): the score stream's grid, loads and logit "
                      "stores with no table work",
            "note": "the practical HBM ceiling of the score stream's own access pattern; medians of "
                    "alternating calls"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(SCORE_KERNELS) if w.name == "gqa8b_decode_b8_32k" else None,
                     "kernel": " + ".join(SCORE_KERNELS) + " (one tq_scores call)"},
        "gpu": torch.cuda.get_device_name(0), "clocks": gpu_clocks(),
    }
    host = None
    if cpu:
        # the oracle's inputs on the host before the device memory is released
        sl = sorted({(0, 0), (0, w.batch - 1), (w.layers - 1, 0), (w.layers - 1, w.batch - 1)})
        host = ({k: K[k].cpu() for k in sl}, {(0, 0): V[0, 0].cpu()}, {k: q[k].cpu() for k in sl})
    del K, V, q, kcodes, vcodes, logits, Kf, Vf
    torch.cuda.empty_cache()
    return res, host


def score_traffic_twin(w, kc, kcodes, logits, stream, scores_call, reps=10):
    """Median times of the traffic twin of the score stream and of the score call itself,
    alternating on the same codes and logits (ms, ms); None where the twin does not apply."""
    import ctypes

    import numpy as np
    import torch
    import vector_quantization_amd as tq

    path = os.path.join(os.path.dirname(tq.LIB_PATH), "libtq_traffic.so")
    if not (os.path.exists(path) and kc.d == 128 and kc.bits == 2 and kc.m == 128 and w.hq == 4 * w.hkv):
        return None
    lib = ctypes.CDLL(path)
    lib.tq_traffic_score_twin.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.tq_traffic_score_twin.restype = ctypes.c_int
    st = ctypes.c_void_p(stream.cuda_stream)

    def twin():
        rc = lib.tq_traffic_score_twin(kcodes.idx.data_ptr(), kcodes.idx.shape[1], kcodes.sign.data_ptr(),
                                       kcodes.sign.shape[1], kcodes.norms.data_ptr(), w.n_seq, w.hq, w.hkv,
                                       w.n_ctx, logits.data_ptr(), st)
        if rc != 0:
            raise RuntimeError(f"traffic twin launch: {rc}")

    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tw, sc = [], []
    for i in range(reps + 2):
        e[0].record(stream)
        twin()
        e[1].record(stream)
        scores_call()
        e[2].record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            tw.append(e[0].elapsed_time(e[1]))
            sc.append(e[1].elapsed_time(e[2]))
    return float(np.median(tw)), float(np.median(sc))


class _Slices:
    """K / V / q restricted to the (layer, batch) slices copied to the host; indexed like them."""

    def __init__(self, d):
        self.d = d

    def __getitem__(self, lb):
        return self.d[lb]


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {a.gpus}); the multi-GPU split of this "
              "path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    if a.workload == "search":
        search_main(a)
        return
    if a.workload == "esm2":
        esm2_main(a)
        return
    if a.workload == "decode_step":
        decode_step_main(a)
        return
    if a.workload == "polar":
        polar_main(a)
        return
    import synth

    w = synth.GQA_DECODE if a.workload == "gqa" else synth.LONG_CTX
    cpu = not a.no_cpu_baseline
    res, host = kv_line(a, w, 2 if a.workload == "gqa" else 3, cpu)
    res["hbm_ceiling"] = hbm_ceiling("cuda")
    if a.calibrate:
        import torch

        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst
    if a.workload == "gqa" and not a.no_configs:
        # every other workload under the same clock: the tiny case, the ESM-2-shaped cache, the
        # 131072-token sequence and the 1M-vector search (its oracle leg stays in --workload search)
        cfg = {}
        log("config 1: tiny")
        cfg["1_tiny"] = tiny_line(a)
        log("config 2: esm2")
        e = esm2_line(a)
        cfg["2_esm2"] = {k: e[k] for k in ("config", "encode_ms", "scores_us", "attend_us", "scores_GBps",
                                           "allpairs_ms", "allpairs_pairs_per_s", "attend_cos_vs_exact",
                                           "turboesm", "cache_bytes")}
        cfg["2_esm2"]["encode_vectors_per_s"] = e["value"]
        log("config 4: long context")
        lr, _ = kv_line(a, synth.LONG_CTX, 3, False)
        cfg["4_long"] = {k: lr[k] for k in ("config", "scores_ms", "scores_hbm_frac", "keys_per_s", "attend_ms",
                                            "attend_GBps", "encode_ms", "encode_vectors_per_s")}
        cfg["4_long"]["scores_GBps"] = lr["value"]
        log("config 5: search")
        sr = search_line(a, cpu=False)
        cfg["5_search"] = {k: sr[k] for k in ("config", "ms_per_step", "recall_at_10", "one_at_10", "encode_ms",
                                              "encode_vectors_per_s", "roofline")}
        cfg["5_search"]["pairs_per_s"] = sr["value"]
        res["configs"] = cfg
    if cpu:
        log("cpu baseline (oracle)")
        K, V, q = (_Slices(h) for h in host)
        res["cpu_baseline"] = cpu_baseline(w, K, q, synth.SEED_ROT_K, synth.SEED_SKETCH_K, V=V)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
