"""Build libtq.so for gfx950 in-tree with hipcc (one object per source, compiled in parallel).

Usage: python -m vector_quantization_amd.build [--jobs N] [--verbose]
The library lands in vector_quantization_amd/lib/libtq.so (and bench.py's measurement aid in
lib/libtq_traffic.so).
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libtq.so")
# measurement aid for bench.py (csrc/probe): the score stream's traffic without its arithmetic
TRAFFIC_SRC = os.path.join(CSRC, "probe", "tq_traffic.hip")
TRAFFIC_LIB = os.path.join(OUT_DIR, "libtq_traffic.so")

ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(HERE, "..", "include")]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


# per-source device flags: the bit-plane scans keep their int32 accumulators in VGPRs (no AGPR
# copies in their epilogues)
EXTRA = {"tq_search.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "tq_scores.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + EXTRA.get(src, []) + ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(jobs=None, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    tmp = TRAFFIC_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + DEVICE + ["-shared", "-x", "hip", TRAFFIC_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on the traffic probe:\n" + r.stderr)
    os.replace(tmp, TRAFFIC_LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
