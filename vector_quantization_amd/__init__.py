"""Python binding of libtq (TurboQuant-style compressed-KV attention on MI355X).

Thin ctypes marshalling over the C ABI declared in include/tq.h: every step of encode,
scoring, attention and search runs in the library's HIP kernels.  PyTorch provides device
memory and the stream.  Importing this package loads ``lib/libtq.so`` and fails loudly when
it is missing (build it with ``python -m vector_quantization_amd.build``).
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libtq.so")

TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2
TQ_ENC_PRE_ROTATED = 1
TQ_OP_SCORES, TQ_OP_ATTEND, TQ_OP_SEARCH, TQ_OP_DECODE_STEP = 0, 1, 2, 3


class TQError(RuntimeError):
    pass


class _Codec(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("m", ctypes.c_int32),
                ("n_rot", ctypes.c_int32), ("vecs_per_rot", ctypes.c_int64),
                ("rot", ctypes.c_void_p), ("sketch", ctypes.c_void_p),
                ("centroids", ctypes.c_void_p), ("thresholds", ctypes.c_void_p),
                ("resid_scale", ctypes.c_float)]


class _Codes(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("idx_stride", ctypes.c_int64),
                ("sign", ctypes.c_void_p), ("sign_stride", ctypes.c_int64),
                ("norms", ctypes.c_void_p)]


class _PolarCodec(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("ab", ctypes.c_int32), ("n_rot", ctypes.c_int32),
                ("vecs_per_rot", ctypes.c_int64), ("rot", ctypes.c_void_p), ("tables", ctypes.c_void_p)]


class _PolarCodes(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_void_p), ("stride", ctypes.c_int64), ("norms", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtq.so not built: {LIB_PATH} is missing "
                          "(run `python -m vector_quantization_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    CP = ctypes.POINTER(_Codec)
    PP = ctypes.POINTER(_PolarCodec)
    sig = {
        "tq_make_rotation": ([U64, I32, P], I32),
        "tq_make_head_rotations": ([U64, P, I32, I32, P], I32),
        "tq_make_sketch": ([U64, I32, I32, P], I32),
        "tq_make_codebook": ([I32, I32, P, P], I32),
        "tq_calibrate_codebook": ([P, I64, I32, P, I32, I32, P, P, P, P], I32),
        "tq_encode": ([CP, P, I32, I64, I64, ctypes.c_uint32, I64, _Codes, P, P], I32),
        "tq_scores": ([CP, P, I64, I32, I32, I64, _Codes, P, P, SZ, P], I32),
        "tq_attend_decode": ([CP, CP, P, I64, I32, I32, I64, _Codes, _Codes, ctypes.c_float, P, P, SZ, P], I32),
        "tq_search_topk": ([CP, P, I64, _Codes, I64, I32, P, P, P, SZ, P], I32),
        "tq_append": ([CP, P, I32, I64, I32, P, I64, ctypes.c_float, _Codes, P], I32),
        "tq_decode_step": ([CP, CP, P, P, P, I32, I64, I32, I32, I64, P, ctypes.c_float, _Codes, _Codes,
                            ctypes.c_float, P, P, SZ, P], I32),
        "tq_workspace_bytes": ([ctypes.c_int, CP, CP, I64, I32, I32, I64], SZ),
        "tq_make_polar_tables": ([I32, I32, P], I32),
        "tq_polar_record_bytes": ([I32, I32], SZ),
        "tq_polar_encode": ([PP, P, I32, I64, I64, ctypes.c_uint32, I64, _PolarCodes, P, P], I32),
        "tq_polar_scores": ([PP, P, I64, I32, I32, I64, _PolarCodes, P, P], I32),
        "tq_polar_attend_workspace_bytes": ([PP, CP, I64, I32, I32, I64], SZ),
        "tq_polar_attend_decode": ([PP, CP, P, I64, I32, I32, I64, _PolarCodes, _Codes, ctypes.c_float, P, P, SZ,
                                    P], I32),
        "tq_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "tq_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()
EXPORTED = ("tq_make_rotation", "tq_make_head_rotations", "tq_make_sketch", "tq_make_codebook",
            "tq_calibrate_codebook", "tq_encode",
            "tq_scores", "tq_attend_decode", "tq_append", "tq_decode_step", "tq_search_topk",
            "tq_workspace_bytes", "tq_status_str", "tq_version", "tq_make_polar_tables",
            "tq_polar_record_bytes", "tq_polar_encode", "tq_polar_scores", "tq_polar_attend_workspace_bytes",
            "tq_polar_attend_decode")


def _check(rc):
    if rc != 0:
        raise TQError(f"libtq status {rc}: {lib.tq_status_str(rc).decode()}")


def version() -> str:
    return lib.tq_version().decode()


# ------------------------------------------------------------------ host codec construction


def make_rotation(seed: int, d: int) -> np.ndarray:
    out = np.empty((d, d), np.float32)
    _check(lib.tq_make_rotation(seed, d, out.ctypes.data))
    return out


def make_head_rotations(seed_pi: int, basis_seeds: Sequence[int], d: int) -> np.ndarray:
    seeds = np.asarray(basis_seeds, dtype=np.uint64)
    out = np.empty((len(seeds), d, d), np.float32)
    _check(lib.tq_make_head_rotations(seed_pi, seeds.ctypes.data, len(seeds), d, out.ctypes.data))
    return out


def make_sketch(seed: int, m: int, d: int) -> np.ndarray:
    out = np.empty((m, d), np.float32)
    _check(lib.tq_make_sketch(seed, m, d, out.ctypes.data))
    return out


def make_codebook(d: int, bits: int):
    c = np.empty(1 << bits, np.float32)
    t = np.empty((1 << bits) - 1, np.float32)
    _check(lib.tq_make_codebook(d, bits, c.ctypes.data, t.ctypes.data))
    return c, t


def calibrate_codebook(u, init, m: int = 1, max_iter: int = 200):
    """Levels, midpoints, mean residual magnitude e and resid_scale = fl32(e m / sqrt(pi/2))
    fitted to the samples u (host, any shape)."""
    u = np.ascontiguousarray(np.asarray(u, dtype=np.float32).ravel())
    init = np.ascontiguousarray(init, dtype=np.float32)
    bits = int(round(np.log2(len(init))))
    c = np.empty(1 << bits, np.float32)
    t = np.empty((1 << bits) - 1, np.float32)
    e = np.empty(2, np.float32)
    _check(lib.tq_calibrate_codebook(u.ctypes.data, u.size, bits, init.ctypes.data, max_iter, m, c.ctypes.data,
                                     t.ctypes.data, e.ctypes.data, e[1:].ctypes.data))
    return c, t, float(e[0]), float(e[1])


# ------------------------------------------------------------------ device objects


def _torch():
    import torch

    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _record_words(bits: int) -> int:
    return (bits + 31) // 32


def min_stride(nbits: int) -> int:
    """Smallest legal plane stride (bytes) for a record of ``nbits`` bits."""
    return 4 * _record_words(nbits) if nbits > 0 else 0


@dataclass
class Codec:
    d: int
    bits: int
    m: int
    rot: object  # torch [n_rot, d, d] fp32 on device
    sketch: Optional[object]
    centroids: object
    thresholds: object
    vecs_per_rot: int = 0
    resid_scale: float = 0.0  # > 0: residual-sign records (tq_codec.resid_scale)

    @property
    def n_rot(self) -> int:
        return int(self.rot.shape[0])

    def c(self) -> _Codec:
        return _Codec(self.d, self.bits, self.m, self.n_rot, self.vecs_per_rot, self.rot.data_ptr(),
                      0 if self.sketch is None else self.sketch.data_ptr(), self.centroids.data_ptr(),
                      self.thresholds.data_ptr(), self.resid_scale)

    @property
    def idx_stride(self) -> int:
        return min_stride(self.d * self.bits)

    @property
    def sign_stride(self) -> int:
        return min_stride(self.m)


def codec_from_arrays(d, bits, m, rot, sketch, centroids, thresholds, vecs_per_rot=0, device="cuda",
                      resid_scale=0.0) -> Codec:
    torch = _torch()
    rot = np.asarray(rot, np.float32)
    if rot.ndim == 2:
        rot = rot[None]

    def dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)

    return Codec(d, bits, m, dev(rot), dev(sketch), dev(centroids), dev(thresholds), vecs_per_rot,
                 float(np.float32(resid_scale)))


def make_codec(d: int, bits: int, m: int, rot_seed: int, sketch_seed: int, basis_seeds=None,
               vecs_per_rot: int = 0, device="cuda") -> Codec:
    """Build a codec with the library's own host constructors and upload it."""
    rot = make_rotation(rot_seed, d) if basis_seeds is None else make_head_rotations(rot_seed, basis_seeds, d)
    sk = make_sketch(sketch_seed, m, d) if m > 0 else None
    c, t = make_codebook(d, bits)
    return codec_from_arrays(d, bits, m, rot, sk, c, t, vecs_per_rot, device)


@dataclass
class Codes:
    idx: object  # torch uint8 [n, idx_stride]
    sign: Optional[object]  # torch uint8 [n, sign_stride]
    norms: object  # torch int32 [n] (uint32 bit patterns)

    def c(self) -> _Codes:
        return _Codes(self.idx.data_ptr(), int(self.idx.shape[1]),
                      0 if self.sign is None else self.sign.data_ptr(),
                      0 if self.sign is None else int(self.sign.shape[1]), self.norms.data_ptr())

    @property
    def n(self) -> int:
        return int(self.idx.shape[0])

    def slice(self, a: int, b: int) -> "Codes":
        return Codes(self.idx[a:b], None if self.sign is None else self.sign[a:b], self.norms[a:b])

    def numpy(self):
        """(idx uint8, sign uint8 or None, norms uint32) on the host."""
        return (self.idx.cpu().numpy(), None if self.sign is None else self.sign.cpu().numpy(),
                self.norms.cpu().numpy().view(np.uint32))

    def nbytes(self, unpadded_codec: Optional[Codec] = None) -> int:
        if unpadded_codec is None:
            s = self.idx.numel() + (0 if self.sign is None else self.sign.numel()) + 4 * self.norms.numel()
            return int(s)
        c = unpadded_codec
        return self.n * ((c.d * c.bits + 7) // 8 + (c.m + 7) // 8 + 4)


def alloc_codes(codec: Codec, n: int, device="cuda") -> Codes:
    torch = _torch()
    idx = torch.empty((n, codec.idx_stride), dtype=torch.uint8, device=device)
    sign = torch.empty((n, codec.sign_stride), dtype=torch.uint8, device=device) if codec.m > 0 else None
    norms = torch.empty((n,), dtype=torch.int32, device=device)
    return Codes(idx, sign, norms)


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None, ctypes.c_void_p(0), 0
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf, ctypes.c_void_p(buf.data_ptr() + off), nbytes


_DT = {"float32": TQ_F32, "float16": TQ_F16, "bfloat16": TQ_BF16}


def encode(codec: Codec, x, pre_rotated: bool = False, first: int = 0, out: Optional[Codes] = None,
           y_tap=None) -> Codes:
    """Encode rows of ``x`` ([n, d] or [..., d], contiguous rows) into ``out`` (allocated if None)."""
    x2 = x.reshape(-1, x.shape[-1])
    if x2.stride(-1) != 1:
        raise ValueError("x rows must be contiguous")
    n = x2.shape[0]
    out = out or alloc_codes(codec, n, x.device)
    dt = _DT[str(x.dtype).replace("torch.", "")]
    flags = TQ_ENC_PRE_ROTATED if pre_rotated else 0
    cc = codec.c()
    _check(lib.tq_encode(ctypes.byref(cc), _ptr(x2), dt, n, x2.stride(0), flags, first, out.c(), _ptr(y_tap),
                         _stream()))
    return out


def scores(codec: Codec, q, codes: Codes, n_keys: int, hkv: int, logits=None):
    """Logits [n_seq, hq, n_keys] for fp32 queries q [n_seq, hq, d] over codes [n_seq][hkv][n_keys]."""
    torch = _torch()
    n_seq, hq, d = q.shape
    q = q.contiguous()
    if logits is None:
        logits = torch.empty((n_seq, hq, n_keys), dtype=torch.float32, device=q.device)
    cc = codec.c()
    need = lib.tq_workspace_bytes(TQ_OP_SCORES, ctypes.byref(cc), None, n_seq, hq, hkv, n_keys)
    buf, ws, wsb = _workspace(need, q.device)
    _check(lib.tq_scores(ctypes.byref(cc), _ptr(q), n_seq, hq, hkv, n_keys, codes.c(), _ptr(logits), ws, wsb,
                         _stream()))
    return logits


def attend_decode(kcodec: Codec, vcodec: Codec, q, kcodes: Codes, vcodes: Codes, n_ctx: int, hkv: int,
                  scale: float, out=None):
    """Attention outputs [n_seq, hq, d] for fp32 queries q [n_seq, hq, d]."""
    torch = _torch()
    n_seq, hq, d = q.shape
    q = q.contiguous()
    if out is None:
        out = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    kc, vc = kcodec.c(), vcodec.c()
    need = lib.tq_workspace_bytes(TQ_OP_ATTEND, ctypes.byref(kc), ctypes.byref(vc), n_seq, hq, hkv, n_ctx)
    buf, ws, wsb = _workspace(need, q.device)
    _check(lib.tq_attend_decode(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), n_seq, hq, hkv, n_ctx, kcodes.c(),
                                vcodes.c(), ctypes.c_float(scale), _ptr(out), ws, wsb, _stream()))
    return out


def append(codec: Codec, x_new, pos, cap: int, rope_base: float, cache: Codes):
    """Append x_new [n_seq, hkv, d] (one vector per sequence and kv head) into ``cache`` laid out
    [n_seq][hkv][cap], at slot pos[s] (int32 [n_seq] on the device), RoPE'd at pos[s] before the
    rotation when rope_base > 0."""
    x = x_new.contiguous()
    n_seq, hkv, d = x.shape
    dt = _DT[str(x.dtype).replace("torch.", "")]
    cc = codec.c()
    _check(lib.tq_append(ctypes.byref(cc), _ptr(x), dt, n_seq, hkv, _ptr(pos), cap, ctypes.c_float(rope_base),
                         cache.c(), _stream()))
    return cache


def decode_step(kcodec: Codec, vcodec: Codec, q, k_new, v_new, pos, cap: int, rope_base: float, kcache: Codes,
                vcache: Codes, scale: float, out=None):
    """One decode step: append k_new / v_new [n_seq, hkv, d] at slot pos[s] (keys RoPE'd), then
    attention of q [n_seq, hq, d] (RoPE'd at pos[s]) over tokens 0 .. pos[s].  Returns out."""
    torch = _torch()
    q, kn, vn = q.contiguous(), k_new.contiguous(), v_new.contiguous()
    n_seq, hq, d = q.shape
    hkv = kn.shape[1]
    if vn.dtype != kn.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    dt = _DT[str(kn.dtype).replace("torch.", "")]
    if out is None:
        out = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    kc, vc = kcodec.c(), vcodec.c()
    need = lib.tq_workspace_bytes(TQ_OP_DECODE_STEP, ctypes.byref(kc), ctypes.byref(vc), n_seq, hq, hkv, cap)
    buf, ws, wsb = _workspace(need, q.device)
    _check(lib.tq_decode_step(ctypes.byref(kc), ctypes.byref(vc), _ptr(q), _ptr(kn), _ptr(vn), dt, n_seq, hq, hkv,
                              cap, _ptr(pos), ctypes.c_float(rope_base), kcache.c(), vcache.c(),
                              ctypes.c_float(scale), _ptr(out), ws, wsb, _stream()))
    return out


def search_topk(codec: Codec, queries, db: Codes, n_db: int, k: int):
    """Top-k (index int64, score fp32) per query by estimated inner product."""
    torch = _torch()
    queries = queries.contiguous()
    n_q = queries.shape[0]
    idx = torch.empty((n_q, k), dtype=torch.int64, device=queries.device)
    sc = torch.empty((n_q, k), dtype=torch.float32, device=queries.device)
    cc = codec.c()
    need = lib.tq_workspace_bytes(TQ_OP_SEARCH, ctypes.byref(cc), None, n_q, k, 0, n_db)
    buf, ws, wsb = _workspace(need, queries.device)
    _check(lib.tq_search_topk(ctypes.byref(cc), _ptr(queries), n_q, db.c(), n_db, k, _ptr(idx), _ptr(sc), ws, wsb,
                              _stream()))
    return idx, sc


# ------------------------------------------------------------------ recursive polar stage 1


def make_polar_tables(d: int, ab: int) -> np.ndarray:
    """Per-level angle tables [L, 4, 2^ab] fp32 (cos, sin of the levels; cos^2, sin^2 of the
    thresholds, zero-padded)."""
    L = int(d).bit_length() - 1
    out = np.empty((L, 4, 1 << ab), np.float32)
    _check(lib.tq_make_polar_tables(d, ab, out.ctypes.data))
    return out


def polar_record_bytes(d: int, ab: int) -> int:
    return int(lib.tq_polar_record_bytes(d, ab))


@dataclass
class PolarCodec:
    d: int
    ab: int
    rot: object     # torch [n_rot, d, d] fp32 on device
    tables: object  # torch [L, 4, 2^ab] fp32 on device
    vecs_per_rot: int = 0

    @property
    def n_rot(self) -> int:
        return int(self.rot.shape[0])

    def c(self) -> _PolarCodec:
        return _PolarCodec(self.d, self.ab, self.n_rot, self.vecs_per_rot, self.rot.data_ptr(),
                           self.tables.data_ptr())

    @property
    def stride(self) -> int:
        return polar_record_bytes(self.d, self.ab)


def polar_codec_from_arrays(d, ab, rot, tables, vecs_per_rot=0, device="cuda") -> PolarCodec:
    torch = _torch()
    rot = np.asarray(rot, np.float32)
    if rot.ndim == 2:
        rot = rot[None]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)

    return PolarCodec(d, ab, dev(rot), dev(tables), vecs_per_rot)


def make_polar_codec(d: int, ab: int, rot_seed: int, basis_seeds=None, vecs_per_rot: int = 0,
                     device="cuda") -> PolarCodec:
    """A polar codec from the library's own host constructors."""
    rot = make_rotation(rot_seed, d) if basis_seeds is None else make_head_rotations(rot_seed, basis_seeds, d)
    return polar_codec_from_arrays(d, ab, rot, make_polar_tables(d, ab), vecs_per_rot, device)


@dataclass
class PolarCodes:
    bits: object   # torch uint8 [n, stride]
    norms: object  # torch int32 [n] (uint32 bit patterns)

    def c(self) -> _PolarCodes:
        return _PolarCodes(self.bits.data_ptr(), int(self.bits.shape[1]), self.norms.data_ptr())

    @property
    def n(self) -> int:
        return int(self.bits.shape[0])

    def numpy(self):
        return self.bits.cpu().numpy(), self.norms.cpu().numpy().view(np.uint32)


def alloc_polar_codes(pc: PolarCodec, n: int, device="cuda", stride: Optional[int] = None) -> PolarCodes:
    torch = _torch()
    bits = torch.empty((n, stride or pc.stride), dtype=torch.uint8, device=device)
    norms = torch.empty((n,), dtype=torch.int32, device=device)
    return PolarCodes(bits, norms)


def polar_encode(pc: PolarCodec, x, pre_rotated: bool = False, first: int = 0, out: Optional[PolarCodes] = None,
                 y_tap=None) -> PolarCodes:
    """Encode rows of ``x`` ([n, d] or [..., d], contiguous rows) with the recursive polar stage."""
    x2 = x.reshape(-1, x.shape[-1])
    if x2.stride(-1) != 1:
        raise ValueError("x rows must be contiguous")
    n = x2.shape[0]
    out = out or alloc_polar_codes(pc, n, x.device)
    dt = _DT[str(x.dtype).replace("torch.", "")]
    flags = TQ_ENC_PRE_ROTATED if pre_rotated else 0
    cc = pc.c()
    _check(lib.tq_polar_encode(ctypes.byref(cc), _ptr(x2), dt, n, x2.stride(0), flags, first, out.c(),
                               _ptr(y_tap), _stream()))
    return out


def polar_scores(pc: PolarCodec, q, codes: PolarCodes, n_keys: int, hkv: int, logits=None):
    """Logits [n_seq, hq, n_keys] = nbar <Pi q, u^> over polar codes [n_seq][hkv][n_keys]."""
    torch = _torch()
    n_seq, hq, d = q.shape
    q = q.contiguous()
    if logits is None:
        logits = torch.empty((n_seq, hq, n_keys), dtype=torch.float32, device=q.device)
    cc = pc.c()
    _check(lib.tq_polar_scores(ctypes.byref(cc), _ptr(q), n_seq, hq, hkv, n_keys, codes.c(), _ptr(logits),
                               _stream()))
    return logits


def polar_attend_decode(pc: PolarCodec, vcodec: Codec, q, kcodes: PolarCodes, vcodes: Codes, n_ctx: int, hkv: int,
                        scale: float, out=None):
    """Attention outputs [n_seq, hq, d] with polar-coded keys and two-stage-coded values."""
    torch = _torch()
    n_seq, hq, d = q.shape
    q = q.contiguous()
    if out is None:
        out = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    pcc, vcc = pc.c(), vcodec.c()
    need = lib.tq_polar_attend_workspace_bytes(ctypes.byref(pcc), ctypes.byref(vcc), n_seq, hq, hkv, n_ctx)
    buf, ws, wsb = _workspace(need, q.device)
    _check(lib.tq_polar_attend_decode(ctypes.byref(pcc), ctypes.byref(vcc), _ptr(q), n_seq, hq, hkv, n_ctx,
                                      kcodes.c(), vcodes.c(), float(scale), _ptr(out), ws, wsb, _stream()))
    return out
