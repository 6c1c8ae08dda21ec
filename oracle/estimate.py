"""Decode side: score estimator, attention over the compressed cache, top-k search.

Test infrastructure only.  All arithmetic is fp64.

Sources (page title, section):
* Estimator.  7minutos.es TurboQuant walkthrough, "Etapa 2 (Corrección Residual)": the
  QJL part of a key is sqrt(pi/2)/m * ||eps|| * S^T sign(S eps), which makes the sign-based
  inner-product estimate unbiased; K~ = K^ + K~_QJL with K^ the dequantised stage-1 key
  (codebook values times the stored norm, rotated back with Pi^T).  The hada.io TurboQuant
  page ("QJL: técnica de 1 bit com overhead zero"): the query stays in high precision.
  In the rotated space this gives, for q~ = Pi q and q^ = S q~,
      s(q, k) = nbar * <q~, c[idx]> + rnbar * sqrt(pi/2)/m * <q^, 2 bits - 1>.
  The walkthrough prints the constant as "(sqrt(pi)/2)/d" and "pi/2d" (garbled); the
  constant that makes E_S[estimate] = <q, r> for Gaussian S with m rows is sqrt(pi/2)/m.
* Attention.  Same walkthrough, opening section: Q.K^T scores, softmax, weights on V.
  TurboESM summary, section 2.E: the decode step reads the codes, unpacks them, applies
  the QJL correction and Pi^T and runs softmax attention, with no dequantised copy kept.
  Here V is dequantised explicitly (its definition), scores use the estimator above.
* Search.  hada.io TurboQuant page, "Desempenho em busca vetorial": rank database
  vectors by estimated inner product; recall 1@k.  sudonull.com "Conclusiones clave":
  the same codes serve vector search.
"""

import math

import numpy as np

from .codec import Codec
from .quantize import Codes, append, rope, unpack


def qjl_scale(m: int) -> float:
    """The unbiasing constant sqrt(pi/2) / m of the QJL inner-product estimate."""
    return math.sqrt(math.pi / 2.0) / m


def prepare_query(q: np.ndarray, codec: Codec, rot: int = 0):
    """q~ = Pi q and q^ = S q~ (fp64) for one query vector."""
    q64 = np.asarray(q, dtype=np.float64)
    qt = codec.rot[rot].astype(np.float64) @ q64
    qh = codec.sketch.astype(np.float64) @ qt if codec.m > 0 else None
    return qt, qh


def scores_one(q: np.ndarray, codes: Codes, codec: Codec, rot: int = 0) -> np.ndarray:
    """Estimated <q, k_n> for every vector n in ``codes`` (unscaled logits)."""
    qt, qh = prepare_query(q, codec, rot)
    index, signs, nbar, rnbar = unpack(codes, codec)
    c = codec.centroids.astype(np.float64)
    s = nbar * (c[index] @ qt)
    if codec.m > 0:
        s = s + rnbar * qjl_scale(codec.m) * (signs @ qh)
    return s


def dequantize(codes: Codes, codec: Codec, first: int = 0) -> np.ndarray:
    """Explicit reconstruction in the original space: Pi^T (nbar c[idx] + QJL part)."""
    index, signs, nbar, rnbar = unpack(codes, codec)
    c = codec.centroids.astype(np.float64)
    rot_space = nbar[:, None] * c[index]
    if codec.m > 0:
        rot_space = rot_space + (rnbar * qjl_scale(codec.m))[:, None] * (
            signs @ codec.sketch.astype(np.float64))
    rid = codec.rot_index(index.shape[0], first)
    out = np.empty_like(rot_space)
    for r in np.unique(rid):
        sel = rid == r
        out[sel] = rot_space[sel] @ codec.rot[r].astype(np.float64)  # rows times Pi = (Pi^T v)^T
    return out


def softmax(logits: np.ndarray) -> np.ndarray:
    z = logits - np.max(logits, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def _slice(codes: Codes, a: int, b: int) -> Codes:
    return Codes(codes.idx[a:b], None if codes.sign is None else codes.sign[a:b], codes.norms[a:b])


def scores(q: np.ndarray, kcodes: Codes, kcodec: Codec, n_keys: int, hkv: int) -> np.ndarray:
    """Logits [S, Hq, N] for queries q [S, Hq, d] over a cache laid out [S][Hkv][N].

    Query head h reads kv head h // (Hq / Hkv).  The rotation of kv block (s, kvh) is the
    codec's rotation for vector index (s * Hkv + kvh) * N.
    """
    S, hq, d = q.shape
    g = hq // hkv
    out = np.empty((S, hq, n_keys), dtype=np.float64)
    for s in range(S):
        for h in range(hq):
            blk = s * hkv + h // g
            rot = int(kcodec.rot_index(1, blk * n_keys)[0])
            out[s, h] = scores_one(q[s, h], _slice(kcodes, blk * n_keys, (blk + 1) * n_keys),
                                   kcodec, rot)
    return out


def attend(q, kcodes, vcodes, kcodec, vcodec, n_ctx, hkv, scale):
    """Decode attention [S, Hq, d]: softmax(scale * estimated logits) times dequantised V."""
    S, hq, d = q.shape
    g = hq // hkv
    logits = scores(q, kcodes, kcodec, n_ctx, hkv)
    p = softmax(scale * logits)
    out = np.empty((S, hq, vcodec.d), dtype=np.float64)
    for s in range(S):
        for kvh in range(hkv):
            blk = s * hkv + kvh
            v = dequantize(_slice(vcodes, blk * n_ctx, (blk + 1) * n_ctx), vcodec, blk * n_ctx)
            out[s, kvh * g:(kvh + 1) * g] = p[s, kvh * g:(kvh + 1) * g] @ v
    return out


def attend_lens(q, kcodes, vcodes, kcodec, vcodec, cap, lens, hkv, scale):
    """Decode attention [S, Hq, d] over a cache of capacity ``cap`` per (sequence, kv head)
    ([S][Hkv][cap]) in which sequence s holds its first lens[s] tokens: softmax over those
    tokens only, times their dequantised V."""
    S, hq, d = q.shape
    g = hq // hkv
    out = np.empty((S, hq, vcodec.d), dtype=np.float64)
    for s in range(S):
        n = int(lens[s])
        for kvh in range(hkv):
            blk = s * hkv + kvh
            a, b = blk * cap, blk * cap + n
            rot = int(kcodec.rot_index(1, a)[0])
            kc = _slice(kcodes, a, b)
            v = dequantize(_slice(vcodes, a, b), vcodec, a)
            for h in range(kvh * g, (kvh + 1) * g):
                p = softmax(scale * scores_one(q[s, h], kc, kcodec, rot))
                out[s, h] = p @ v
    return out


def decode_step(q, k_new, v_new, kcodes, vcodes, kcodec, vcodec, cap, pos, rope_base, hkv, scale):
    """One decode step over a growing cache [S][Hkv][cap]: sequence s appends its new key (RoPE
    at pos[s]) and value at slot pos[s], then its queries (RoPE at pos[s]) attend over tokens
    0 .. pos[s].  Returns (outputs [S, Hq, d], updated K codes, updated V codes); the inputs
    are not modified."""
    S, hq, d = q.shape
    pos = np.asarray(pos, dtype=np.int64)
    slots = ((np.arange(S)[:, None] * hkv + np.arange(hkv)[None, :]) * cap + pos[:, None]).reshape(-1)
    kpos = np.repeat(pos, hkv)
    out_codes = []
    for codes, codec, x, base in ((kcodes, kcodec, k_new, rope_base), (vcodes, vcodec, v_new, 0.0)):
        new = append(np.asarray(x).reshape(S * hkv, codec.d), codec, slots, kpos, base,
                     idx_stride=codes.idx.shape[1],
                     sign_stride=None if codes.sign is None else codes.sign.shape[1])
        c2 = Codes(codes.idx.copy(), None if codes.sign is None else codes.sign.copy(), codes.norms.copy())
        c2.idx[slots] = new.idx
        if c2.sign is not None:
            c2.sign[slots] = new.sign
        c2.norms[slots] = new.norms
        out_codes.append(c2)
    qr = np.asarray(q, dtype=np.float64)
    if rope_base > 0:
        qr = rope(qr.reshape(S * hq, d), np.repeat(pos, hq), rope_base).reshape(S, hq, d)
    out = attend_lens(qr, out_codes[0], out_codes[1], kcodec, vcodec, cap, pos + 1, hkv, scale)
    return out, out_codes[0], out_codes[1]


def attend_materialised(q, kcodes, vcodes, kcodec, vcodec, n_ctx, hkv, scale):
    """Second route: textbook softmax(scale q K~^T) V~ over explicitly dequantised K~ and V~."""
    S, hq, d = q.shape
    g = hq // hkv
    out = np.empty((S, hq, vcodec.d), dtype=np.float64)
    for s in range(S):
        for kvh in range(hkv):
            blk = s * hkv + kvh
            kt = dequantize(_slice(kcodes, blk * n_ctx, (blk + 1) * n_ctx), kcodec, blk * n_ctx)
            vt = dequantize(_slice(vcodes, blk * n_ctx, (blk + 1) * n_ctx), vcodec, blk * n_ctx)
            qs = np.asarray(q[s, kvh * g:(kvh + 1) * g], dtype=np.float64)
            out[s, kvh * g:(kvh + 1) * g] = softmax(scale * (qs @ kt.T)) @ vt
    return out


def topk_rows(score_rows: np.ndarray, k: int):
    """Per row, the k best (score descending, index ascending): (index int64, score)."""
    n = score_rows.shape[1]
    idx = np.empty((score_rows.shape[0], k), dtype=np.int64)
    for i, row in enumerate(score_rows):
        order = np.lexsort((np.arange(n), -row))[:k]
        idx[i] = order
    return idx, np.take_along_axis(score_rows, idx, axis=1)


def search_scores(queries: np.ndarray, db: Codes, codec: Codec, chunk: int = 65536) -> np.ndarray:
    """Estimated <q, x_n> for every query and database row ([Q, n_db]; single shared rotation)."""
    qs = np.asarray(queries, dtype=np.float64)
    qt = qs @ codec.rot[0].astype(np.float64).T
    qh = qt @ codec.sketch.astype(np.float64).T if codec.m > 0 else None
    c = codec.centroids.astype(np.float64)
    n = db.norms.shape[0]
    out = np.empty((qs.shape[0], n), dtype=np.float64)
    for a in range(0, n, chunk):
        part = _slice(db, a, min(n, a + chunk))
        index, signs, nbar, rnbar = unpack(part, codec)
        s = nbar[None, :] * (qt @ c[index].T)
        if codec.m > 0:
            s = s + (rnbar * qjl_scale(codec.m))[None, :] * (qh @ signs.T)
        out[:, a:a + index.shape[0]] = s
    return out


def search_topk(queries: np.ndarray, db: Codes, codec: Codec, k: int):
    """Top-k database vectors per query by estimated inner product (single shared rotation)."""
    return topk_rows(search_scores(queries, db, codec), k)


def exact_topk(queries: np.ndarray, db: np.ndarray, k: int):
    """Ground truth: top-k by exact fp64 inner product."""
    rows = np.asarray(queries, dtype=np.float64) @ np.asarray(db, dtype=np.float64).T
    return topk_rows(rows, k)


def recall_at_k(found: np.ndarray, truth: np.ndarray) -> float:
    """Mean fraction of the true top-k found (recall@k)."""
    k = truth.shape[1]
    return float(np.mean([len(set(a) & set(b)) / k for a, b in zip(found, truth)]))


def one_at_k(found: np.ndarray, truth: np.ndarray) -> float:
    """Mean indicator that the true best vector is among the found k (recall 1@k)."""
    return float(np.mean([t[0] in set(a) for a, t in zip(found, truth)]))
