// C ABI entry points of libtq: argument validation, then the launchers of the .hip units.
// Every check runs on the host before any launch; see include/tq.h for the contract.

#include <cmath>
#include <cstdint>

#include "tq_internal.h"

namespace {

using tq::CodecView;
using tq::CodesView;

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// vector width (bytes) the kernels use for a record of `words` 32-bit words
inline int64_t vec_bytes(int64_t words) { return words % 4 == 0 ? 16 : (words % 2 == 0 ? 8 : 4); }

int check_codec(const tq_codec *c) {
  if (!c) return TQ_EINVAL;
  if (!tq::supported_d(c->d) || !tq::supported_bits(c->bits) || !tq::supported_m(c->d, c->m))
    return TQ_EUNSUPPORTED;
  if (!c->rot || !c->centroids || !c->thresholds || c->n_rot < 1 || c->vecs_per_rot < 0) return TQ_EINVAL;
  if (c->m > 0 && !c->sketch) return TQ_EINVAL;
  if (!(c->resid_scale >= 0.0f) || c->resid_scale == INFINITY || (c->resid_scale > 0.0f && c->m == 0))
    return TQ_EINVAL;
  if (!aligned(c->rot, 16) || (c->sketch && !aligned(c->sketch, 16))) return TQ_EALIGN;
  return TQ_OK;
}

int check_codes(const tq_codec *c, const tq_codes &k) {
  if (!k.idx || !k.norms) return TQ_EINVAL;
  const int64_t iw = ((int64_t)c->d * c->bits + 31) / 32;
  if (k.idx_stride < 4 * iw) return TQ_EINVAL;
  if (k.idx_stride % vec_bytes(iw) != 0 || !aligned(k.idx, 16) || !aligned(k.norms, 4)) return TQ_EALIGN;
  if (c->m > 0) {
    const int64_t sw = ((int64_t)c->m + 31) / 32;
    if (!k.sign) return TQ_EINVAL;
    if (k.sign_stride < 4 * sw) return TQ_EINVAL;
    if (k.sign_stride % vec_bytes(sw) != 0 || !aligned(k.sign, 16)) return TQ_EALIGN;
  }
  return TQ_OK;
}

}  // namespace

extern "C" int tq_encode(const tq_codec *codec, const void *x, tq_dtype dt, int64_t n, int64_t ld_x,
                         uint32_t flags, int64_t first, tq_codes out, float *y_tap, void *stream) {
  int rc = check_codec(codec);
  if (rc != TQ_OK) return rc;
  if (n < 0 || first < 0) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  if (!x || ld_x < codec->d) return TQ_EINVAL;
  if (dt != TQ_F32 && dt != TQ_F16 && dt != TQ_BF16) return TQ_EINVAL;
  const bool pre = (flags & TQ_ENC_PRE_ROTATED) != 0;
  if ((flags & ~TQ_ENC_PRE_ROTATED) != 0) return TQ_EINVAL;
  if (pre && dt != TQ_F32) return TQ_EINVAL;
  rc = check_codes(codec, out);
  if (rc != TQ_OK) return rc;
  return tq::launch_encode(tq::view(*codec), x, (int)dt, n, ld_x, pre, first, tq::view(out), y_tap, stream);
}

extern "C" size_t tq_workspace_bytes(int op, const tq_codec *kc, const tq_codec *vc, int64_t n_seq, int32_t hq,
                                     int32_t hkv, int64_t n) {
  if (!kc || n_seq < 0 || n < 0) return 0;
  const tq::ScoreShape s{n_seq, hq, hkv, n};
  switch (op) {
    case TQ_OP_SCORES: return tq::scores_workspace(tq::view(*kc), s);
    case TQ_OP_ATTEND:
    case TQ_OP_DECODE_STEP: return vc ? tq::attend_workspace(tq::view(*kc), tq::view(*vc), s) : 0;
    case TQ_OP_SEARCH: return tq::search_workspace(tq::view(*kc), n_seq, hq, n);
    default: return 0;
  }
}

extern "C" int tq_scores(const tq_codec *kc, const float *q, int64_t n_seq, int32_t hq, int32_t hkv,
                         int64_t n_keys, tq_codes k, float *logits, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_codec(kc);
  if (rc != TQ_OK) return rc;
  if (n_seq < 0 || n_keys < 0 || hq < 1 || hkv < 1 || hq % hkv != 0) return TQ_EINVAL;
  if (n_seq == 0 || n_keys == 0) return TQ_OK;
  if (!q || !logits) return TQ_EINVAL;
  rc = check_codes(kc, k);
  if (rc != TQ_OK) return rc;
  const tq::ScoreShape s{n_seq, hq, hkv, n_keys};
  const size_t need = tq::scores_workspace(tq::view(*kc), s);
  if (need > 0) {
    if (!ws || ws_bytes < need) return TQ_EWORKSPACE;
    if (!aligned(ws, 256)) return TQ_EALIGN;
  }
  return tq::launch_scores(tq::view(*kc), q, s, tq::view(k), logits, ws, ws_bytes, stream);
}

extern "C" int tq_attend_decode(const tq_codec *kc, const tq_codec *vc, const float *q, int64_t n_seq, int32_t hq,
                                int32_t hkv, int64_t n_ctx, tq_codes k, tq_codes v, float scale, float *out,
                                void *ws, size_t ws_bytes, void *stream) {
  int rc = check_codec(kc);
  if (rc != TQ_OK) return rc;
  rc = check_codec(vc);
  if (rc != TQ_OK) return rc;
  if (kc->d != vc->d) return TQ_EINVAL;
  if (n_seq < 0 || n_ctx < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return TQ_EINVAL;
  if (n_seq == 0) return TQ_OK;
  if (!q || !out) return TQ_EINVAL;
  rc = check_codes(kc, k);
  if (rc != TQ_OK) return rc;
  rc = check_codes(vc, v);
  if (rc != TQ_OK) return rc;
  const tq::ScoreShape s{n_seq, hq, hkv, n_ctx};
  rc = tq::attend_preflight(tq::view(*kc), tq::view(*vc), s);
  if (rc != TQ_OK) return rc;
  const size_t need = tq::attend_workspace(tq::view(*kc), tq::view(*vc), s);
  if (!ws || ws_bytes < need) return TQ_EWORKSPACE;
  if (!aligned(ws, 256)) return TQ_EALIGN;
  return tq::launch_attend(tq::view(*kc), tq::view(*vc), q, s, tq::view(k), tq::view(v), scale, out, ws,
                           ws_bytes, stream);
}

extern "C" int tq_append(const tq_codec *c, const void *x_new, tq_dtype dt, int64_t n_seq, int32_t hkv,
                         const int32_t *pos, int64_t cap, float rope_base, tq_codes cache, void *stream) {
  int rc = check_codec(c);
  if (rc != TQ_OK) return rc;
  if (n_seq < 0 || hkv < 1 || cap < 1 || !(rope_base >= 0.0f)) return TQ_EINVAL;
  if (n_seq == 0) return TQ_OK;
  if (!x_new || !pos) return TQ_EINVAL;
  if (dt != TQ_F32 && dt != TQ_F16 && dt != TQ_BF16) return TQ_EINVAL;
  rc = check_codes(c, cache);
  if (rc != TQ_OK) return rc;
  return tq::launch_append(tq::view(*c), x_new, (int)dt, n_seq, hkv, pos, cap, rope_base, tq::view(cache), stream);
}

namespace tq {

// tq_decode_step; every check before the first launch.  With `scratch` set, the workspace is
// not an argument: once the arguments are checked, scratch() gives the library's own buffer and
// its size, and a call that needs more returns TQ_ESCRATCH.
int decode_step_impl(const tq_codec *kc, const tq_codec *vc, const float *q, const void *k_new, const void *v_new,
                     tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv, int64_t cap, const int32_t *pos,
                     float rope_base, tq_codes kcache, tq_codes vcache, float scale, float *out, void *ws,
                     size_t ws_bytes, void *stream, int (*scratch)(void **ws, size_t *bytes)) {
  int rc = check_codec(kc);
  if (rc != TQ_OK) return rc;
  rc = check_codec(vc);
  if (rc != TQ_OK) return rc;
  if (kc->d != vc->d) return TQ_EINVAL;
  if (n_seq < 0 || cap < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || !(rope_base >= 0.0f)) return TQ_EINVAL;
  if (n_seq == 0) return TQ_OK;
  if (!q || !out || !k_new || !v_new || !pos) return TQ_EINVAL;
  if (dt != TQ_F32 && dt != TQ_F16 && dt != TQ_BF16) return TQ_EINVAL;
  rc = check_codes(kc, kcache);
  if (rc != TQ_OK) return rc;
  rc = check_codes(vc, vcache);
  if (rc != TQ_OK) return rc;
  const ScoreShape s{n_seq, hq, hkv, cap};
  // every check of the attention, and of both appends, before the first launch: an unsupported
  // combination must leave the caches untouched
  rc = attend_preflight(view(*kc), view(*vc), s);
  if (rc != TQ_OK) return rc;
  const size_t need = attend_workspace(view(*kc), view(*vc), s);
  if (scratch != nullptr) {
    rc = scratch(&ws, &ws_bytes);
    if (rc != TQ_OK) return rc;
    if (need > ws_bytes) return TQ_ESCRATCH;
  }
  if (!ws || ws_bytes < need) return TQ_EWORKSPACE;
  if (!aligned(ws, 256)) return TQ_EALIGN;
  rc = launch_append(view(*kc), k_new, (int)dt, n_seq, hkv, pos, cap, rope_base, view(kcache), stream);
  if (rc != TQ_OK) return rc;
  rc = launch_append(view(*vc), v_new, (int)dt, n_seq, hkv, pos, cap, 0.0f, view(vcache), stream);
  if (rc != TQ_OK) return rc;
  return launch_attend(view(*kc), view(*vc), q, s, view(kcache), view(vcache), scale, out, ws, ws_bytes, stream,
                       pos, rope_base);
}

}  // namespace tq

extern "C" int tq_decode_step(const tq_codec *kc, const tq_codec *vc, const float *q, const void *k_new,
                              const void *v_new, tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv,
                              int64_t cap, const int32_t *pos, float rope_base, tq_codes kcache, tq_codes vcache,
                              float scale, float *out, void *ws, size_t ws_bytes, void *stream) {
  return tq::decode_step_impl(kc, vc, q, k_new, v_new, dt, n_seq, hq, hkv, cap, pos, rope_base, kcache, vcache,
                              scale, out, ws, ws_bytes, stream, nullptr);
}

extern "C" int tq_search_topk(const tq_codec *c, const float *queries, int64_t n_q, tq_codes db, int64_t n_db,
                              int32_t k, int64_t *out_idx, float *out_score, void *ws, size_t ws_bytes,
                              void *stream) {
  int rc = check_codec(c);
  if (rc != TQ_OK) return rc;
  if (c->n_rot != 1) return TQ_EINVAL;
  if (n_q < 0 || n_db < 1 || k < 1 || k > 32 || k > n_db) return TQ_EINVAL;
  if (n_q == 0) return TQ_OK;
  if (!queries || !out_idx || !out_score) return TQ_EINVAL;
  rc = check_codes(c, db);
  if (rc != TQ_OK) return rc;
  const size_t need = tq::search_workspace(tq::view(*c), n_q, k, n_db);
  if (need > 0 && (!ws || ws_bytes < need)) return TQ_EWORKSPACE;
  if (ws && !aligned(ws, 256)) return TQ_EALIGN;
  return tq::launch_search(tq::view(*c), queries, n_q, tq::view(db), n_db, k, out_idx, out_score, ws, ws_bytes,
                           stream);
}

namespace {

int check_polar(const tq_polar_codec *pc) {
  if (!pc) return TQ_EINVAL;
  if (!tq::supported_polar(pc->d, pc->ab) || !tq::supported_polar_m(pc->d, pc->m)) return TQ_EUNSUPPORTED;
  if (!pc->rot || !pc->tables || pc->n_rot < 1 || pc->vecs_per_rot < 0) return TQ_EINVAL;
  if (pc->m > 0 && !pc->sketch) return TQ_EINVAL;
  if (!aligned(pc->rot, 16) || !aligned(pc->tables, 4) || (pc->sketch && !aligned(pc->sketch, 16))) return TQ_EALIGN;
  return TQ_OK;
}

int check_polar_codes(const tq_polar_codec *pc, const tq_polar_codes &k) {
  if (!k.bits || !k.norms) return TQ_EINVAL;
  const int64_t words = (tq::polar_record_bits(pc->d, pc->ab) + 31) / 32;
  if (k.stride < 4 * words) return TQ_EINVAL;
  if (k.stride % vec_bytes(words) != 0 || !aligned(k.bits, 16) || !aligned(k.norms, 4)) return TQ_EALIGN;
  if (pc->m > 0) {
    const int64_t sw = ((int64_t)pc->m + 31) / 32;
    if (!k.sign) return TQ_EINVAL;
    if (k.sign_stride < 4 * sw) return TQ_EINVAL;
    if (k.sign_stride % vec_bytes(sw) != 0 || !aligned(k.sign, 16)) return TQ_EALIGN;
  }
  return TQ_OK;
}

}  // namespace

extern "C" size_t tq_polar_record_bytes(int32_t d, int32_t ab) {
  if (d < 4 || d > 1024 || (d & (d - 1)) != 0 || ab < 1 || ab > 8) return 0;
  return (size_t)(4 * ((tq::polar_record_bits(d, ab) + 31) / 32));
}

extern "C" int tq_polar_encode(const tq_polar_codec *pc, const void *x, tq_dtype dt, int64_t n, int64_t ld_x,
                               uint32_t flags, int64_t first, tq_polar_codes out, float *y_tap, void *stream) {
  int rc = check_polar(pc);
  if (rc != TQ_OK) return rc;
  if (n < 0 || first < 0) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  if (!x || ld_x < pc->d) return TQ_EINVAL;
  if (dt != TQ_F32 && dt != TQ_F16 && dt != TQ_BF16) return TQ_EINVAL;
  const bool pre = (flags & TQ_ENC_PRE_ROTATED) != 0;
  if ((flags & ~TQ_ENC_PRE_ROTATED) != 0) return TQ_EINVAL;
  if (pre && dt != TQ_F32) return TQ_EINVAL;
  rc = check_polar_codes(pc, out);
  if (rc != TQ_OK) return rc;
  return tq::launch_polar_encode(tq::view(*pc), x, (int)dt, n, ld_x, pre, first, tq::view(out), y_tap, stream);
}

namespace {

size_t polar_attend_ws(const tq_polar_codec *pc, const tq_codec *vc, int64_t n_seq, int32_t hq, int32_t hkv,
                       int64_t n_ctx) {
  const tq::ScoreShape s{n_seq, hq, hkv, n_ctx};
  const size_t lg = (size_t)n_seq * (size_t)hq * (size_t)n_ctx * sizeof(float);
  (void)pc;
  return (lg + 255) / 256 * 256 + tq::attend_logits_workspace(tq::view(*vc), s);
}

}  // namespace

extern "C" size_t tq_polar_attend_workspace_bytes(const tq_polar_codec *pc, const tq_codec *vc, int64_t n_seq,
                                                  int32_t hq, int32_t hkv, int64_t n_ctx) {
  if (!pc || !vc || n_seq < 0 || n_ctx < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return 0;
  return polar_attend_ws(pc, vc, n_seq, hq, hkv, n_ctx);
}

extern "C" int tq_polar_attend_decode(const tq_polar_codec *pc, const tq_codec *vc, const float *q, int64_t n_seq,
                                      int32_t hq, int32_t hkv, int64_t n_ctx, tq_polar_codes k, tq_codes v,
                                      float scale, float *out, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_polar(pc);
  if (rc != TQ_OK) return rc;
  rc = check_codec(vc);
  if (rc != TQ_OK) return rc;
  if (pc->d != vc->d) return TQ_EINVAL;
  if (n_seq < 0 || n_ctx < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return TQ_EINVAL;
  if (n_seq == 0) return TQ_OK;
  if (!q || !out) return TQ_EINVAL;
  rc = check_polar_codes(pc, k);
  if (rc != TQ_OK) return rc;
  rc = check_codes(vc, v);
  if (rc != TQ_OK) return rc;
  const tq::ScoreShape s{n_seq, hq, hkv, n_ctx};
  rc = tq::attend_logits_preflight(tq::view(*vc), s);  // before the score launch
  if (rc != TQ_OK) return rc;
  const size_t need = polar_attend_ws(pc, vc, n_seq, hq, hkv, n_ctx);
  if (!ws || ws_bytes < need) return TQ_EWORKSPACE;
  if (!aligned(ws, 256)) return TQ_EALIGN;
  float *lg = reinterpret_cast<float *>(ws);
  const size_t lg_bytes = (size_t)n_seq * (size_t)hq * (size_t)n_ctx * sizeof(float);
  void *part = reinterpret_cast<uint8_t *>(ws) + (lg_bytes + 255) / 256 * 256;
  rc = tq::launch_polar_scores(tq::view(*pc), q, s, tq::view(k), lg, stream);
  if (rc != TQ_OK) return rc;
  return tq::launch_attend_logits(tq::view(*vc), lg, s, tq::view(v), scale, out, part, stream);
}

extern "C" int tq_polar_append(const tq_polar_codec *pc, const void *x_new, tq_dtype dt, int64_t n_seq, int32_t hkv,
                               const int32_t *pos, int64_t cap, float rope_base, tq_polar_codes cache, void *stream) {
  int rc = check_polar(pc);
  if (rc != TQ_OK) return rc;
  if (n_seq < 0 || hkv < 1 || cap < 1 || !(rope_base >= 0.0f)) return TQ_EINVAL;
  if (n_seq == 0) return TQ_OK;
  if (!x_new || !pos) return TQ_EINVAL;
  if (dt != TQ_F32 && dt != TQ_F16 && dt != TQ_BF16) return TQ_EINVAL;
  rc = check_polar_codes(pc, cache);
  if (rc != TQ_OK) return rc;
  return tq::launch_polar_append(tq::view(*pc), x_new, (int)dt, n_seq, hkv, pos, cap, rope_base, tq::view(cache),
                                 stream);
}

extern "C" size_t tq_polar_search_workspace_bytes(const tq_polar_codec *pc, int64_t n_q, int32_t k, int64_t n_db) {
  if (check_polar(pc) != TQ_OK || n_q < 0 || n_db < 1 || k < 1 || k > 32) return 0;
  return tq::polar_search_workspace(tq::view(*pc), n_q, k, n_db);
}

extern "C" int tq_polar_search_topk(const tq_polar_codec *pc, const float *queries, int64_t n_q, tq_polar_codes db,
                                    int64_t n_db, int32_t k, int64_t *out_idx, float *out_score, void *ws,
                                    size_t ws_bytes, void *stream) {
  int rc = check_polar(pc);
  if (rc != TQ_OK) return rc;
  if (pc->n_rot != 1) return TQ_EINVAL;
  if (n_q < 0 || n_db < 1 || k < 1 || k > 32 || k > n_db) return TQ_EINVAL;
  if (n_q == 0) return TQ_OK;
  if (!queries || !out_idx || !out_score) return TQ_EINVAL;
  rc = check_polar_codes(pc, db);
  if (rc != TQ_OK) return rc;
  const size_t need = tq::polar_search_workspace(tq::view(*pc), n_q, k, n_db);
  if (need > 0 && (!ws || ws_bytes < need)) return TQ_EWORKSPACE;
  if (ws && !aligned(ws, 256)) return TQ_EALIGN;
  return tq::launch_polar_search(tq::view(*pc), queries, n_q, tq::view(db), n_db, k, out_idx, out_score, ws,
                                 stream);
}

namespace {

size_t polar_step_ws(const tq_polar_codec *pc, const tq_codec *vc, int64_t n_seq, int32_t hq, int32_t hkv,
                     int64_t cap) {
  return polar_attend_ws(pc, vc, n_seq, hq, hkv, cap);
}

}  // namespace

extern "C" size_t tq_polar_decode_step_workspace_bytes(const tq_polar_codec *pc, const tq_codec *vc, int64_t n_seq,
                                                       int32_t hq, int32_t hkv, int64_t cap) {
  if (!pc || !vc || n_seq < 0 || cap < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return 0;
  return polar_step_ws(pc, vc, n_seq, hq, hkv, cap);
}

extern "C" int tq_polar_decode_step(const tq_polar_codec *pc, const tq_codec *vc, const float *q, const void *k_new,
                                    const void *v_new, tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv,
                                    int64_t cap, const int32_t *pos, float rope_base, tq_polar_codes kcache,
                                    tq_codes vcache, float scale, float *out, void *ws, size_t ws_bytes,
                                    void *stream) {
  int rc = check_polar(pc);
  if (rc != TQ_OK) return rc;
  rc = check_codec(vc);
  if (rc != TQ_OK) return rc;
  if (pc->d != vc->d) return TQ_EINVAL;
  if (n_seq < 0 || cap < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || !(rope_base >= 0.0f)) return TQ_EINVAL;
  if (n_seq == 0) return TQ_OK;
  if (!q || !out || !k_new || !v_new || !pos) return TQ_EINVAL;
  if (dt != TQ_F32 && dt != TQ_F16 && dt != TQ_BF16) return TQ_EINVAL;
  rc = check_polar_codes(pc, kcache);
  if (rc != TQ_OK) return rc;
  rc = check_codes(vc, vcache);
  if (rc != TQ_OK) return rc;
  const tq::ScoreShape s{n_seq, hq, hkv, cap};
  // every check before the first launch: an unsupported call leaves the caches untouched (the
  // score grid is at most n_seq * hq * ceil(cap / 256) workgroups)
  rc = tq::attend_logits_preflight(tq::view(*vc), s);
  if (rc != TQ_OK) return rc;
  if (!tq::grid_fits(n_seq * hq * ((cap + 255) / 256))) return TQ_EUNSUPPORTED;
  const size_t need = polar_step_ws(pc, vc, n_seq, hq, hkv, cap);
  if (!ws || ws_bytes < need) return TQ_EWORKSPACE;
  if (!aligned(ws, 256)) return TQ_EALIGN;
  rc = tq::launch_polar_append(tq::view(*pc), k_new, (int)dt, n_seq, hkv, pos, cap, rope_base, tq::view(kcache),
                               stream);
  if (rc != TQ_OK) return rc;
  rc = tq::launch_append(tq::view(*vc), v_new, (int)dt, n_seq, hkv, pos, cap, 0.0f, tq::view(vcache), stream);
  if (rc != TQ_OK) return rc;
  float *lg = reinterpret_cast<float *>(ws);
  const size_t lg_bytes = (size_t)n_seq * (size_t)hq * (size_t)cap * sizeof(float);
  void *part = reinterpret_cast<uint8_t *>(ws) + (lg_bytes + 255) / 256 * 256;
  rc = tq::launch_polar_scores(tq::view(*pc), q, s, tq::view(kcache), lg, stream, pos, rope_base);
  if (rc != TQ_OK) return rc;
  return tq::launch_attend_logits(tq::view(*vc), lg, s, tq::view(vcache), scale, out, part, stream, pos);
}

extern "C" int tq_polar_scores(const tq_polar_codec *pc, const float *q, int64_t n_seq, int32_t hq, int32_t hkv,
                               int64_t n_keys, tq_polar_codes k, float *logits, void *stream) {
  int rc = check_polar(pc);
  if (rc != TQ_OK) return rc;
  if (n_seq < 0 || n_keys < 0 || hq < 1 || hkv < 1 || hq % hkv != 0) return TQ_EINVAL;
  if (n_seq == 0 || n_keys == 0) return TQ_OK;
  if (!q || !logits) return TQ_EINVAL;
  rc = check_polar_codes(pc, k);
  if (rc != TQ_OK) return rc;
  const tq::ScoreShape s{n_seq, hq, hkv, n_keys};
  return tq::launch_polar_scores(tq::view(*pc), q, s, tq::view(k), logits, stream);
}
