// Internal declarations shared by libtq's translation units (not part of the C ABI).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/tq.h"

namespace tq {

// host codec construction (tq_host.cpp)
void gaussian_fill(uint64_t seed, int64_t count, double *out);
void haar_rotation64(uint64_t seed, int d, std::vector<double> &q);
int lloyd_max_codebook(int d, int bits, std::vector<double> &c, std::vector<double> &t);

// Everything a kernel needs about one codec, by value.
struct CodecView {
  int d, bits, m, n_rot;
  int64_t vecs_per_rot;
  const float *rot, *sketch, *centroids, *thresholds;
  float resid_scale;
};

struct CodesView {
  uint8_t *idx;
  int64_t idx_stride;
  uint8_t *sign;
  int64_t sign_stride;
  uint32_t *norms;
};

inline CodecView view(const tq_codec &c) {
  return CodecView{c.d, c.bits, c.m, c.n_rot, c.vecs_per_rot, c.rot, c.sketch, c.centroids, c.thresholds,
                   c.resid_scale};
}
inline CodesView view(const tq_codes &c) {
  return CodesView{c.idx, c.idx_stride, c.sign, c.sign_stride, c.norms};
}

// launchers (one per .hip translation unit); return a tq_status
int launch_encode(const CodecView &c, const void *x, int dt, int64_t n, int64_t ld_x, bool pre_rotated,
                  int64_t first, const CodesView &out, float *y_tap, void *stream);
// one new vector per (sequence, kv head) into record (s * hkv + h) * cap + pos[s]; RoPE at pos[s]
// before the rotation when rope_base > 0
int launch_append(const CodecView &c, const void *x, int dt, int64_t n_seq, int hkv, const int32_t *pos,
                  int64_t cap, float rope_base, const CodesView &out, void *stream);

struct ScoreShape {
  int64_t n_seq;
  int hq, hkv;
  int64_t n;
};
size_t scores_workspace(const CodecView &kc, const ScoreShape &s);
int launch_scores(const CodecView &kc, const float *q, const ScoreShape &s, const CodesView &k,
                  float *logits, void *ws, size_t ws_bytes, void *stream);

size_t attend_workspace(const CodecView &kc, const CodecView &vc, const ScoreShape &s);
// pos != nullptr: sequence s attends over tokens 0 .. pos[s] of its s.n slots, and its queries
// are turned by RoPE at pos[s] first when rope_base > 0
int launch_attend(const CodecView &kc, const CodecView &vc, const float *q, const ScoreShape &s,
                  const CodesView &k, const CodesView &v, float scale, float *out, void *ws,
                  size_t ws_bytes, void *stream, const int32_t *pos = nullptr, float rope_base = 0.0f);

// TQ_OK when launch_attend (resp. launch_attend_logits) builds the codecs' combination and its
// grids fit the launch limits, TQ_EUNSUPPORTED otherwise; host only, launches nothing -- the
// entry points call them before any launch, so that an unsupported call changes no memory
int attend_preflight(const CodecView &kc, const CodecView &vc, const ScoreShape &s);
int attend_logits_preflight(const CodecView &vc, const ScoreShape &s);

// attention from given logits [n_seq][hq][n] (keys scored elsewhere) over value codes
size_t attend_logits_workspace(const CodecView &vc, const ScoreShape &s);
// pos != nullptr: sequence s attends over tokens 0 .. pos[s] (none, a zero output, when pos[s] is
// outside [0, s.n)); logits past them are not read
int launch_attend_logits(const CodecView &vc, const float *logits, const ScoreShape &s, const CodesView &v,
                         float scale, float *out, void *ws, void *stream, const int32_t *pos = nullptr);

// tq_decode_step behind its C entry point (all argument checks, then the launches), shared with
// the entry point that takes its workspace from the library's static scratch array: with
// `scratch` set, ws and ws_bytes come from scratch() once the arguments are checked
int decode_step_impl(const tq_codec *kc, const tq_codec *vc, const float *q, const void *k_new, const void *v_new,
                     tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv, int64_t cap, const int32_t *pos,
                     float rope_base, tq_codes kcache, tq_codes vcache, float scale, float *out, void *ws,
                     size_t ws_bytes, void *stream, int (*scratch)(void **ws, size_t *bytes));

size_t search_workspace(const CodecView &c, int64_t n_q, int k, int64_t n_db);
int launch_search(const CodecView &c, const float *queries, int64_t n_q, const CodesView &db,
                  int64_t n_db, int k, int64_t *out_idx, float *out_score, void *ws, size_t ws_bytes,
                  void *stream);

// recursive polar stage 1 (tq_polar.hip)
struct PolarView {
  int d, ab, n_rot;
  int64_t vecs_per_rot;
  const float *rot, *tables;
  int m;
  const float *sketch;
};
struct PolarCodesView {
  uint8_t *bits;
  int64_t stride;
  uint32_t *norms;
  uint8_t *sign;
  int64_t sign_stride;
};
inline PolarView view(const tq_polar_codec &c) {
  return PolarView{c.d, c.ab, c.n_rot, c.vecs_per_rot, c.rot, c.tables, c.m, c.sketch};
}
inline PolarCodesView view(const tq_polar_codes &c) {
  return PolarCodesView{c.bits, c.stride, c.norms, c.sign, c.sign_stride};
}
// bits of one record: (d/2)(2 + ab) pair fields and (d/2 - 1) ab node fields
inline int64_t polar_record_bits(int d, int ab) { return (int64_t)(d / 2) * (2 + ab) + (int64_t)(d / 2 - 1) * ab; }
int polar_angle_levels(int k, int L, std::vector<double> &c);
int launch_polar_encode(const PolarView &pc, const void *x, int dt, int64_t n, int64_t ld_x, bool pre_rotated,
                        int64_t first, const PolarCodesView &out, float *y_tap, void *stream);
// the MFMA encoder with the polar epilogue; TQ_EUNSUPPORTED where it does not apply
int launch_polar_mfma(const PolarView &pc, const void *x, int dt, int64_t n, int64_t ld_x, bool pre_rotated,
                      int64_t first, const PolarCodesView &out, float *y_tap, void *stream);
// pos != nullptr: sequence s scores keys 0 .. pos[s] only (RoPE of its queries at pos[s] with
// rope_base > 0); the other logits of the row are left unwritten
int launch_polar_scores(const PolarView &pc, const float *q, const ScoreShape &s, const PolarCodesView &k,
                        float *logits, void *stream, const int32_t *pos = nullptr, float rope_base = 0.0f);
int launch_polar_append(const PolarView &pc, const void *x, int dt, int64_t n_seq, int hkv, const int32_t *pos,
                        int64_t cap, float rope_base, const PolarCodesView &out, void *stream);
size_t polar_search_workspace(const PolarView &pc, int64_t n_q, int k, int64_t n_db);
int launch_polar_search(const PolarView &pc, const float *queries, int64_t n_q, const PolarCodesView &db,
                        int64_t n_db, int k, int64_t *out_idx, float *out_score, void *ws, void *stream);
// merge of per-slice top-k lists part_s/part_i [n_q][n_slices][k] into out [n_q][k] (tq_search.hip)
int launch_topk_merge(const float *part_s, const int32_t *part_i, int64_t n_q, int n_slices, int k,
                      int64_t *out_idx, float *out_score, void *stream);
inline bool supported_polar(int d, int ab) { return (d == 64 || d == 128 || d == 256) && ab >= 2 && ab <= 4; }
// the QJL stage on the polar residual: m = d at d = 64, 128
inline bool supported_polar_m(int d, int m) { return m == 0 || (m == d && (d == 64 || d == 128)); }

// A 1-D grid of `blocks` workgroups is within the launch limit (2^31 - 1); launchers return
// TQ_EUNSUPPORTED for shapes beyond it instead of truncating the count.
inline bool grid_fits(int64_t blocks) { return blocks >= 0 && blocks <= 0x7FFFFFFF; }

// supported device configurations
inline bool supported_d(int d) { return d == 64 || d == 128 || d == 200; }
inline bool supported_bits(int b) { return b >= 2 && b <= 4; }
inline bool supported_m(int d, int m) { return m == 0 || m == d; }

}  // namespace tq
