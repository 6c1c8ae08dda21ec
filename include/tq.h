/*
 * tq.h -- C ABI of libtq: TurboQuant-style two-stage compression of attention K/V vectors
 * and attention / top-k search computed from the compressed codes, on AMD MI355X (gfx950).
 *
 * The method (sources: the pages' titles and sections):
 *   stage 1  7minutos.es TurboQuant walkthrough, "Etapa 1 (PolarQuant)": rotate with a random
 *            orthogonal Pi, quantise each coordinate of the direction with a Lloyd-Max codebook
 *            for the Beta law of a rotated coordinate, store indices; sudonull.com "Cómo
 *            funciona PolarQuant": the radius (norm) is stored beside the direction.
 *   stage 2  same walkthrough, "Etapa 2 (Corrección Residual)": the residual's sign sketch
 *            sign(S r) under a Gaussian projection S, plus the residual's L2 norm.
 *   decode   same walkthrough, the K~_QJL formula and K~ = K^ + K~_QJL; hada.io TurboQuant
 *            page, "QJL: técnica de 1 bit com overhead zero": the query stays in high precision;
 *            TurboESM summary, section 2.E: scores, online softmax and the weighted sum of V
 *            over the compressed cache without materialising a dequantised copy.
 *   search   hada.io page, "Desempenho em busca vetorial": inner-product top-k from the codes.
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless the parameter name starts with host_.
 *   - The caller owns all memory.  No call allocates or frees device memory and none
 *     synchronises; kernels are enqueued on `stream` (a hipStream_t, NULL = default stream).
 *   - Argument checks run on the host before any launch and return a negative status; a
 *     failed launch returns TQ_EHIP.  Faults inside kernels surface at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.
 *   - Calls are reentrant: the library keeps no mutable global state (one exception:
 *     tq_decode_step_noalloc shares one static scratch array per GPU between its calls).
 *   - Inputs must be finite.  A vector norm of 65520 or more does not fit fp16 and is out of
 *     contract (it is stored as +inf).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* NULL pointer, negative size, inconsistent shapes          */
  TQ_EUNSUPPORTED = -2, /* (d, bits, m, heads-per-group, dtype) not built            */
  TQ_EALIGN = -3,       /* plane stride or pointer alignment violated                */
  TQ_EWORKSPACE = -4,   /* workspace NULL or smaller than tq_workspace_bytes         */
  TQ_EHIP = -5,         /* a HIP launch failed                                       */
  TQ_ESCRATCH = -6      /* the call needs more than the static scratch maximum        */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 } tq_dtype;

/* Shared codec of one (d, bits, m) configuration.  Borrowed device pointers.
 *   rot         [n_rot][d][d] fp32 row-major, y = rot[r] x (Haar Pi, or Pi composed with a
 *               per-head basis: TurboESM summary, section 2.B, one rotation per layer/head).
 *   sketch      [m][d] fp32 row-major Gaussian S (NULL when m == 0: stage 1 only).
 *   centroids   [2^bits] fp32 ascending Lloyd-Max levels of the unit-direction coordinate.
 *   thresholds  [2^bits - 1] fp32 midpoints between adjacent centroids, ascending (the
 *               encoder finds #{j : y >= nbar t_j} by binary descent, which relies on it).
 *   vecs_per_rot  vector v of a cache uses rot[min(v / vecs_per_rot, n_rot - 1)]; 0 or
 *               n_rot == 1 means rot[0] for all.
 *   resid_scale 0: the high half of a record's norm word is fp16(||r||) (walkthrough "Etapa 2").
 *               > 0 (needs m > 0): it is fp16(nbar * resid_scale), exactly rounded -- the
 *               TurboESM residual-sign correction (TurboESM summary, section 2.D): with S = I
 *               (m = d) and resid_scale = e m / sqrt(pi/2), e the calibrated mean residual
 *               magnitude (tq_calibrate_codebook), the QJL term of every estimator becomes
 *               nbar e sign(r_i) per coordinate, x~ = x^ + sign * e.  Finite.              */
typedef struct {
  int32_t d, bits, m;
  int32_t n_rot;
  int64_t vecs_per_rot;
  const float *rot;
  const float *sketch;
  const float *centroids;
  const float *thresholds;
  float resid_scale;
} tq_codec;

/* Compressed vectors as three planes (structure of arrays), caller-allocated.
 *   idx    [n][idx_stride] bytes: the bits-per-coordinate index stream, coordinate i at bit
 *          bits*i, least significant bit first, little-endian bytes; pad bits and bytes zero.
 *          idx_stride >= ceil(d*bits/8) and a multiple of 4.
 *   sign   [n][sign_stride] bytes: QJL bit j = [ (S r)_j >= 0 ], same bit order; NULL when
 *          m == 0.  sign_stride >= ceil(m/8) and a multiple of 4.
 *   norms  [n] uint32: low 16 bits fp16 ||x|| (round to nearest even of the exact norm), high
 *          16 bits fp16 ||r|| (the stage-1 residual in the rotated space).
 * Plane base pointers must be 16-byte aligned.                                              */
typedef struct {
  uint8_t *idx;
  int64_t idx_stride;
  uint8_t *sign;
  int64_t sign_stride;
  uint32_t *norms;
} tq_codes;

/* ---------------------------------------------------------------- codec construction (host) */

/* Haar-random orthogonal d x d matrix (fp32, row-major) from `seed`: QR (Householder, fp64)
 * of a Gaussian matrix drawn from the SplitMix64 stream `seed` (Box-Muller pairs, row-major
 * fill), with the signs of R's diagonal moved into Q.  Walkthrough "Etapa 1": y = R x with R
 * a random orthogonal matrix.  host_out: [d][d].  3 <= d <= 1024.                          */
int tq_make_rotation(uint64_t seed, int32_t d, float *host_out);

/* n_rot rotations Pi @ B_r (composed in fp64, stored fp32) with Pi = Haar(seed_pi) and
 * B_r = Haar(host_basis_seeds[r]).  host_out: [n_rot][d][d].                                */
int tq_make_head_rotations(uint64_t seed_pi, const uint64_t *host_basis_seeds, int32_t n_rot,
                           int32_t d, float *host_out);

/* Gaussian QJL projection S (fp32 [m][d] row-major) from the SplitMix64 stream `seed`
 * (walkthrough "Etapa 2": a random projection matrix S).                                    */
int tq_make_sketch(uint64_t seed, int32_t m, int32_t d, float *host_out);

/* Lloyd-Max codebook with 2^bits levels for the density (1-x^2)^((d-3)/2)/B(1/2,(d-1)/2) of
 * one coordinate of a uniform unit vector (walkthrough "Etapa 1": the Beta law and the
 * Lloyd-Max iteration; the codebook depends only on (d, bits)).  fp64 iteration with
 * Gauss-Legendre cell integrals, symmetrised, rounded to fp32.
 * host_centroids: [2^bits] ascending; host_thresholds: [2^bits - 1].  1 <= bits <= 8.       */
int tq_make_codebook(int32_t d, int32_t bits, float *host_centroids, float *host_thresholds);

/* A codebook calibrated on data (TurboESM summary, section 2.C: separate K and V tables fitted
 * to each matrix's statistics; the Lloyd rule of walkthrough "Etapa 1" applied to a sample).
 *   host_u        [n] samples of rotated directions u = Pi x / ||x|| (host memory).
 *   host_init     [2^bits] ascending starting levels (e.g. tq_make_codebook's).
 *   max_iter      rounds at most (>= 1); a round stops the loop when no level moved by more
 *                 than 1e-12 of the largest.  Each round: midpoints t_j between the levels,
 *                 cell of u = #{j : u >= t_j}, each level replaced by its cell's mean (in
 *                 fp64; an empty cell keeps its level).
 *   host_centroids [2^bits] out, fp32 of the final levels; host_thresholds [2^bits - 1] out,
 *                 fp32 of their midpoints; host_ebar out: the mean over the samples of
 *                 |u - level of its cell| (the TurboESM mean residual magnitude e);
 *                 host_resid_scale out (may be NULL): fl32(e * m / sqrt(pi/2)), the
 *                 tq_codec.resid_scale of a residual-sign codec with m = d sign bits.
 * 1 <= bits <= 8, n >= 1, m >= 1.  Host only, no device work.                              */
int tq_calibrate_codebook(const float *host_u, int64_t n, int32_t bits, const float *host_init, int32_t max_iter,
                          int32_t m, float *host_centroids, float *host_thresholds, float *host_ebar,
                          float *host_resid_scale);

/* ---------------------------------------------------------------- device operations */

/* Encode n vectors (stages 1 and 2; walkthrough "Etapa 1" and "Etapa 2").
 *   x        [n] rows of ld_x elements of type dt (row v starts at x + v*ld_x elements).
 *   flags    TQ_ENC_PRE_ROTATED: x already holds y = Pi x as fp32 (dt must be TQ_F32); the
 *            stored norm is then that of y.  Otherwise the norm is that of x and y = Pi x is
 *            computed on the device.
 *   first    index of x's first row in the whole cache (selects the per-block rotation).
 *   y_tap    optional [n][d] fp32 output of the rotated vectors used (NULL to skip).
 * Per vector: n16 = fp16(||x||); idx_i = #{ j : y_i >= fl32(nbar * t_j) }; r_i =
 * fl32(y_i - fl32(nbar * c[idx_i])); rn16 = fp16(||r||); sign bits of S r (exact sign).
 * Supported (d, bits, m): d in {64, 128, 200}, bits in {2, 3, 4}, m in {0, d}.             */
#define TQ_ENC_PRE_ROTATED 1u
int tq_encode(const tq_codec *codec, const void *x, tq_dtype dt, int64_t n, int64_t ld_x,
              uint32_t flags, int64_t first, tq_codes out, float *y_tap, void *stream);

/* Estimated logits of every (query head, key) pair (spec estimator):
 *   s = nbar * <Pi q, c[idx]> + rnbar * sqrt(pi/2)/m * <S Pi q, 2 bits - 1>
 * (walkthrough "Etapa 2", K~ = K^ + K~_QJL, taken in the rotated space).
 *   q       [n_seq][hq][d] fp32 queries (post-RoPE).  The cache k holds [n_seq][hkv][n_keys]
 *           vectors; query head h reads kv head h / (hq / hkv) (hq % hkv == 0).
 *   logits  [n_seq][hq][n_keys] fp32, unscaled (no 1/sqrt(d)).
 *   ws      workspace of tq_workspace_bytes(TQ_OP_SCORES, ...) bytes, 256-byte aligned; that
 *           size is 0 (each workgroup prepares Pi q and S Pi q itself), and ws may be NULL.   */
int tq_scores(const tq_codec *kc, const float *q, int64_t n_seq, int32_t hq, int32_t hkv,
              int64_t n_keys, tq_codes k, float *logits, void *ws, size_t ws_bytes, void *stream);

/* One decode step of attention over the compressed cache (TurboESM summary, section 2.E):
 * out[s][h] = sum_n softmax_n(scale * s_n) * v~_n, with s_n the estimate of tq_scores and
 * v~_n = Pi_V^T (nbar_n c_V[idx_n] + [m_V > 0] sqrt(pi/2)/m_V rnbar_n S_V^T (2 bits_n - 1)).
 *   q [n_seq][hq][d] fp32; caches [n_seq][hkv][n_ctx]; out [n_seq][hq][d] fp32.
 *   kc, vc may differ in bits and m (e.g. 2-bit + QJL keys, 3-bit values), not in d.       */
int tq_attend_decode(const tq_codec *kc, const tq_codec *vc, const float *q, int64_t n_seq,
                     int32_t hq, int32_t hkv, int64_t n_ctx, tq_codes k, tq_codes v, float scale,
                     float *out, void *ws, size_t ws_bytes, void *stream);

/* Append one new vector per (sequence, kv head) to a growing compressed cache laid out
 * [n_seq][hkv][cap] (walkthrough "Etapa 1": the codes stay in the cache until the token is
 * evicted; TurboESM summary, "Metodologia" A: RoPE first, then the orthogonal rotation, which
 * keeps the attention scores).
 *   x_new      [n_seq][hkv][d] device rows of type dt (contiguous).
 *   pos        [n_seq] int32 device: the position of sequence s's new token, which is also its
 *              slot: row (s, h) is encoded into record (s * hkv + h) * cap + pos[s].  Rows whose
 *              position is outside [0, cap) are skipped (device data, not checked on the host).
 *   rope_base  > 0: the rotation sees RoPE(x, pos[s]) -- coordinate i < d/2 turns with
 *              i + d/2 by the angle pos * rope_base^(-2i/d), computed in fp64 -- while the
 *              stored norm stays fp16(||x||) (RoPE keeps norms).  0: no RoPE (values).
 * The codes are those of tq_encode otherwise (per-block rotations select the block of the
 * record written).  Writes only the appended records.                                       */
int tq_append(const tq_codec *c, const void *x_new, tq_dtype dt, int64_t n_seq, int32_t hkv,
              const int32_t *pos, int64_t cap, float rope_base, tq_codes cache, void *stream);

/* One decode step over growing caches of capacity cap per (sequence, kv head): tq_append of
 * the new keys (RoPE at pos[s] when rope_base > 0) and values (no RoPE) into slot pos[s], then
 * tq_attend_decode of the queries, turned by RoPE at pos[s] when rope_base > 0, over tokens
 * 0 .. pos[s] of their sequence only.  A sequence whose pos[s] is outside [0, cap) appends
 * nothing and gets a zero output.
 *   q [n_seq][hq][d] fp32; k_new, v_new [n_seq][hkv][d] of type dt; out [n_seq][hq][d] fp32.
 *   ws  workspace of tq_workspace_bytes(TQ_OP_DECODE_STEP, kc, vc, n_seq, hq, hkv, cap) bytes,
 *       256-byte aligned.                                                                    */
int tq_decode_step(const tq_codec *kc, const tq_codec *vc, const float *q, const void *k_new,
                   const void *v_new, tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv,
                   int64_t cap, const int32_t *pos, float rope_base, tq_codes kcache,
                   tq_codes vcache, float scale, float *out, void *ws, size_t ws_bytes,
                   void *stream);

/* tq_decode_step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same checks, kernels and results,
 * with no workspace argument.  The workspace is the library's own scratch array, a static device
 * array of TQ_NOALLOC_SCRATCH_BYTES per GPU (reserved when the library's code is loaded on that
 * GPU, held until the process ends); this call allocates and frees nothing.  A call whose
 * tq_workspace_bytes(TQ_OP_DECODE_STEP, ...) exceeds it returns TQ_ESCRATCH before any launch
 * (the 8B-class step at batch 256 x capacity 32768 needs about 16 MiB).  Every call on one GPU
 * uses that GPU's array: calls that overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  Nothing in the array needs clearing between calls (each
 * call writes every scratch value it reads).  The first call on a device looks up that device's
 * copy of the array (the calling thread's current device).                                 */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int tq_decode_step_noalloc(const tq_codec *kc, const tq_codec *vc, const float *q, const void *k_new,
                           const void *v_new, tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv,
                           int64_t cap, const int32_t *pos, float rope_base, tq_codes kcache,
                           tq_codes vcache, float scale, float *out, void *stream);

/* Inner-product top-k search over an encoded database (one shared rotation):
 * for each query the k database rows with the largest estimated <q, x> (ties: smaller row
 * index first).  queries [n_q][d] fp32; out_idx [n_q][k] int64; out_score [n_q][k] fp32.
 * 1 <= k <= 32.                                                                              */
int tq_search_topk(const tq_codec *c, const float *queries, int64_t n_q, tq_codes db,
                   int64_t n_db, int32_t k, int64_t *out_idx, float *out_score, void *ws,
                   size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- recursive polar stage 1
 *
 * The recursive form of the polar stage (hada.io TurboQuant page, "PolarQuant: um novo
 * 'ângulo' para compressão"; sudonull.com "Cómo funciona PolarQuant"): after the rotation
 * y = Pi x (d = 2^L), coordinate pairs (y_2j, y_2j+1) become (radius, angle), the radii are
 * paired and turned to polar form again, level by level, until one radius remains.  Every
 * angle psi = atan2(r_b, r_a) lies in [0, pi/2] with a known law (children of k = 2^(l-1)
 * coordinates at level l: density proportional to sin^(k-1) psi cos^(k-1) psi), so each level
 * has a fixed Lloyd-Max table and no vector carries a scale besides its radius fp16(||x||).
 * Decode: u^ from the root (value 1) down, child a = parent cos psi^, child b = parent sin psi^;
 * a level-1 pair gives (sign_a r cos psi^, sign_b r sin psi^); x^ = ||x|| Pi^T u^.
 *
 * With a sketch (m > 0) the codec is the pages' two-stage composition with this polar stage
 * first (hada.io page, "Estrutura de compressão em 2 etapas" and "Etapa 2: eliminação do erro
 * oculto"): the QJL stage of tq_encode on the polar stage's residual in the rotated space,
 * r_i = fl32(y_i - fl32(nbar u^_i)) with u^ computed in fp32 from the root down (one rounding
 * per product, in the order above), rn16 = fp16(||r||) exactly rounded, and the exact sign bits
 * of S r; scores add rnbar sqrt(pi/2)/m <S Pi q, 2 bits - 1> as in tq_scores.
 *
 * Tables [L][4][2^ab] fp32, level l = 1..L at (l-1) * 4 * 2^ab:
 *   [0, n)    cos psi^_j      [n, 2n)   sin psi^_j      (psi^_j ascending, n = 2^ab)
 *   [2n, 3n)  cos^2 tau_j     [3n, 4n)  sin^2 tau_j     (tau_j = (psi^_j + psi^_j+1)/2, j < n-1;
 *                                                        the last entry of each is 0 padding)  */
typedef struct {
  int32_t d;  /* 64, 128 or 256 on the device */
  int32_t ab; /* angle bits per node: 2, 3 or 4 on the device */
  int32_t n_rot;
  int64_t vecs_per_rot; /* as tq_codec.vecs_per_rot */
  const float *rot;     /* [n_rot][d][d] fp32, 16-byte aligned */
  const float *tables;  /* [L][4][2^ab] fp32 as above */
  int32_t m;            /* 0: polar stage only; d: QJL stage on the residual (d = 64, 128) */
  const float *sketch;  /* [m][d] fp32 Gaussian S, 16-byte aligned (NULL when m == 0) */
} tq_polar_codec;

/* Compressed vectors of the polar stage.
 *   bits   [n][stride] bytes, one bitstream per vector, least significant bit first: pair j at
 *          bit (2 + ab) j as [sign of y_2j (1 = negative), sign of y_2j+1, angle index (ab
 *          bits)], then the node indices of levels 2, 3, ..., L in order, ab bits each; pad
 *          bits and bytes zero.  stride >= tq_polar_record_bytes(d, ab), a multiple of 16 when
 *          that size is a multiple of 16 (else of 8, else of 4); 16-byte aligned base.
 *   norms  [n] uint32: fp16 ||x|| (round to nearest even of the exact norm) in the low half; the
 *          high half 0, or with m > 0 fp16 ||r|| (round to nearest even of the exact norm).
 *   sign   [n][sign_stride] bytes with m > 0: bit j = [ (S r)_j >= 0 ], LSB first, pad bytes
 *          zero; sign_stride >= m/8, a multiple of 16 (m = 128) or 8 (m = 64); 16-byte aligned.
 *          NULL when m == 0.                                                                   */
typedef struct {
  uint8_t *bits;
  int64_t stride;
  uint32_t *norms;
  uint8_t *sign;
  int64_t sign_stride;
} tq_polar_codes;

/* Per-level angle tables (layout above) for d = 2^L (4 <= d <= 1024) and ab angle bits
 * (1 <= ab <= 4): Lloyd-Max on each level's law in fp64 (Gauss-Legendre cell integrals, the
 * law's quantiles as the start; level 1, the uniform law, in closed form), symmetrised about
 * pi/4, rounded to fp32.  host_tables: L * 4 * 2^ab floats.  Host only; up to a few seconds
 * at d = 1024, ab = 4.                                                                       */
int tq_make_polar_tables(int32_t d, int32_t ab, float *host_tables);

/* Bytes of one record's bitstream: 4 * ceil(((d/2)(2 + ab) + (d/2 - 1) ab) / 32); 0 for
 * d or ab out of range.                                                                      */
size_t tq_polar_record_bytes(int32_t d, int32_t ab);

/* Encode n vectors with the recursive polar stage (and, with m > 0, the QJL stage on its
 * residual).
 *   x, dt, ld_x, flags, first, y_tap as tq_encode (TQ_ENC_PRE_ROTATED: x holds y as fp32).
 * Per vector: n16 = fp16(||x||).  Level 1: A = fl32(y_2j^2), B = fl32(y_2j+1^2); level l > 1: A,
 * B the children's fl32(A + B).  A node's index is #{ j : fl32(B cos^2 tau_j) >= fl32(A sin^2
 * tau_j) } with the level's table -- the number of thresholds below psi, decided without
 * computing an angle.                                                                        */
int tq_polar_encode(const tq_polar_codec *pc, const void *x, tq_dtype dt, int64_t n, int64_t ld_x,
                    uint32_t flags, int64_t first, tq_polar_codes out, float *y_tap, void *stream);

/* Append one new vector per (sequence, kv head) to a growing cache of polar records laid out
 * [n_seq][hkv][cap]: the steps of tq_append with the polar stage (TurboESM summary,
 * "Metodologia" A: RoPE first, then the orthogonal rotation; walkthrough "Etapa 1": the codes
 * stay in the cache).  x_new [n_seq][hkv][d] device rows of type dt (contiguous); pos [n_seq]
 * int32 device, the position and slot of sequence s's token (row (s, h) goes to record
 * (s hkv + h) cap + pos[s], whose block selects the rotation; positions outside [0, cap) are
 * skipped); rope_base > 0 turns x by RoPE at pos[s] in fp64 before the rotation (as tq_append),
 * 0 for none.  The stored radius is fp16(||x||).  With m > 0 the QJL stage follows as in
 * tq_polar_encode.  Writes only the appended records.                                       */
int tq_polar_append(const tq_polar_codec *pc, const void *x_new, tq_dtype dt, int64_t n_seq, int32_t hkv,
                    const int32_t *pos, int64_t cap, float rope_base, tq_polar_codes cache, void *stream);

/* One decode step with polar-coded keys and two-stage-coded values over growing caches of
 * capacity cap per (sequence, kv head): tq_polar_append of the new keys (RoPE at pos[s] when
 * rope_base > 0) and tq_append of the new values (no RoPE) into slot pos[s], then attention of
 * the queries, turned by RoPE at pos[s] when rope_base > 0, over tokens 0 .. pos[s] of their
 * sequence only: softmax of scale times the estimate of tq_polar_scores, times the values as
 * tq_polar_attend_decode.  A sequence whose pos[s] is outside [0, cap) appends nothing and gets
 * a zero output (TurboESM summary, "Metodologia" A and section 2.E; walkthrough "Etapa 1").
 *   q [n_seq][hq][d] fp32; k_new, v_new [n_seq][hkv][d] of type dt; pos [n_seq] int32 device;
 *   kcache [n_seq][hkv][cap] polar records, vcache [n_seq][hkv][cap] codes; out [n_seq][hq][d].
 *   ws  workspace of tq_polar_decode_step_workspace_bytes bytes, 256-byte aligned: logits
 *       [n_seq][hq][cap] fp32 (only tokens 0 .. pos[s] written), then the per-chunk states.
 * Every check runs before the first launch; an unsupported call changes no memory.          */
size_t tq_polar_decode_step_workspace_bytes(const tq_polar_codec *pc, const tq_codec *vc, int64_t n_seq,
                                            int32_t hq, int32_t hkv, int64_t cap);
int tq_polar_decode_step(const tq_polar_codec *pc, const tq_codec *vc, const float *q, const void *k_new,
                         const void *v_new, tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv, int64_t cap,
                         const int32_t *pos, float rope_base, tq_polar_codes kcache, tq_codes vcache, float scale,
                         float *out, void *ws, size_t ws_bytes, void *stream);

/* Inner-product top-k search over a database of polar records (hada.io TurboQuant page,
 * "Desempenho em busca vetorial"): per query the k records with the largest estimate of
 * tq_polar_scores (ties: smaller row first).  One shared rotation (n_rot = 1).
 *   queries [n_q][d] fp32; db [n_db] records; out_idx [n_q][k] int64; out_score [n_q][k] fp32;
 *   1 <= k <= min(32, n_db), n_db < 2^31 - 1.
 *   ws  workspace of tq_polar_search_workspace_bytes bytes (may be 0: then ws may be NULL),
 *       256-byte aligned: the per-slice lists when the database is split.                   */
size_t tq_polar_search_workspace_bytes(const tq_polar_codec *pc, int64_t n_q, int32_t k, int64_t n_db);
int tq_polar_search_topk(const tq_polar_codec *pc, const float *queries, int64_t n_q, tq_polar_codes db,
                         int64_t n_db, int32_t k, int64_t *out_idx, float *out_score, void *ws, size_t ws_bytes,
                         void *stream);

/* Logits of every (query head, key) pair: nbar <Pi q, u^> (the query stays in fp32), plus
 * rnbar sqrt(pi/2)/m <S Pi q, 2 bits - 1> with the QJL stage.
 *   q [n_seq][hq][d] fp32, keys [n_seq][hkv][n_keys] records, logits [n_seq][hq][n_keys] fp32
 *   (unscaled); query head h reads kv head h / (hq / hkv).  The rotation of kv block
 *   (s, h) is that of record (s hkv + h) n_keys, as in tq_scores.  No workspace.              */
int tq_polar_scores(const tq_polar_codec *pc, const float *q, int64_t n_seq, int32_t hq, int32_t hkv,
                    int64_t n_keys, tq_polar_codes k, float *logits, void *stream);

/* One decode step of attention with polar-coded keys and two-stage-coded values: the logits of
 * tq_polar_scores, then the online softmax and the value sum of tq_attend_decode (TurboESM
 * summary, section 2.E) over vc's codes:
 * out[s][h] = sum_n softmax_n(scale * s_n) * v~_n, s_n the logit of tq_polar_scores.
 *   pc, vc of the same d (vc: 2 or 3 bits, m in {0, d}); q [n_seq][hq][d] fp32; keys k and values v
 *   [n_seq][hkv][n_ctx]; out [n_seq][hq][d] fp32.
 *   ws  workspace of tq_polar_attend_workspace_bytes bytes, 256-byte aligned: the logits
 *       [n_seq][hq][n_ctx] fp32, then the per-chunk partial states.                          */
size_t tq_polar_attend_workspace_bytes(const tq_polar_codec *pc, const tq_codec *vc, int64_t n_seq, int32_t hq,
                                       int32_t hkv, int64_t n_ctx);
int tq_polar_attend_decode(const tq_polar_codec *pc, const tq_codec *vc, const float *q, int64_t n_seq,
                           int32_t hq, int32_t hkv, int64_t n_ctx, tq_polar_codes k, tq_codes v, float scale,
                           float *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- helpers */

#define TQ_OP_SCORES 0
#define TQ_OP_ATTEND 1
#define TQ_OP_SEARCH 2
#define TQ_OP_DECODE_STEP 3
/* Workspace bytes for `op` (0 when none).  SCORES/ATTEND/DECODE_STEP: n_seq, hq, hkv,
 * n = n_keys/n_ctx/cap, vc used by ATTEND and DECODE_STEP only (may be NULL otherwise).
 * SEARCH: n_seq = n_q, hq = k, n = n_db.                                                     */
size_t tq_workspace_bytes(int op, const tq_codec *kc, const tq_codec *vc, int64_t n_seq,
                          int32_t hq, int32_t hkv, int64_t n);

/* Static description of a status code. */
const char *tq_status_str(int status);

/* Library version string. */
const char *tq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
