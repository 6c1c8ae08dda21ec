// Recursive polar stage 1: encode (radius + angle tree) and scores over its codes.
//
// Sources: hada.io TurboQuant page, "PolarQuant: um novo 'ângulo' para compressão" (coordinate
// pairs to polar form, the radii paired and turned to polar form again until one radius
// remains; the angles are quantised on a fixed grid for their known, concentrated law, with no
// per-vector normalisation); sudonull.com "Cómo funciona PolarQuant" (a random rotation first;
// the radius carries the magnitude and the angles the direction).
//
// Tree of a rotated vector y (d = 2^L): level 1 pairs (y_2j, y_2j+1) -- two sign bits and the
// angle atan2(|y_2j+1|, |y_2j|); level l + 1 pairs the level-l radii (2i, 2i+1) -- the angle
// atan2(r_2i+1, r_2i).  Each level has its own Lloyd-Max angle table (the law of a node whose
// children hold k = 2^(l-1) coordinates, density proportional to sin^(k-1) cos^(k-1)).  No angle
// is computed: with A, B the children's fp32 sums of squares (leaves fl32(y^2), a node
// fl32(A + B)), the index is the number of thresholds tau_j with fl32(B cos^2 tau_j) >=
// fl32(A sin^2 tau_j) -- psi >= tau in squared, angle-free form.  The radius is fp16(||x||).
//
// Record (LSB first, one bitstream): pair j at bit (2 + ab) j as [sign of y_2j (1 = negative),
// sign of y_2j+1, angle index]; then the node indices of levels 2 .. L in order, ab bits each;
// pad bits zero.  Norm word: fp16 ||x|| in the low half, 0 in the high half.
//
// polar_encode_kernel: one wavefront per vector (rotation as the standard encoder's); the
// levels are decided in LDS, one node per lane, and lane w packs word w of the record.  With a
// sketch (M = D), the QJL stage follows on the residual: the reconstruction u^ is expanded from
// the root down in LDS (one node per lane, fp32 products), r = fl32(y - fl32(nbar u^)), its exact
// fp16 norm and the exact signs of S r as in the two-stage encoder.
// polar_score_kernel: one workgroup per (sequence, kv head, head subgroup, key chunk).  It
// rotates its G query heads, then tabulates for every pair j and every value f of the pair
// field the leaf term (+-cos psi^ q_2j +- sin psi^ q_2j+1) of each head, G floats per (j, f).  A
// key's logit is nbar sum_j r_j T[j][f_j], with r_j the product of the node cos/sin factors on
// the path to pair j, expanded from the root down in registers (one thread per key).  With the
// QJL stage, tables of 4-bit sign groups U_p[beta] = sum_t q^_4p+t (2 bit_t(beta) - 1) of the
// sketched query add rnbar sqrt(pi/2)/m sum_p U_p[sign nibble p] (16 entries per group keep four
// heads' tables small enough for several workgroups per CU).
// polar_search_scan: the same tables for G queries of a search, one workgroup per (query group,
// database slice), a top-k list per wave and query as in the two-stage search.

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_qprep.h"
#include "tq_topk.h"

namespace tq {

template <int D, int AB>
struct PolarLayout {
  static constexpr int LV = D == 64 ? 6 : D == 128 ? 7 : 8;  // levels
  static constexpr int NP = D / 2;                            // pairs
  static constexpr int WP = 2 + AB;                           // pair field width
  static constexpr int P0 = NP * WP;                          // first node bit
  static constexpr int NBITS = P0 + (NP - 1) * AB;
  static constexpr int NW = (NBITS + 31) / 32;                // record words
  static constexpr int NA = 1 << AB;                          // angle levels
  static constexpr int NF = 1 << WP;                          // pair field values
  // first bit of node i of level l >= 2 (levels 2 .. l - 1 hold NP - D / 2^(l-1) nodes)
  static constexpr int node_bit(int l, int i) { return P0 + AB * (NP - (D >> (l - 1)) + i); }
};

// Field of `width` bits at bit p of the words w (p constant after unrolling).
template <int NW>
__device__ __forceinline__ uint32_t bit_field(const uint32_t (&w)[NW], int p, int width) {
  const int i = p >> 5, o = p & 31;
  const uint32_t mask = (1u << width) - 1u;
  if (o + width <= 32 || i + 1 >= NW) return (w[i] >> o) & mask;
  return __builtin_amdgcn_alignbit(w[i + 1], w[i], o) & mask;
}

// ------------------------------------------------------------------ encode

struct PolarEncArgs {
  const void *x;
  int64_t ld_x, n, first;
  const float *rot;
  int n_rot;
  int64_t vecs_per_rot;
  const float *tables;  // [L][4][2^ab]: cos, sin, cos^2 tau, sin^2 tau per level
  uint8_t *bits;
  int64_t stride;
  uint32_t *norms;
  float *y_tap;
  const float *sketch;  // [M][D] with the QJL stage
  uint8_t *sign;
  int64_t sign_stride;
  // append mode (pos != nullptr): input row v = s * hkv + h goes to record v * cap + pos[s]
  // (skipped when pos[s] is outside [0, cap)), whose block selects the rotation; with
  // rope_base > 0 the rotation sees RoPE(x, pos[s])
  const int32_t *pos;
  int64_t cap;
  int hkv;
  float rope_base;
};

constexpr int kPolarEncWaves = 4;

template <int D>
struct PolarEncLds {
  float xs[D];
  float ys[D];
  float sum[2][D / 2];  // children's sums of squares; then the node values of the reconstruction
  uint32_t field[D];  // pair fields [0, D/2), node fields of levels 2.. from D/2
  float rs[D];        // the residual of the QJL stage
  double terms[D + 2];
  double buf[D + 2];
};

// Index of a node with children sums of squares A, B: thresholds passed (ties go up).
template <int NA>
__device__ __forceinline__ uint32_t polar_decide(float A, float B, const float *c2, const float *s2) {
  uint32_t k = 0;
#pragma unroll
  for (int j = 0; j < NA - 1; ++j) k += (__fmul_rn(B, c2[j]) >= __fmul_rn(A, s2[j])) ? 1u : 0u;
  return k;
}

template <int D, int AB, int M, int TIN, bool PRE>
__global__ __launch_bounds__(kWave *kPolarEncWaves) void polar_encode_kernel(PolarEncArgs a) {
  using P = PolarLayout<D, AB>;
  constexpr int C = D / kWave;
  static_assert(M == 0 || M == D, "the QJL stage takes m = d");
  __shared__ PolarEncLds<D> lds_all[kPolarEncWaves];
  __shared__ float tc2[P::LV][P::NA], ts2[P::LV][P::NA];
  __shared__ float tco[M > 0 ? P::LV : 1][P::NA], tsi[M > 0 ? P::LV : 1][P::NA];  // cos, sin of the levels
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  PolarEncLds<D> &s = lds_all[wid];
  for (int e = threadIdx.x; e < P::LV * P::NA; e += blockDim.x) {
    const int l = e / P::NA, j = e % P::NA;
    tc2[l][j] = a.tables[(l * 4 + 2) * P::NA + j];
    ts2[l][j] = a.tables[(l * 4 + 3) * P::NA + j];
    if constexpr (M > 0) {
      tco[l][j] = a.tables[(l * 4) * P::NA + j];
      tsi[l][j] = a.tables[(l * 4 + 1) * P::NA + j];
    }
  }
  __syncthreads();
  const int sw = (int)(a.stride >> 2);

  for (int64_t v = (int64_t)blockIdx.x * kPolarEncWaves + wid; v < a.n; v += (int64_t)gridDim.x * kPolarEncWaves) {
    int64_t rec = v;  // the record written
    int64_t p = 0;    // the position (append mode)
    if (a.pos != nullptr) {
      p = a.pos[v / a.hkv];
      if (p < 0 || p >= a.cap) continue;  // uniform: one vector per wavefront
      rec = v * a.cap + p;
    }
    // ---- load and rotate
    float y[C], nsrc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) nsrc[c] = load_in<TIN>(a.x, v * a.ld_x + lane + kWave * c);
    if constexpr (PRE) {
#pragma unroll
      for (int c = 0; c < C; ++c) y[c] = nsrc[c];
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) s.xs[lane + kWave * c] = nsrc[c];
      wave_lds_fence();
      if (a.pos != nullptr && a.rope_base > 0.0f) wave_rope_lds<D>(s.xs, p, a.rope_base);
      int64_t rid = 0;
      if (a.n_rot > 1 && a.vecs_per_rot > 0) {
        rid = (a.first + rec) / a.vecs_per_rot;
        if (rid > a.n_rot - 1) rid = a.n_rot - 1;
      }
      const float *R = a.rot + rid * (int64_t)D * D;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float4 *row = reinterpret_cast<const float4 *>(R + (int64_t)(lane + kWave * c) * D);
        float acc = 0.0f;
        for (int k4 = 0; k4 < D / 4; ++k4) {
          const float4 p = row[k4];
          acc = fmaf(p.x, s.xs[4 * k4 + 0], acc);
          acc = fmaf(p.y, s.xs[4 * k4 + 1], acc);
          acc = fmaf(p.z, s.xs[4 * k4 + 2], acc);
          acc = fmaf(p.w, s.xs[4 * k4 + 3], acc);
        }
        y[c] = acc;
      }
    }
    if (a.y_tap) {
#pragma unroll
      for (int c = 0; c < C; ++c) a.y_tap[v * D + lane + kWave * c] = y[c];
    }
    const uint32_t n16 = wave_norm_f16<D, C>(nsrc, s.terms, s.buf);
#pragma unroll
    for (int c = 0; c < C; ++c) s.ys[lane + kWave * c] = y[c];
    wave_lds_fence();

    // ---- level 1: signs, angle index, radius^2 of every pair
    for (int j = lane; j < P::NP; j += kWave) {
      const float ya = s.ys[2 * j], yb = s.ys[2 * j + 1];
      const float A = __fmul_rn(ya, ya), B = __fmul_rn(yb, yb);
      const uint32_t k = polar_decide<P::NA>(A, B, tc2[0], ts2[0]);
      s.field[j] = (ya < 0.0f ? 1u : 0u) | (yb < 0.0f ? 2u : 0u) | (k << 2);
      s.sum[0][j] = __fadd_rn(A, B);
    }
    wave_lds_fence();
    // ---- levels 2 .. L: one node per lane
    int src = 0, nbase = P::NP;
#pragma unroll
    for (int l = 2; l <= P::LV; ++l) {
      const int nn = D >> l;
      for (int i = lane; i < nn; i += kWave) {
        const float A = s.sum[src][2 * i], B = s.sum[src][2 * i + 1];
        s.field[nbase + i] = polar_decide<P::NA>(A, B, tc2[l - 1], ts2[l - 1]);
        s.sum[src ^ 1][i] = __fadd_rn(A, B);
      }
      nbase += nn;
      src ^= 1;
      wave_lds_fence();
    }

    // ---- pack: lane w assembles word w
    for (int w = lane; w < sw; w += kWave) {
      uint32_t word = 0;
      const int b0 = 32 * w, b1 = b0 + 32;
      if (b0 < P::P0) {
        const int j0 = b0 / P::WP;
        int j1 = (b1 - 1) / P::WP;
        if (j1 > P::NP - 1) j1 = P::NP - 1;
        for (int j = j0; j <= j1; ++j) {
          const int off = P::WP * j - b0;
          const uint32_t f = s.field[j];
          word |= off >= 0 ? (f << off) : (f >> (-off));
        }
      }
      if (b1 > P::P0 && b0 < P::NBITS) {
        const int i0 = b0 > P::P0 ? (b0 - P::P0) / AB : 0;
        int i1 = (b1 - 1 - P::P0) / AB;
        if (i1 > P::NP - 2) i1 = P::NP - 2;
        for (int i = i0; i <= i1; ++i) {
          const int off = P::P0 + AB * i - b0;
          const uint32_t f = s.field[P::NP + i];
          word |= off >= 0 ? (f << off) : (f >> (-off));
        }
      }
      reinterpret_cast<uint32_t *>(a.bits + rec * a.stride)[w] = word;
    }
    uint32_t hi = 0u;
    if constexpr (M > 0) {
      // ---- the reconstruction u^ from the root down: node values in s.sum (ping-pong)
      if (lane == 0) s.sum[0][0] = 1.0f;
      wave_lds_fence();
      int cur = 0;
#pragma unroll
      for (int l = P::LV; l >= 2; --l) {
        const int nn = D >> l;  // nodes of level l
        const int f0 = P::NP + (P::NP - (D >> (l - 1)));  // first field of level l
        for (int i = lane; i < nn; i += kWave) {
          const uint32_t k = s.field[f0 + i];
          const float pv = s.sum[cur][i];
          s.sum[cur ^ 1][2 * i] = __fmul_rn(pv, tco[l - 1][k]);
          s.sum[cur ^ 1][2 * i + 1] = __fmul_rn(pv, tsi[l - 1][k]);
        }
        cur ^= 1;
        wave_lds_fence();
      }
      // ---- residual r_i = fl32(y_i - fl32(nbar u^_i)) on the lane's coordinates
      const float nbar = f16_bits_to_float(n16);
      float r[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int i = lane + kWave * c;
        const uint32_t f = s.field[i >> 1];
        const uint32_t k = f >> 2;
        const float rad = s.sum[cur][i >> 1];
        float u = (i & 1) ? __fmul_rn(rad, tsi[0][k]) : __fmul_rn(rad, tco[0][k]);
        if (f & ((i & 1) ? 2u : 1u)) u = -u;
        r[c] = __fsub_rn(s.ys[i], __fmul_rn(nbar, u));
        s.rs[i] = r[c];
      }
      const uint32_t rn16 = wave_norm_f16<D, C>(r, s.terms, s.buf);
      wave_lds_fence();
      wave_sign_words<D, M>(a.sketch, s.rs, s.terms, s.buf,
                            reinterpret_cast<uint32_t *>(a.sign + rec * a.sign_stride), (int)(a.sign_stride >> 2));
      hi = rn16;
    }
    if (lane == 0) a.norms[rec] = (hi << 16) | n16;
    wave_lds_fence();
  }
}

template <int D, int AB, int M, int TIN, bool PRE>
static int launch_polar_encode_t(const PolarEncArgs &a, hipStream_t st) {
  const int64_t want = (a.n + kPolarEncWaves - 1) / kPolarEncWaves;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL((polar_encode_kernel<D, AB, M, TIN, PRE>), dim3(blocks), dim3(kWave * kPolarEncWaves), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

template <int D, int AB, int M>
static int launch_polar_encode_dam(const PolarEncArgs &a, int dt, bool pre, hipStream_t st) {
  if (pre) return launch_polar_encode_t<D, AB, M, TQ_F32, true>(a, st);
  if (dt == TQ_F32) return launch_polar_encode_t<D, AB, M, TQ_F32, false>(a, st);
  if (dt == TQ_F16) return launch_polar_encode_t<D, AB, M, TQ_F16, false>(a, st);
  return launch_polar_encode_t<D, AB, M, TQ_BF16, false>(a, st);
}

template <int D, int AB>
static int launch_polar_encode_da(const PolarEncArgs &a, int m, int dt, bool pre, hipStream_t st) {
  if (m == 0) return launch_polar_encode_dam<D, AB, 0>(a, dt, pre, st);
  if constexpr (D == 64 || D == 128) {
    if (m == D) return launch_polar_encode_dam<D, AB, D>(a, dt, pre, st);
  }
  return TQ_EUNSUPPORTED;
}

int launch_polar_encode(const PolarView &pc, const void *x, int dt, int64_t n, int64_t ld_x, bool pre_rotated,
                        int64_t first, const PolarCodesView &out, float *y_tap, void *stream) {
  if (n == 0) return TQ_OK;
  {
    const int rc = launch_polar_mfma(pc, x, dt, n, ld_x, pre_rotated, first, out, y_tap, stream);
    if (rc != TQ_EUNSUPPORTED) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  PolarEncArgs a{x, ld_x, n, first, pc.rot, pc.n_rot, pc.vecs_per_rot, pc.tables, out.bits, out.stride,
                 out.norms, y_tap, pc.sketch, out.sign, out.sign_stride};
#define TQ_PE(DD, AA) \
  if (pc.d == DD && pc.ab == AA) return launch_polar_encode_da<DD, AA>(a, pc.m, dt, pre_rotated, st);
  TQ_PE(64, 2) TQ_PE(64, 3) TQ_PE(64, 4) TQ_PE(128, 2) TQ_PE(128, 3) TQ_PE(128, 4)
  TQ_PE(256, 2) TQ_PE(256, 3) TQ_PE(256, 4)
#undef TQ_PE
  return TQ_EUNSUPPORTED;
}

int launch_polar_append(const PolarView &pc, const void *x, int dt, int64_t n_seq, int hkv, const int32_t *pos,
                        int64_t cap, float rope_base, const PolarCodesView &out, void *stream) {
  const int64_t n = n_seq * hkv;
  if (n == 0) return TQ_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  PolarEncArgs a{x, pc.d, n, 0, pc.rot, pc.n_rot, pc.vecs_per_rot, pc.tables, out.bits, out.stride,
                 out.norms, nullptr, pc.sketch, out.sign, out.sign_stride, pos, cap, hkv, rope_base};
#define TQ_PE(DD, AA) \
  if (pc.d == DD && pc.ab == AA) return launch_polar_encode_da<DD, AA>(a, pc.m, dt, false, st);
  TQ_PE(64, 2) TQ_PE(64, 3) TQ_PE(64, 4) TQ_PE(128, 2) TQ_PE(128, 3) TQ_PE(128, 4)
  TQ_PE(256, 2) TQ_PE(256, 3) TQ_PE(256, 4)
#undef TQ_PE
  return TQ_EUNSUPPORTED;
}

// ------------------------------------------------------------------ scores

struct PolarScoreArgs {
  const float *q, *rot, *tables;
  int n_rot;
  int64_t vecs_per_rot;
  int64_t n_seq, n_keys;
  int hq, hkv, nsub, n_chunks, chunk;
  const uint8_t *bits;
  int64_t stride;
  const uint32_t *norms;
  float *logits;
  const float *sketch;  // the QJL stage (M > 0): S [M][D], sign planes
  const uint8_t *sign;
  int64_t sign_stride;
  // decode step (pos != nullptr): sequence s scores its keys 0 .. pos[s] only (none when pos[s]
  // is outside [0, n_keys)), with its queries turned by RoPE at pos[s] when rope_base > 0
  const int32_t *pos;
  float rope_base;
};

// Logits of record v for G query heads from the LDS tables (layouts as polar_score_kernel's):
// nbar sum_j r_j T[j][f_j], plus rnbar sqrt(pi/2)/m sum_p U_p[sign nibble p] with the QJL stage.
// sign bits per lookup of the QJL term's tables, and entries per table
constexpr int kPolarSB = 4;
constexpr int kPolarSE = 1 << kPolarSB;

template <int D, int AB, int M, int G>
__device__ __forceinline__ void polar_record_logits(const uint8_t *bits, int64_t stride, const uint32_t *norms,
                                                    const uint8_t *sign, int64_t sign_stride, int64_t v,
                                                    const float *lut, const float *qlut,
                                                    const float2 (*cs)[PolarLayout<D, AB>::NA], float (&out)[G]) {
  using P = PolarLayout<D, AB>;
  uint32_t w[P::NW];
  load_words<P::NW>(bits + v * stride, w);
  const uint32_t nw = norms[v];
  // radii of the level-1 pairs, expanded from the root (radius 1) down; r[i] holds node i of
  // the current level, children written in place from the back
  float r[P::NP];
  r[0] = 1.0f;
#pragma unroll
  for (int l = P::LV; l >= 2; --l) {
#pragma unroll
    for (int i = (D >> l) - 1; i >= 0; --i) {
      const float2 c = cs[l - 1][bit_field<P::NW>(w, P::node_bit(l, i), AB)];
      const float ri = r[i];
      r[2 * i] = ri * c.x;
      r[2 * i + 1] = ri * c.y;
    }
  }
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0f;
#pragma unroll
  for (int j = 0; j < P::NP; ++j) {
    const uint32_t f = bit_field<P::NW>(w, P::WP * j, P::WP);
    const float *e = lut + (j * P::NF + (int)f) * G;
    if constexpr (G % 4 == 0) {
#pragma unroll
      for (int g = 0; g < G; g += 4) {
        const float4 tv = *reinterpret_cast<const float4 *>(e + g);
        acc[g] = fmaf(r[j], tv.x, acc[g]);
        acc[g + 1] = fmaf(r[j], tv.y, acc[g + 1]);
        acc[g + 2] = fmaf(r[j], tv.z, acc[g + 2]);
        acc[g + 3] = fmaf(r[j], tv.w, acc[g + 3]);
      }
    } else if constexpr (G == 2) {
      const float2 tv = *reinterpret_cast<const float2 *>(e);
      acc[0] = fmaf(r[j], tv.x, acc[0]);
      acc[1] = fmaf(r[j], tv.y, acc[1]);
    } else {
      acc[0] = fmaf(r[j], e[0], acc[0]);
    }
  }
  const float nbar = f16_bits_to_float(nw & 0xFFFFu);
  if constexpr (M > 0) {
    constexpr int NQ = M / kPolarSB;
    constexpr int PW = 32 / kPolarSB;  // groups per sign word
    constexpr int SW = (M + 31) / 32;
    uint32_t sw[SW];
    load_words<SW>(sign + v * sign_stride, sw);
    float aq[G];
#pragma unroll
    for (int g = 0; g < G; ++g) aq[g] = 0.0f;
#pragma unroll
    for (int p = 0; p < NQ; ++p) {
      const int code = (sw[p / PW] >> (kPolarSB * (p % PW))) & (kPolarSE - 1);
      const float *e = qlut + (p * kPolarSE + code) * G;
      if constexpr (G % 4 == 0) {
#pragma unroll
        for (int g = 0; g < G; g += 4) {
          const float4 tv = *reinterpret_cast<const float4 *>(e + g);
          aq[g] += tv.x;
          aq[g + 1] += tv.y;
          aq[g + 2] += tv.z;
          aq[g + 3] += tv.w;
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) aq[g] += e[g];
      }
    }
    const float rq = f16_bits_to_float(nw >> 16) * (1.2533141373155003f / (float)(M > 0 ? M : 1));
#pragma unroll
    for (int h = 0; h < G; ++h) out[h] = fmaf(rq, aq[h], nbar * acc[h]);
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) out[h] = nbar * acc[h];
  }
}

// The LDS tables of G query heads from their rotated (qt [G][D]) and sketched (qh [G][M])
// forms: leaf terms (j, f, g) = (+-cos psi^_k) q_2j + (+-sin psi^_k) q_2j+1 with f = sa | sb << 1
// | k << 2, and the sign-byte tables.  Ends synchronised.
template <int D, int AB, int M, int G, int NT>
__device__ void build_polar_tables(float *lut, float *qlut, const float2 (*cs)[PolarLayout<D, AB>::NA],
                                   const float *qt, const float *qh) {
  using P = PolarLayout<D, AB>;
  if constexpr (M > 0) {
    for (int e = threadIdx.x; e < (M / kPolarSB) * kPolarSE * G; e += NT) {
      const int g = e % G, beta = (e / G) % kPolarSE, p = e / (G * kPolarSE);
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < kPolarSB; ++t) {
        const float y = qh[g * M + kPolarSB * p + t];
        acc += ((beta >> t) & 1) ? y : -y;
      }
      qlut[e] = acc;
    }
  }
  for (int e = threadIdx.x; e < P::NP * P::NF * G; e += NT) {
    const int g = e % G, f = (e / G) % P::NF, j = e / (G * P::NF);
    const float2 t = cs[0][f >> 2];
    const float c = (f & 1) ? -t.x : t.x, sn = (f & 2) ? -t.y : t.y;
    lut[e] = fmaf(sn, qt[g * D + 2 * j + 1], c * qt[g * D + 2 * j]);
  }
  __syncthreads();
}

// LDS tables of G heads: the leaf terms, and with the QJL stage the sign-group tables
// U_p[beta] = sum_t q^_{4p+t} (2 bit_t(beta) - 1), G floats per entry
template <int D, int AB, int M, int G>
constexpr int polar_lut_bytes() {
  return PolarLayout<D, AB>::NP * PolarLayout<D, AB>::NF * G * 4 + (M / kPolarSB) * kPolarSE * G * 4;
}

template <int D, int AB, int M, int G, int NT>
__global__ __launch_bounds__(NT) void polar_score_kernel(PolarScoreArgs a) {
  using P = PolarLayout<D, AB>;
  constexpr int NQ = M / kPolarSB;
  __shared__ __align__(16) float lut[P::NP * P::NF * G];
  __shared__ __align__(16) float qlut[M > 0 ? NQ * kPolarSE * G : 4];
  __shared__ float2 cs[P::LV][P::NA];
  __shared__ float qs[G * D];
  __shared__ float qt[G * D];
  __shared__ float qh[G * (M > 0 ? M : 1)];

  const int64_t b = blockIdx.x;
  const int chunk = (int)(b % a.n_chunks);
  const int64_t rest = b / a.n_chunks;
  const int sub = (int)(rest % a.nsub);
  const int64_t blk = rest / a.nsub;  // s * hkv + kvh
  const int64_t s = blk / a.hkv;
  const int kvh = (int)(blk % a.hkv);
  const int h0 = kvh * (a.hq / a.hkv) + sub * G;
  const int64_t qrow = s * a.hq + h0;

  int64_t len = a.n_keys, p = -1;
  if (a.pos != nullptr) {
    p = a.pos[s];
    len = (p >= 0 && p < a.n_keys) ? p + 1 : 0;
  }
  const int64_t t0 = (int64_t)chunk * a.chunk;
  int64_t t1 = t0 + a.chunk;
  if (t1 > len) t1 = len;
  if (t0 >= t1) return;  // uniform over the workgroup: no key of this chunk is scored

  int64_t rid = 0;  // the rotation of this kv block
  if (a.n_rot > 1 && a.vecs_per_rot > 0) {
    rid = (blk * a.n_keys) / a.vecs_per_rot;
    if (rid > a.n_rot - 1) rid = a.n_rot - 1;
  }
  QueryPrep<D, M, G, NT> prep;
  prep.issue(a.q + qrow * D, a.rot + rid * (int64_t)D * D, a.sketch);
  for (int e = threadIdx.x; e < P::LV * P::NA; e += NT) {
    const int l = e / P::NA, j = e % P::NA;
    cs[l][j] = make_float2(a.tables[l * 4 * P::NA + j], a.tables[(l * 4 + 1) * P::NA + j]);
  }
  prep.finish(qs, qt, qh, p, a.rope_base);  // ends synchronised
  build_polar_tables<D, AB, M, G, NT>(lut, qlut, cs, qt, qh);

  const int64_t vbase = blk * a.n_keys;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += NT) {
    float lg[G];
    polar_record_logits<D, AB, M, G>(a.bits, a.stride, a.norms, a.sign, a.sign_stride, vbase + t, lut, qlut, cs, lg);
#pragma unroll
    for (int h = 0; h < G; ++h) a.logits[(qrow + h) * a.n_keys + t] = lg[h];
  }
}

template <int D, int AB, int M, int G>
static int launch_polar_score_g(const PolarScoreArgs &a0, int64_t n_seq, int hq, int hkv, int64_t n,
                                hipStream_t st) {
  constexpr int NT = 256;
  PolarScoreArgs a = a0;
  a.nsub = (hq / hkv) / G;
  a.chunk = 16384;
  if (n < a.chunk) a.chunk = (int)((n + NT - 1) / NT * NT);
  a.n_chunks = (int)((n + a.chunk - 1) / a.chunk);
  const int64_t blocks = n_seq * hkv * a.nsub * a.n_chunks;
  if (!grid_fits(blocks)) return TQ_EUNSUPPORTED;
  hipLaunchKernelGGL((polar_score_kernel<D, AB, M, G, NT>), dim3((unsigned)blocks), dim3(NT), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

// query heads per table: the largest of 8, 4, 2, 1 dividing the group whose tables fit 64 KiB
template <int D, int AB, int M>
static int launch_polar_score_dam(const PolarScoreArgs &a, int64_t n_seq, int hq, int hkv, int64_t n,
                                  hipStream_t st) {
  const int g = hq / hkv;
  constexpr int kMax = 64 * 1024;
  if constexpr (polar_lut_bytes<D, AB, M, 8>() <= kMax) {
    if (g % 8 == 0) return launch_polar_score_g<D, AB, M, 8>(a, n_seq, hq, hkv, n, st);
  }
  if constexpr (polar_lut_bytes<D, AB, M, 4>() <= kMax) {
    if (g % 4 == 0) return launch_polar_score_g<D, AB, M, 4>(a, n_seq, hq, hkv, n, st);
  }
  if constexpr (polar_lut_bytes<D, AB, M, 2>() <= kMax) {
    if (g % 2 == 0) return launch_polar_score_g<D, AB, M, 2>(a, n_seq, hq, hkv, n, st);
  }
  return launch_polar_score_g<D, AB, M, 1>(a, n_seq, hq, hkv, n, st);
}

template <int D, int AB>
static int launch_polar_score_da(const PolarScoreArgs &a, int m, int64_t n_seq, int hq, int hkv, int64_t n,
                                 hipStream_t st) {
  if (m == 0) return launch_polar_score_dam<D, AB, 0>(a, n_seq, hq, hkv, n, st);
  if constexpr (D == 64 || D == 128) {
    if (m == D) return launch_polar_score_dam<D, AB, D>(a, n_seq, hq, hkv, n, st);
  }
  return TQ_EUNSUPPORTED;
}

int launch_polar_scores(const PolarView &pc, const float *q, const ScoreShape &s, const PolarCodesView &k,
                        float *logits, void *stream, const int32_t *pos, float rope_base) {
  if (s.n == 0 || s.n_seq == 0) return TQ_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  PolarScoreArgs a{q, pc.rot, pc.tables, pc.n_rot, pc.vecs_per_rot, s.n_seq, s.n, s.hq, s.hkv, 0, 1, 0,
                   k.bits, k.stride, k.norms, logits, pc.sketch, k.sign, k.sign_stride, pos, rope_base};
#define TQ_PS(DD, AA) \
  if (pc.d == DD && pc.ab == AA) return launch_polar_score_da<DD, AA>(a, pc.m, s.n_seq, s.hq, s.hkv, s.n, st);
  TQ_PS(64, 2) TQ_PS(64, 3) TQ_PS(64, 4) TQ_PS(128, 2) TQ_PS(128, 3) TQ_PS(128, 4)
  TQ_PS(256, 2) TQ_PS(256, 3) TQ_PS(256, 4)
#undef TQ_PS
  return TQ_EUNSUPPORTED;
}

// ------------------------------------------------------------------ search

struct PolarSearchArgs {
  const float *q, *rot, *tables, *sketch;
  int64_t n_q, n_db;
  int k, n_slices;
  int64_t slice;
  const uint8_t *bits;
  int64_t stride;
  const uint32_t *norms;
  const uint8_t *sign;
  int64_t sign_stride;
  float *part_s;     // [n_q][n_slices][k] when n_slices > 1
  int32_t *part_i;
  int64_t *out_idx;  // [n_q][k] when n_slices == 1
  float *out_score;
};

constexpr int kPolarSearchNT = 512;

template <int D, int AB, int M, int G, int NT>
__global__ __launch_bounds__(NT) void polar_search_scan(PolarSearchArgs a) {
  using P = PolarLayout<D, AB>;
  constexpr int NW = NT / kWave;
  static_assert(NW >= G, "one wave per query merges the lists");
  __shared__ __align__(16) float lut[P::NP * P::NF * G];
  __shared__ __align__(16) float qlut[M > 0 ? (M / kPolarSB) * kPolarSE * G : 4];
  __shared__ float2 cs[P::LV][P::NA];
  __shared__ float qs[G * D];
  __shared__ float qt[G * D];
  __shared__ float qh[G * (M > 0 ? M : 1)];
  __shared__ float wls[NW * G * 32];
  __shared__ int32_t wli[NW * G * 32];

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const int slice = (int)(blockIdx.x % a.n_slices);
  const int64_t q0 = (int64_t)(blockIdx.x / a.n_slices) * G;
  const int rows = a.n_q - q0 < G ? (int)(a.n_q - q0) : G;  // the last group may be partial
  QueryPrep<D, M, G, NT> prep;
  prep.issue(a.q + q0 * D, a.rot, a.sketch, rows);
  for (int e = tid; e < P::LV * P::NA; e += NT) {
    const int l = e / P::NA, j = e % P::NA;
    cs[l][j] = make_float2(a.tables[l * 4 * P::NA + j], a.tables[(l * 4 + 1) * P::NA + j]);
  }
  prep.finish(qs, qt, qh);  // ends synchronised
  build_polar_tables<D, AB, M, G, NT>(lut, qlut, cs, qt, qh);

  const int k = a.k;
  float ls[G], tau[G];
  int32_t li[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ls[h] = -INFINITY;
    li[h] = 0x7FFFFFFF;
    tau[h] = -INFINITY;
  }
  const int64_t v0 = (int64_t)slice * a.slice;
  int64_t v1 = v0 + a.slice;
  if (v1 > a.n_db) v1 = a.n_db;
  for (int64_t base = v0; base < v1; base += NT) {
    const int64_t v = base + tid;
    const bool valid = v < v1;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = -INFINITY;
    if (valid) polar_record_logits<D, AB, M, G>(a.bits, a.stride, a.norms, a.sign, a.sign_stride, v, lut, qlut, cs, sc);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint64_t m = __ballot(valid && sc[h] >= tau[h]);
      while (m) {
        const int j = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const float c = __shfl(sc[h], j, kWave);
        list_insert(ls[h], li[h], c, (int32_t)(base + wid * kWave + j), k);
        tau[h] = __shfl(ls[h], k - 1, kWave);
      }
    }
  }

  // merge the waves' lists: wave h (< G) merges query h
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (lane < k) {
      wls[(wid * G + h) * 32 + lane] = ls[h];
      wli[(wid * G + h) * 32 + lane] = li[h];
    }
  __syncthreads();
  if (wid < G && wid < rows) {
    const int h = wid;
    float ms = lane < k ? wls[h * 32 + lane] : -INFINITY;
    int32_t mi = lane < k ? wli[h * 32 + lane] : 0x7FFFFFFF;
    for (int w = 1; w < NW; ++w)
      for (int i = 0; i < k; ++i) list_insert(ms, mi, wls[(w * G + h) * 32 + i], wli[(w * G + h) * 32 + i], k);
    const int64_t qi = q0 + h;
    if (lane < k) {
      if (a.n_slices == 1) {
        a.out_idx[qi * k + lane] = mi;
        a.out_score[qi * k + lane] = ms;
      } else {
        a.part_s[(qi * a.n_slices + slice) * k + lane] = ms;
        a.part_i[(qi * a.n_slices + slice) * k + lane] = mi;
      }
    }
  }
}

// queries per workgroup: the largest of 4, 2, 1 whose tables fit 64 KiB
static int polar_search_group(const PolarView &pc) {
  const int64_t per = (int64_t)(pc.d / 2) * (1 << (2 + pc.ab)) * 4 + (int64_t)(pc.m / kPolarSB) * kPolarSE * 4;
  for (int g = 4; g > 1; g /= 2)
    if (per * g <= 64 * 1024) return g;
  return 1;
}

// about 2048 workgroups over (query group, slice); slices of at least 4 NT rows
static void polar_search_split(int64_t n_q, int g, int64_t n_db, int &n_slices, int64_t &slice) {
  const int64_t groups = (n_q + g - 1) / g;
  int64_t want = (2048 + groups - 1) / groups;
  const int64_t max_slices = (n_db + 4 * kPolarSearchNT - 1) / (4 * kPolarSearchNT);
  if (want > max_slices) want = max_slices;
  if (want < 1) want = 1;
  slice = (n_db + want - 1) / want;
  n_slices = (int)((n_db + slice - 1) / slice);
}

size_t polar_search_workspace(const PolarView &pc, int64_t n_q, int k, int64_t n_db) {
  int ns;
  int64_t sl;
  polar_search_split(n_q, polar_search_group(pc), n_db, ns, sl);
  return ns > 1 ? (size_t)n_q * ns * k * (sizeof(float) + sizeof(int32_t)) : 0;
}

template <int D, int AB, int M>
static int launch_polar_search_dam(const PolarSearchArgs &a, int g, hipStream_t st) {
  constexpr int NT = kPolarSearchNT;
  const int64_t blocks = (a.n_q + g - 1) / g * a.n_slices;
  if (!grid_fits(blocks)) return TQ_EUNSUPPORTED;
  if (g == 4) {
    if constexpr (polar_lut_bytes<D, AB, M, 4>() <= 64 * 1024) {
      hipLaunchKernelGGL((polar_search_scan<D, AB, M, 4, NT>), dim3((unsigned)blocks), dim3(NT), 0, st, a);
      return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
    }
    return TQ_EUNSUPPORTED;
  }
  if (g == 2) {
    if constexpr (polar_lut_bytes<D, AB, M, 2>() <= 64 * 1024) {
      hipLaunchKernelGGL((polar_search_scan<D, AB, M, 2, NT>), dim3((unsigned)blocks), dim3(NT), 0, st, a);
      return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
    }
    return TQ_EUNSUPPORTED;
  }
  hipLaunchKernelGGL((polar_search_scan<D, AB, M, 1, NT>), dim3((unsigned)blocks), dim3(NT), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

template <int D, int AB>
static int launch_polar_search_da(const PolarSearchArgs &a, int m, int g, hipStream_t st) {
  if (m == 0) return launch_polar_search_dam<D, AB, 0>(a, g, st);
  if constexpr (D == 64 || D == 128) {
    if (m == D) return launch_polar_search_dam<D, AB, D>(a, g, st);
  }
  return TQ_EUNSUPPORTED;
}

int launch_polar_search(const PolarView &pc, const float *queries, int64_t n_q, const PolarCodesView &db,
                        int64_t n_db, int k, int64_t *out_idx, float *out_score, void *ws, void *stream) {
  if (n_q == 0) return TQ_OK;
  if (n_db > 0x7FFFFFFELL) return TQ_EUNSUPPORTED;  // rows are int32 in the lists
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int g = polar_search_group(pc);
  int ns;
  int64_t sl;
  polar_search_split(n_q, g, n_db, ns, sl);
  float *part_s = reinterpret_cast<float *>(ws);
  int32_t *part_i = ns > 1 ? reinterpret_cast<int32_t *>(part_s + (size_t)n_q * ns * k) : nullptr;
  PolarSearchArgs a{queries, pc.rot, pc.tables, pc.sketch, n_q, n_db, k, ns, sl, db.bits, db.stride, db.norms,
                    db.sign, db.sign_stride, part_s, part_i, out_idx, out_score};
  int rc = TQ_EUNSUPPORTED;
#define TQ_PQ(DD, AA) \
  if (pc.d == DD && pc.ab == AA) rc = launch_polar_search_da<DD, AA>(a, pc.m, g, st); else
  TQ_PQ(64, 2) TQ_PQ(64, 3) TQ_PQ(64, 4) TQ_PQ(128, 2) TQ_PQ(128, 3) TQ_PQ(128, 4)
  TQ_PQ(256, 2) TQ_PQ(256, 3) TQ_PQ(256, 4) {}
#undef TQ_PQ
  if (rc != TQ_OK) return rc;
  if (ns > 1) return launch_topk_merge(part_s, part_i, n_q, ns, k, out_idx, out_score, stream);
  return TQ_OK;
}

}  // namespace tq
