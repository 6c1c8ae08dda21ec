// Encode kernel: stage 1 (norm, rotation, Lloyd-Max index) and stage 2 (residual, QJL signs).
//
// Sources: 7minutos.es TurboQuant walkthrough, "Etapa 1 (PolarQuant)" (rotate, quantise each
// coordinate with the Lloyd-Max codebook, store indices) and "Etapa 2 (Corrección Residual)"
// (residual, signs of the Gaussian projection S r, residual L2 norm); sudonull.com "Cómo
// funciona PolarQuant" (the radius is stored beside the direction).
//
// Stored values per vector v:
//   n16  = fp16 RNE of the exact norm of the input (of y in pre-rotated mode);
//   idx_i = #{ j : y_i >= fl32(nbar * t_j) }, nbar = float(n16);
//   r_i  = fl32(y_i - fl32(nbar * c[idx_i]));  rn16 = fp16 RNE of the exact norm of r;
//   bit_j = [ sum_k S_jk r_k >= 0 ] in exact arithmetic.
// The fp32 steps are single IEEE operations (this file is built with -ffp-contract=off).
// The norms and signs come from fp64 sums whose rounding-error bound decides them; when it
// cannot, an exact expansion sum decides (Shewchuk's Grow-Expansion), so the stored bits are
// those of the exact real quantities.
//
// encode_kernel (any d, per-vector rotations, unaligned input): one wavefront per vector.
// Lane l owns coordinates l + 64c (c < ceil(d/64)) and sketch rows l + 64c.  The index stream is packed from an LDS copy of the codes, the sign
// stream straight from wave ballots (lane l -> bit l).

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

struct EncArgs {
  const void *x;
  int64_t ld_x, n, first;
  const float *rot;
  int n_rot;
  int64_t vecs_per_rot;
  const float *sketch, *centroids, *thresholds;
  uint8_t *idx;
  int64_t idx_stride;
  uint8_t *sign;
  int64_t sign_stride;
  uint32_t *norms;
  float *y_tap;
  // append mode (pos != nullptr, encode_kernel only): input row v = s * hkv + h is stored at
  // record v * cap + pos[s] (rows whose position is outside [0, cap) are skipped), and with
  // rope_base > 0 the rotation sees RoPE(x, pos[s])
  const int32_t *pos;
  int64_t cap;
  int hkv;
  float rope_base;
  // > 0: the norm word's high half is fp16(nbar * resid_scale) instead of fp16(||r||)
  float resid_scale;
};

// The high half of the norm word: fp16(||r||), or with resid_scale > 0 fp16(nbar * resid_scale)
// (the product of an fp16 and an fp32 value is exact in fp64; one rounding to fp16).
__device__ __forceinline__ uint32_t hi_word(uint32_t rn16, float nbar, float resid_scale) {
  return resid_scale > 0.0f ? f64_to_f16_rne((double)nbar * (double)resid_scale) : rn16;
}

constexpr int kEncWaves = 4;

template <int D>
struct EncLds {
  float xs[D];
  float rs[D];
  uint8_t code[D + 4];
  double terms[D + 2];
  double buf[D + 2];
};

template <int D, int BITS, int M, int TIN, bool PRE>
__global__ __launch_bounds__(kWave *kEncWaves) void encode_kernel(EncArgs a) {
  constexpr int C = (D + kWave - 1) / kWave;
  constexpr int L = 1 << BITS;
  __shared__ EncLds<D> lds_all[kEncWaves];
  __shared__ float cbs[L];
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  EncLds<D> &s = lds_all[wid];
  if (threadIdx.x < L) cbs[threadIdx.x] = a.centroids[threadIdx.x];
  float th[L - 1];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) th[j] = a.thresholds[j];
  __syncthreads();

  const int iw = (int)(a.idx_stride >> 2);
  const int sw = M > 0 ? (int)(a.sign_stride >> 2) : 0;

  for (int64_t v = (int64_t)blockIdx.x * kEncWaves + wid; v < a.n; v += (int64_t)gridDim.x * kEncWaves) {
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
    for (int c = 0; c < C; ++c) {
      const int i = lane + kWave * c;
      nsrc[c] = (i < D) ? load_in<TIN>(a.x, v * a.ld_x + i) : 0.0f;
    }
    if constexpr (PRE) {
#pragma unroll
      for (int c = 0; c < C; ++c) y[c] = nsrc[c];
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (lane + kWave * c < D) s.xs[lane + kWave * c] = nsrc[c];
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
        const int i = lane + kWave * c;
        float acc = 0.0f;
        if (i < D) {
          const float4 *row = reinterpret_cast<const float4 *>(R + (int64_t)i * D);
          for (int k4 = 0; k4 < D / 4; ++k4) {
            const float4 p = row[k4];
            acc = fmaf(p.x, s.xs[4 * k4 + 0], acc);
            acc = fmaf(p.y, s.xs[4 * k4 + 1], acc);
            acc = fmaf(p.z, s.xs[4 * k4 + 2], acc);
            acc = fmaf(p.w, s.xs[4 * k4 + 3], acc);
          }
        }
        y[c] = acc;
      }
    }
    if (a.y_tap) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (lane + kWave * c < D) a.y_tap[v * D + lane + kWave * c] = y[c];
    }

    // ---- stage 1: norm and indices
    const uint32_t n16 = wave_norm_f16<D, C>(nsrc, s.terms, s.buf);
    const float nbar = f16_bits_to_float(n16);
    float thr[L - 1];
#pragma unroll
    for (int j = 0; j < L - 1; ++j) thr[j] = __fmul_rn(nbar, th[j]);
    float r[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = lane + kWave * c;
      int q = 0;
#pragma unroll
      for (int j = 0; j < L - 1; ++j) q += (y[c] >= thr[j]) ? 1 : 0;
      r[c] = 0.0f;
      if (i < D) {
        s.code[i] = (uint8_t)q;
        r[c] = __fsub_rn(y[c], __fmul_rn(nbar, cbs[q]));
        s.rs[i] = r[c];
      }
    }
    // ---- stage 2: residual norm and signs
    const uint32_t rn16 = wave_norm_f16<D, C>(r, s.terms, s.buf);
    wave_lds_fence();

    // pack the index stream: lane w assembles 32-bit word w
    for (int w = lane; w < iw; w += kWave) {
      uint32_t word = 0;
      const int b0 = 32 * w;
      if (b0 < D * BITS) {
        const int i0 = b0 / BITS;
        int i1 = (b0 + 31) / BITS;
        if (i1 > D - 1) i1 = D - 1;
        for (int i = i0; i <= i1; ++i) {
          const int off = BITS * i - b0;
          const uint32_t cv = s.code[i];
          word |= off >= 0 ? (cv << off) : (cv >> (-off));
        }
      }
      reinterpret_cast<uint32_t *>(a.idx + rec * a.idx_stride)[w] = word;
    }

    if constexpr (M > 0)
      wave_sign_words<D, M>(a.sketch, s.rs, s.terms, s.buf, reinterpret_cast<uint32_t *>(a.sign + rec * a.sign_stride),
                            sw);
    if (lane == 0) a.norms[rec] = (hi_word(rn16, nbar, a.resid_scale) << 16) | n16;
    wave_lds_fence();
  }
}

// ------------------------------------------------------------------ several vectors per wavefront
//
// encode_multi: the encoder of encode_kernel for one shared rotation outside append mode, with
// the wavefronts of a workgroup taking MV_W x MV_E vectors at a time (MV_E per wavefront), so
// that Pi and S pass through the CU once per MV_W x MV_E vectors instead of once per vector
// (encode_kernel streams all 320 KB of both per 200-coordinate vector through the cache, 64
// rows at a time, one 16-byte piece of each row per load).  The workgroup stages MV_KC columns
// of Pi (then of S) in LDS, double-buffered and read by every wavefront; lane l owns rotation
// rows and sketch rows l + 64c for its wavefront's MV_E vectors, which sit in LDS and are read
// as broadcast float4s.
//   - y: the same fp32 FMA chain per row as encode_kernel (k ascending), so the rotated values,
//     and with them the records, are those encode_kernel writes;
//   - norms, indices and residual: encode_kernel's steps, one vector after the other;
//   - signs: z = S r by an fp32 FMA chain, whose error is at most gamma_D sum_k |S_jk r_k| <=
//     2 (D + 2) 2^-24 ||S_j|| ||r|| (Cauchy-Schwarz), with ||S_j|| computed once per wavefront and
//     ||r|| bounded from its exact fp16 norm; outside that band the sign of z is the sign of the
//     exact dot product.  Inside it (or where r = 0) the wavefront takes the exact products in
//     fp64 and decides from their fp64 sum and its error bound, or else by the exact expansion.

constexpr int kMultiWaves = 4;  // MV_W
constexpr int kMultiVec = 8;    // MV_E
constexpr int kMultiCols = 8;   // MV_KC: columns of Pi or S per staged chunk
constexpr int kMultiStride = 12;  // floats per staged row: 16-byte reads of 16 lanes on distinct banks

template <int D>
struct MultiLds {
  float xs[kMultiVec][D];  // the inputs; after the rotation, the residuals
  uint8_t code[kMultiVec][D + 4];
  double terms[D + 2];
  double buf[D + 2];
};

// Columns [kc * MV_KC, kc * MV_KC + MV_KC) of the rows x D matrix W into dst[row * stride + col],
// by the whole workgroup (two float4 per row).
template <int D>
__device__ __forceinline__ void multi_fetch(const float *W, int rows, int kc, float4 (&r)[2], int nthreads) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int f = threadIdx.x + nthreads * it;
    r[it] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (f < 2 * rows) r[it] = reinterpret_cast<const float4 *>(W + (int64_t)(f >> 1) * D + kc * kMultiCols)[f & 1];
  }
}
__device__ __forceinline__ void multi_stage(float *dst, int rows, const float4 (&r)[2], int nthreads) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int f = threadIdx.x + nthreads * it;
    if (f < 2 * rows) *reinterpret_cast<float4 *>(dst + (f >> 1) * kMultiStride + 4 * (f & 1)) = r[it];
  }
}

// acc[e][c] += sum over the chunk's columns of W[row(c)][k] * xs[e][k], k ascending, for the
// lane's rows l + 64c (rows >= nrows read row 0 of the chunk; the caller discards them).
template <int D, int CR>
__device__ __forceinline__ void multi_chunk(const float *wl, const float (*xs)[D], int kc, int nrows,
                                            float (&acc)[kMultiVec][CR]) {
  const int lane = lane_id();
  float4 p[CR][2];
#pragma unroll
  for (int c = 0; c < CR; ++c) {
    const int i = lane + kWave * c;
    const float *row = wl + (i < nrows ? i : 0) * kMultiStride;
    p[c][0] = *reinterpret_cast<const float4 *>(row);
    p[c][1] = *reinterpret_cast<const float4 *>(row + 4);
  }
#pragma unroll
  for (int e = 0; e < kMultiVec; ++e) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 xv = *reinterpret_cast<const float4 *>(&xs[e][kc * kMultiCols + 4 * h]);
#pragma unroll
      for (int c = 0; c < CR; ++c) {
        float a = acc[e][c];
        a = fmaf(p[c][h].x, xv.x, a);
        a = fmaf(p[c][h].y, xv.y, a);
        a = fmaf(p[c][h].z, xv.z, a);
        a = fmaf(p[c][h].w, xv.w, a);
        acc[e][c] = a;
      }
    }
  }
}

// acc = W xs over all D columns, W (rows x D) staged chunk by chunk in the two buffers wl; the
// whole workgroup calls it (barriers inside).
template <int D, int CR>
__device__ void multi_product(const float *W, int rows, float *wl0, float *wl1, const float (*xs)[D],
                              float (&acc)[kMultiVec][CR]) {
  constexpr int NC = D / kMultiCols;
  constexpr int NTH = kWave * kMultiWaves;
  float4 r[2];
  multi_fetch<D>(W, rows, 0, r, NTH);
  __syncthreads();  // every wavefront is done with both buffers
  multi_stage(wl0, rows, r, NTH);
  __syncthreads();
  for (int kc = 0; kc < NC; ++kc) {
    float *cur = (kc & 1) ? wl1 : wl0;
    float *nxt = (kc & 1) ? wl0 : wl1;
    if (kc + 1 < NC) multi_fetch<D>(W, rows, kc + 1, r, NTH);
    multi_chunk<D, CR>(cur, xs, kc, rows, acc);
    if (kc + 1 < NC) multi_stage(nxt, rows, r, NTH);
    __syncthreads();
  }
}

template <int D, int BITS, int M, int TIN, bool PRE>
__global__ __launch_bounds__(kWave *kMultiWaves) void encode_multi(EncArgs a) {
  constexpr int C = (D + kWave - 1) / kWave;
  constexpr int CM = (M + kWave - 1) / kWave;
  constexpr int EV = kMultiVec;
  constexpr int L = 1 << BITS;
  constexpr int ROWS = D > M ? D : M;
  static_assert(D % kMultiCols == 0 && ROWS <= kWave * kMultiWaves, "staged chunks");
  __shared__ __align__(16) MultiLds<D> lds_all[kMultiWaves];
  __shared__ __align__(16) float wl[2][ROWS * kMultiStride];
  __shared__ float cbs[L];
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  MultiLds<D> &s = lds_all[wid];
  if (threadIdx.x < L) cbs[threadIdx.x] = a.centroids[threadIdx.x];
  float th[L - 1];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) th[j] = a.thresholds[j];
  __syncthreads();

  // 2 (D + 2) 2^-24 ||S_j|| (1 + 2^-16) for the lane's sketch rows
  float band[CM > 0 ? CM : 1];
#pragma unroll
  for (int c = 0; c < (CM > 0 ? CM : 1); ++c) {
    band[c] = 0.0f;
    if constexpr (M > 0) {
      const int j = lane + kWave * c;
      if (j < M) {
        double ss = 0.0;
        for (int k = 0; k < D; ++k) {
          const double v = a.sketch[(int64_t)j * D + k];
          ss += v * v;
        }
        band[c] = (float)(sqrt(ss) * (2.0 * (D + 2) * 0x1p-24) * (1.0 + 0x1p-16));
      }
    }
  }

  const int iw = (int)(a.idx_stride >> 2);
  const int sw = M > 0 ? (int)(a.sign_stride >> 2) : 0;
  const int64_t groups = (a.n + EV * kMultiWaves - 1) / (EV * kMultiWaves);

  // uniform over the workgroup: every wavefront runs the same number of staged products
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t v0 = (grp * kMultiWaves + wid) * EV;
    // ---- load, the exact norms of the inputs, and the inputs staged for the rotation
    float y[EV][C];
    uint32_t n16[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      float xin[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int i = lane + kWave * c;
        xin[c] = (i < D && v0 + e < a.n) ? load_in<TIN>(a.x, (v0 + e) * a.ld_x + i) : 0.0f;
        if (!PRE && i < D) s.xs[e][i] = xin[c];
        y[e][c] = xin[c];
      }
      n16[e] = wave_norm_f16<D, C>(xin, s.terms, s.buf);
    }
    if constexpr (!PRE) {
#pragma unroll
      for (int e = 0; e < EV; ++e)
#pragma unroll
        for (int c = 0; c < C; ++c) y[e][c] = 0.0f;
      wave_lds_fence();
      multi_product<D, C>(a.rot, D, wl[0], wl[1], s.xs, y);  // ends with a barrier
#pragma unroll
      for (int e = 0; e < EV; ++e)
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (lane + kWave * c >= D) y[e][c] = 0.0f;
    }
    if (a.y_tap) {
#pragma unroll
      for (int e = 0; e < EV; ++e)
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (lane + kWave * c < D && v0 + e < a.n) a.y_tap[(v0 + e) * D + lane + kWave * c] = y[e][c];
    }

    // ---- stage 1 and the residual, one vector after the other
    uint32_t nw[EV];
    float rbound[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      const float nbar = f16_bits_to_float(n16[e]);
      float thr[L - 1];
#pragma unroll
      for (int j = 0; j < L - 1; ++j) thr[j] = __fmul_rn(nbar, th[j]);
      float r[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int i = lane + kWave * c;
        int q = 0;
#pragma unroll
        for (int j = 0; j < L - 1; ++j) q += (y[e][c] >= thr[j]) ? 1 : 0;
        r[c] = 0.0f;
        if (i < D) {
          s.code[e][i] = (uint8_t)q;
          r[c] = __fsub_rn(y[e][c], __fmul_rn(nbar, cbs[q]));
          s.xs[e][i] = r[c];
        }
      }
      const uint32_t rn16 = wave_norm_f16<D, C>(r, s.terms, s.buf);
      nw[e] = (hi_word(rn16, nbar, a.resid_scale) << 16) | n16[e];
      // ||r|| <= fp16(||r||) + max(2^-11 ||r||, 2^-25) < fp16(||r||) * 1.001 + 2^-25 (the fp16 word
      // is the correctly rounded norm: half a spacing, relative for normal values, 2^-25 below)
      rbound[e] = fmaf(f16_bits_to_float(rn16), 1.001f, 0x1p-25f);
    }
    wave_lds_fence();

    // ---- index words
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      if (v0 + e >= a.n) break;  // uniform over the wavefront
      for (int w = lane; w < iw; w += kWave) {
        uint32_t word = 0;
        const int b0 = 32 * w;
        if (b0 < D * BITS) {
          const int i0 = b0 / BITS;
          int i1 = (b0 + 31) / BITS;
          if (i1 > D - 1) i1 = D - 1;
          for (int i = i0; i <= i1; ++i) {
            const int off = BITS * i - b0;
            const uint32_t cv = s.code[e][i];
            word |= off >= 0 ? (cv << off) : (cv >> (-off));
          }
        }
        reinterpret_cast<uint32_t *>(a.idx + (v0 + e) * a.idx_stride)[w] = word;
      }
      if (lane == 0) a.norms[v0 + e] = nw[e];
    }

    // ---- stage 2: sign words
    if constexpr (M > 0) {
      float z[EV][CM];
#pragma unroll
      for (int e = 0; e < EV; ++e)
#pragma unroll
        for (int c = 0; c < CM; ++c) z[e][c] = 0.0f;
      multi_product<D, CM>(a.sketch, M, wl[0], wl[1], s.xs, z);  // ends with a barrier
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        if (v0 + e >= a.n) break;  // uniform over the wavefront
        uint64_t masks[CM];
#pragma unroll
        for (int c = 0; c < CM; ++c) {
          const int j = lane + kWave * c;
          bool bit = z[e][c] >= 0.0f;
          const bool amb = (j < M) && !(fabsf(z[e][c]) > band[c] * rbound[e]);
          uint64_t am = __ballot(amb);
          while (am) {  // rows the fp32 band cannot decide, one at a time
            const int src = __ffsll((unsigned long long)am) - 1;
            const int j0 = src + kWave * c;
            for (int k = lane; k < D; k += kWave) s.terms[k] = (double)a.sketch[(int64_t)j0 * D + k] * (double)s.xs[e][k];
            wave_lds_fence();
            int sg = 0;
            if (lane == 0) {
              double zz = 0.0, bb = 0.0;
              for (int k = 0; k < D; ++k) {
                zz += s.terms[k];
                bb += fabs(s.terms[k]);
              }
              if (fabs(zz) > 2.0 * (D + 2) * 0x1p-53 * bb) sg = zz > 0.0 ? 1 : -1;
              else if (bb == 0.0) sg = 0;
              else sg = expansion_sign(s.terms, D, s.buf);
            }
            wave_lds_fence();
            sg = __shfl(sg, 0, kWave);
            if (lane == src) bit = sg >= 0;
            am &= am - 1;
          }
          masks[c] = __ballot((j < M) && bit);
        }
        uint32_t *out = reinterpret_cast<uint32_t *>(a.sign + (v0 + e) * a.sign_stride);
        for (int w = lane; w < sw; w += kWave) {
          uint32_t word = 0;
#pragma unroll
          for (int c = 0; c < CM; ++c)
            if ((w >> 1) == c) word = (w & 1) ? (uint32_t)(masks[c] >> 32) : (uint32_t)masks[c];
          out[w] = word;
        }
      }
    }
    wave_lds_fence();  // the next group overwrites this wavefront's LDS
  }
}

// ------------------------------------------------------------------ MFMA encode (d = 64, 128)
//
// Persistent workgroups of NW wavefronts; every wavefront runs its own passes of 32 vectors
// (two 16-vector tiles) with no workgroup barrier after set-up.  At set-up the workgroup
// splits Pi and S into bf16 hi + lo parts and stores them in LDS as MFMA A fragments of
// v_mfma_f32_16x16x32_bf16 (lane l holds A[l%16][8(l/16) + 0..7]).  The input is the B
// operand (lane l holds B[8(l/16) + j][l%16] = x[vector l%16][32 ks + 8(l/16) + j]), read from
// HBM straight into registers as one 16-byte chunk per lane and k-step.
//
// The rows of Pi and S are stored permuted: row m of 16-row tile t is output coordinate
// tile_coord(t, m).  The MFMA result D[4(l/16) + i][l%16] of the tile pair (2u, 2u+1) then
// gives lane l the 8 consecutive coordinates 32u + 8(l/16) + 0..7 of vector l%16 -- the same
// coordinates the lane holds of the input, and exactly the B operand of the next product.
// So per vector, four lanes (l%16 fixed) each own 32 coordinates through the whole pass:
//   1. exact fp16 norm of the input: fp64 sum over the lane's values, reduced over the four
//      lanes; where the fp64 bound cannot decide, Shewchuk's expansion (one lane);
//   2. y = Pi x: hi*x + lo*x (+ hi*x_lo when the input is not bf16), fp32 accumulation;
//   3. indices and residual on the lane's own coordinates; the index fields of the four
//      lanes are OR-combined by lane shuffles into whole words;
//   4. exact fp16 norm of the residual, as in 1;
//   5. z = S r by the same split MFMA (S_hi r_hi + S_hi r_lo + S_lo r_hi).  Its error is below
//      2^-13 ||S_j|| ||r|| (bf16 split error 3 * 2^-16 plus 3d fp32 additions); outside that
//      band the sign of z is the sign of the exact dot product; inside it the wavefront
//      computes the fp64 dot product with its error bound and, if still undecided, the exact
//      expansion.  Each lane's 8 sketch rows form one byte of the sign stream.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Output coordinate of row m of 16-row tile t (see above).
__device__ __forceinline__ int tile_coord(int t, int m) {
  return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}

// bf16 hi/lo split of 8 floats: hi = RNE(x), lo = RNE(x - hi); x - hi is exact in fp32.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)__fsub_rn(x[j], (float)h);
  }
}

// fp16 candidate for sqrt(s) and whether the fp64 sum s (error <= (D+2) u s) decides it.
template <int D>
__device__ __forceinline__ uint32_t f16_norm_candidate(double s, bool &ok) {
  const double slack = 4.0 * (D + 2) * 0x1p-53;
  const uint32_t h = f64_to_f16_rne(sqrt(s));
  ok = h < 0x7C00u;
  if (ok) {
    const double vh = f16_bits_to_double_ext(h);
    const double up = 0.5 * (vh + f16_bits_to_double_ext(h + 1));
    if (!(s < up * up * (1.0 - slack))) ok = false;
    if (h > 0) {
      const double dn = 0.5 * (vh + f16_bits_to_double_ext(h - 1));
      if (!(s > dn * dn * (1.0 + slack))) ok = false;
    }
  }
  return h;
}

// fp16 candidate for sqrt(s) where s is within relative 8 * 2^-24 of the exact sum of squares
// (fp32 partial sums of at most 8 terms, combined in fp64), and whether s decides it.  The
// squared fp16 midpoints are exact in fp32.  Below 2^-60 the exact norm is under 2^-29.9
// (even if fp32 underflow was flushed), which rounds to 0.
__device__ __forceinline__ uint32_t f16_norm_fast(double s, bool &ok) {
  const float sf = (float)s;
  if (sf < 0x1p-60f) {
    ok = true;
    return 0u;
  }
  const uint32_t h = (uint32_t)__half_as_ushort(__float2half_rn(__builtin_amdgcn_sqrtf(sf)));
  const float v = __half2float(__ushort_as_half((unsigned short)h));
  const float vu = h >= 0x7BFFu ? 65536.0f : __half2float(__ushort_as_half((unsigned short)(h + 1)));
  const float vd = h == 0u ? 0.0f : __half2float(__ushort_as_half((unsigned short)(h - 1)));
  const float mu = 0.5f * (v + vu), md = 0.5f * (v + vd);
  const double e = 20.0 * 0x1p-24;  // 2.5 times the partial sums' error bound
  ok = sf <= 0x1p32f && h < 0x7C00u && s < (double)(mu * mu) * (1.0 - e) &&
       (h == 0u || s > (double)(md * md) * (1.0 + e));
  return h;
}

// idx = #{ j : y >= thr[j] } for ascending thr, by binary descent: bit b of idx compares y
// with the threshold that splits what the higher bits left; the candidates of each level are
// selected from registers as soon as the bit above is known.
template <int BITS>
__device__ __forceinline__ uint32_t quantize_index(float y, const float (&t)[(1 << BITS) - 1]) {
  static_assert(BITS >= 2 && BITS <= 4, "index widths");
  if constexpr (BITS == 2) {
    const bool b1 = y >= t[1];
    const bool b0 = y >= (b1 ? t[2] : t[0]);
    return (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
  } else if constexpr (BITS == 3) {
    const bool b2 = y >= t[3];
    const float c1 = b2 ? t[5] : t[1];
    const float ca = b2 ? t[6] : t[2];
    const float cb = b2 ? t[4] : t[0];
    const bool b1 = y >= c1;
    const bool b0 = y >= (b1 ? ca : cb);
    return (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
  } else {
    const bool b3 = y >= t[7];
    const float c2 = b3 ? t[11] : t[3];
    const float p1a = b3 ? t[13] : t[5], p1b = b3 ? t[9] : t[1];
    const float p11 = b3 ? t[14] : t[6], p10 = b3 ? t[12] : t[4];
    const float p01 = b3 ? t[10] : t[2], p00 = b3 ? t[8] : t[0];
    const bool b2 = y >= c2;
    const float c1 = b2 ? p1a : p1b;
    const float q1 = b2 ? p11 : p01, q0 = b2 ? p10 : p00;
    const bool b1 = y >= c1;
    const bool b0 = y >= (b1 ? q1 : q0);
    return (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
  }
}

// An opaque copy of x: conversions of it inside a rarely taken loop stay in that loop instead of
// being hoisted in front of it, where they would hold two registers per element for the whole
// pass.
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Exact fp16 RNE of sqrt(sum of terms[0..cnt)), starting from candidate h: compares the exact
// sum with squared fp16 midpoints (each exact in fp64).  terms needs cnt + 1 entries, buf
// cnt + 1.  Run by one lane.
__device__ uint32_t f16_norm_exact(double *terms, int cnt, uint32_t h, double *buf) {
  uint32_t hh = h >= 0x7C00u ? 0x7BFFu : h;
  while (hh < 0x7C00u) {
    const double mu = 0.5 * (f16_bits_to_double_ext(hh) + f16_bits_to_double_ext(hh + 1));
    terms[cnt] = -(mu * mu);
    const int cmp = expansion_sign(terms, cnt + 1, buf);
    if (cmp > 0 || (cmp == 0 && ((hh + 1) & 1u) == 0)) ++hh;
    else break;
  }
  while (hh > 0) {
    const double mu = 0.5 * (f16_bits_to_double_ext(hh - 1) + f16_bits_to_double_ext(hh));
    terms[cnt] = -(mu * mu);
    const int cmp = expansion_sign(terms, cnt + 1, buf);
    if (cmp < 0 || (cmp == 0 && ((hh - 1) & 1u) == 0)) --hh;
    else break;
  }
  return hh;
}

// Store the A fragments of the row-permuted, bf16-split matrix W [rows][D] (fp32, row-major):
// frag[((t * KS + ks) * 2 + hl) * 64 + lane] = 8 bf16 of part hl (0 = hi, 1 = lo) of
// W[tile_coord(t, lane % 16)][32 ks + 8 (lane / 16) + 0..7].
template <int D>
__device__ void build_afrags(const float *W, int rows, uint4 *frag, int nthreads) {
  constexpr int KS = D / 32;
  for (int e = threadIdx.x; e < (rows / 16) * KS * 64; e += nthreads) {
    const int lane = e % 64, ks = (e / 64) % KS, t = e / (64 * KS);
    const float *src = W + (int64_t)tile_coord(t, lane % 16) * D + 32 * ks + 8 * (lane / 16);
    float v[8];
    const float4 a = reinterpret_cast<const float4 *>(src)[0], b = reinterpret_cast<const float4 *>(src)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    bf16x8 hi, lo;
    split8(v, hi, lo);
    frag[((t * KS + ks) * 2 + 0) * 64 + lane] = __builtin_bit_cast(uint4, hi);
    frag[((t * KS + ks) * 2 + 1) * 64 + lane] = __builtin_bit_cast(uint4, lo);
  }
}

__device__ __forceinline__ bf16x8 afrag(const uint4 *frag, int t, int ks, int hl, int KS) {
  return __builtin_bit_cast(bf16x8, frag[((t * KS + ks) * 2 + hl) * 64 + lane_id()]);
}

// The 8 input elements of a lane for one k-step, as floats.
template <int TIN, int U4>
__device__ __forceinline__ void raw_to_f32(const uint4 (&r)[U4], float (&x)[8]) {
  if constexpr (U4 == 2) {
    const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(w[j]);
  } else {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      if constexpr (TIN == TQ_F16) x[j] = __half2float(__ushort_as_half((unsigned short)h));
      else x[j] = bf16_bits_to_float((uint16_t)h);
    }
  }
}

// 16-vector tiles per wavefront pass: two share each Pi / S fragment read from LDS.  At d = 128
// an input that needs a lo part takes one (else the registers spill), and so does a codec
// without sketch, whose one-tile passes fit 4 wavefronts per SIMD (latency is what bounds it).
// ---- recursive polar stage as the MFMA encoder's epilogue (tq_polar_encode, d = 64, 128)
//
// Same record and decisions as polar_encode_kernel: A, B the children's fp32 sums of squares,
// index #{ j : fl32(B cos^2 tau_j) >= fl32(A sin^2 tau_j) } with the level's table.  Lane
// (n, g) holds coordinates 32u + 8g + 0..7 of vector n, so levels 1-3 (pairs, quads, octets)
// stay in the lane; level 4 pairs lanes g, g ^ 1 (one shuffle), level 5 lanes g, g ^ 2, and the
// levels above combine the lane's own octet groups u.  A node's field goes into the staged
// record (LDS, zeroed per tile) by an LDS OR; every lane of a vector computes the shared nodes
// with the same operands, and one of them stores each.

template <int D>
constexpr int log2_d() { return D == 64 ? 6 : D == 128 ? 7 : 8; }

// OR `width` (<= 32) bits of val into the LDS record at bit p.
__device__ __forceinline__ void or_field(uint32_t *rec, int p, uint32_t val, int width) {
  const int w = p >> 5, o = p & 31;
  atomicOr(&rec[w], val << o);
  if (o + width > 32) atomicOr(&rec[w + 1], val >> (32 - o));
}

// Thresholds of one level (cos^2 tau, sin^2 tau) from the LDS copy of the tables.
template <int NA>
struct PolarLevelTh {
  float c2[NA - 1], s2[NA - 1];
  __device__ __forceinline__ void load(const float *ptab, int level) {
#pragma unroll
    for (int j = 0; j < NA - 1; ++j) {
      c2[j] = ptab[(2 * level) * NA + j];
      s2[j] = ptab[(2 * level + 1) * NA + j];
    }
  }
  __device__ __forceinline__ uint32_t decide(float A, float B) const {
    uint32_t k = 0;
#pragma unroll
    for (int j = 0; j < NA - 1; ++j) k += (__fmul_rn(B, c2[j]) >= __fmul_rn(A, s2[j])) ? 1u : 0u;
    return k;
  }
};

// QJL: the records are followed by the stage-1 residual on the lane's own coordinates, which
// replaces yv: u^ from the root down (fp32 products in the order of the decoder: a node's value
// times its level's cos or sin, the children of the lane's own nodes only), r = fl32(y -
// fl32(nbar u^)); the norm words are then left to the caller.  pcs: cos and sin of every
// level, [level][2][2^AB].
template <int D, int AB, int NV, int KS, bool QJL>
__device__ void polar_tail(float (&yv)[NV][KS][8], const uint32_t (&n16)[NV], int64_t v0, const EncArgs &a,
                           uint32_t *stg, const float *ptab, const float *pcs) {
  constexpr int NA = 1 << AB, WP = 2 + AB, NP = D / 2, P0 = NP * WP;
  constexpr int NWD = (P0 + (NP - 1) * AB + 31) / 32;  // record words
  constexpr int LV = log2_d<D>();
  static_assert(KS == D / 32 && (D == 64 || D == 128), "lane layout");
  const int lane = lane_id(), n = lane & 15, g = lane >> 4;
  const int sw = (int)(a.idx_stride >> 2);
  uint32_t *bitsw = reinterpret_cast<uint32_t *>(a.idx);
  auto node_bit = [](int l, int i) { return P0 + AB * (NP - (D >> (l - 1)) + i); };
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    for (int e = lane; e < 16 * NWD; e += kWave) stg[e] = 0u;
    wave_lds_fence();
    uint32_t *rec = stg + n * NWD;
    // level 1: pairs 16u + 4g + p (p < 4), one run of 4 fields per octet
    float s1[KS][4];
    uint32_t f1[KS][4], k2s[KS][2], k3s[KS], k4s[KS], k5s[KS], khs[LV + 1][(D >> 6) > 0 ? (D >> 6) : 1];
    {
      PolarLevelTh<NA> th;
      th.load(ptab, 0);
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        uint32_t run = 0u;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float ya = yv[t][u][2 * p], yb = yv[t][u][2 * p + 1];
          const float A = __fmul_rn(ya, ya), B = __fmul_rn(yb, yb);
          const uint32_t f = (ya < 0.0f ? 1u : 0u) | (yb < 0.0f ? 2u : 0u) | (th.decide(A, B) << 2);
          f1[u][p] = f;
          run |= f << (WP * p);
          s1[u][p] = __fadd_rn(A, B);
        }
        or_field(rec, WP * (16 * u + 4 * g), run, 4 * WP);
      }
    }
    // level 2: nodes 8u + 2g + {0, 1}
    float s2[KS][2];
    {
      PolarLevelTh<NA> th;
      th.load(ptab, 1);
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const uint32_t k0 = th.decide(s1[u][0], s1[u][1]), k1 = th.decide(s1[u][2], s1[u][3]);
        k2s[u][0] = k0;
        k2s[u][1] = k1;
        s2[u][0] = __fadd_rn(s1[u][0], s1[u][1]);
        s2[u][1] = __fadd_rn(s1[u][2], s1[u][3]);
        or_field(rec, node_bit(2, 8 * u + 2 * g), k0 | (k1 << AB), 2 * AB);
      }
    }
    // level 3: node 4u + g
    float s3[KS];
    {
      PolarLevelTh<NA> th;
      th.load(ptab, 2);
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        k3s[u] = th.decide(s2[u][0], s2[u][1]);
        or_field(rec, node_bit(3, 4 * u + g), k3s[u], AB);
        s3[u] = __fadd_rn(s2[u][0], s2[u][1]);
      }
    }
    // level 4: node 2u + (g >> 1) from the level-3 nodes of lanes g & ~1 (A) and g | 1 (B)
    float s4[KS];
    {
      PolarLevelTh<NA> th;
      th.load(ptab, 3);
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const float o = __shfl_xor(s3[u], 16, kWave);
        const float A = (g & 1) ? o : s3[u], B = (g & 1) ? s3[u] : o;
        const uint32_t k = th.decide(A, B);
        k4s[u] = k;
        if ((g & 1) == 0) or_field(rec, node_bit(4, 2 * u + (g >> 1)), k, AB);
        s4[u] = __fadd_rn(A, B);
      }
    }
    // level 5: node u from the level-4 nodes of lanes g & ~2 (A) and g | 2 (B)
    float cur[KS];
    {
      PolarLevelTh<NA> th;
      th.load(ptab, 4);
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const float o = __shfl_xor(s4[u], 32, kWave);
        const float A = (g & 2) ? o : s4[u], B = (g & 2) ? s4[u] : o;
        const uint32_t k = th.decide(A, B);
        k5s[u] = k;
        if (g == 0) or_field(rec, node_bit(5, u), k, AB);
        cur[u] = __fadd_rn(A, B);
      }
    }
    // levels 6 .. L: the octet groups u within the lane (every lane holds the same values)
#pragma unroll
    for (int l = 6; l <= LV; ++l) {
      PolarLevelTh<NA> th;
      th.load(ptab, l - 1);
      const int cnt = D >> l;
#pragma unroll
      for (int i = 0; i < cnt; ++i) {
        const uint32_t k = th.decide(cur[2 * i], cur[2 * i + 1]);
        khs[l][i] = k;
        if (g == 0) or_field(rec, node_bit(l, i), k, AB);
        cur[i] = __fadd_rn(cur[2 * i], cur[2 * i + 1]);
      }
    }
    wave_lds_fence();
    // the tile's 16 records -> HBM (pad words zero), then the norm words
    for (int e = lane; e < 16 * sw; e += kWave) {
      const int vv = e / sw, w = e % sw;
      const int64_t v = v0 + 16 * t + vv;
      if (v < a.n) bitsw[v * sw + w] = w < NWD ? stg[vv * NWD + w] : 0u;
    }
    wave_lds_fence();
    if constexpr (QJL) {
      constexpr int NA2 = 2 * NA;
      auto cs = [&](int level, bool sn, uint32_t k) { return pcs[(level - 1) * NA2 + (sn ? NA : 0) + k]; };
      // level-5 node values from the root (every lane the same), then the lane's own subtree
      float v5[KS];
      v5[0] = 1.0f;
#pragma unroll
      for (int l = LV; l >= 6; --l) {
#pragma unroll
        for (int i = (D >> l) - 1; i >= 0; --i) {
          const float pv = v5[i];
          v5[2 * i] = __fmul_rn(pv, cs(l, false, khs[l][i]));
          v5[2 * i + 1] = __fmul_rn(pv, cs(l, true, khs[l][i]));
        }
      }
      const float nbar = f16_bits_to_float(n16[t]);
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const float v4 = __fmul_rn(v5[u], cs(5, ((g >> 1) & 1) != 0, k5s[u]));
        const float v3 = __fmul_rn(v4, cs(4, (g & 1) != 0, k4s[u]));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float v2 = __fmul_rn(v3, cs(3, c != 0, k3s[u]));
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float rp = __fmul_rn(v2, cs(2, e != 0, k2s[u][c]));
            const int p = 2 * c + e;
            const uint32_t f = f1[u][p], k = f >> 2;
            float ua = __fmul_rn(rp, cs(1, false, k)), ub = __fmul_rn(rp, cs(1, true, k));
            if (f & 1u) ua = -ua;
            if (f & 2u) ub = -ub;
            yv[t][u][2 * p] = __fsub_rn(yv[t][u][2 * p], __fmul_rn(nbar, ua));
            yv[t][u][2 * p + 1] = __fsub_rn(yv[t][u][2 * p + 1], __fmul_rn(nbar, ub));
          }
        }
      }
    } else {
      const int64_t v = v0 + 16 * t + n;
      if (g == 0 && v < a.n) a.norms[v] = n16[t];
    }
  }
}

// 16-vector tiles per wavefront pass: one at d = 128 (the registers of a second tile cost more
// occupancy than its shared work saves), two at d = 64
template <int D, int M, int TIN, bool PRE>
constexpr int enc_tiles() {
  return (D == 128) ? 1 : 2;
}
// wavefronts per workgroup (one workgroup per CU, the A fragments in LDS): 16 where the pass
// fits 128 VGPRs, 12 where it fits 168 and the fragments of Pi and S leave room for 12
// wavefronts' staging (bf16 2-bit keys with a sketch)
template <int D, int BITS, int M, int TIN, bool PRE>
constexpr int enc_waves() {
  return (D == 128 && M == 0 && !PRE && TIN == TQ_BF16 && BITS <= 3)   ? 16
         : (D == 128 && M == D && !PRE && TIN == TQ_BF16 && BITS == 2) ? 12
                                                                        : 8;
}

// AB > 0: the recursive polar stage with AB angle bits (M = 0; a.thresholds holds the polar
// tables, a.idx / a.idx_stride the records) in place of steps 3-5.
template <int D, int BITS, int M, int TIN, bool PRE, int NW, bool ROTS, int AB = 0>
__global__ __launch_bounds__(NW * 64) void encode_mfma(EncArgs a) {
  constexpr int KS = D / 32;   // k-steps; also 8-coordinate groups u per lane
  constexpr int CT = D / 16;   // 16-row tiles of y
  constexpr int MT = M / 16;   // 16-row tiles of z
  constexpr int L = 1 << BITS;
  constexpr bool XLO = !PRE && TIN != TQ_BF16;            // input needs a lo part
  constexpr int NV = enc_tiles<D, M, TIN, PRE>();
  constexpr int U4 = (PRE || TIN == TQ_F32) ? 2 : 1;      // 16-byte chunks per 8 elements
  constexpr int EB = (PRE || TIN == TQ_F32) ? 4 : 2;
  constexpr int IWV = D * BITS / 32;                       // index words per vector
  static_assert(D % 32 == 0 && (M == 0 || M == D), "supported shapes");

  __shared__ uint4 fpi[PRE ? 1 : CT * KS * 2 * 64];
  __shared__ uint4 fsk[M > 0 ? MT * KS * 2 * 64 : 1];
  // per wavefront: the exact-fallback terms and buffer, also the staging of packed records
  __shared__ __align__(16) double wscr[NW][2 * (D + 2)];
  __shared__ float cbs[L];
  __shared__ float smax_s;
  // polar: cos^2 tau and sin^2 tau of every level, [level][2][2^AB]
  __shared__ float ptab[AB > 0 ? log2_d<D>() * 2 * (1 << AB) : 1];
  static_assert(AB == 0 || ((M == 0 || M == D) && 16 * ((D / 2 * (2 + AB) + (D / 2 - 1) * AB + 31) / 32) * 4 <=
                                                       2 * (D + 2) * 8),
                "polar records of a tile fit the staging");
  // polar with the QJL stage: cos and sin of every level, [level][2][2^AB]
  __shared__ float pcs[AB > 0 && M > 0 ? log2_d<D>() * 2 * (1 << AB) : 1];

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  double *xt = wscr[wid], *xb = wscr[wid] + (D + 2);
  uint8_t *stg = reinterpret_cast<uint8_t *>(wscr[wid]);
  constexpr int IB = D * BITS / 8;  // index bytes per vector
  constexpr int SB = M / 8;         // sign bytes per vector
  static_assert(NV * 16 * IB <= 2 * (D + 2) * 8 && NV * 16 * SB <= 2 * (D + 2) * 8, "staging fits");
  if constexpr (AB == 0) {
    if (tid < L) cbs[tid] = a.centroids[tid];
  } else {
    constexpr int NA = 1 << AB;
    for (int e = tid; e < log2_d<D>() * 2 * NA; e += NW * 64) {
      const int l = e / (2 * NA), r = e % (2 * NA);  // r < NA: cos^2 tau, else sin^2 tau
      ptab[e] = a.thresholds[(l * 4 + 2) * NA + r];
      if constexpr (M > 0) pcs[e] = a.thresholds[(l * 4) * NA + r];  // r < NA: cos, else sin
    }
  }
  if constexpr (!PRE && !ROTS) build_afrags<D>(a.rot, D, fpi, NW * 64);
  if constexpr (M > 0) {
    build_afrags<D>(a.sketch, M, fsk, NW * 64);
    if (wid == 0) {
      float mx = 0.0f;
      for (int q = lane; q < M; q += kWave) {
        double ss = 0.0;
        for (int k = 0; k < D; ++k) {
          const double v = a.sketch[(int64_t)q * D + k];
          ss += v * v;
        }
        mx = fmaxf(mx, (float)sqrt(ss));
      }
      mx = wave_max(mx);
      if (lane == 0) smax_s = mx * (1.0f + 0x1p-20f);
    }
  }
  float th[L - 1];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) th[j] = AB == 0 ? a.thresholds[j] : 0.0f;
  __syncthreads();
  const float smax = M > 0 ? smax_s : 0.0f;

  const int iw_all = (int)(a.idx_stride >> 2);
  const int sw_all = M > 0 ? (int)(a.sign_stride >> 2) : 0;
  uint32_t *idxw = reinterpret_cast<uint32_t *>(a.idx);
  uint32_t *sgnw = reinterpret_cast<uint32_t *>(a.sign);
  const int64_t wstep = (int64_t)gridDim.x * NW * 16 * NV;

  uint4 raw[NV][KS][U4];
  auto load_pass = [&](int64_t v0) {
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int64_t v = v0 + 16 * t + n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int w = 0; w < U4; ++w) {
          raw[t][ks][w] = make_uint4(0u, 0u, 0u, 0u);
          if (v < a.n)
            raw[t][ks][w] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(a.x) +
                                                             (v * a.ld_x + 32 * ks + 8 * g + 4 * w) * EB);
        }
    }
  };

  // One pass: vectors v0 .. v0 + 16 NV - 1; the input of the pass at vnext is loaded meanwhile.
  auto pass = [&](const int64_t v0, const int64_t vnext) {
    // ---- 1. exact fp16 norm of the input (of y in pre-rotated mode)
    uint32_t n16[NV];
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      double s = 0.0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float p = 0.0f;  // 8 squares, at most 8 roundings
        if constexpr (!PRE && TIN == TQ_BF16) {
          const uint32_t w[4] = {raw[t][ks][0].x, raw[t][ks][0].y, raw[t][ks][0].z, raw[t][ks][0].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 v = __builtin_bit_cast(bf16x2, w[i]);
            p = __builtin_amdgcn_fdot2_f32_bf16(v, v, p, false);
          }
        } else if constexpr (!PRE && TIN == TQ_F16) {
          const uint32_t w[4] = {raw[t][ks][0].x, raw[t][ks][0].y, raw[t][ks][0].z, raw[t][ks][0].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x2 v = __builtin_bit_cast(f16x2, w[i]);
            p = __builtin_amdgcn_fdot2(v, v, p, false);
          }
        } else {
          float x[8];
          raw_to_f32<TQ_F32, U4>(raw[t][ks], x);
#pragma unroll
          for (int j = 0; j < 8; ++j) p = fmaf(x[j], x[j], p);
        }
        s += (double)p;
      }
      s += __shfl_xor(s, 16, kWave);
      s += __shfl_xor(s, 32, kWave);
      bool ok;
      n16[t] = f16_norm_fast(s, ok);
      if (__ballot(!ok)) {
        // fp64 sum (error <= (D+2) u s), then the exact expansion where even that cannot decide
        double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float x[8];
          raw_to_f32<PRE ? TQ_F32 : TIN, U4>(raw[t][ks], x);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const double xj = opaque(x[j]);
            s4[j & 3] = fma(xj, xj, s4[j & 3]);
          }
        }
        double s64 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s64 += __shfl_xor(s64, 16, kWave);
        s64 += __shfl_xor(s64, 32, kWave);
        bool ok64;
        const uint32_t h64 = f16_norm_candidate<D>(s64, ok64);
        if (!ok) n16[t] = h64;
        uint64_t bad = __ballot(!ok && !ok64 && g == 0);
        while (bad) {
          const int n0 = __ffsll((unsigned long long)bad) - 1;
          if (n == n0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              float x[8];
              raw_to_f32<PRE ? TQ_F32 : TIN, U4>(raw[t][ks], x);
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const double xj = opaque(x[j]);
                xt[8 * KS * g + 8 * ks + j] = xj * xj;
              }
            }
          }
          wave_lds_fence();
          uint32_t h = 0;
          if (lane == n0) h = f16_norm_exact(xt, D, n16[t], xb);
          wave_lds_fence();
          h = (uint32_t)__shfl((int)h, n0, kWave);
          if (n == n0) n16[t] = h;
          bad &= bad - 1;
        }
      }
    }

    // ---- 2. y = Pi x (coordinates 32u + 8g + j of vector 16t + n in yv[t][u][j])
    float yv[NV][KS][8];
    if constexpr (PRE) {
#pragma unroll
      for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) raw_to_f32<TQ_F32, U4>(raw[t][ks], yv[t][ks]);
    } else {
      bf16x8 xh[NV][KS], xl[XLO ? NV : 1][XLO ? KS : 1];
#pragma unroll
      for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (TIN == TQ_BF16) {
            xh[t][ks] = __builtin_bit_cast(bf16x8, raw[t][ks][0]);
          } else {
            float x[8];
            raw_to_f32<TIN, U4>(raw[t][ks], x);
            split8(x, xh[t][ks], xl[t][ks]);
          }
        }
      f32x4 acc[NV][CT];
#pragma unroll
      for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[t][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // the hi and lo parts in separate sweeps: consecutive MFMAs update different tiles
#pragma unroll
      for (int hl = 0; hl < (XLO ? 3 : 2); ++hl)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const bf16x8 af = afrag(fpi, ct, ks, hl == 1 ? 1 : 0, KS);
#pragma unroll
            for (int t = 0; t < NV; ++t) {
              if constexpr (XLO) {
                acc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, hl == 2 ? xl[t][ks] : xh[t][ks], acc[t][ct], 0, 0, 0);
              } else {
                acc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xh[t][ks], acc[t][ct], 0, 0, 0);
              }
            }
          }
#pragma unroll
      for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int u = 0; u < KS; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) yv[t][u][j] = acc[t][2 * u + (j >> 2)][j & 3];
    }
    // the next pass's input is in flight while this one finishes (with a sketch, only once the
    // z products are issued: its registers are free then)
    if constexpr (M == 0) load_pass(vnext);
    if (a.y_tap) {
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int64_t v = v0 + 16 * t + n;
        if (v < a.n) {
#pragma unroll
          for (int u = 0; u < KS; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) a.y_tap[v * D + 32 * u + 8 * g + j] = yv[t][u][j];
        }
      }
    }
    if constexpr (AB > 0) {
      polar_tail<D, AB, NV, KS, (M > 0)>(yv, n16, v0, a, reinterpret_cast<uint32_t *>(wscr[wid]), ptab, pcs);
      if constexpr (M == 0) return;
    }
    // ---- 4. exact fp16 norm of the residual of tile t from s2, the fp64 sum of the lanes' fp32
    // partial sums of 8 squares (within 8u of the exact sum): the fp64 sum where that cannot
    // decide, then the exact expansion (one vector at a time)
    uint32_t rn16[NV];
    double rn2[NV];
    auto resid_norm = [&](const int t, double s2) {
      s2 += __shfl_xor(s2, 16, kWave);
      s2 += __shfl_xor(s2, 32, kWave);
      bool ok;
      rn16[t] = f16_norm_fast(s2, ok);
      if (__ballot(!ok)) {
        double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int u = 0; u < KS; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const double rj = opaque(yv[t][u][j]);
            s4[j & 3] = fma(rj, rj, s4[j & 3]);
          }
        double s64 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s64 += __shfl_xor(s64, 16, kWave);
        s64 += __shfl_xor(s64, 32, kWave);
        s2 = s64;
        bool ok64;
        const uint32_t h64 = f16_norm_candidate<D>(s64, ok64);
        if (!ok) rn16[t] = h64;
        uint64_t bad = __ballot(!ok && !ok64 && g == 0);
        while (bad) {
          const int n0 = __ffsll((unsigned long long)bad) - 1;
          if (n == n0) {
#pragma unroll
            for (int u = 0; u < KS; ++u)
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const double rj = opaque(yv[t][u][j]);
                xt[8 * KS * g + 8 * u + j] = rj * rj;
              }
          }
          wave_lds_fence();
          uint32_t h = 0;
          if (lane == n0) h = f16_norm_exact(xt, D, rn16[t], xb);
          wave_lds_fence();
          h = (uint32_t)__shfl((int)h, n0, kWave);
          if (n == n0) rn16[t] = h;
          bad &= bad - 1;
        }
      }
      rn2[t] = s2;
    };
    if constexpr (AB > 0) {
      // the QJL stage on the polar residual (yv): its norm, then the signs below
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        double s2 = 0.0;
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) p = fmaf(yv[t][u][j], yv[t][u][j], p);
          s2 += (double)p;
        }
        resid_norm(t, s2);
        const int64_t v = v0 + 16 * t + n;
        if (g == 0 && v < a.n) a.norms[v] = (rn16[t] << 16) | n16[t];
      }
    } else {
      // ---- 3. indices and residual (their norm by resid_norm)
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const float nbar = f16_bits_to_float(n16[t]);
        float thr[L - 1];
#pragma unroll
        for (int j = 0; j < L - 1; ++j) thr[j] = __fmul_rn(nbar, th[j]);
        double s2 = 0.0;
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          uint32_t qv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) qv[j] = quantize_index<BITS>(yv[t][u][j], thr);
          uint32_t field = 0u;  // 8 * BITS bits: coordinates 32u + 8g + 0..7
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float r = __fsub_rn(yv[t][u][j], __fmul_rn(nbar, cbs[qv[j]]));
            yv[t][u][j] = r;
            p = fmaf(r, r, p);
            field |= qv[j] << (BITS * j);
          }
          s2 += (double)p;
          // the field is bytes BITS (4u + g) .. + BITS - 1 of the vector's index record
          uint8_t *dst = stg + IB * (16 * t + n) + BITS * (4 * u + g);
          if constexpr (BITS == 2) {
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)field;
          } else if constexpr (BITS == 4) {
            *reinterpret_cast<uint32_t *>(dst) = field;
          } else {
            dst[0] = (uint8_t)field;
            dst[1] = (uint8_t)(field >> 8);
            dst[2] = (uint8_t)(field >> 16);
          }
        }
        // staged index records of tile t -> HBM, 8 bytes per lane and step
        wave_lds_fence();
        for (int e = lane; e < 16 * IB / 8; e += kWave) {
          const int vv = e / (IB / 8), w = e % (IB / 8);
          const int64_t v = v0 + 16 * t + vv;
          if (v < a.n)
            *reinterpret_cast<uint2 *>(a.idx + v * a.idx_stride + 8 * w) =
                *reinterpret_cast<const uint2 *>(stg + IB * (16 * t + vv) + 8 * w);
        }
        wave_lds_fence();
        const int64_t v = v0 + 16 * t + n;
        if (g == 0 && v < a.n)
          for (int w = IWV; w < iw_all; ++w) idxw[v * iw_all + w] = 0u;
        resid_norm(t, s2);
        if (g == 0 && v < a.n) a.norms[v] = (hi_word(rn16[t], f16_bits_to_float(n16[t]), a.resid_scale) << 16) | n16[t];
      }
    }

    // ---- 5. sign bits of z = S r
    if constexpr (M > 0) {
      constexpr int NB = M / 32;  // sign bytes per lane per tile: sketch rows 32b + 8g + 0..7
      float tau[NV];
      double rbound[NV];
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        // A tiny r (products near the fp32 underflow) leaves every sign to the fp64 path,
        // except r = 0 exactly: then z = 0 exactly and every bit is 1.
        const bool tiny = rn2[t] < 1e-30;
        bool zero = false;
        if (__ballot(tiny)) {
          float rmax = 0.0f;
#pragma unroll
          for (int u = 0; u < KS; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) rmax = fmaxf(rmax, fabsf(yv[t][u][j]));
          rmax = fmaxf(rmax, __shfl_xor(rmax, 16, kWave));
          rmax = fmaxf(rmax, __shfl_xor(rmax, 32, kWave));
          zero = rmax == 0.0f;
        }
        tau[t] = zero ? -1.0f : (tiny ? INFINITY : 0x1p-13f * smax * (float)sqrt(rn2[t]));
        // an upper bound on smax ||r|| for the fp64 test: rn2 is the sum of squares within
        // relative 2^-19 (fp32 partial sums of 8 squares; squares below the fp32 range add at
        // most 2^-19 of a sum >= 1e-30); a tiny r leaves every undecided row to the expansion
        rbound[t] = tiny ? INFINITY : (double)smax * sqrt(rn2[t]) * (1.0 + 0x1p-16);
      }
      uint32_t sb[NV][NB];
      // one 16-vector tile at a time: z for every sketch tile, r split into bf16 hi/lo one
      // k-step at a time
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        f32x4 z[NB][2];
#pragma unroll
        for (int b = 0; b < NB; ++b) z[b][0] = z[b][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          bf16x8 rh, rl;
          split8(yv[t][u], rh, rl);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const bf16x8 h0 = afrag(fsk, 2 * b, u, 0, KS), l0 = afrag(fsk, 2 * b, u, 1, KS);
            const bf16x8 h1 = afrag(fsk, 2 * b + 1, u, 0, KS), l1 = afrag(fsk, 2 * b + 1, u, 1, KS);
            z[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, rh, z[b][0], 0, 0, 0);
            z[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, rh, z[b][1], 0, 0, 0);
            z[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, rl, z[b][0], 0, 0, 0);
            z[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, rl, z[b][1], 0, 0, 0);
            z[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l0, rh, z[b][0], 0, 0, 0);
            z[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l1, rh, z[b][1], 0, 0, 0);
          }
        }
        if (t == NV - 1) load_pass(vnext);
        // bit = 1 - sign bit of z (a z of either zero is undecided, so this is z >= 0 wherever
        // it is used); undecided when |z| <= tau
        uint32_t am[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          uint32_t neg = 0u, amb = 0u;
          // rows 4h + i from the top down: each step shifts one bit in
#pragma unroll
          for (int k = 7; k >= 0; --k) {
            const float zz = z[b][k >> 2][k & 3];
            neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(zz), 31);
            amb = 2u * amb + (fabsf(zz) <= tau[t] ? 1u : 0u);
          }
          sb[t][b] = neg ^ 0xFFu;
          am[b] = amb;
        }
        // Undecided signs, all vectors of the tile at once: the four lanes of a vector agree on
        // its lowest undecided sketch row q, each takes the fp64 products over its own 32
        // coordinates, and two exchanges give the dot product and its error bound.
        for (;;) {
          int myq = 0xFF;
#pragma unroll
          for (int b = NB - 1; b >= 0; --b)
            if (am[b]) myq = 32 * b + 8 * g + (__ffs(am[b]) - 1);
          int q = min(myq, __shfl_xor(myq, 16, kWave));
          q = min(q, __shfl_xor(q, 32, kWave));
          if (__ballot(q != 0xFF) == 0) break;
          const bool act = q != 0xFF;
          double ps = 0.0;
          if (act) {
#pragma unroll
            for (int u = 0; u < KS; ++u) {
              const float4 *srow = reinterpret_cast<const float4 *>(a.sketch + (int64_t)q * D + 32 * u + 8 * g);
              const float4 s0 = srow[0], s1 = srow[1];
              const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
              for (int j = 0; j < 8; ++j) ps = fma((double)sv[j], (double)opaque(yv[t][u][j]), ps);
            }
          }
          ps += __shfl_xor(ps, 16, kWave);
          ps += __shfl_xor(ps, 32, kWave);
          // D/4 fused steps per lane and two exchanges, each rounding once: error <= (D/4 + 2)
          // 2^-53 sum_k |S_qk r_k| <= (D/4 + 2) 2^-53 ||S_q|| ||r||, with smax >= ||S_q|| and
          // rbound >= ||r|| (the test below allows 2 (D + 2) 2^-53 of it)
          const bool dec = fabs(ps) > 2.0 * (D + 2) * 0x1p-53 * rbound[t];
          int sg = ps > 0.0 ? 1 : -1;
          // where even fp64 cannot decide: the exact expansion, one vector at a time
          uint64_t und = __ballot(act && !dec && g == 0);
          while (und) {
            const int n0 = __ffsll((unsigned long long)und) - 1;
            const int q0 = __shfl(q, n0, kWave);
            if (n == n0) {
#pragma unroll
              for (int u = 0; u < KS; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                  xt[8 * KS * g + 8 * u + j] =
                      (double)a.sketch[(int64_t)q0 * D + 32 * u + 8 * g + j] * (double)opaque(yv[t][u][j]);
            }
            wave_lds_fence();
            int e = 0;
            if (lane == n0) e = expansion_sign(xt, D, xb);
            wave_lds_fence();
            e = __shfl(e, n0, kWave);
            if (n == n0) sg = e >= 0 ? 1 : -1;
            und &= und - 1;
          }
          // the lane holding row q records the bit
          if (act && g == ((q >> 3) & 3)) {
            const int b0 = q >> 5, bit = q & 7;
#pragma unroll
            for (int b = 0; b < NB; ++b)
              if (b == b0) {
                sb[t][b] = (sb[t][b] & ~(1u << bit)) | ((sg >= 0 ? 1u : 0u) << bit);
                am[b] &= ~(1u << bit);
              }
          }
        }
      }
      // sign byte b of lane g is byte 4b + g of the vector's sign record
#pragma unroll
      for (int t = 0; t < NV; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) stg[SB * (16 * t + n) + 4 * b + g] = (uint8_t)sb[t][b];
      wave_lds_fence();
      for (int e = lane; e < NV * 16 * SB / 8; e += kWave) {
        const int vv = e / (SB / 8), w = e % (SB / 8);
        const int64_t v = v0 + vv;
        if (v < a.n)
          *reinterpret_cast<uint2 *>(a.sign + v * a.sign_stride + 8 * w) =
              *reinterpret_cast<const uint2 *>(stg + SB * vv + 8 * w);
      }
      wave_lds_fence();
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int64_t v = v0 + 16 * t + n;
        if (v < a.n && g == 0)
          for (int w = NB; w < sw_all; ++w) sgnw[v * sw_all + w] = 0u;
      }
    }
  };

  if constexpr (!ROTS) {
    int64_t v0 = ((int64_t)blockIdx.x * NW + wid) * 16 * NV;
    load_pass(v0);
    for (; v0 < a.n; v0 += wstep) pass(v0, v0 + wstep);
  } else {
    // Per-block rotations: a workgroup takes whole rotation blocks (vectors v with
    // (first + v) / vecs_per_rot = rb; the last rotation also takes everything beyond), rebuilds
    // the Pi fragments for each, and its wavefronts split the block's passes.  The launcher
    // guarantees that first and vecs_per_rot are multiples of 32, so no pass straddles blocks.
    const int64_t vpr = a.vecs_per_rot;
    const int64_t step = (int64_t)NW * 16 * NV;
    for (int64_t rb = blockIdx.x;; rb += gridDim.x) {
      int64_t bs = rb * vpr - a.first;
      if (bs < 0) bs = 0;
      if (bs >= a.n) break;
      const bool last = rb >= a.n_rot - 1;
      int64_t be = last ? a.n : (rb + 1) * vpr - a.first;
      if (be > a.n) be = a.n;
      __syncthreads();  // every wavefront is done with the previous block's fragments
      build_afrags<D>(a.rot + (last ? a.n_rot - 1 : rb) * (int64_t)D * D, D, fpi, NW * 64);
      __syncthreads();
      int64_t v0 = bs + (int64_t)wid * 16 * NV;
      load_pass(v0);
      for (; v0 < be; v0 += step) pass(v0, v0 + step < be ? v0 + step : a.n);
      if (last) break;
    }
  }
}

template <int D, int BITS, int M, int TIN, bool PRE, bool ROTS = false, int AB = 0>
static void launch_mfma(const EncArgs &a, hipStream_t st) {
  constexpr int NW = ROTS ? 8 : enc_waves<D, BITS, M, TIN, PRE>();
  constexpr int PER_BLOCK = NW * 16 * enc_tiles<D, M, TIN, PRE>();
  int64_t blocks = ROTS ? a.n_rot : (a.n + PER_BLOCK - 1) / PER_BLOCK;
  if (blocks > 256) blocks = 256;
  hipLaunchKernelGGL((encode_mfma<D, BITS, M, TIN, PRE, NW, ROTS, AB>), dim3((unsigned)blocks), dim3(NW * 64), 0, st, a);
}

// The recursive polar stage on the MFMA encoder (d = 64, 128; input rows 16-byte aligned; with
// per-block rotations, blocks and first multiples of 32 and, at d = 128, bf16 input), with or
// without the QJL stage on its residual (M = D).  Returns TQ_EUNSUPPORTED where these do not
// hold (the caller then takes polar_encode_kernel).
template <int D, int AB, int M>
static int launch_polar_mfma_da(const EncArgs &a, int dt, bool pre, hipStream_t st) {
  const int eb = dt == TQ_F32 ? 4 : 2;
  const bool vec_ok = ((uintptr_t)a.x % 16 == 0) && ((a.ld_x * eb) % 16 == 0);
  const bool rots = a.n_rot > 1 && a.vecs_per_rot > 0;
  if (!vec_ok) return TQ_EUNSUPPORTED;
  if (rots) {
    if (pre || a.vecs_per_rot % 32 != 0 || a.first % 32 != 0 || (D == 128 && dt != TQ_BF16)) return TQ_EUNSUPPORTED;
    if (dt == TQ_BF16) launch_mfma<D, 2, M, TQ_BF16, false, true, AB>(a, st);
    else if constexpr (D == 64) {
      if (dt == TQ_F32) launch_mfma<D, 2, M, TQ_F32, false, true, AB>(a, st);
      else launch_mfma<D, 2, M, TQ_F16, false, true, AB>(a, st);
    }
  } else if (pre) {
    launch_mfma<D, 2, M, TQ_F32, true, false, AB>(a, st);
  } else if (dt == TQ_F32) {
    launch_mfma<D, 2, M, TQ_F32, false, false, AB>(a, st);
  } else if (dt == TQ_F16) {
    launch_mfma<D, 2, M, TQ_F16, false, false, AB>(a, st);
  } else {
    launch_mfma<D, 2, M, TQ_BF16, false, false, AB>(a, st);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

int launch_polar_mfma(const PolarView &pc, const void *x, int dt, int64_t n, int64_t ld_x, bool pre, int64_t first,
                      const PolarCodesView &out, float *y_tap, void *stream) {
  EncArgs a{x, ld_x, n, first, pc.rot, pc.n_rot, pc.vecs_per_rot, pc.sketch, nullptr, pc.tables,
            out.bits, out.stride, out.sign, out.sign_stride, out.norms, y_tap, nullptr, 0, 0, 0.0f, 0.0f};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#define TQ_PM(DD, AA)                                                              \
  if (pc.d == DD && pc.ab == AA) {                                                 \
    if (pc.m == 0) return launch_polar_mfma_da<DD, AA, 0>(a, dt, pre, st);         \
    if (pc.m == DD) return launch_polar_mfma_da<DD, AA, DD>(a, dt, pre, st);       \
    return TQ_EUNSUPPORTED;                                                        \
  }
  TQ_PM(64, 2) TQ_PM(64, 3) TQ_PM(64, 4) TQ_PM(128, 2) TQ_PM(128, 3) TQ_PM(128, 4)
#undef TQ_PM
  return TQ_EUNSUPPORTED;
}

template <int D, int BITS, int M>
static int launch_enc_dm(const EncArgs &a, int dt, bool pre, hipStream_t st) {
  if constexpr (D == 64 || D == 128) {
    if (a.pos == nullptr) {  // append mode takes encode_kernel below
      const int eb = dt == TQ_F32 ? 4 : 2;
      const bool vec_ok = ((uintptr_t)a.x % 16 == 0) && ((a.ld_x * eb) % 16 == 0);
      const bool rots = a.n_rot > 1 && a.vecs_per_rot > 0;
      // per-block rotations on the MFMA path where the blocks align with passes (and, at d = 128,
      // for bf16 input, whose registers leave room for the block loop)
      if (rots && vec_ok && !pre && a.vecs_per_rot % 32 == 0 && a.first % 32 == 0 && (D == 64 || dt == TQ_BF16)) {
        if constexpr (D == 64) {
          if (dt == TQ_F32) launch_mfma<D, BITS, M, TQ_F32, false, true>(a, st);
          else if (dt == TQ_F16) launch_mfma<D, BITS, M, TQ_F16, false, true>(a, st);
          else if (dt == TQ_BF16) launch_mfma<D, BITS, M, TQ_BF16, false, true>(a, st);
          else return TQ_EINVAL;
        } else {
          launch_mfma<D, BITS, M, TQ_BF16, false, true>(a, st);
        }
        return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
      }
      if (!rots && vec_ok) {
        if (pre) {
          if (dt != TQ_F32) return TQ_EINVAL;
          launch_mfma<D, BITS, M, TQ_F32, true>(a, st);
        } else if (dt == TQ_F32) {
          launch_mfma<D, BITS, M, TQ_F32, false>(a, st);
        } else if (dt == TQ_F16) {
          launch_mfma<D, BITS, M, TQ_F16, false>(a, st);
        } else if (dt == TQ_BF16) {
          launch_mfma<D, BITS, M, TQ_BF16, false>(a, st);
        } else {
          return TQ_EINVAL;
        }
        return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
      }
    }
  }
  if constexpr (D % 32 != 0) {
    // one shared rotation outside append mode: several vectors per wavefront
    if (a.pos == nullptr && !(a.n_rot > 1 && a.vecs_per_rot > 0)) {
      int64_t blocks = (a.n + kMultiVec * kMultiWaves - 1) / (kMultiVec * kMultiWaves);
      if (blocks > 256 * 2) blocks = 256 * 2;
      dim3 grid((unsigned)blocks), block(kWave * kMultiWaves);
      if (pre) {
        if (dt != TQ_F32) return TQ_EINVAL;
        hipLaunchKernelGGL((encode_multi<D, BITS, M, TQ_F32, true>), grid, block, 0, st, a);
      } else if (dt == TQ_F32) {
        hipLaunchKernelGGL((encode_multi<D, BITS, M, TQ_F32, false>), grid, block, 0, st, a);
      } else if (dt == TQ_F16) {
        hipLaunchKernelGGL((encode_multi<D, BITS, M, TQ_F16, false>), grid, block, 0, st, a);
      } else if (dt == TQ_BF16) {
        hipLaunchKernelGGL((encode_multi<D, BITS, M, TQ_BF16, false>), grid, block, 0, st, a);
      } else {
        return TQ_EINVAL;
      }
      return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
    }
  }
  int64_t blocks = (a.n + kEncWaves - 1) / kEncWaves;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(kWave * kEncWaves);
  if (pre) {
    if (dt != TQ_F32) return TQ_EINVAL;
    hipLaunchKernelGGL((encode_kernel<D, BITS, M, TQ_F32, true>), grid, block, 0, st, a);
  } else if (dt == TQ_F32) {
    hipLaunchKernelGGL((encode_kernel<D, BITS, M, TQ_F32, false>), grid, block, 0, st, a);
  } else if (dt == TQ_F16) {
    hipLaunchKernelGGL((encode_kernel<D, BITS, M, TQ_F16, false>), grid, block, 0, st, a);
  } else if (dt == TQ_BF16) {
    hipLaunchKernelGGL((encode_kernel<D, BITS, M, TQ_BF16, false>), grid, block, 0, st, a);
  } else {
    return TQ_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

template <int D, int BITS>
static int launch_enc_d(const EncArgs &a, int m, int dt, bool pre, hipStream_t st) {
  if (m == 0) return launch_enc_dm<D, BITS, 0>(a, dt, pre, st);
  if (m == D) return launch_enc_dm<D, BITS, D>(a, dt, pre, st);
  return TQ_EUNSUPPORTED;
}

template <int D>
static int launch_enc_bits(const EncArgs &a, int bits, int m, int dt, bool pre, hipStream_t st) {
  switch (bits) {
    case 2: return launch_enc_d<D, 2>(a, m, dt, pre, st);
    case 3: return launch_enc_d<D, 3>(a, m, dt, pre, st);
    case 4: return launch_enc_d<D, 4>(a, m, dt, pre, st);
    default: return TQ_EUNSUPPORTED;
  }
}

int launch_append(const CodecView &c, const void *x, int dt, int64_t n_seq, int hkv, const int32_t *pos,
                  int64_t cap, float rope_base, const CodesView &out, void *stream) {
  if (n_seq == 0) return TQ_OK;
  EncArgs a{x, c.d, n_seq * hkv, 0, c.rot, c.n_rot, c.vecs_per_rot, c.sketch, c.centroids, c.thresholds,
            out.idx, out.idx_stride, out.sign, out.sign_stride, out.norms, nullptr, pos, cap, hkv, rope_base,
            c.resid_scale};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (c.d) {
    case 64: return launch_enc_bits<64>(a, c.bits, c.m, dt, false, st);
    case 128: return launch_enc_bits<128>(a, c.bits, c.m, dt, false, st);
    case 200: return launch_enc_bits<200>(a, c.bits, c.m, dt, false, st);
    default: return TQ_EUNSUPPORTED;
  }
}

int launch_encode(const CodecView &c, const void *x, int dt, int64_t n, int64_t ld_x, bool pre_rotated,
                  int64_t first, const CodesView &out, float *y_tap, void *stream) {
  if (n == 0) return TQ_OK;
  EncArgs a{x, ld_x, n, first, c.rot, c.n_rot, c.vecs_per_rot, c.sketch, c.centroids, c.thresholds,
            out.idx, out.idx_stride, out.sign, out.sign_stride, out.norms, y_tap, nullptr, 0, 0, 0.0f,
            c.resid_scale};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (c.d) {
    case 64: return launch_enc_bits<64>(a, c.bits, c.m, dt, pre_rotated, st);
    case 128: return launch_enc_bits<128>(a, c.bits, c.m, dt, pre_rotated, st);
    case 200: return launch_enc_bits<200>(a, c.bits, c.m, dt, pre_rotated, st);
    default: return TQ_EUNSUPPORTED;
  }
}

}  // namespace tq
