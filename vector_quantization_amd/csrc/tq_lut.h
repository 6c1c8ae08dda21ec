// Lookup-table scoring of compressed keys against full-precision queries.
//
// The estimator (7minutos.es TurboQuant walkthrough, "Etapa 2 (Corrección Residual)", K~ =
// K^ + K~_QJL, taken in the rotated space; hada.io TurboQuant page: the query stays in high
// precision) is
//     s = nbar * sum_i q~_i c[idx_i] + rnbar * sqrt(pi/2)/m * sum_j q^_j (2 b_j - 1)
// with q~ = Pi q and q^ = S q~.  Both sums split over fixed groups of index bits: a group of
// GB bits holds CPG = GB / bits coordinates (GB = 8 for 2- and 4-bit codes, 6 for 3-bit
// codes) and a sign byte holds 8 sketch rows.  For one query, each group position p has a
// table T_p[beta] = sum over the group's coordinates of q~_i c[code_i(beta)], and each sign
// byte position a table U_p[beta] = sum_t q^_{8p+t} (2 bit_t(beta) - 1).  Scoring a key is
// then one LDS lookup per group, summed in fp32.
//
// Several query heads that read the same kv head (GQA) share one lookup: an entry holds G
// heads' values.  G = 1 and 2 store fp32; G = 4 stores fp16 values scaled per head by a
// power of two (so the largest possible entry is about 2^14), which keeps the LDS footprint
// at 8 bytes per entry; sums stay fp32.
#pragma once

#include "tq_device.h"

namespace tq {

template <int D, int BITS, int M, int G>
struct Lut {
  static constexpr int L = 1 << BITS;
  static constexpr int GB = (BITS == 3) ? 6 : 8;
  static constexpr int CPG = GB / BITS;
  static constexpr int NG = D / CPG;
  static constexpr int TS = 1 << GB;
  static constexpr int NQ = M / 8;
  static constexpr bool F16 = (G == 4);
  static constexpr int EB = (G == 1) ? 4 : 8;  // entry bytes
  static constexpr int MSE_BYTES = NG * TS * EB;
  static constexpr int QJL_BYTES = NQ * 256 * EB;
  static constexpr int BYTES = MSE_BYTES + QJL_BYTES;
  static constexpr int IW = (D * BITS + 31) / 32;  // index words per key
  static constexpr int SW = (M + 31) / 32;         // sign words per key
  static_assert(D % CPG == 0, "d must be a multiple of the coordinates per lookup");
  static_assert(M % 8 == 0, "m must be a multiple of 8");
};

template <int G>
struct HeadScales {
  float inv_m[G];  // undo the per-head fp16 table scaling (1 for fp32 tables)
  float inv_q[G];
};

// Power-of-two scale 2^e with 2^e * bound <= 2^14 (bound > 0), as float.
__device__ __forceinline__ float pow2_scale_for(float bound) {
  if (!(bound > 0.0f)) return 1.0f;
  int e;
  (void)frexpf(bound, &e);  // bound < 2^e
  int s = 14 - e;
  s = s > 100 ? 100 : (s < -100 ? -100 : s);
  return ldexpf(1.0f, s);
}

// Build the tables of G query heads in LDS.  qt [G][D] and qh [G][M] (fp32) and the codebook
// cb [L] are in LDS; scale_m/scale_q are the per-head table scales (1 for fp32 tables).
// All threads of the block participate; the caller synchronises afterwards.
template <int D, int BITS, int M, int G, int NT>
__device__ void build_luts(uint8_t *mse, uint8_t *qjl, const float *qt, const float *qh, const float *cb,
                           const float *scale_m, const float *scale_q) {
  using C = Lut<D, BITS, M, G>;
  for (int e = threadIdx.x; e < C::NG * C::TS; e += NT) {
    const int p = e / C::TS, beta = e % C::TS;
    float v[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < C::CPG; ++t) {
        const int code = (beta >> (BITS * t)) & (C::L - 1);
        acc = fmaf(qt[h * D + C::CPG * p + t], cb[code], acc);
      }
      v[h] = acc * scale_m[h];
    }
    if constexpr (G == 1) {
      reinterpret_cast<float *>(mse)[e] = v[0];
    } else if constexpr (G == 2) {
      reinterpret_cast<float2 *>(mse)[e] = make_float2(v[0], v[1]);
    } else {
      const uint32_t lo = (uint32_t)__half_as_ushort(__float2half_rn(v[0])) |
                          ((uint32_t)__half_as_ushort(__float2half_rn(v[1])) << 16);
      const uint32_t hi = (uint32_t)__half_as_ushort(__float2half_rn(v[2])) |
                          ((uint32_t)__half_as_ushort(__float2half_rn(v[3])) << 16);
      reinterpret_cast<uint2 *>(mse)[e] = make_uint2(lo, hi);
    }
  }
  if constexpr (M > 0) {
    for (int e = threadIdx.x; e < C::NQ * 256; e += NT) {
      const int p = e >> 8, beta = e & 255;
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x = qh[h * M + 8 * p + t];
          acc += ((beta >> t) & 1) ? x : -x;
        }
        v[h] = acc * scale_q[h];
      }
      if constexpr (G == 1) {
        reinterpret_cast<float *>(qjl)[e] = v[0];
      } else if constexpr (G == 2) {
        reinterpret_cast<float2 *>(qjl)[e] = make_float2(v[0], v[1]);
      } else {
        const uint32_t lo = (uint32_t)__half_as_ushort(__float2half_rn(v[0])) |
                            ((uint32_t)__half_as_ushort(__float2half_rn(v[1])) << 16);
        const uint32_t hi = (uint32_t)__half_as_ushort(__float2half_rn(v[2])) |
                            ((uint32_t)__half_as_ushort(__float2half_rn(v[3])) << 16);
        reinterpret_cast<uint2 *>(qjl)[e] = make_uint2(lo, hi);
      }
    }
  }
}

// Per-head table scales: fp32 tables use 1; fp16 tables use 2^e so that the largest entry
// bound (CPG max|c| max|q~| or 8 max|q^|) maps to at most 2^14.  Computed by every wave
// redundantly from qt/qh in LDS (values identical across waves).
template <int D, int BITS, int M, int G>
__device__ void table_scales(const float *qt, const float *qh, float cmax, float *scale_m, float *scale_q,
                             HeadScales<G> &hs) {
  using C = Lut<D, BITS, M, G>;
  const int lane = lane_id();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float sm = 1.0f, sq = 1.0f;
    if constexpr (C::F16) {
      float a = 0.0f;
      for (int i = lane; i < D; i += kWave) a = fmaxf(a, fabsf(qt[h * D + i]));
      a = wave_max(a);
      sm = pow2_scale_for(a * cmax * C::CPG);
      if constexpr (M > 0) {
        float b = 0.0f;
        for (int i = lane; i < M; i += kWave) b = fmaxf(b, fabsf(qh[h * M + i]));
        b = wave_max(b);
        sq = pow2_scale_for(b * 8.0f);
      }
    }
    scale_m[h] = sm;
    scale_q[h] = sq;
    hs.inv_m[h] = 1.0f / sm;
    hs.inv_q[h] = 1.0f / sq;
  }
}

// acc[h] += entry[h] * inv[h].  For fp16 entries this is one v_fma_mix_f32 per head (the
// fp16 operand is widened inside the FMA; inv is the exact power-of-two descale).
template <int G, bool F16>
__device__ __forceinline__ void lut_accumulate(const uint8_t *tab, int entry, float (&acc)[G], const float (&inv)[G]) {
  if constexpr (G == 1) {
    acc[0] += reinterpret_cast<const float *>(tab)[entry];
  } else if constexpr (G == 2) {
    const float2 e = reinterpret_cast<const float2 *>(tab)[entry];
    acc[0] += e.x;
    acc[1] += e.y;
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint2 e = reinterpret_cast<const uint2 *>(tab)[entry];
    const h2 p = __builtin_bit_cast(h2, e.x);
    const h2 q = __builtin_bit_cast(h2, e.y);
    acc[0] = __builtin_fmaf((float)p.x, inv[0], acc[0]);
    acc[1] = __builtin_fmaf((float)p.y, inv[1], acc[1]);
    acc[2] = __builtin_fmaf((float)q.x, inv[2], acc[2]);
    acc[3] = __builtin_fmaf((float)q.y, inv[3], acc[3]);
  }
}

// Index group p of a key whose index words are in registers.
template <int BITS, int IW, int GB>
__device__ __forceinline__ int group_code(const uint32_t (&w)[IW], int p) {
  const int bit = p * GB;
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + GB > 32 && wi + 1 < IW) v |= w[wi + 1] << (32 - sh);
  return (int)(v & ((1u << GB) - 1));
}

// Score one key against the G heads whose tables are in LDS.  Returns the two sums (index
// part and sign part) per head, descaled to query units.
template <int D, int BITS, int M, int G>
__device__ __forceinline__ void lut_score(const uint32_t (&iw)[Lut<D, BITS, M, G>::IW],
                                          const uint32_t (&sw)[Lut<D, BITS, M, G>::SW > 0 ? Lut<D, BITS, M, G>::SW : 1],
                                          const uint8_t *mse, const uint8_t *qjl, const HeadScales<G> &hs,
                                          float (&am)[G], float (&aq)[G]) {
  using C = Lut<D, BITS, M, G>;
#pragma unroll
  for (int h = 0; h < G; ++h) am[h] = aq[h] = 0.0f;
#pragma unroll
  for (int p = 0; p < C::NG; ++p) {
    const int code = group_code<BITS, C::IW, C::GB>(iw, p);
    lut_accumulate<G, C::F16>(mse, p * C::TS + code, am, hs.inv_m);
  }
  if constexpr (M > 0) {
#pragma unroll
    for (int p = 0; p < C::NQ; ++p) {
      const int byte = (sw[p >> 2] >> (8 * (p & 3))) & 0xFF;
      lut_accumulate<G, C::F16>(qjl, p * 256 + byte, aq, hs.inv_q);
    }
  }
}

}  // namespace tq
