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
// heads' values.  G = 1 and 2 store fp32.  G = 4 stores each head's value as a 16-bit
// fixed-point integer (8 bytes per entry, so the four heads' tables of a 128-dimensional
// 2-bit + QJL key fit LDS), scaled per head and table so that the largest entry the table can
// hold maps to 32767; the 16-bit values are summed exactly in 32-bit integers and converted
// once per key.  The only rounding is the quantisation of each entry, at most half a unit of
// (largest entry) / 32767.
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
  static constexpr bool I16 = (G == 4);
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

// Four scaled values -> four 16-bit fixed-point integers (round to nearest, clamped to
// [-32767, 32767]), packed: v_cvt_pk_i16_i32 saturates at 32767, the explicit lower clamp keeps
// -32768 out.
__device__ __forceinline__ uint2 pack_i16x4(const float (&v)[4]) {
  int q[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) q[h] = (int)__builtin_rintf(fmaxf(v[h], -32767.0f));
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(q[0], q[1])),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(q[2], q[3])));
}

// Store one table entry of G heads (already scaled) at index e.
template <int G>
__device__ __forceinline__ void store_entry(uint8_t *tab, int e, const float (&v)[G]) {
  if constexpr (G == 1) {
    reinterpret_cast<float *>(tab)[e] = v[0];
  } else if constexpr (G == 2) {
    reinterpret_cast<float2 *>(tab)[e] = make_float2(v[0], v[1]);
  } else {
    reinterpret_cast<uint2 *>(tab)[e] = pack_i16x4(v);
  }
}

// LDS scratch of the half-table builder: for every index group and sign byte, the tables of its
// low and high halves (HS = 2^(GB/2) entries for an index group, 16 for a sign byte), G floats
// per entry.
template <int D, int BITS, int M, int G>
constexpr int lut_half_bytes() {
  using C = Lut<D, BITS, M, G>;
  return (C::NG * 2 * (1 << (C::GB / 2)) + C::NQ * 2 * 16) * G * 4;
}

// Build the tables of G query heads in LDS.  qt [G][D] and qh [G][M] (fp32) and the codebook
// cb [L] are in LDS; scale_m/scale_q are the per-head table scales (1 for fp32 tables).
// All threads of the block participate; the caller synchronises afterwards.
//
// With LDS scratch `half` (lut_half_bytes, 16-byte aligned), every entry is the sum of the
// entries of its two half-groups -- T_p[beta] = Tlo_p[beta mod HS] + Thi_p[beta / HS], and the
// same for the sign bytes -- which are built first.  This is the same sum of the same products,
// grouped in two, and costs two reads and one add per head instead of CPG (or 8) products.
// With half == nullptr each entry is summed directly.
template <int D, int BITS, int M, int G, int NT>
__device__ void build_luts(uint8_t *mse, uint8_t *qjl, const float *qt, const float *qh, const float *cb,
                           const float *scale_m, const float *scale_q, float *half = nullptr) {
  using C = Lut<D, BITS, M, G>;
  if (half != nullptr) {
    constexpr int HB = C::GB / 2;          // bits per half-group
    constexpr int HS = 1 << HB;            // entries per half table
    constexpr int HC = C::CPG / 2;         // coordinates per half-group
    static_assert(C::CPG % 2 == 0, "index groups split into two halves");
    constexpr int NHM = C::NG * 2 * HS;    // index half entries: [p][half][x]
    constexpr int NHQ = C::NQ * 2 * 16;    // sign half entries: [p][half][x]
    float *hm = half, *hq = half + NHM * G;
    for (int e = threadIdx.x; e < NHM + NHQ; e += NT) {
      float v[G];
      if (e < NHM) {
        const int p = e / (2 * HS), hf = (e / HS) & 1, x = e % HS;
        const int i0 = C::CPG * p + HC * hf;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.0f;
#pragma unroll
          for (int t = 0; t < HC; ++t) acc = fmaf(qt[h * D + i0 + t], cb[(x >> (BITS * t)) & (C::L - 1)], acc);
          v[h] = acc;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) hm[e * G + h] = v[h];
      } else if constexpr (M > 0) {
        const int f = e - NHM;
        const int p = f >> 5, hf = (f >> 4) & 1, x = f & 15;
        const int j0 = 8 * p + 4 * hf;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float y = qh[h * M + j0 + t];
            acc += ((x >> t) & 1) ? y : -y;
          }
          hq[f * G + h] = acc;
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < C::NG * C::TS; e += NT) {
      const int p = e / C::TS, beta = e % C::TS;
      const float *lo = hm + ((p * 2) * HS + (beta & (HS - 1))) * G;
      const float *hi = hm + ((p * 2 + 1) * HS + (beta >> HB)) * G;
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) v[h] = (lo[h] + hi[h]) * scale_m[h];
      store_entry<G>(mse, e, v);
    }
    if constexpr (M > 0) {
      for (int e = threadIdx.x; e < C::NQ * 256; e += NT) {
        const int p = e >> 8, beta = e & 255;
        const float *lo = hq + ((p * 2) * 16 + (beta & 15)) * G;
        const float *hi = hq + ((p * 2 + 1) * 16 + (beta >> 4)) * G;
        float v[G];
#pragma unroll
        for (int h = 0; h < G; ++h) v[h] = (lo[h] + hi[h]) * scale_q[h];
        store_entry<G>(qjl, e, v);
      }
    }
    return;
  }
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
      reinterpret_cast<uint2 *>(mse)[e] = pack_i16x4(v);
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
        reinterpret_cast<uint2 *>(qjl)[e] = pack_i16x4(v);
      }
    }
  }
}

// Per-head table scales.  fp32 tables use 1.  16-bit tables map the largest entry a table
// can hold -- max over positions of cmax * sum |q~| over the position's coordinates for the
// index tables, sum |q^| over the byte's rows for the sign tables -- to 32767.  Every wave
// computes the values redundantly from qt/qh in LDS (identical across waves).
template <int D, int BITS, int M, int G>
__device__ void table_scales(const float *qt, const float *qh, float cmax, float *scale_m, float *scale_q,
                             HeadScales<G> &hs) {
  using C = Lut<D, BITS, M, G>;
  const int lane = lane_id();
  // per-lane partial maxima of every head first, then the 2G wavefront reductions (DPP, no LDS)
  float pa[G], pb[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    pa[h] = pb[h] = 0.0f;
    if constexpr (C::I16) {
      for (int p = lane; p < C::NG; p += kWave) {
        float t = 0.0f;
#pragma unroll
        for (int u = 0; u < C::CPG; ++u) t += fabsf(qt[h * D + C::CPG * p + u]);
        pa[h] = fmaxf(pa[h], t);
      }
      if constexpr (M > 0) {
        for (int p = lane; p < C::NQ; p += kWave) {
          float t = 0.0f;
#pragma unroll
          for (int u = 0; u < 8; ++u) t += fabsf(qh[h * M + 8 * p + u]);
          pb[h] = fmaxf(pb[h], t);
        }
      }
    }
  }
  if constexpr (C::I16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pa[h] = wave_max_dpp(pa[h]);
      if constexpr (M > 0) pb[h] = wave_max_dpp(pb[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float sm = 1.0f, sq = 1.0f, im = 1.0f, iq = 1.0f;
    if constexpr (C::I16) {
      const float a = pa[h] * cmax;
      if (a > 0.0f) {
        sm = 32767.0f / a;
        im = a / 32767.0f;
      }
      if constexpr (M > 0) {
        const float b = pb[h];
        if (b > 0.0f) {
          sq = 32767.0f / b;
          iq = b / 32767.0f;
        }
      }
    }
    scale_m[h] = sm;
    scale_q[h] = sq;
    hs.inv_m[h] = im;
    hs.inv_q[h] = iq;
  }
}

// The per-head scales for a workgroup: wavefront 0 computes them (table_scales) and publishes
// them in LDS as sc[4G] = {scale_m[G], scale_q[G], inv_m[G], inv_q[G]}; after the barrier every
// thread takes its HeadScales from there.  One wavefront instead of all of them keeps the LDS
// reads and shuffles of the reductions off the other wavefronts.  Ends synchronised.
template <int D, int BITS, int M, int G>
__device__ void block_table_scales(const float *qt, const float *qh, const float *cb, float *sc, HeadScales<G> &hs) {
  using C = Lut<D, BITS, M, G>;
  if (threadIdx.x < kWave) {
    const float cmax = fmaxf(fabsf(cb[0]), fabsf(cb[C::L - 1]));
    float sm[G], sq[G];
    HeadScales<G> h0;
    table_scales<D, BITS, M, G>(qt, qh, cmax, sm, sq, h0);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sc[h] = sm[h];
        sc[G + h] = sq[h];
        sc[2 * G + h] = h0.inv_m[h];
        sc[3 * G + h] = h0.inv_q[h];
      }
    }
  }
  __syncthreads();
  // block-uniform: read into scalar registers, which keeps them out of the key loops' VGPRs
#pragma unroll
  for (int h = 0; h < G; ++h) {
    hs.inv_m[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sc[2 * G + h])));
    hs.inv_q[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sc[3 * G + h])));
  }
}

// A block-uniform byte offset the compiler cannot treat as a constant.  The sign tables start at
// the index tables' size, 64 KB for 2-bit keys at d = 128: with a constant base every sign
// group's address (beyond the 16-bit immediate offset of an LDS read) would take a register of
// its own; with this one base register each group's offset fits the reads' immediate field.
__device__ __forceinline__ int opaque_offset(int off) {
  asm volatile("" : "+s"(off));
  return off;
}

// acc[h] += entry[h] for fp32 tables (G = 1, 2); iacc[h] += entry[h] for 16-bit tables
// (G = 4: one v_dot2c_i32_i16 per head, the entry pair dotted with (1, 0) or (0, 1)).
template <int G>
__device__ __forceinline__ void lut_accumulate(const uint8_t *tab, int entry, float (&acc)[G], int (&iacc)[G]) {
  if constexpr (G == 1) {
    acc[0] += reinterpret_cast<const float *>(tab)[entry];
  } else if constexpr (G == 2) {
    const float2 e = reinterpret_cast<const float2 *>(tab)[entry];
    acc[0] += e.x;
    acc[1] += e.y;
  } else {
    typedef short s2 __attribute__((ext_vector_type(2)));
    const s2 lo = {1, 0}, hi = {0, 1};
    const uint2 e = reinterpret_cast<const uint2 *>(tab)[entry];
    const s2 x = __builtin_bit_cast(s2, e.x), y = __builtin_bit_cast(s2, e.y);
    iacc[0] = __builtin_amdgcn_sdot2(x, lo, iacc[0], false);
    iacc[1] = __builtin_amdgcn_sdot2(x, hi, iacc[1], false);
    iacc[2] = __builtin_amdgcn_sdot2(y, lo, iacc[2], false);
    iacc[3] = __builtin_amdgcn_sdot2(y, hi, iacc[3], false);
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
// part and sign part) per head, in query units.
template <int D, int BITS, int M, int G>
__device__ __forceinline__ void lut_score(const uint32_t (&iw)[Lut<D, BITS, M, G>::IW],
                                          const uint32_t (&sw)[Lut<D, BITS, M, G>::SW > 0 ? Lut<D, BITS, M, G>::SW : 1],
                                          const uint8_t *mse, const uint8_t *qjl, const HeadScales<G> &hs,
                                          float (&am)[G], float (&aq)[G]) {
  using C = Lut<D, BITS, M, G>;
  int im[G], iq[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    am[h] = aq[h] = 0.0f;
    im[h] = iq[h] = 0;
  }
  if constexpr (C::I16) {
    // 16-bit entries: the reads of a batch of groups are all issued before any is summed, so
    // that many table reads are in flight at once whatever else the caller keeps in registers
    constexpr int NT_ = C::NG + C::NQ;
    constexpr int B = 16;
#pragma unroll
    for (int p0 = 0; p0 < NT_; p0 += B) {
      uint2 e[B];
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int p = p0 + k;
        if (p < C::NG) {
          e[k] = reinterpret_cast<const uint2 *>(mse)[p * C::TS + group_code<BITS, C::IW, C::GB>(iw, p)];
        } else if constexpr (M > 0) {
          if (p < NT_) {
            const int q = p - C::NG;
            e[k] = reinterpret_cast<const uint2 *>(qjl)[q * 256 + ((sw[q >> 2] >> (8 * (q & 3))) & 0xFF)];
          }
        }
      }
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int p = p0 + k;
        if (p >= NT_) continue;
        typedef short s2 __attribute__((ext_vector_type(2)));
        const s2 lo = {1, 0}, hi = {0, 1};
        const s2 x = __builtin_bit_cast(s2, e[k].x), y = __builtin_bit_cast(s2, e[k].y);
        int *acc = p < C::NG ? im : iq;
        acc[0] = __builtin_amdgcn_sdot2(x, lo, acc[0], false);
        acc[1] = __builtin_amdgcn_sdot2(x, hi, acc[1], false);
        acc[2] = __builtin_amdgcn_sdot2(y, lo, acc[2], false);
        acc[3] = __builtin_amdgcn_sdot2(y, hi, acc[3], false);
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < C::NG; ++p) {
      const int code = group_code<BITS, C::IW, C::GB>(iw, p);
      lut_accumulate<G>(mse, p * C::TS + code, am, im);
    }
    if constexpr (M > 0) {
#pragma unroll
      for (int p = 0; p < C::NQ; ++p) {
        const int byte = (sw[p >> 2] >> (8 * (p & 3))) & 0xFF;
        lut_accumulate<G>(qjl, p * 256 + byte, aq, iq);
      }
    }
  }
  if constexpr (C::I16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      am[h] = (float)im[h] * hs.inv_m[h];
      aq[h] = (float)iq[h] * hs.inv_q[h];
    }
  }
}

}  // namespace tq
