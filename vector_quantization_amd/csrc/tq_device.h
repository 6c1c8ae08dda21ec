// Device helpers for libtq kernels on gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <cstdint>

#include "../../include/tq.h"

namespace tq {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  return __half2float(__ushort_as_half((unsigned short)(b & 0xFFFFu)));
}

__host__ __device__ __forceinline__ double f16_bits_to_double_ext(uint32_t bits) {
  // value of a non-negative fp16 pattern; 0x7C00 stands for 65536 (the overflow step)
  if (bits >= 0x7C00u) return 65536.0;
  const uint32_t e = bits >> 10, f = bits & 0x3FFu;
  if (e == 0) return (double)f * 0x1p-24;
  return ((double)(1024u + f)) * ldexp(1.0, (int)e - 25);
}

// Round a non-negative double to the nearest fp16 (ties to even); >= 65520 gives +inf.
__device__ __forceinline__ uint32_t f64_to_f16_rne(double v) {
  if (!(v < 65520.0)) return 0x7C00u;
  if (v < 0x1p-14) return (uint32_t)rint(v * 0x1p24);  // subnormal grid 2^-24 (may reach 0x400)
  int e2;
  (void)frexp(v, &e2);          // v = f 2^e2, f in [0.5, 1)
  const int E = e2 - 1;         // v in [2^E, 2^(E+1)), -14 <= E <= 15
  const double q = ldexp(v, 10 - E);  // [1024, 2048)
  const uint32_t r = (uint32_t)rint(q);
  return (uint32_t)((E + 15) << 10) + (r - 1024u);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over aligned groups of K lanes (K = 1, 2, 4, 8 or 16), result in every lane of the group,
// with DPP moves inside 16-lane rows instead of LDS permutes: two quad permutations give the sum
// of each quad; the half-row mirror pairs each lane with one of the other quad of its 8 lanes,
// the row mirror with one of the other 8 lanes of its row.
template <int K>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8 || K == 16, "groups of up to 16 lanes");
  if constexpr (K >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  if constexpr (K >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  if constexpr (K >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  if constexpr (K >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Max over the whole wavefront, uniform result: DPP within each 16-lane row (as group_sum_dpp),
// then the four row maxima read as scalars.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- exact sums

// Knuth's TwoSum: s + e == a + b exactly.
__device__ __forceinline__ void two_sum(double a, double b, double &s, double &e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Exact sign (-1, 0, +1) of the sum of n doubles, each exact, by Shewchuk's Grow-Expansion
// with zero elimination ("Adaptive Precision Floating-Point Arithmetic and Fast Robust
// Geometric Predicates", 1997): the running sum is kept as a non-overlapping expansion in
// increasing magnitude, whose last component carries the sign.  buf holds n doubles.
// Run by one lane.
__device__ inline int expansion_sign(const double *terms, int n, double *buf) {
  int len = 0;
  for (int k = 0; k < n; ++k) {
    double q = terms[k];
    int out = 0;
    for (int i = 0; i < len; ++i) {
      double s, h;
      two_sum(q, buf[i], s, h);
      q = s;
      if (h != 0.0) buf[out++] = h;
    }
    if (q != 0.0) buf[out++] = q;
    len = out;
  }
  if (len == 0) return 0;
  return buf[len - 1] > 0.0 ? 1 : -1;
}

// ---------------------------------------------------------------- encoder helpers

template <int TIN>
__device__ __forceinline__ float load_in(const void *p, int64_t off) {
  if constexpr (TIN == TQ_F32) return reinterpret_cast<const float *>(p)[off];
  else if constexpr (TIN == TQ_F16) return __half2float(reinterpret_cast<const __half *>(p)[off]);
  else return bf16_bits_to_float(reinterpret_cast<const uint16_t *>(p)[off]);
}

// fp16 bits of the exactly rounded norm of the D values held C per lane.
template <int D, int C>
__device__ uint32_t wave_norm_f16(const float (&v)[C], double *terms, double *buf) {
  const int lane = lane_id();
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (lane + kWave * c < D) s += (double)v[c] * (double)v[c];
  s = wave_sum(s);  // every lane holds the same value (the butterfly is symmetric)
  const double slack = 4.0 * (D + 2) * 0x1p-53;
  uint32_t h = f64_to_f16_rne(sqrt(s));
  bool ok = h < 0x7C00u;
  if (ok) {
    const double vh = f16_bits_to_double_ext(h);
    const double up = 0.5 * (vh + f16_bits_to_double_ext(h + 1));
    if (!(s < up * up * (1.0 - slack))) ok = false;
    if (h > 0) {
      const double dn = 0.5 * (vh + f16_bits_to_double_ext(h - 1));
      if (!(s > dn * dn * (1.0 + slack))) ok = false;
    }
  }
  if (ok) return h;
  // Exact decision: compare the exact sum of squares with squared midpoints.
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (lane + kWave * c < D) terms[lane + kWave * c] = (double)v[c] * (double)v[c];
  wave_lds_fence();
  uint32_t hh = h >= 0x7C00u ? 0x7BFFu : h;
  if (lane == 0) {
    while (hh < 0x7C00u) {
      const double mu = 0.5 * (f16_bits_to_double_ext(hh) + f16_bits_to_double_ext(hh + 1));
      terms[D] = -(mu * mu);
      const int cmp = expansion_sign(terms, D + 1, buf);
      if (cmp > 0 || (cmp == 0 && ((hh + 1) & 1u) == 0)) ++hh;
      else break;
    }
    while (hh > 0) {
      const double mu = 0.5 * (f16_bits_to_double_ext(hh - 1) + f16_bits_to_double_ext(hh));
      terms[D] = -(mu * mu);
      const int cmp = expansion_sign(terms, D + 1, buf);
      if (cmp < 0 || (cmp == 0 && ((hh - 1) & 1u) == 0)) --hh;
      else break;
    }
  }
  wave_lds_fence();
  return (uint32_t)__shfl((int)hh, 0, kWave);
}

// RoPE of the D-vector x (LDS) at position p: coordinate i < D/2 turns with i + D/2 by the angle
// p * base^(-2i/D), in fp64; `first` and `step` spread the D/2 pairs over the calling threads.
template <int D>
__device__ __forceinline__ void rope_pairs(float *x, int64_t p, float base, int first, int step) {
  const double lb = log2((double)base);
  for (int i = first; i < D / 2; i += step) {
    const double ang = (double)p * exp2(-2.0 * i / D * lb);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double x0 = x[i], x1 = x[i + D / 2];
    x[i] = (float)(x0 * cs - x1 * sn);
    x[i + D / 2] = (float)(x0 * sn + x1 * cs);
  }
}

// RoPE of one vector held in LDS, by one wavefront (TurboESM summary, "Metodologia" A: the
// positional rotation comes before the orthogonal one); ends with the wave's LDS fence.
template <int D>
__device__ void wave_rope_lds(float *xs, int64_t p, float rope_base) {
  rope_pairs<D>(xs, p, rope_base, lane_id(), kWave);
  wave_lds_fence();
}

// The sign words of one vector's QJL stage, by one wavefront: bit j (lane j + 64c's row) is
// [ sum_k S_jk r_k >= 0 ] of the exact real dot product, for r in LDS (rs[D], fp32).  Lane j
// sums its rows' fp64 products (each exact) with an error bound; rows whose sum the bound cannot
// decide are settled one at a time by the exact expansion (terms and buf: LDS scratch of D + 2
// doubles).  The sign stream (sw words) is written to out, pad bits zero.
template <int D, int M>
__device__ void wave_sign_words(const float *sketch, const float *rs, double *terms, double *buf, uint32_t *out,
                                int sw) {
  constexpr int CM = (M + kWave - 1) / kWave;
  const int lane = lane_id();
  uint64_t masks[CM > 0 ? CM : 1];
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    const int j = lane + kWave * c;
    double z = 0.0, bound = 0.0;
    if (j < M) {
      const float4 *row = reinterpret_cast<const float4 *>(sketch + (int64_t)j * D);
      for (int k4 = 0; k4 < D / 4; ++k4) {
        const float4 p = row[k4];
        const double t0 = (double)p.x * (double)rs[4 * k4 + 0];
        const double t1 = (double)p.y * (double)rs[4 * k4 + 1];
        const double t2 = (double)p.z * (double)rs[4 * k4 + 2];
        const double t3 = (double)p.w * (double)rs[4 * k4 + 3];
        z += t0; z += t1; z += t2; z += t3;
        bound += fabs(t0) + fabs(t1) + fabs(t2) + fabs(t3);
      }
    }
    bool bit = z >= 0.0;
    bool amb = (j < M) && (fabs(z) <= 2.0 * (D + 2) * 0x1p-53 * bound);
    // rows whose fp64 sum cannot decide the sign: exact expansion, one row at a time
    uint64_t am = __ballot(amb);
    while (am) {
      const int src = __ffsll((unsigned long long)am) - 1;
      const int j0 = src + kWave * c;
      for (int k = lane; k < D; k += kWave) terms[k] = (double)sketch[(int64_t)j0 * D + k] * (double)rs[k];
      wave_lds_fence();
      int sg = 0;
      if (lane == 0) sg = expansion_sign(terms, D, buf);
      wave_lds_fence();
      sg = __shfl(sg, 0, kWave);
      if (lane == src) bit = sg >= 0;
      am &= am - 1;
    }
    masks[c] = __ballot((j < M) && bit);
  }
  for (int w = lane; w < sw; w += kWave) {
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      if ((w >> 1) == c) word = (w & 1) ? (uint32_t)(masks[c] >> 32) : (uint32_t)masks[c];
    }
    out[w] = word;
  }
}

// The W 32-bit words of one record at p, in 16-, 8- or 4-byte loads by W (record strides
// and base pointers aligned to that width).
template <int W>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t (&w)[W]) {
  if constexpr (W % 4 == 0) {
    const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = p4[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (W % 2 == 0) {
    const uint2 *p2 = reinterpret_cast<const uint2 *>(p);
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const uint2 v = p2[i];
      w[2 * i] = v.x; w[2 * i + 1] = v.y;
    }
  } else {
    const uint32_t *p1 = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p1[i];
  }
}

}  // namespace tq
