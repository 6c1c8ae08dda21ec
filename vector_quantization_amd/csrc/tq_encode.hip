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
// Layout: one wavefront per vector.  Lane l owns coordinates l + 64c (c < ceil(d/64)) and
// sketch rows l + 64c.  The index stream is packed from an LDS copy of the codes, the sign
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
};

constexpr int kEncWaves = 4;

template <int D>
struct EncLds {
  float xs[D];
  float rs[D];
  uint8_t code[D + 4];
  double terms[D + 2];
  double buf[D + 2];
};

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

template <int D, int BITS, int M, int TIN, bool PRE>
__global__ __launch_bounds__(kWave *kEncWaves) void encode_kernel(EncArgs a) {
  constexpr int C = (D + kWave - 1) / kWave;
  constexpr int CM = (M + kWave - 1) / kWave;
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
      int64_t rid = 0;
      if (a.n_rot > 1 && a.vecs_per_rot > 0) {
        rid = (a.first + v) / a.vecs_per_rot;
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
      reinterpret_cast<uint32_t *>(a.idx + v * a.idx_stride)[w] = word;
    }

    if constexpr (M > 0) {
      uint64_t masks[CM > 0 ? CM : 1];
#pragma unroll
      for (int c = 0; c < CM; ++c) {
        const int j = lane + kWave * c;
        double z = 0.0, bound = 0.0;
        if (j < M) {
          const float4 *row = reinterpret_cast<const float4 *>(a.sketch + (int64_t)j * D);
          for (int k4 = 0; k4 < D / 4; ++k4) {
            const float4 p = row[k4];
            const double t0 = (double)p.x * (double)s.rs[4 * k4 + 0];
            const double t1 = (double)p.y * (double)s.rs[4 * k4 + 1];
            const double t2 = (double)p.z * (double)s.rs[4 * k4 + 2];
            const double t3 = (double)p.w * (double)s.rs[4 * k4 + 3];
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
          for (int k = lane; k < D; k += kWave)
            s.terms[k] = (double)a.sketch[(int64_t)j0 * D + k] * (double)s.rs[k];
          wave_lds_fence();
          int sg = 0;
          if (lane == 0) sg = expansion_sign(s.terms, D, s.buf);
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
        reinterpret_cast<uint32_t *>(a.sign + v * a.sign_stride)[w] = word;
      }
    }
    if (lane == 0) a.norms[v] = (rn16 << 16) | n16;
    wave_lds_fence();
  }
}

template <int D, int BITS, int M>
static int launch_enc_dm(const EncArgs &a, int dt, bool pre, hipStream_t st) {
  const int64_t waves = (a.n + 0) ;
  int64_t blocks = (waves + kEncWaves - 1) / kEncWaves;
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

int launch_encode(const CodecView &c, const void *x, int dt, int64_t n, int64_t ld_x, bool pre_rotated,
                  int64_t first, const CodesView &out, float *y_tap, void *stream) {
  if (n == 0) return TQ_OK;
  EncArgs a{x, ld_x, n, first, c.rot, c.n_rot, c.vecs_per_rot, c.sketch, c.centroids, c.thresholds,
            out.idx, out.idx_stride, out.sign, out.sign_stride, out.norms, y_tap};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (c.d) {
    case 64: return launch_enc_bits<64>(a, c.bits, c.m, dt, pre_rotated, st);
    case 128: return launch_enc_bits<128>(a, c.bits, c.m, dt, pre_rotated, st);
    case 200: return launch_enc_bits<200>(a, c.bits, c.m, dt, pre_rotated, st);
    default: return TQ_EUNSUPPORTED;
  }
}

}  // namespace tq
