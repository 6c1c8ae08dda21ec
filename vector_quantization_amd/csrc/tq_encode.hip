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

// ------------------------------------------------------------------ MFMA encode (d = 64, 128)
//
// Persistent workgroups of NTH threads.  Each wavefront keeps, in registers, the bf16 hi/lo
// split of its column slice of Pi^T and of S^T as MFMA B operands (loaded once).  Per tile
// of T vectors (T * d = 8192 elements):
//   1. the inputs go to LDS as fp32 (exact) and as a bf16 hi/lo split (A operand);
//   2. the exact fp16 norm of each input row (32 coordinates per thread, fp64 sums, exact
//      fallback as in encode_kernel);
//   3. y = x Pi^T with v_mfma_f32_16x16x16bf16_1k: hi*hi + hi*lo (+ lo*hi when the input is
//      not bf16), fp32 accumulation -- y within about 2^-16 of the exact product;
//   4. indices, residual and its exact fp16 norm, 32 coordinates per thread, index words
//      assembled in registers;
//   5. z = r S^T by the same split MFMA.  Its error is below 2^-13 ||S_j|| ||r||, so z decides
//      the sign bit outside that band; inside it a wavefront computes the fp64 dot product
//      and, if that is still undecided, the exact expansion -- the bit is always the sign of
//      the exact real dot product, as in encode_kernel.

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  const uint32_t h = bf16_rne_bits(x);
  hi = (uint16_t)h;
  lo = (uint16_t)bf16_rne_bits(__fsub_rn(x, bf16_bits_f(h)));
}

// B fragment of a 16x16x16 MFMA for rows n (output) and k-step ks of a row-major [rows][D]
// fp32 matrix W, B[k][n] = W[n][k]: lane l holds W[n0 + l%16][16 ks + 4 (l/16) + 0..3].
template <int D>
__device__ __forceinline__ void load_bfrag(const float *W, int n0, int ks, bf16x4 &hi, bf16x4 &lo) {
  const int l = lane_id();
  const float4 w = *reinterpret_cast<const float4 *>(W + (int64_t)(n0 + (l & 15)) * D + 16 * ks + 4 * (l >> 4));
  const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint16_t h, o;
    split_bf16(wv[j], h, o);
    hi[j] = (short)h;
    lo[j] = (short)o;
  }
}

template <int TPV>
__device__ __forceinline__ double group_sum(double v) {
  if constexpr (TPV >= 2) v += __shfl_xor(v, 1, kWave);
  if constexpr (TPV >= 4) v += __shfl_xor(v, 2, kWave);
  return v;
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

template <int D, int BITS, int M, int TIN, bool PRE, int NTH>
__global__ __launch_bounds__(NTH) void encode_mfma(EncArgs a) {
  constexpr int NW = NTH / kWave;  // wavefronts; each owns NCT / NW column tiles of y and z
  constexpr int T = NTH * 32 / D;  // vectors per tile (128)
  constexpr int TPV = D / 32;      // scalar threads per vector, 32 coordinates each
  constexpr int NRT = T / 16;
  constexpr int NCT = D / 16;
  constexpr int WCT = NCT / NW;
  constexpr int NKS = D / 16;
  constexpr int MCT = M / 16;
  constexpr int WMCT = M > 0 ? MCT / NW : 1;
  constexpr bool XLO = !PRE && TIN != TQ_BF16;  // input needs a lo part in bf16
  constexpr int L = 1 << BITS;
  constexpr int LDA = D + 8;
  constexpr int LDF = D + 1;
  constexpr int C = D / kWave;
  static_assert(NCT % NW == 0 && WCT >= 1 && (M == 0 || M == D), "supported shapes");

  __shared__ __align__(16) uint16_t ah[T * LDA];
  __shared__ __align__(16) uint16_t al[T * LDA];
  __shared__ float fv[T * LDF];
  __shared__ uint32_t nws[T];
  __shared__ float rn2[T];
  __shared__ uint32_t flag[T];
  __shared__ uint16_t sbits[T * (M > 0 ? MCT : 1)];
  __shared__ double xterms[NW][D + 2];
  __shared__ double xbuf[NW][D + 2];
  __shared__ float cbs[L], ths[L];

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  if (tid < L) cbs[tid] = a.centroids[tid];
  if (tid < L - 1) ths[tid] = a.thresholds[tid];

  bf16x4 ph[WCT][NKS], pl[WCT][NKS];
  bf16x4 sh[WMCT][NKS], sl[WMCT][NKS];
  float snorm[WMCT];
  if constexpr (!PRE) {
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) load_bfrag<D>(a.rot, 16 * (wid * WCT + ct), ks, ph[ct][ks], pl[ct][ks]);
  }
  if constexpr (M > 0) {
#pragma unroll
    for (int mc = 0; mc < WMCT; ++mc) {
      const int n0 = 16 * (wid * WMCT + mc);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) load_bfrag<D>(a.sketch, n0, ks, sh[mc][ks], sl[mc][ks]);
      double q = 0.0;
      for (int k = 0; k < D; ++k) {
        const double v = a.sketch[(int64_t)(n0 + (lane & 15)) * D + k];
        q += v * v;
      }
      snorm[mc] = (float)sqrt(q) * (1.0f + 0x1p-20f);
    }
  }
  __syncthreads();
  float thr_unused = ths[0];
  (void)thr_unused;

  const int vr = tid / TPV, ch = tid % TPV;
  const int iw_all = (int)(a.idx_stride >> 2);
  const int sw_all = M > 0 ? (int)(a.sign_stride >> 2) : 0;
  uint32_t *idxw = reinterpret_cast<uint32_t *>(a.idx);
  uint32_t *sgnw = reinterpret_cast<uint32_t *>(a.sign);

  // The tile is read as 16-byte chunks (8 bf16/fp16 or 4 fp32 elements of one row); the next
  // tile's chunks are loaded into registers while the current tile is processed.
  constexpr int EB = (TIN == TQ_F32) ? 4 : 2;
  constexpr int EPC = 16 / EB;               // elements per chunk
  constexpr int NCH = T * D / EPC / NTH;     // chunks per thread
  static_assert(D % EPC == 0 && (T * D / EPC) % NTH == 0, "tile chunking");
  uint4 pre[NCH];
  auto load_tile = [&](int64_t t0v) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int e = (tid + i * NTH) * EPC;
      const int64_t v = t0v + e / D;
      pre[i] = make_uint4(0u, 0u, 0u, 0u);
      if (v < a.n)
        pre[i] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(a.x) + (v * a.ld_x + e % D) * EB);
    }
  };
  load_tile((int64_t)blockIdx.x * T);
  for (int64_t tile = blockIdx.x; tile * T < a.n; tile += gridDim.x) {
    const int64_t v0 = tile * T;
    // ---- 1. the prefetched tile to LDS (fp32 values and the bf16 hi/lo split)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int e = (tid + i * NTH) * EPC;
      const int r = e / D, c0 = e % D;
      const uint32_t w[4] = {pre[i].x, pre[i].y, pre[i].z, pre[i].w};
#pragma unroll
      for (int u = 0; u < EPC; ++u) {
        float x;
        if constexpr (TIN == TQ_F32) x = __uint_as_float(w[u]);
        else if constexpr (TIN == TQ_F16) x = __half2float(__ushort_as_half((unsigned short)(w[u >> 1] >> (16 * (u & 1)))));
        else x = bf16_bits_to_float((uint16_t)(w[u >> 1] >> (16 * (u & 1))));
        const int c = c0 + u;
        fv[r * LDF + c] = x;
        if constexpr (!PRE) {
          uint16_t hi, lo;
          split_bf16(x, hi, lo);
          ah[r * LDA + c] = hi;
          if constexpr (XLO) al[r * LDA + c] = lo;
        } else {
          if (a.y_tap && v0 + r < a.n) a.y_tap[(v0 + r) * D + c] = x;
        }
      }
    }
    load_tile((tile + gridDim.x) * T);
    __syncthreads();
    // ---- 2. exact fp16 norm of the input rows
    {
      double s = 0.0;
#pragma unroll 8
      for (int k = 0; k < 32; ++k) {
        const double x = fv[vr * LDF + ch * 32 + k];
        s += x * x;
      }
      s = group_sum<TPV>(s);
      bool ok;
      const uint32_t h = f16_norm_candidate<D>(s, ok);
      if (ch == 0) {
        nws[vr] = h;
        flag[vr] = ok ? 0u : 1u;
      }
    }
    __syncthreads();
    for (int r = wid; r < T; r += NW) {
      if (flag[r]) {
        float xv[C];
#pragma unroll
        for (int c = 0; c < C; ++c) xv[c] = fv[r * LDF + lane + kWave * c];
        const uint32_t h = wave_norm_f16<D, C>(xv, xterms[wid], xbuf[wid]);
        if (lane == 0) nws[r] = h;
      }
    }
    __syncthreads();
    // ---- 3. y = x Pi^T
    if constexpr (!PRE) {
      f32x4 acc[NRT][WCT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) acc[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // k-step outermost, row tiles innermost: consecutive MFMAs update independent tiles
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const bf16x4 xh = *reinterpret_cast<const bf16x4 *>(&ah[(16 * rt + (lane & 15)) * LDA + 16 * ks + 4 * (lane >> 4)]);
            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, ph[ct][ks], acc[rt][ct], 0, 0, 0);
          }
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const bf16x4 xh = *reinterpret_cast<const bf16x4 *>(&ah[(16 * rt + (lane & 15)) * LDA + 16 * ks + 4 * (lane >> 4)]);
            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, pl[ct][ks], acc[rt][ct], 0, 0, 0);
          }
          if constexpr (XLO) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
              const bf16x4 xl = *reinterpret_cast<const bf16x4 *>(&al[(16 * rt + (lane & 15)) * LDA + 16 * ks + 4 * (lane >> 4)]);
              acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xl, ph[ct][ks], acc[rt][ct], 0, 0, 0);
            }
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * (lane >> 4) + i;
            const int col = 16 * (wid * WCT + ct) + (lane & 15);
            fv[row * LDF + col] = acc[rt][ct][i];
            if (a.y_tap && v0 + row < a.n) a.y_tap[(v0 + row) * D + col] = acc[rt][ct][i];
          }
      __syncthreads();
    }
    // ---- 4. indices and residual, 32 coordinates per thread
    {
      const uint32_t n16 = nws[vr];
      const float nbar = f16_bits_to_float(n16);
      float thr[L - 1];
#pragma unroll
      for (int j = 0; j < L - 1; ++j) thr[j] = __fmul_rn(nbar, ths[j]);
      uint64_t w0 = 0, w1 = 0;  // the thread's 32 * BITS index bits (at most 128)
      double s2 = 0.0;
#pragma unroll 4
      for (int k = 0; k < 32; ++k) {
        const int col = ch * 32 + k;
        const float y = fv[vr * LDF + col];
        uint32_t q = 0;
#pragma unroll
        for (int j = 0; j < L - 1; ++j) q += (y >= thr[j]) ? 1u : 0u;
        const float r = __fsub_rn(y, __fmul_rn(nbar, cbs[q]));
        fv[vr * LDF + col] = r;
        if constexpr (M > 0) {
          uint16_t hi, lo;
          split_bf16(r, hi, lo);
          ah[vr * LDA + col] = hi;
          al[vr * LDA + col] = lo;
        }
        s2 += (double)r * (double)r;
        const int b = BITS * k;
        if (b < 64) {
          w0 |= (uint64_t)q << b;
          if (b + BITS > 64) w1 |= (uint64_t)q >> (64 - b);
        } else {
          w1 |= (uint64_t)q << (b - 64);
        }
      }
      const int64_t v = v0 + vr;
      if (v < a.n) {
        const uint32_t wds[4] = {(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
#pragma unroll
        for (int w = 0; w < BITS; ++w) idxw[v * iw_all + ch * BITS + w] = wds[w];
        if (ch == 0)
          for (int w = D * BITS / 32; w < iw_all; ++w) idxw[v * iw_all + w] = 0u;
      }
      s2 = group_sum<TPV>(s2);
      bool ok;
      const uint32_t h = f16_norm_candidate<D>(s2, ok);
      if (ch == 0) {
        nws[vr] = n16 | (h << 16);
        flag[vr] = ok ? 0u : 1u;
        rn2[vr] = (float)s2;
      }
    }
    __syncthreads();
    for (int r = wid; r < T; r += NW) {
      if (flag[r]) {
        float xv[C];
#pragma unroll
        for (int c = 0; c < C; ++c) xv[c] = fv[r * LDF + lane + kWave * c];
        const uint32_t h = wave_norm_f16<D, C>(xv, xterms[wid], xbuf[wid]);
        if (lane == 0) nws[r] = (nws[r] & 0xFFFFu) | (h << 16);
      }
    }
    __syncthreads();
    // ---- 5. sign bits of z = r S^T
    if constexpr (M > 0) {
      f32x4 acc[NRT][WMCT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int mc = 0; mc < WMCT; ++mc) acc[rt][mc] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int mc = 0; mc < WMCT; ++mc) {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const bf16x4 rh = *reinterpret_cast<const bf16x4 *>(&ah[(16 * rt + (lane & 15)) * LDA + 16 * ks + 4 * (lane >> 4)]);
            acc[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(rh, sh[mc][ks], acc[rt][mc], 0, 0, 0);
          }
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const bf16x4 rl = *reinterpret_cast<const bf16x4 *>(&al[(16 * rt + (lane & 15)) * LDA + 16 * ks + 4 * (lane >> 4)]);
            acc[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(rl, sh[mc][ks], acc[rt][mc], 0, 0, 0);
          }
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const bf16x4 rh = *reinterpret_cast<const bf16x4 *>(&ah[(16 * rt + (lane & 15)) * LDA + 16 * ks + 4 * (lane >> 4)]);
            acc[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(rh, sl[mc][ks], acc[rt][mc], 0, 0, 0);
          }
        }
      }
      static_assert(NRT * WMCT * 4 <= 32, "one bit per accumulator element in a 32-bit mask");
      // pass 1: sign and "undecided" flag of every accumulator element, as per-lane bit masks
      uint32_t bitm = 0u, ambm = 0u;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int mc = 0; mc < WMCT; ++mc)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (rt * WMCT + mc) * 4 + i;
            const int row = 16 * rt + 4 * (lane >> 4) + i;
            const float z = acc[rt][mc][i];
            const float r2 = rn2[row];
            const float tau = r2 < 1e-30f ? INFINITY : 0x1p-13f * snorm[mc] * sqrtf(r2);
            bitm |= (z >= 0.0f ? 1u : 0u) << e;
            ambm |= (fabsf(z) <= tau ? 1u : 0u) << e;
          }
      // pass 2: undecided elements, one at a time for the whole wavefront: fp64 dot product
      // with its error bound, then the exact expansion if the bound still does not decide
      uint64_t pend = __ballot(ambm != 0u);
      while (pend) {
        const int src = __ffsll((unsigned long long)pend) - 1;
        const uint32_t sm = (uint32_t)__shfl((int)ambm, src, kWave);
        const int e = __ffs(sm) - 1;
        const int i = e & 3, mc = (e >> 2) % WMCT, rt = (e >> 2) / WMCT;
        const int srow = 16 * rt + 4 * (src >> 4) + i;
        const int j = 16 * (wid * WMCT + mc) + (src & 15);
        double ps = 0.0, pa = 0.0;
        for (int k = lane; k < D; k += kWave) {
          const double p = (double)a.sketch[(int64_t)j * D + k] * (double)fv[srow * LDF + k];
          ps += p;
          pa += fabs(p);
        }
        ps = wave_sum(ps);
        pa = wave_sum(pa);
        int sg;
        if (fabs(ps) > 2.0 * (D + 2) * 0x1p-53 * pa) {
          sg = ps > 0.0 ? 1 : -1;
        } else {
          for (int k = lane; k < D; k += kWave)
            xterms[wid][k] = (double)a.sketch[(int64_t)j * D + k] * (double)fv[srow * LDF + k];
          wave_lds_fence();
          sg = 0;
          if (lane == 0) sg = expansion_sign(xterms[wid], D, xbuf[wid]);
          wave_lds_fence();
          sg = __shfl(sg, 0, kWave);
        }
        if (lane == src) {
          bitm = (bitm & ~(1u << e)) | ((sg >= 0 ? 1u : 0u) << e);
          ambm &= ~(1u << e);
        }
        pend = __ballot(ambm != 0u);
      }
      // pass 3: 16-bit chunks of sketch rows per vector
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int mc = 0; mc < WMCT; ++mc)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (rt * WMCT + mc) * 4 + i;
            const uint64_t bm = __ballot((bitm >> e) & 1u);
            if (lane < 4) {
              const int rowg = 16 * rt + 4 * lane + i;
              sbits[rowg * MCT + wid * WMCT + mc] = (uint16_t)((bm >> (16 * lane)) & 0xFFFFu);
            }
          }
      __syncthreads();
      for (int e = tid; e < T * sw_all; e += NTH) {
        const int r = e / sw_all, w = e % sw_all;
        const int64_t v = v0 + r;
        if (v < a.n) {
          uint32_t word = 0u;
          if (2 * w < MCT) word = sbits[r * MCT + 2 * w];
          if (2 * w + 1 < MCT) word |= (uint32_t)sbits[r * MCT + 2 * w + 1] << 16;
          sgnw[v * sw_all + w] = word;
        }
      }
    }
    for (int r = tid; r < T; r += NTH)
      if (v0 + r < a.n) a.norms[v0 + r] = nws[r];
    __syncthreads();
  }
}

template <int D, int BITS, int M, int TIN, bool PRE>
static void launch_mfma(const EncArgs &a, hipStream_t st) {
  constexpr int NTH = D == 128 ? 512 : 256;  // tiles of 128 vectors; 16 columns of y per wavefront
  constexpr int T = NTH * 32 / D;
  int64_t tiles = (a.n + T - 1) / T;
  if (tiles > 256 * 2) tiles = 256 * 2;
  hipLaunchKernelGGL((encode_mfma<D, BITS, M, TIN, PRE, NTH>), dim3((unsigned)tiles), dim3(NTH), 0, st, a);
}

template <int D, int BITS, int M>
static int launch_enc_dm(const EncArgs &a, int dt, bool pre, hipStream_t st) {
  if constexpr (D == 64 || D == 128) {
    const int eb = dt == TQ_F32 ? 4 : 2;
    const bool vec_ok = ((uintptr_t)a.x % 16 == 0) && ((a.ld_x * eb) % 16 == 0);
    if ((a.n_rot == 1 || a.vecs_per_rot == 0) && vec_ok) {
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
