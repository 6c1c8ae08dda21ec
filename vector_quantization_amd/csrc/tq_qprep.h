// Per-workgroup query preparation: the rotated (and sketched) queries of a group of query
// heads, computed by the whole workgroup into LDS.
#pragma once

#include "tq_device.h"

namespace tq {

// q~ = R q and q^ = S q~ for the G consecutive query heads at q (fp32, global), by the whole
// workgroup: KSL threads per output row each sum KPER products, then combine by shuffles
// (KSL is a power of two, so a row's threads are aligned lanes of one wavefront).
// issue() requests every global operand at once -- the queries and, where each thread owns one
// (row, slice) of both products, its KPER weights of R and of S, kept in registers -- so that
// the prologue waits for one memory latency instead of a chain of them.  finish() computes:
// qs is LDS scratch of G * D floats; qt [G][D] and qh [G][M] are LDS outputs.  With rope_base > 0
// and rope_p >= 0 the queries are first turned by RoPE at position rope_p (rope_pairs).  It ends
// synchronised.
template <int D, int M, int G, int NT>
struct QueryPrep {
  static constexpr int ROWS = D > M ? D : M;
  static constexpr int KSL = (NT / ROWS >= 16) ? 16 : (NT / ROWS >= 8) ? 8 : (NT / ROWS >= 4) ? 4 : (NT / ROWS >= 2) ? 2 : 1;
  static constexpr int KPER = (D + KSL - 1) / KSL;
  static constexpr bool REG = NT / KSL >= ROWS && KPER * KSL == D && KPER <= 16;
  static constexpr int NWR = REG ? KPER : 1;
  static constexpr int QN = (G * D + NT - 1) / NT;
  float qv[QN];
  float wr[NWR], wsk[NWR];
  const float *R, *S;

  // rows < G: only the first `rows` query rows are read, the others taken as zero
  __device__ __forceinline__ void issue(const float *q, const float *R_, const float *S_, int rows = G) {
    R = R_;
    S = S_;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int e = tid + i * NT;
      qv[i] = e < rows * D ? q[e] : 0.0f;
    }
    if constexpr (REG) {
      const int r = tid / KSL, sl = tid % KSL;
#pragma unroll
      for (int kk = 0; kk < KPER; ++kk) {
        wr[kk] = r < D ? R[(int64_t)r * D + sl * KPER + kk] : 0.0f;
        if constexpr (M > 0) wsk[kk] = r < M ? S[(int64_t)r * D + sl * KPER + kk] : 0.0f;
      }
    }
  }

  __device__ void finish(float *qs, float *qt, float *qh, int64_t rope_p = -1, float rope_base = 0.0f) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int e = tid + i * NT;
      if (e < G * D) qs[e] = qv[i];
    }
    __syncthreads();
    if (rope_base > 0.0f && rope_p >= 0) {  // uniform over the workgroup
      for (int e = tid; e < G * (D / 2); e += NT) rope_pairs<D>(qs + (e / (D / 2)) * D, rope_p, rope_base, e % (D / 2), D / 2);
      __syncthreads();
    }
    auto reduce_store = [&](float(&acc)[G], int r, int rows, float *out) {
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = group_sum_dpp<KSL>(acc[h]);
      if (r < rows && tid % KSL == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) out[h * rows + r] = acc[h];
    };
    auto matvec_reg = [&](const float(&w)[NWR], int rows, const float *in, float *out) {
      const int r = tid / KSL, sl = tid % KSL;
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KPER; ++kk)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(w[kk], in[h * D + sl * KPER + kk], acc[h]);
      reduce_store(acc, r, rows, out);
    };
    auto matvec = [&](const float *W, int rows, const float *in, float *out) {
      for (int r0 = 0; r0 < rows; r0 += NT / KSL) {
        const int r = r0 + tid / KSL, sl = tid % KSL;
        float acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0.0f;
        if (r < rows) {
#pragma unroll 4
          for (int kk = 0; kk < KPER; ++kk) {
            const int k = sl * KPER + kk;
            if (k < D) {
              const float w = W[(int64_t)r * D + k];
#pragma unroll
              for (int h = 0; h < G; ++h) acc[h] = fmaf(w, in[h * D + k], acc[h]);
            }
          }
        }
        reduce_store(acc, r, rows, out);
      }
    };
    if constexpr (REG) matvec_reg(wr, D, qs, qt);
    else matvec(R, D, qs, qt);
    __syncthreads();
    if constexpr (M > 0) {
      if constexpr (REG) matvec_reg(wsk, M, qt, qh);
      else matvec(S, M, qt, qh);
      __syncthreads();
    }
  }
};

}  // namespace tq
