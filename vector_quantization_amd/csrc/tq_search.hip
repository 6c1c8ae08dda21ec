// Inner-product top-k search over encoded database vectors.
//
// Sources: hada.io TurboQuant page, "Desempenho em busca vetorial": the codes serve vector
// search; recall 1@k counts how often the true best inner product is among the approximate
// top k.  sudonull.com "Conclusiones clave": the same compression serves vector search / RAG.
// Scores are the estimator of tq_scores (tq_lut.h); ranking is by score descending, then by
// database row ascending.
//
// search_scan: one workgroup per (group of G queries, database slice) builds the G queries'
// lookup tables, scores its slice (one database vector per thread per step) and keeps, per
// wave and query, a sorted top-k list spread over the lanes (lane i holds entry i).  A
// candidate enters only if it beats the current k-th entry; inserting is one ballot, one
// shuffle and a select per lane.  The waves' lists are merged in LDS at the end.
// search_merge: one wave per query merges the slices' lists when the database was split.

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_lut.h"

namespace tq {

int qprep(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh, hipStream_t st,
          const int32_t *pos = nullptr, float rope_base = 0.0f);

struct SearchArgs {
  const float *qt, *qh, *centroids;
  int64_t n_q, n_db;
  int k, n_slices;
  int64_t slice;
  const uint8_t *idx;
  int64_t idx_stride;
  const uint8_t *sign;
  int64_t sign_stride;
  const uint32_t *norms;
  float *part_s;      // [n_q][n_slices][k] when n_slices > 1
  int32_t *part_i;
  int64_t *out_idx;   // [n_q][k] when n_slices == 1
  float *out_score;
};

// a better than b: higher score, then smaller row
__device__ __forceinline__ bool better(float as, int32_t ai, float bs, int32_t bi) {
  return as > bs || (as == bs && ai < bi);
}

// Insert the wave-uniform candidate (cs, ci) into the lane-distributed sorted list (ls, li)
// of length k (lanes >= k are unused).
__device__ __forceinline__ void list_insert(float &ls, int32_t &li, float cs, int32_t ci, int k) {
  const int lane = lane_id();
  const bool b = lane < k && better(ls, li, cs, ci);
  const int pos = __popcll(__ballot(b));
  if (pos >= k) return;
  const float us = __shfl_up(ls, 1, kWave);
  const int32_t ui = __shfl_up(li, 1, kWave);
  if (lane > pos) {
    ls = us;
    li = ui;
  } else if (lane == pos) {
    ls = cs;
    li = ci;
  }
}

template <int W>
__device__ __forceinline__ void load_words_s(const uint8_t *p, uint32_t (&w)[W]) {
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

template <int D, int BITS, int M, int G, int NT>
__global__ __launch_bounds__(NT) void search_scan(SearchArgs a) {
  using C = Lut<D, BITS, M, G>;
  constexpr int SWN = C::SW > 0 ? C::SW : 1;
  constexpr int NW = NT / kWave;
  __shared__ __align__(16) uint8_t tabs[C::BYTES];
  __shared__ float qt[G * D];
  __shared__ float qh[G * (M > 0 ? M : 1)];
  __shared__ float cb[C::L];
  __shared__ float sc[4 * G];

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const int slice = (int)(blockIdx.x % a.n_slices);
  const int64_t qg = blockIdx.x / a.n_slices;
  const int64_t q0 = qg * G;
  for (int i = tid; i < G * D; i += NT) {
    int64_t qi = q0 + i / D;
    if (qi > a.n_q - 1) qi = a.n_q - 1;
    qt[i] = a.qt[qi * D + i % D];
  }
  if constexpr (M > 0)
    for (int i = tid; i < G * M; i += NT) {
      int64_t qi = q0 + i / M;
      if (qi > a.n_q - 1) qi = a.n_q - 1;
      qh[i] = a.qh[qi * M + i % M];
    }
  if (tid < C::L) cb[tid] = a.centroids[tid];
  __syncthreads();
  HeadScales<G> hs;
  block_table_scales<D, BITS, M, G>(qt, qh, cb, sc, hs);
  build_luts<D, BITS, M, G, NT>(tabs, tabs + C::MSE_BYTES, qt, qh, cb, sc, sc + G);
  __syncthreads();

  const int k = a.k;
  const float kappa = M > 0 ? 1.2533141373155003f / (float)(M > 0 ? M : 1) : 0.0f;
  float ls[G];
  int32_t li[G];
  float tau[G];
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
    if (valid) {
      uint32_t iw[C::IW];
      uint32_t sw[SWN];
      load_words_s<C::IW>(a.idx + v * a.idx_stride, iw);
      if constexpr (M > 0) load_words_s<C::SW>(a.sign + v * a.sign_stride, sw);
      const uint32_t nw = a.norms[v];
      float am[G], aq[G];
      lut_score<D, BITS, M, G>(iw, sw, tabs, tabs + C::MSE_BYTES, hs, am, aq);
      const float nbar = f16_bits_to_float(nw & 0xFFFFu);
      const float rq = f16_bits_to_float(nw >> 16) * kappa;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sc[h] = nbar * am[h];
        if constexpr (M > 0) sc[h] = fmaf(rq, aq[h], sc[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint64_t m = __ballot(valid && sc[h] >= tau[h]);
      while (m) {
        const int j = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const float cs = __shfl(sc[h], j, kWave);
        const int32_t ci = (int32_t)(base + wid * kWave + j);
        list_insert(ls[h], li[h], cs, ci, k);
        tau[h] = __shfl(ls[h], k - 1, kWave);
      }
    }
  }

  // merge the waves' lists: wave h (< G) merges query h
  __syncthreads();
  float *wls = reinterpret_cast<float *>(tabs);
  int32_t *wli = reinterpret_cast<int32_t *>(tabs + NW * G * 32 * sizeof(float));
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (lane < k) {
      wls[(wid * G + h) * 32 + lane] = ls[h];
      wli[(wid * G + h) * 32 + lane] = li[h];
    }
  __syncthreads();
  if (wid < G) {
    const int h = wid;
    float ms = lane < k ? wls[h * 32 + lane] : -INFINITY;
    int32_t mi = lane < k ? wli[h * 32 + lane] : 0x7FFFFFFF;
    for (int w = 1; w < NW; ++w) {
      for (int i = 0; i < k; ++i) {
        const float cs = wls[(w * G + h) * 32 + i];
        const int32_t ci = wli[(w * G + h) * 32 + i];
        list_insert(ms, mi, cs, ci, k);
      }
    }
    const int64_t qi = q0 + h;
    if (qi < a.n_q && lane < k) {
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

__global__ __launch_bounds__(256) void search_merge(SearchArgs a) {
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int64_t qi = (int64_t)blockIdx.x * 4 + wid;
  if (qi >= a.n_q) return;
  const int k = a.k;
  const float *ps = a.part_s + qi * a.n_slices * k;
  const int32_t *pi = a.part_i + qi * a.n_slices * k;
  float ms = lane < k ? ps[lane] : -INFINITY;
  int32_t mi = lane < k ? pi[lane] : 0x7FFFFFFF;
  for (int s = 1; s < a.n_slices; ++s)
    for (int i = 0; i < k; ++i) list_insert(ms, mi, ps[s * k + i], pi[s * k + i], k);
  if (lane < k) {
    a.out_idx[qi * k + lane] = mi;
    a.out_score[qi * k + lane] = ms;
  }
}

// ------------------------------------------------------------------ host side

constexpr int kSearchNT = 1024;
constexpr int kSearchG = 4;

static void search_split(int64_t n_q, int64_t n_db, int &n_slices, int64_t &slice) {
  const int64_t groups = (n_q + kSearchG - 1) / kSearchG;
  int64_t want = (2048 + groups - 1) / groups;
  const int64_t max_slices = (n_db + 4 * kSearchNT - 1) / (4 * kSearchNT);
  if (want > max_slices) want = max_slices;
  if (want < 1) want = 1;
  slice = (n_db + want - 1) / want;
  n_slices = (int)((n_db + slice - 1) / slice);
}

size_t search_workspace(const CodecView &c, int64_t n_q, int k, int64_t n_db) {
  int ns;
  int64_t sl;
  search_split(n_q, n_db, ns, sl);
  const size_t q = (size_t)n_q * (size_t)(c.d + c.m) * sizeof(float);
  const size_t q_al = (q + 255) / 256 * 256;
  return q_al + (ns > 1 ? (size_t)n_q * ns * k * (sizeof(float) + sizeof(int32_t)) : 0);
}

template <int D, int BITS, int M>
static int launch_scan(const SearchArgs &a, hipStream_t st) {
  const int64_t groups = (a.n_q + kSearchG - 1) / kSearchG;
  hipLaunchKernelGGL((search_scan<D, BITS, M, kSearchG, kSearchNT>), dim3((unsigned)(groups * a.n_slices)),
                     dim3(kSearchNT), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

int launch_search(const CodecView &c, const float *queries, int64_t n_q, const CodesView &db, int64_t n_db, int k,
                  int64_t *out_idx, float *out_score, void *ws, size_t ws_bytes, void *stream) {
  (void)ws_bytes;
  if (n_db > 0x7FFFFFFELL) return TQ_EUNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int ns;
  int64_t sl;
  search_split(n_q, n_db, ns, sl);
  float *qt = reinterpret_cast<float *>(ws);
  float *qh = qt + (size_t)n_q * c.d;
  const size_t q = (size_t)n_q * (size_t)(c.d + c.m) * sizeof(float);
  uint8_t *pbase = reinterpret_cast<uint8_t *>(ws) + (q + 255) / 256 * 256;
  float *part_s = reinterpret_cast<float *>(pbase);
  int32_t *part_i = reinterpret_cast<int32_t *>(pbase + (size_t)n_q * ns * k * sizeof(float));
  const ScoreShape s{n_q, 1, 1, n_db};
  int rc = qprep(c, queries, s, qt, qh, st);
  if (rc != TQ_OK) return rc;
  SearchArgs a{qt, qh, c.centroids, n_q, n_db, k, ns, sl, db.idx, db.idx_stride, db.sign, db.sign_stride, db.norms,
               part_s, part_i, out_idx, out_score};
  const int D = c.d, B = c.bits, M = c.m;
  rc = TQ_EUNSUPPORTED;
#define TQ_SR(DD, BB, MM) if (D == DD && B == BB && M == MM) rc = launch_scan<DD, BB, MM>(a, st); else
  TQ_SR(64, 2, 64) TQ_SR(64, 3, 64) TQ_SR(128, 2, 128) TQ_SR(128, 3, 0) TQ_SR(200, 2, 200) TQ_SR(200, 3, 0) {}
#undef TQ_SR
  if (rc != TQ_OK) return rc;
  if (ns > 1) {
    hipLaunchKernelGGL(search_merge, dim3((unsigned)((n_q + 3) / 4)), dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  }
  return TQ_OK;
}

}  // namespace tq
