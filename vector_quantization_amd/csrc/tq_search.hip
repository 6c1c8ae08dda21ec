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
#include "tq_planes.h"
#include "tq_topk.h"

namespace tq {

int qprep(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh, hipStream_t st,
          const int32_t *pos = nullptr, float rope_base = 0.0f);
int qprep_limbs(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh, uint8_t *limbs,
                hipStream_t st);

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
  const uint8_t *limbs;  // search_planes: per query, its int8 limbs and constants (planes_limbs)
};

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
  const uint8_t *qjl_tabs = tabs + opaque_offset(C::MSE_BYTES);
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
      load_words<C::IW>(a.idx + v * a.idx_stride, iw);
      if constexpr (M > 0) load_words<C::SW>(a.sign + v * a.sign_stride, sw);
      const uint32_t nw = a.norms[v];
      float am[G], aq[G];
      lut_score<D, BITS, M, G>(iw, sw, tabs, qjl_tabs, hs, am, aq);
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
  float tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ms), k - 1));
  // the other slices' entries 64 at a time; only those reaching the current k-th are inserted
  const int64_t total = (int64_t)a.n_slices * k;
  for (int64_t b = k; b < total; b += kWave) {
    const int64_t e = b + lane;
    const float cs = e < total ? ps[e] : -INFINITY;
    const int32_t ci = e < total ? pi[e] : 0x7FFFFFFF;
    uint64_t m = __ballot(e < total && cs >= tau);
    while (m) {
      const int src = __builtin_ctzll(m);
      m &= m - 1;
      const float us = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), src));
      const int32_t ui = __builtin_amdgcn_readlane(ci, src);
      if (!(us >= tau)) continue;
      list_insert(ms, mi, us, ui, k);
      tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ms), k - 1));
    }
  }
  if (lane < k) {
    a.out_idx[qi * k + lane] = mi;
    a.out_score[qi * k + lane] = ms;
  }
}

// ------------------------------------------------------------------ batched queries on the matrix cores
//
// search_planes (tq_planes.h): a workgroup's four wavefronts hold 64 queries and walk the rows
// of a database slice; each wavefront keeps its 16 queries' top-k lists in LDS, with the k-th
// best score of each query as the entry threshold.  Launched twice, ASYM false and true: the
// launch whose ASYM does not match the codebook returns at once, so each variant is compiled for
// its own planes only.
template <int D, int BITS, int M, bool ASYM>
__global__ __launch_bounds__(kSpW * kWave) void search_planes(SearchArgs a) {
  constexpr int NK = (D + 63) / 64;  // 64-coordinate steps of the index term
  constexpr int NKM = (M + 63) / 64;  // of the sign term
  constexpr int NKM1 = NKM > 0 ? NKM : 1;
  constexpr int NP = n_planes<BITS, ASYM>();
  __shared__ float lsc[kSpW][16][32];
  __shared__ int32_t lix[kSpW][16][32];

  double wd[1 << BITS];
  if (walsh_weights<BITS>(a.centroids, wd) != ASYM) return;

  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int g = lane >> 4, col = lane & 15;
  const int64_t n_groups = (a.n_q + 16 * kSpW - 1) / (16 * kSpW);
  const int slice = (int)(blockIdx.x / n_groups);
  const int64_t qw = (int64_t)(blockIdx.x % n_groups) * (16 * kSpW) + 16 * wid;  // this wavefront's queries
  if (qw >= a.n_q) return;
  const int k = a.k;
  for (int e = lane; e < 16 * 32; e += kWave) {
    lsc[wid][e >> 5][e & 31] = -INFINITY;
    lix[wid][e >> 5][e & 31] = 0x7FFFFFFF;
  }

  PlaneQuery<NK, NKM1, NP> pq;
  load_plane_query<D, BITS, M, ASYM>(a.limbs, qw + col, qw + col < a.n_q, wd, pq);

  const int64_t v0 = (int64_t)slice * a.slice;
  int64_t v1 = v0 + a.slice;
  if (v1 > a.n_db) v1 = a.n_db;
  const RowPlanes rp{a.idx, a.idx_stride, a.sign, a.sign_stride, a.norms};
  float tau = -INFINITY;  // the k-th best score of query col so far
  float(*ls)[32] = lsc[wid];
  int32_t(*li)[32] = lix[wid];
  planes_rows<D, BITS, M, ASYM>(rp, pq, v0, v1, [&](int64_t t0, int left, const float(&s)[4]) {
    bool cand = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) cand |= pq.qok && 4 * g + i < left && s[i] >= tau;
    // candidates, one row position at a time; the source lane's values are read as scalars
    if (__ballot(cand)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint64_t m = __ballot(pq.qok && 4 * g + i < left && s[i] >= tau);
        while (m) {  // rare once the lists hold k entries
          const int src = __builtin_ctzll(m);
          m &= m - 1;
          const float cs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s[i]), src));
          const float ct = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tau), src));
          if (!(cs >= ct)) continue;  // the threshold rose since the ballot
          const int qc2 = src & 15;
          const int32_t ci = (int32_t)(t0 + 4 * (src >> 4) + i);
          const float nt = list_insert_lds(ls[qc2], li[qc2], cs, ci, k);
          if (col == qc2) tau = nt;
        }
      }
    }
  });

  for (int qc2 = 0; qc2 < 16; ++qc2) {
    const int64_t qo = qw + qc2;
    if (qo >= a.n_q) break;
    if (lane < k) {
      const float ms = lsc[wid][qc2][lane];
      const int32_t mi = lix[wid][qc2][lane];
      if (a.n_slices == 1) {
        a.out_idx[qo * k + lane] = mi;
        a.out_score[qo * k + lane] = ms;
      } else {
        a.part_s[(qo * a.n_slices + slice) * k + lane] = ms;
        a.part_i[(qo * a.n_slices + slice) * k + lane] = mi;
      }
    }
  }
}

// ------------------------------------------------------------------ host side

constexpr int kSearchNT = 1024;
constexpr int kSearchG = 4;

// queries from which the matrix-core scan is used
constexpr int64_t kSpMinQ = 32;
// rows per slice at most (with plane strides up to 256 bytes a slice's bytes stay below 2^31,
// the reach of the scan's 32-bit buffer offsets)
constexpr int64_t kSpMaxRows = (int64_t)1 << 23;

static void search_split(int64_t n_q, int64_t n_db, int &n_slices, int64_t &slice) {
  if (n_q >= kSpMinQ) {
    // bit-plane scan: workgroups of 64 queries; about 4096 workgroups, slices of at least 2048
    // rows (128 row tiles), a multiple of 16 rows
    const int64_t groups = (n_q + 16 * kSpW - 1) / (16 * kSpW);
    int64_t want = (4096 + groups - 1) / groups;
    const int64_t max_slices = (n_db + kSpMinRows - 1) / kSpMinRows;
    if (want > max_slices) want = max_slices;
    if (want < 1) want = 1;
    slice = (n_db + want - 1) / want;
    if (slice > kSpMaxRows) slice = kSpMaxRows;
    slice = (slice + 15) / 16 * 16;
    n_slices = (int)((n_db + slice - 1) / slice);
    return;
  }
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
  const size_t part = ns > 1 ? (size_t)n_q * ns * k * (sizeof(float) + sizeof(int32_t)) : 0;
  const size_t limbs = n_q >= kSpMinQ ? (size_t)n_q * limb_record_bytes(c.d, c.m) : 0;
  return q_al + (part + 255) / 256 * 256 + limbs;
}

template <int D, int BITS, int M>
static int launch_scan(const SearchArgs &a, hipStream_t st) {
  if (a.limbs != nullptr) {
    const int64_t groups = (a.n_q + 16 * kSpW - 1) / (16 * kSpW);
    if (!grid_fits(groups * a.n_slices)) return TQ_EUNSUPPORTED;
    hipLaunchKernelGGL((search_planes<D, BITS, M, false>), dim3((unsigned)(groups * a.n_slices)),
                       dim3(kSpW * kWave), 0, st, a);
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
    hipLaunchKernelGGL((search_planes<D, BITS, M, true>), dim3((unsigned)(groups * a.n_slices)),
                       dim3(kSpW * kWave), 0, st, a);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
  }
  const int64_t groups = (a.n_q + kSearchG - 1) / kSearchG;
  if (!grid_fits(groups * a.n_slices)) return TQ_EUNSUPPORTED;
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
  const size_t part = ns > 1 ? (size_t)n_q * ns * k * (sizeof(float) + sizeof(int32_t)) : 0;
  uint8_t *limbs = pbase + (part + 255) / 256 * 256;
  const ScoreShape s{n_q, 1, 1, n_db};
  // the matrix-core scan from kSpMinQ queries on (plane strides up to 256 bytes keep a slice's
  // bytes within its 32-bit buffer offsets); it needs the queries' limb records, the table scan
  // q~ and q^
  const bool planes = n_q >= kSpMinQ && db.idx_stride <= 256 && db.sign_stride <= 256;
  int rc = planes ? qprep_limbs(c, queries, s, qt, qh, limbs, st) : qprep(c, queries, s, qt, qh, st);
  if (rc != TQ_OK) return rc;
  SearchArgs a{qt, qh, c.centroids, n_q, n_db, k, ns, sl, db.idx, db.idx_stride, db.sign, db.sign_stride, db.norms,
               part_s, part_i, out_idx, out_score, planes ? limbs : nullptr};
  const int D = c.d, B = c.bits, M = c.m;
  rc = TQ_EUNSUPPORTED;
#define TQ_SR(DD, BB, MM) if (D == DD && B == BB && M == MM) rc = launch_scan<DD, BB, MM>(a, st); else
  TQ_SR(64, 2, 64) TQ_SR(64, 3, 64) TQ_SR(128, 2, 128) TQ_SR(128, 3, 0) TQ_SR(200, 2, 200) TQ_SR(200, 3, 0) {}
#undef TQ_SR
  if (rc != TQ_OK) return rc;
  if (ns > 1) return launch_topk_merge(part_s, part_i, n_q, ns, k, out_idx, out_score, stream);
  return TQ_OK;
}

int launch_topk_merge(const float *part_s, const int32_t *part_i, int64_t n_q, int n_slices, int k,
                      int64_t *out_idx, float *out_score, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  SearchArgs a{};
  a.n_q = n_q;
  a.k = k;
  a.n_slices = n_slices;
  a.part_s = const_cast<float *>(part_s);
  a.part_i = const_cast<int32_t *>(part_i);
  a.out_idx = out_idx;
  a.out_score = out_score;
  hipLaunchKernelGGL(search_merge, dim3((unsigned)((n_q + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
