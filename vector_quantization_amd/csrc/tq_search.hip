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
  const uint8_t *limbs;  // search_planes: per query, its int8 limbs and constants (search_limbs)
};

// a better than b: higher score, then smaller row
__device__ __forceinline__ bool better(float as, int32_t ai, float bs, int32_t bi) {
  return as > bs || (as == bs && ai < bi);
}

// Shift a value up by one lane across the wavefront (DPP wave_shr:1; lane 0 gets 0).
__device__ __forceinline__ int32_t wave_shr1(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x138, 0xF, 0xF, false);
}

// Insert the wave-uniform candidate (cs, ci) into the lane-distributed sorted list (ls, li)
// of length k (lanes >= k are unused).
__device__ __forceinline__ void list_insert(float &ls, int32_t &li, float cs, int32_t ci, int k) {
  const int lane = lane_id();
  const bool b = lane < k && better(ls, li, cs, ci);
  const int pos = __popcll(__ballot(b));
  if (pos >= k) return;
  const float us = __int_as_float(wave_shr1(__float_as_int(ls)));
  const int32_t ui = wave_shr1(li);
  if (lane > pos) {
    ls = us;
    li = ui;
  } else if (lane == pos) {
    ls = cs;
    li = ci;
  }
}

// Insert the wave-uniform candidate (cs, ci) into the sorted list of length k held in LDS
// (entry i at ls[i], li[i]); returns the list's k-th score afterwards.
__device__ __forceinline__ float list_insert_lds(float *lsp, int32_t *lip, float cs, int32_t ci, int k) {
  const int lane = lane_id();
  float ls = lane < k ? lsp[lane] : -INFINITY;
  int32_t li = lane < k ? lip[lane] : 0x7FFFFFFF;
  const int pos = __popcll(__ballot(lane < k && better(ls, li, cs, ci)));
  if (pos < k) {
    const float us = __int_as_float(wave_shr1(__float_as_int(ls)));
    const int32_t ui = wave_shr1(li);
    if (lane > pos) {
      ls = us;
      li = ui;
    } else if (lane == pos) {
      ls = cs;
      li = ci;
    }
    if (lane >= pos && lane < k) {
      lsp[lane] = ls;
      lip[lane] = li;
    }
  }
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), k - 1));
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
// search_planes: with many queries, the estimate of a tile of 16 rows x 16 queries is a matrix
// product on the matrix cores, taken over bit planes so that no table lookup is needed.
//
// Index term.  Write each code's bits as signs s_p = 2 b_p - 1.  Any function of the code is a
// combination of the sign products chi_S = prod_{p in S} s_p over the subsets S of the bits
// (the Walsh expansion), so c[idx] = w_0 + sum_S w_S chi_S with w_S = 2^-bits sum_code c[code]
// chi_S(code).  A codebook symmetric about zero (c[L-1-j] = -c[j], as for the Lloyd-Max levels
// of the symmetric coordinate law) has w_S = 0 for every even |S|: two planes for 2 bits, four
// for 3.  Other codebooks add the even planes (a second kernel variant).  Then
//   sum_i c[idx_i] q~_i = w_0 Q + sum_S w_S (2 P_S - Q),  P_S = sum_i [chi_S,i = +1] q~_i,
// with Q = sum_i q~_i.  Sign term likewise: sum_j (2 b_j - 1) q^_j = 2 P - Q^.  For 2-bit codes
// the planes taken are the b0 bits and the code values b0 + 2 b1 (2 P_b1 = P_code - P_b0), which
// one shift of the index word serves with two masks.
//
// Products.  A plane's bits (or code values) as bytes are the int8 A operand of
// v_mfma_i32_16x16x64_i8; the query is the B operand as two int8 limbs,
//   q~_i ~= sigma (L0_i + L1_i / 254),  sigma = max_i |q~_i| / 127,
// (representation error <= sigma / 508 per coordinate), so every product sum is an exact
// integer, P_S = sigma / 254 (254 A0_S + A1_S) with A0/A1 the limb sums, and 254 A0 + A1 stays
// below 2^24 and converts exactly.  Per 64 coordinates a plane costs two products: 2-bit index +
// QJL signs at d = m = 200 take 24 per tile.  The K order of the products is chosen so that a
// lane's A bytes are its index or sign word shifted and masked (k_position).
//
// Rows.  A workgroup's four wavefronts hold 64 queries (16 each) and walk the same rows of a
// database slice, so each row is fetched once per 64 queries; the next tile's words are loaded
// while this one is scored.  Each wavefront keeps its queries' top-k lists in LDS, with the k-th
// best score of each query as the entry threshold; the slices' lists are merged by search_merge.
typedef int32_t si32x4 __attribute__((ext_vector_type(4)));

constexpr int kSpW = 4;  // wavefronts per workgroup (16 queries each)

// A raw buffer resource over [base, base + bytes) (bytes < 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// The 16 plane bits of a 3-bit code field (bit 3c for code c) as an int8 x 16 operand, code c
// at byte c: four bits at a time, a 24-bit multiply puts copy k at shift 5k, landing bit 3k on
// bit 8k, and no two copies' bits meet, so the mask leaves the four bits alone.
__device__ __forceinline__ si32x4 plane_bytes3(uint64_t P) {
  si32x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) r[t] = (int32_t)(__umul24((uint32_t)(P >> (12 * t)) & 0xFFFu, 0x8421u) & 0x01010101u);
  return r;
}

// Where the MFMA's K index puts each coordinate.  Lane group g holds K positions 16 g + 4 t + j
// (dword t, byte j) of a 64-coordinate step; the K order is free as long as A and B agree, so it
// is chosen to make the bits of dword t a shift and a mask away:
//   KL_CONTIG  coordinate 16 g + 4 t + j (3-bit codes: decoded with the multiply spread)
//   KL_CODE2   coordinate 16 g + t + 4 j: in the index word of lane group g the plane bit of
//              coordinate c sits at bit 2c, so dword t is (word >> 2t) & 0x01010101
//   KL_SIGN    coordinate 32 (g >> 1) + 8 j + 4 (g & 1) + t: sign word 2 ks + (g >> 1) shifted
//              by 4 (g & 1) + t and masked
enum { KL_CONTIG = 0, KL_CODE2 = 1, KL_SIGN = 2 };

__device__ __forceinline__ int k_position(int layout, int c) {  // c: coordinate within the step
  if (layout == KL_CODE2) return 16 * (c >> 4) + 4 * (c & 3) + ((c >> 2) & 3);
  if (layout == KL_SIGN) return 16 * (2 * (c >> 5) + ((c >> 2) & 1)) + 4 * (c & 3) + ((c >> 3) & 3);
  return c;
}

// A query's limb record: L0 and L1 of q~ (NK * 64 bytes each, in the index term's K order),
// then those of q^ (NKM * 64 each, K order KL_SIGN), then sigma, sigma^ (float) and 254 Q0 + Q1
// of each (int32).  Coordinates past d (m) are zero.
__host__ __device__ constexpr int limb_record_bytes(int d, int m) {
  return 128 * ((d + 63) / 64 + (m + 63) / 64) + 16;
}

// One wavefront per query: lane l takes coordinates 64 ks + l.
template <int LEN, int NK, int LAYOUT>
__device__ __forceinline__ void limbs_of(const float *row, uint8_t *l0, uint8_t *l1, float &sigma, int32_t &qc) {
  const int lane = lane_id();
  float mx = 0.0f;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int i = 64 * ks + lane;
    if (i < LEN) mx = fmaxf(mx, fabsf(row[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  sigma = mx / 127.0f;
  const float inv = mx > 0.0f ? 127.0f / mx : 0.0f;
  int32_t s0 = 0, s1 = 0;
  const int pos = k_position(LAYOUT, lane);
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int i = 64 * ks + lane;
    const float u = i < LEN ? row[i] * inv : 0.0f;
    const float r0 = fminf(fmaxf(__builtin_rintf(u), -127.0f), 127.0f);
    const float r1 = fminf(fmaxf(__builtin_rintf((u - r0) * 254.0f), -127.0f), 127.0f);
    l0[64 * ks + pos] = (uint8_t)(int8_t)r0;
    l1[64 * ks + pos] = (uint8_t)(int8_t)r1;
    s0 += (int32_t)r0;
    s1 += (int32_t)r1;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    s0 += __shfl_xor(s0, o, kWave);
    s1 += __shfl_xor(s1, o, kWave);
  }
  qc = 254 * s0 + s1;
}

template <int D, int BITS, int M>
__global__ __launch_bounds__(256) void search_limbs(const float *qt, const float *qh, int64_t n_q, uint8_t *limbs) {
  constexpr int NK = (D + 63) / 64, NKM = (M + 63) / 64;
  const int64_t qi = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (qi >= n_q) return;
  uint8_t *rec = limbs + qi * limb_record_bytes(D, M);
  float sig, sigh = 0.0f;
  int32_t qc, qch = 0;
  limbs_of<D, NK, BITS == 2 ? KL_CODE2 : KL_CONTIG>(qt + qi * D, rec, rec + 64 * NK, sig, qc);
  if constexpr (M > 0)
    limbs_of<M, NKM, KL_SIGN>(qh + qi * M, rec + 128 * NK, rec + 128 * NK + 64 * NKM, sigh, qch);
  if (lane_id() == 0) {
    float *cf = reinterpret_cast<float *>(rec + 128 * (NK + NKM));
    cf[0] = sig;
    cf[1] = sigh;
    reinterpret_cast<int32_t *>(cf)[2] = qc;
    reinterpret_cast<int32_t *>(cf)[3] = qch;
  }
}

// The queries' side of search_planes, per lane (column q, group g).
template <int NK, int NKM1, int NP>
struct PlaneQuery {
  si32x4 bq0[NK], bq1[NK];      // limbs of q~ (K positions 16 g + 0..15 of each step)
  si32x4 bh0[NKM1], bh1[NKM1];  // limbs of q^
  float cp[NP];                 // per A plane: the weight of its limb sum T = 254 A0 + A1
  float a0;                     // the index term's constant
  float ssk, sq;                // sign term sqrt(pi/2)/m (2 P - Q^) = ssk T + sq
  bool qok;
};

// A planes of the index term.  2-bit codes: the b0 bits and the code values b0 + 2 b1 (one
// shift serves both masks), plus b0 xnor b1 for an asymmetric codebook.  3-bit codes: one plane
// per Walsh subset S (the odd ones, plus the even ones for an asymmetric codebook), plane S - 1.
template <int BITS, bool ASYM>
constexpr int n_planes() {
  return BITS == 2 ? (ASYM ? 3 : 2) : (1 << BITS) - 1;
}

// Walk rows [v0, v1) in tiles of 16, scoring them against the wavefront's 16 queries and
// keeping their lists (lsc/lix: [16][32]) and thresholds.  ASYM adds the even Walsh planes.
template <int D, int BITS, int M, bool ASYM, int NK, int NKM1, int NP>
__device__ __forceinline__ void planes_rows(const SearchArgs &a, const PlaneQuery<NK, NKM1, NP> &pq, int64_t v0,
                                            int64_t v1, float (*lsc)[32], int32_t (*lix)[32]) {
  constexpr int NKM = (M + 63) / 64;
  constexpr int L = 1 << BITS;
  constexpr int IW = (D * BITS + 31) / 32;    // index words per row
  constexpr int SWW = (M + 31) / 32;          // sign words per row
  constexpr int WPS = BITS == 3 ? 2 : 1;      // index words a lane needs per step
  constexpr uint64_t PMASK3 = 0x0000249249249249ull;  // bit 0 of each 3-bit code
  const int lane = lane_id(), g = lane >> 4, col = lane & 15;
  const int k = a.k;

  // buffer resources over this slice's rows: the row of a tile is a scalar offset, the word a
  // lane reads a constant one; reads past the slice return 0 (those rows are masked, and
  // coordinates past d meet zero query values)
  const __amdgpu_buffer_rsrc_t ridx = slice_rsrc(a.idx + v0 * a.idx_stride, (v1 - v0) * a.idx_stride);
  const __amdgpu_buffer_rsrc_t rsgn = slice_rsrc(M > 0 ? a.sign + v0 * a.sign_stride : a.idx, (v1 - v0) * a.sign_stride);
  const __amdgpu_buffer_rsrc_t rnrm = slice_rsrc(a.norms + v0, (v1 - v0) * 4);
  const uint32_t istr = (uint32_t)a.idx_stride, sstr = (uint32_t)a.sign_stride;
  uint32_t ioff[NK * WPS], soff[NKM1];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int wi = (BITS * (64 * ks + 16 * g)) >> 5;
#pragma unroll
    for (int u = 0; u < WPS; ++u) ioff[ks * WPS + u] = col * istr + 4 * (wi + u < IW ? wi + u : IW - 1);
  }
#pragma unroll
  for (int ks = 0; ks < NKM1; ++ks) {
    const int wi = 2 * ks + (g >> 1);
    soff[ks] = col * sstr + 4 * (wi < SWW ? wi : SWW - 1);
  }
  struct Words {
    uint32_t iw[NK * WPS], sw[NKM1], nw[4];
  };
  auto load_tile = [&](int64_t t0, Words &w) {
    const uint32_t r = (uint32_t)(t0 - v0);
#pragma unroll
    for (int u = 0; u < NK * WPS; ++u) w.iw[u] = __builtin_amdgcn_raw_buffer_load_b32(ridx, ioff[u], r * istr, 0);
    if constexpr (M > 0) {
#pragma unroll
      for (int ks = 0; ks < NKM; ++ks) w.sw[ks] = __builtin_amdgcn_raw_buffer_load_b32(rsgn, soff[ks], r * sstr, 0);
    }
    const si32x4 n4 = __builtin_bit_cast(si32x4, __builtin_amdgcn_raw_buffer_load_b128(rnrm, 16 * g, 4 * r, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) w.nw[i] = (uint32_t)n4[i];
  };

  float tau = -INFINITY;  // the k-th best score of query col so far
  auto process = [&](int64_t t0, const Words &w) {
    si32x4 acc[NP][2], accs[2];
    const si32x4 z = {0, 0, 0, 0};
    auto mfma2 = [&](si32x4(&c)[2], const si32x4 &A, const si32x4 &b0, const si32x4 &b1, bool first) {
      c[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, b0, first ? z : c[0], 0, 0, 0);
      c[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, b1, first ? z : c[1], 0, 0, 0);
    };
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      if constexpr (BITS == 2) {
        // the 16 codes of coordinates 64 ks + 16 g + 0..15 (code c at bits 2c, 2c + 1); dword t
        // byte j holds code t + 4 j
        const uint32_t wd0 = w.iw[ks];
        si32x4 Ab, Ac;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t x = wd0 >> (2 * t);
          Ab[t] = (int32_t)(x & 0x01010101u);
          Ac[t] = (int32_t)(x & 0x03030303u);
        }
        mfma2(acc[0], Ab, pq.bq0[ks], pq.bq1[ks], ks == 0);
        mfma2(acc[1], Ac, pq.bq0[ks], pq.bq1[ks], ks == 0);
        if constexpr (ASYM) {
          const uint32_t xn = ~(wd0 ^ (wd0 >> 1));
          si32x4 Ax;
#pragma unroll
          for (int t = 0; t < 4; ++t) Ax[t] = (int32_t)((xn >> (2 * t)) & 0x01010101u);
          mfma2(acc[NP - 1], Ax, pq.bq0[ks], pq.bq1[ks], ks == 0);
        }
      } else {
        // the 16 codes of coordinates 64 ks + 16 g + 0..15 as 48 bits
        const int sh = (BITS * (64 * ks + 16 * g)) & 31;
        const uint64_t f = ((uint64_t)w.iw[ks * WPS] | ((uint64_t)w.iw[ks * WPS + 1] << 32)) >> sh;
        uint64_t base[BITS];
#pragma unroll
        for (int p = 0; p < BITS; ++p) base[p] = (f >> p) & PMASK3;
#pragma unroll
        for (int S = 1; S < L; ++S) {
          const bool even = (__builtin_popcount((unsigned)S) & 1) == 0;
          if (even && !ASYM) continue;
          uint64_t X = even ? PMASK3 : 0;
#pragma unroll
          for (int p = 0; p < BITS; ++p)
            if (S & (1 << p)) X ^= base[p];
          mfma2(acc[S - 1], plane_bytes3(X), pq.bq0[ks], pq.bq1[ks], ks == 0);
        }
      }
    }
    if constexpr (M > 0) {
#pragma unroll
      for (int ks = 0; ks < NKM; ++ks) {
        // sign word 2 ks + (g >> 1): dword t takes bits 4 (g & 1) + t + 8 j
        const uint32_t sw = w.sw[ks] >> (4 * (g & 1));
        si32x4 A;
#pragma unroll
        for (int t = 0; t < 4; ++t) A[t] = (int32_t)((sw >> t) & 0x01010101u);
        mfma2(accs, A, pq.bh0[ks], pq.bh1[ks], ks == 0);
      }
    }

    // D layout: rows t0 + 4 g + i, query col
    const int left = (int)(v1 - t0 < 16 ? v1 - t0 : 16);  // valid rows of this tile
    float s[4];
    bool cand = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float u = pq.a0;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (BITS == 3 && !ASYM && (__builtin_popcount((unsigned)(p + 1)) & 1) == 0) continue;
        u = fmaf(pq.cp[p], (float)(__mul24(acc[p][0][i], 254) + acc[p][1][i]), u);  // exact: below 2^24
      }
      s[i] = f16_bits_to_float(w.nw[i] & 0xFFFFu) * u;
      if constexpr (M > 0) {
        const float v = fmaf(pq.ssk, (float)(__mul24(accs[0][i], 254) + accs[1][i]), pq.sq);
        s[i] = fmaf(f16_bits_to_float(w.nw[i] >> 16), v, s[i]);
      }
      cand |= pq.qok && 4 * g + i < left && s[i] >= tau;
    }
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
          const float nt = list_insert_lds(lsc[qc2], lix[qc2], cs, ci, k);
          if (col == qc2) tau = nt;
        }
      }
    }
  };

  // two word buffers in turn: the next tile's loads are in flight while this one is scored
  // (issued unconditionally, past the slice they read zeros, so that every path waits for the
  // same loads)
  Words wa, wb;
  load_tile(v0, wa);
  for (int64_t t0 = v0; t0 < v1; t0 += 32) {
    load_tile(t0 + 16, wb);
    process(t0, wa);
    if (t0 + 16 >= v1) break;
    load_tile(t0 + 32, wa);
    process(t0 + 16, wb);
  }
}

// Launched twice, ASYM false and true: the launch whose ASYM does not match the codebook
// returns at once, so each variant is compiled for its own planes only.
template <int D, int BITS, int M, bool ASYM>
__global__ __launch_bounds__(kSpW * kWave) void search_planes(SearchArgs a) {
  constexpr int NK = (D + 63) / 64;           // 64-coordinate steps of the index term
  constexpr int NKM = (M + 63) / 64;          // of the sign term
  constexpr int NKM1 = NKM > 0 ? NKM : 1;
  constexpr int L = 1 << BITS;
  __shared__ float lsc[kSpW][16][32];
  __shared__ int32_t lix[kSpW][16][32];

  // Walsh weights of the codebook (fp64: sums of the fp32 levels, exact for a symmetric one)
  double wd[L];
#pragma unroll
  for (int S = 0; S < L; ++S) {
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < L; ++c) {
      const bool neg = (__builtin_popcount((unsigned)(S & ~c)) & 1) != 0;  // chi_S(c) = -1 iff odd # of zero bits in S
      acc += neg ? -(double)a.centroids[c] : (double)a.centroids[c];
    }
    wd[S] = acc / (double)L;
  }
  bool asym = wd[0] != 0.0;
#pragma unroll
  for (int S = 1; S < L; ++S)
    if ((__builtin_popcount((unsigned)S) & 1) == 0 && wd[S] != 0.0) asym = true;
  if (asym != ASYM) return;

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

  // B operands and the constants of this lane's query; absent queries get zeros
  constexpr int NP = n_planes<BITS, ASYM>();
  PlaneQuery<NK, NKM1, NP> pq;
  const int64_t qi = qw + col;
  pq.qok = qi < a.n_q;
  float sig, sigh;
  int32_t qc, qch;
  {
    // unconditional loads (of query 0 for absent ones) then a select: the operands are complete
    // and in registers before the row loop starts
    const bool ok = pq.qok;
    const uint8_t *rec = a.limbs + (ok ? qi : 0) * limb_record_bytes(D, M);
    const si32x4 z = {0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const si32x4 l0 = *reinterpret_cast<const si32x4 *>(rec + 64 * ks + 16 * g);
      const si32x4 l1 = *reinterpret_cast<const si32x4 *>(rec + 64 * NK + 64 * ks + 16 * g);
      pq.bq0[ks] = ok ? l0 : z;
      pq.bq1[ks] = ok ? l1 : z;
    }
#pragma unroll
    for (int ks = 0; ks < NKM1; ++ks) {
      if (ks < NKM) {
        const si32x4 h0 = *reinterpret_cast<const si32x4 *>(rec + 128 * NK + 64 * ks + 16 * g);
        const si32x4 h1 = *reinterpret_cast<const si32x4 *>(rec + 128 * NK + 64 * NKM + 64 * ks + 16 * g);
        pq.bh0[ks] = ok ? h0 : z;
        pq.bh1[ks] = ok ? h1 : z;
      } else {
        pq.bh0[ks] = pq.bh1[ks] = z;
      }
    }
    const float4 cf = *reinterpret_cast<const float4 *>(rec + 128 * (NK + NKM));
    sig = ok ? cf.x : 0.0f;
    sigh = ok ? cf.y : 0.0f;
    qc = ok ? __float_as_int(cf.z) : 0;
    qch = ok ? __float_as_int(cf.w) : 0;
  }
  // With T_S = 254 A0_S + A1_S (so P_S = sigma / 254 T_S) and qc = 254 Q0 + Q1:
  //   index term = sigma / 254 [sum_S w_S 2 T_S + (w_0 - sum_S w_S) qc]
  // over the planes used; for 2-bit codes 2 P_b1 = P_code - P_b0.
  const double s254 = (double)sig / 254.0;
  double used = 0.0;
  if constexpr (BITS == 2) {
    pq.cp[0] = (float)((2.0 * wd[1] - wd[2]) * s254);  // b0 plane
    pq.cp[1] = (float)(wd[2] * s254);                  // code plane
    used = wd[1] + wd[2];
    if constexpr (ASYM) {
      pq.cp[2] = (float)(2.0 * wd[3] * s254);
      used += wd[3];
    }
  } else {
#pragma unroll
    for (int S = 1; S < L; ++S) {
      const bool even = (__builtin_popcount((unsigned)S) & 1) == 0;
      pq.cp[S - 1] = (even && !ASYM) ? 0.0f : (float)(2.0 * wd[S] * s254);
      if (!(even && !ASYM)) used += wd[S];
    }
  }
  pq.a0 = (float)((wd[0] - used) * s254 * (double)qc);
  // sign term: sqrt(pi/2)/m (2 P - Q^) = sqrt(pi/2)/m sigma^ / 254 (2 T - qch)
  const double kq = M > 0 ? 1.2533141373155003 / (double)(M > 0 ? M : 1) * (double)sigh / 254.0 : 0.0;
  pq.ssk = (float)(2.0 * kq);
  pq.sq = (float)(-kq * (double)qch);

  const int64_t v0 = (int64_t)slice * a.slice;
  int64_t v1 = v0 + a.slice;
  if (v1 > a.n_db) v1 = a.n_db;
  planes_rows<D, BITS, M, ASYM>(a, pq, v0, v1, lsc[wid], lix[wid]);

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

static void search_split(int64_t n_q, int64_t n_db, int &n_slices, int64_t &slice) {
  if (n_q >= kSpMinQ) {
    // bit-plane scan: workgroups of 64 queries; about 4096 workgroups, slices of at least 2048
    // rows (128 row tiles), a multiple of 16 rows
    const int64_t groups = (n_q + 16 * kSpW - 1) / (16 * kSpW);
    int64_t want = (4096 + groups - 1) / groups;
    const int64_t max_slices = (n_db + 2047) / 2048;
    if (want > max_slices) want = max_slices;
    if (want < 1) want = 1;
    slice = (n_db + want - 1) / want;
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
  if (a.n_q >= kSpMinQ) {
    hipLaunchKernelGGL((search_limbs<D, BITS, M>), dim3((unsigned)((a.n_q + 3) / 4)), dim3(256), 0, st, a.qt, a.qh, a.n_q,
                       const_cast<uint8_t *>(a.limbs));
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
    const int64_t groups = (a.n_q + 16 * kSpW - 1) / (16 * kSpW);
    hipLaunchKernelGGL((search_planes<D, BITS, M, false>), dim3((unsigned)(groups * a.n_slices)),
                       dim3(kSpW * kWave), 0, st, a);
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
    hipLaunchKernelGGL((search_planes<D, BITS, M, true>), dim3((unsigned)(groups * a.n_slices)),
                       dim3(kSpW * kWave), 0, st, a);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
  }
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
  const size_t part = ns > 1 ? (size_t)n_q * ns * k * (sizeof(float) + sizeof(int32_t)) : 0;
  uint8_t *limbs = pbase + (part + 255) / 256 * 256;
  const ScoreShape s{n_q, 1, 1, n_db};
  int rc = qprep(c, queries, s, qt, qh, st);
  if (rc != TQ_OK) return rc;
  SearchArgs a{qt, qh, c.centroids, n_q, n_db, k, ns, sl, db.idx, db.idx_stride, db.sign, db.sign_stride, db.norms,
               part_s, part_i, out_idx, out_score, limbs};
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
