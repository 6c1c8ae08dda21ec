// Bit-plane matrix products for many queries at once, shared by the batched search
// (tq_search.hip: search_planes) and the batched scoring (tq_scores.hip: score_planes).
//
// Sources: the estimator is that of tq_scores (walkthrough "Etapa 2": K~ = K^ + K~_QJL, in the
// rotated space).  Many queries share one pass over the codes in the search of the hada.io page
// ("Desempenho em busca vetorial") and when every token of a sequence queries every cached key,
// the all-pairs shape of a bidirectional protein model over one sequence (TurboESM summary,
// section 3: ESM-2 650M, 33 layers x 20 heads, 1024 tokens).
//
// With many queries, the estimate of a tile of 16 rows x 16 queries is a matrix product on the
// matrix cores, taken over bit planes so that no table lookup is needed.
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
// Rows.  A workgroup's four wavefronts hold 64 queries (16 each) and walk the same rows, so
// each row is fetched once per 64 queries; the next tile's words are loaded while this one is
// scored, and each tile's 16 x 16 scores go to a sink (top-k lists, or logits).

#pragma once

#include "tq_device.h"

namespace tq {

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

// One wavefront per query: lane l takes coordinates 64 ks + l (row may point to LDS); the limb
// bytes go to l0 / l1 in the K order `layout` (LDS staging).
template <int LEN, int NK>
__device__ __forceinline__ void limbs_of(const float *row, int layout, uint8_t *l0, uint8_t *l1, float &sigma,
                                         int32_t &qc) {
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
  const int pos = k_position(layout, lane);
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

// The limb record of one query from its q~ (D) and q^ (M) rows; one wavefront.  The record is
// assembled in `stage` (LDS, limb_record_bytes(D, M) bytes for this wavefront) and written out
// with 16-byte stores.
template <int D, int M>
__device__ __forceinline__ void write_limb_record(const float *qt_row, const float *qh_row, int bits, uint8_t *stage,
                                                  uint8_t *rec) {
  constexpr int NK = (D + 63) / 64, NKM = (M + 63) / 64;
  constexpr int R = limb_record_bytes(D, M);
  float sig, sigh = 0.0f;
  int32_t qc, qch = 0;
  limbs_of<D, NK>(qt_row, bits == 2 ? KL_CODE2 : KL_CONTIG, stage, stage + 64 * NK, sig, qc);
  if constexpr (M > 0) limbs_of<M, NKM>(qh_row, KL_SIGN, stage + 128 * NK, stage + 128 * NK + 64 * NKM, sigh, qch);
  const int lane = lane_id();
  if (lane == 0) {
    float *cf = reinterpret_cast<float *>(stage + 128 * (NK + NKM));
    cf[0] = sig;
    cf[1] = sigh;
    reinterpret_cast<int32_t *>(cf)[2] = qc;
    reinterpret_cast<int32_t *>(cf)[3] = qch;
  }
  wave_lds_fence();
  for (int e = lane; e < R / 16; e += kWave)
    reinterpret_cast<uint4 *>(rec)[e] = reinterpret_cast<const uint4 *>(stage)[e];
  wave_lds_fence();  // the stage is reused by the wavefront's next record
}

// limbs_of for four queries at once, one per 16-lane group of the wavefront: lane 16 g + s
// takes coordinates s, s + 16, ... of query g's row, and the maximum and the limb sums are
// reduced over the group's 16 lanes.  The same values as limbs_of, byte for byte.
template <int LEN, int NK>
__device__ __forceinline__ void limbs_of16(const float *row, int layout, uint8_t *l0, uint8_t *l1, float &sigma,
                                           int32_t &qc) {
  const int sl = lane_id() & 15;
  constexpr int NC = 4 * NK;  // coordinates per lane
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = sl + 16 * i;
    if (c < LEN) mx = fmaxf(mx, fabsf(row[c]));
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  sigma = mx / 127.0f;
  const float inv = mx > 0.0f ? 127.0f / mx : 0.0f;
  int32_t s0 = 0, s1 = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = sl + 16 * i;
    const float u = c < LEN ? row[c] * inv : 0.0f;
    const float r0 = fminf(fmaxf(__builtin_rintf(u), -127.0f), 127.0f);
    const float r1 = fminf(fmaxf(__builtin_rintf((u - r0) * 254.0f), -127.0f), 127.0f);
    const int b = 64 * (i >> 2) + k_position(layout, sl + 16 * (i & 3));
    l0[b] = (uint8_t)(int8_t)r0;
    l1[b] = (uint8_t)(int8_t)r1;
    s0 += (int32_t)r0;
    s1 += (int32_t)r1;
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    s0 += __shfl_xor(s0, o, 16);
    s1 += __shfl_xor(s1, o, 16);
  }
  qc = 254 * s0 + s1;
}

// The limb records of four consecutive queries, rows qt0 + g qt_stride and qh0 + g qh_stride
// (LDS), one per 16-lane group; assembled in `stage` (4 records) and written to rec0 (the
// first of four consecutive records) for the first n_valid of them.
template <int D, int M>
__device__ __forceinline__ void write_limb_records4(const float *qt0, int qt_stride, const float *qh0, int qh_stride,
                                                    int n_valid, int bits, uint8_t *stage, uint8_t *rec0) {
  constexpr int NK = (D + 63) / 64, NKM = (M + 63) / 64;
  constexpr int R = limb_record_bytes(D, M);
  static_assert(R % 16 == 0, "records in 16-byte words");
  const int lane = lane_id(), g = lane >> 4;
  uint8_t *st = stage + g * R;
  float sig, sigh = 0.0f;
  int32_t qc, qch = 0;
  limbs_of16<D, NK>(qt0 + g * qt_stride, bits == 2 ? KL_CODE2 : KL_CONTIG, st, st + 64 * NK, sig, qc);
  if constexpr (M > 0) limbs_of16<M, NKM>(qh0 + g * qh_stride, KL_SIGN, st + 128 * NK, st + 128 * NK + 64 * NKM, sigh, qch);
  if ((lane & 15) == 0) {
    float *cf = reinterpret_cast<float *>(st + 128 * (NK + NKM));
    cf[0] = sig;
    cf[1] = sigh;
    reinterpret_cast<int32_t *>(cf)[2] = qc;
    reinterpret_cast<int32_t *>(cf)[3] = qch;
  }
  wave_lds_fence();
  for (int e = lane; e < 4 * (R / 16); e += kWave)
    if (e / (R / 16) < n_valid) reinterpret_cast<uint4 *>(rec0)[e] = reinterpret_cast<const uint4 *>(stage)[e];
  wave_lds_fence();  // the stage is reused by the wavefront's next records
}

// The limb records of n_q queries from q~ [n_q][D] and q^ [n_q][M]; one wavefront per query.
template <int D, int M>
__global__ __launch_bounds__(256) void planes_limbs(const float *qt, const float *qh, int64_t n_q, int bits,
                                                    uint8_t *limbs) {
  __shared__ __align__(16) uint8_t stage[4][limb_record_bytes(D, M)];
  const int64_t qi = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (qi >= n_q) return;
  write_limb_record<D, M>(qt + qi * D, M > 0 ? qh + qi * M : nullptr, bits, stage[threadIdx.x / kWave],
                          limbs + qi * limb_record_bytes(D, M));
}

// The queries' side of a bit-plane scan, per lane (column q, group g).
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

// The rows a scan reads: the three code planes, based at the first row of the range it walks.
struct RowPlanes {
  const uint8_t *idx;
  int64_t idx_stride;
  const uint8_t *sign;
  int64_t sign_stride;
  const uint32_t *norms;
};

// Walk rows [v0, v1) of rp in tiles of 16, scoring them against the wavefront's 16 queries;
// sink(t0, left, s) receives each tile's scores (lane: rows t0 + 4 g + i, i = 0..3, of query
// col; left = the tile's valid rows).  ASYM adds the even Walsh planes.
template <int D, int BITS, int M, bool ASYM, int NK, int NKM1, int NP, typename Sink>
__device__ __forceinline__ void planes_rows(const RowPlanes &rp, const PlaneQuery<NK, NKM1, NP> &pq, int64_t v0,
                                            int64_t v1, Sink &&sink) {
  constexpr int NKM = (M + 63) / 64;
  constexpr int L = 1 << BITS;
  constexpr int IW = (D * BITS + 31) / 32;    // index words per row
  constexpr int SWW = (M + 31) / 32;          // sign words per row
  constexpr int WPS = BITS == 3 ? 2 : 1;      // index words a lane needs per step
  constexpr uint64_t PMASK3 = 0x0000249249249249ull;  // bit 0 of each 3-bit code
  const int lane = lane_id(), g = lane >> 4, col = lane & 15;

  // buffer resources over this slice's rows: the row of a tile is a scalar offset, the word a
  // lane reads a constant one; reads past the slice return 0 (those rows are masked, and
  // coordinates past d meet zero query values)
  const __amdgpu_buffer_rsrc_t ridx = slice_rsrc(rp.idx + v0 * rp.idx_stride, (v1 - v0) * rp.idx_stride);
  const __amdgpu_buffer_rsrc_t rsgn = slice_rsrc(M > 0 ? rp.sign + v0 * rp.sign_stride : rp.idx, (v1 - v0) * rp.sign_stride);
  const __amdgpu_buffer_rsrc_t rnrm = slice_rsrc(rp.norms + v0, (v1 - v0) * 4);
  const uint32_t istr = (uint32_t)rp.idx_stride, sstr = (uint32_t)rp.sign_stride;
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
    }
    sink(t0, left, s);
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

// Walsh weights of the codebook, w_S = 2^-bits sum_code c[code] chi_S(code), in fp64 (sums of the
// fp32 levels, exact for a symmetric codebook); returns whether an even |S| (or S = {}) has a
// nonzero weight.
template <int BITS>
__device__ __forceinline__ bool walsh_weights(const float *centroids, double (&wd)[1 << BITS]) {
  constexpr int L = 1 << BITS;
#pragma unroll
  for (int S = 0; S < L; ++S) {
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < L; ++c) {
      const bool neg = (__builtin_popcount((unsigned)(S & ~c)) & 1) != 0;  // chi_S(c) = -1: odd # of zero bits in S
      acc += neg ? -(double)centroids[c] : (double)centroids[c];
    }
    wd[S] = acc / (double)L;
  }
  bool asym = wd[0] != 0.0;
#pragma unroll
  for (int S = 1; S < L; ++S)
    if ((__builtin_popcount((unsigned)S) & 1) == 0 && wd[S] != 0.0) asym = true;
  return asym;
}

// The B operands and constants of query record qi (absent queries, ok false, get zeros; their
// loads read record 0, then a select: the operands are complete and in registers before the
// row loop starts).
template <int D, int BITS, int M, bool ASYM, int NK, int NKM1, int NP>
__device__ __forceinline__ void load_plane_query(const uint8_t *limbs, int64_t qi, bool ok,
                                                 const double (&wd)[1 << BITS], PlaneQuery<NK, NKM1, NP> &pq) {
  constexpr int NKM = (M + 63) / 64;
  constexpr int L = 1 << BITS;
  const int g = lane_id() >> 4;
  pq.qok = ok;
  const uint8_t *rec = limbs + (ok ? qi : 0) * limb_record_bytes(D, M);
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
  const float sig = ok ? cf.x : 0.0f, sigh = ok ? cf.y : 0.0f;
  const int32_t qc = ok ? __float_as_int(cf.z) : 0, qch = ok ? __float_as_int(cf.w) : 0;
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
}

// Rows per workgroup at least: the split of rows over workgroups stops there.
constexpr int64_t kSpMinRows = 2048;

}  // namespace tq
