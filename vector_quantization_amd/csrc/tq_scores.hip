// Query preparation and the score stream over a compressed key cache.
//
// Sources: 7minutos.es TurboQuant walkthrough, "Etapa 2 (Corrección Residual)" (the QJL term
// sqrt(pi/2)/m ||r|| S^T sign(S r) and K~ = K^ + K~_QJL); hada.io TurboQuant page, "QJL:
// técnica de 1 bit com overhead zero" (high-precision query against 1-bit data); sudonull.com
// "Cómo funciona PolarQuant" (norm times quantised direction).  The estimate is evaluated in
// the rotated space: <q, k~> = nbar <Pi q, c[idx]> + rnbar sqrt(pi/2)/m <S Pi q, 2 bits - 1>.
//
// qprep (used by attention and search): q~ = Pi_r q and q^ = S q~ in fp32 for every query head.
// score: one workgroup per (sequence, kv head, head subgroup, key chunk) computes q~ and q^ of
// its G query heads itself (Pi and S come from L2), builds their lookup tables in LDS
// (tq_lut.h), then streams the chunk's code planes from HBM, one key per thread per step, and
// writes fp32 logits for the G heads.

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_lut.h"
#include "tq_planes.h"
#include "tq_qprep.h"

namespace tq {

struct QprepArgs {
  const float *q;
  int64_t n_heads;  // n_seq * hq
  int hq, hkv;
  int64_t n_keys;   // vectors per kv block (selects the block's rotation)
  const float *rot;
  int n_rot;
  int64_t vecs_per_rot;
  const float *sketch;
  float *qt, *qh;
  const int32_t *pos;  // with rope_base > 0: RoPE of the queries of sequence s at pos[s]
  float rope_base;
  uint8_t *limbs;      // qprep_tiled: when set, write the limb records (tq_planes.h) instead of q~, q^
  int bits;            // their index-term K order
};

template <int D, int M>
__global__ __launch_bounds__(256) void qprep_kernel(QprepArgs a) {
  constexpr int C = (D + kWave - 1) / kWave;
  constexpr int CM = (M + kWave - 1) / kWave;
  __shared__ float qs[4][D];
  __shared__ float ts[4][D];
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int64_t hidx = (int64_t)blockIdx.x * 4 + wid;
  if (hidx >= a.n_heads) return;
  const int64_t s = hidx / a.hq;
  const int h = (int)(hidx % a.hq);
  const int64_t blk = s * a.hkv + h / (a.hq / a.hkv);
  int64_t rid = 0;
  if (a.n_rot > 1 && a.vecs_per_rot > 0) {
    rid = (blk * a.n_keys) / a.vecs_per_rot;
    if (rid > a.n_rot - 1) rid = a.n_rot - 1;
  }
  const float *R = a.rot + rid * (int64_t)D * D;
  for (int i = lane; i < D; i += kWave) qs[wid][i] = a.q[hidx * D + i];
  wave_lds_fence();
  if (a.pos != nullptr && a.rope_base > 0.0f) {
    rope_pairs<D>(qs[wid], a.pos[s], a.rope_base, lane, kWave);
    wave_lds_fence();
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i = lane + kWave * c;
    if (i < D) {
      float acc = 0.0f;
      for (int k = 0; k < D; ++k) acc = fmaf(R[(int64_t)i * D + k], qs[wid][k], acc);
      ts[wid][i] = acc;
      a.qt[hidx * D + i] = acc;
    }
  }
  if constexpr (M > 0) {
    wave_lds_fence();
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      const int j = lane + kWave * c;
      if (j < M) {
        float acc = 0.0f;
        for (int k = 0; k < D; ++k) acc = fmaf(a.sketch[(int64_t)j * D + k], ts[wid][k], acc);
        a.qh[hidx * M + j] = acc;
      }
    }
  }
}

// Tiled variant for 16 query heads that share one rotation (one shared rotation, or per-block
// rotations with a multiple of 16 query heads per kv head): a block takes the 16 heads and
// computes q~ = q Pi^T, then q^ = q~ S^T, staging column tiles of Pi (or S) transposed in LDS
// so that the output columns are read without bank conflicts.  The next tile is requested into
// registers before the current one is used, so the block waits for one memory latency per
// tile at most, and tiles of 32 columns (d a multiple of 32; else 8) keep the tile count low:
// the prologue of a decode step is this chain of tiles.
constexpr int kQpHeads = 16;
constexpr int kQpHeadsMany = 64;
constexpr int kQpKt = 8;  // a multiple of 4 dividing every supported d
template <int D>
constexpr int qp_kt() { return D % 32 == 0 ? 32 : kQpKt; }

template <int D, int M, int HEADS>
__global__ __launch_bounds__(256) void qprep_tiled(QprepArgs a) {
  constexpr int NOUT = D > M ? D : M;
  constexpr int TPC = (256 / NOUT) >= 1 ? 256 / NOUT : 1;  // threads per output column
  constexpr int HPT = HEADS / TPC;                         // heads per thread
  // rows padded to a multiple of 4 floats: a thread reads four consecutive k of a head at once
  // (every lane of a wavefront the same head, one broadcast read)
  constexpr int QSW = (D + 4) / 4 * 4;
  __shared__ __align__(16) float qs[HEADS][QSW];
  __shared__ float qhs[HEADS][(M > 0 ? M : 1) + 1];
  constexpr int KT = qp_kt<D>();
  constexpr int TLD = (NOUT * KT + 255) / 256;  // tile elements per thread
  __shared__ float rt[KT][NOUT + 1];
  const int tid = threadIdx.x;
  const int64_t h0 = (int64_t)blockIdx.x * HEADS;
  // the rotation of the key block that head h0 reads (the same for all HEADS heads)
  const float *rot = a.rot;
  if (a.n_rot > 1 && a.vecs_per_rot > 0) {
    const int64_t kvb = (h0 / a.hq) * a.hkv + (h0 % a.hq) / (a.hq / a.hkv);
    int64_t r = kvb * a.n_keys / a.vecs_per_rot;
    if (r > a.n_rot - 1) r = a.n_rot - 1;
    rot += r * D * D;
  }
  // tile k0 of W (rows x D): columns k0 .. k0 + KT - 1 into registers, then transposed into rt
  float pre[TLD];
  auto fetch = [&](const float *W, int rows, int k0) {
#pragma unroll
    for (int u = 0; u < TLD; ++u) {
      const int e = tid + 256 * u;
      pre[u] = e < rows * KT ? W[(int64_t)(e / KT) * D + k0 + e % KT] : 0.0f;
    }
  };
  auto stage = [&](int rows) {
#pragma unroll
    for (int u = 0; u < TLD; ++u) {
      const int e = tid + 256 * u;
      if (e < rows * KT) rt[e % KT][e / KT] = pre[u];
    }
  };
  fetch(rot, D, 0);
  for (int e = tid; e < HEADS * D; e += 256) {
    int64_t h = h0 + e / D;
    if (h > a.n_heads - 1) h = a.n_heads - 1;
    qs[e / D][e % D] = a.q[h * D + e % D];
  }
  if (a.pos != nullptr && a.rope_base > 0.0f) {
    __syncthreads();
    // 16 threads per head
    const int hh = tid / 16;
    int64_t h = h0 + hh;
    if (h > a.n_heads - 1) h = a.n_heads - 1;
    rope_pairs<D>(qs[hh], a.pos[h / a.hq], a.rope_base, tid % 16, 16);
  }
  const int col = tid % NOUT;
  const int hs = tid / NOUT;
  const bool active = hs < TPC;
  float acc[HPT];
  // out[col] = sum_k W[col][k] in[k] over the staged tiles of W, k ascending (the next tile in
  // flight while the current one is used)
  auto product = [&](const float *W, int rows) {
#pragma unroll
    for (int j = 0; j < HPT; ++j) acc[j] = 0.0f;
    for (int k0 = 0; k0 < D; k0 += KT) {
      __syncthreads();
      stage(rows);
      __syncthreads();
      if (k0 + KT < D) fetch(W, rows, k0 + KT);
      if (active && col < rows) {
#pragma unroll
        for (int k4 = 0; k4 < KT; k4 += 4) {
          float r[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) r[t] = rt[k4 + t][col];
#pragma unroll
          for (int j = 0; j < HPT; ++j) {
            const float4 x = *reinterpret_cast<const float4 *>(&qs[hs * HPT + j][k0 + k4]);
            acc[j] = fmaf(r[0], x.x, acc[j]);
            acc[j] = fmaf(r[1], x.y, acc[j]);
            acc[j] = fmaf(r[2], x.z, acc[j]);
            acc[j] = fmaf(r[3], x.w, acc[j]);
          }
        }
      }
    }
  };
  // ---- q~ = q Pi^T
  product(rot, D);
  if constexpr (M > 0) fetch(a.sketch, M, 0);  // the first tile of S while q~ is stored
  __syncthreads();
  if (active && col < D) {
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
      const int64_t h = h0 + hs * HPT + j;
      qs[hs * HPT + j][col] = acc[j];
      if (h < a.n_heads && a.limbs == nullptr) a.qt[h * D + col] = acc[j];
    }
  }
  if constexpr (M > 0) {
    // ---- q^ = q~ S^T
    product(a.sketch, M);
    if (active && col < M) {
#pragma unroll
      for (int j = 0; j < HPT; ++j) {
        const int64_t h = h0 + hs * HPT + j;
        qhs[hs * HPT + j][col] = acc[j];
        if (h < a.n_heads && a.limbs == nullptr) a.qh[h * M + col] = acc[j];
      }
    }
  }
  if (a.limbs != nullptr) {
    // four heads per wavefront (16 lanes each): the limb records straight from LDS
    static_assert(HEADS % 4 == 0, "heads in groups of four");
    __shared__ __align__(16) uint8_t stage[256 / kWave][4 * limb_record_bytes(D, M)];
    __syncthreads();
    for (int hh = 4 * (threadIdx.x / kWave); hh < HEADS; hh += 4 * (256 / kWave)) {
      const int64_t h = h0 + hh;
      const int64_t left = a.n_heads - h;
      if (left > 0)
        write_limb_records4<D, M>(qs[hh], QSW, M > 0 ? qhs[hh] : nullptr, (M > 0 ? M : 1) + 1,
                                  left < 4 ? (int)left : 4, a.bits, stage[threadIdx.x / kWave],
                                  a.limbs + h * limb_record_bytes(D, M));
    }
  }
}

struct ScoreArgs {
  const float *q, *rot, *sketch, *centroids;
  int n_rot;
  int64_t vecs_per_rot;
  int64_t n_seq, n_keys;
  int hq, hkv, nsub, n_chunks, chunk;
  const uint8_t *idx;
  int64_t idx_stride;
  const uint8_t *sign;
  int64_t sign_stride;
  const uint32_t *norms;
  float *logits;
};

// LDS of a score workgroup besides the tables: the queries, their two transforms, the
// codebook and the scales.
template <int D, int BITS, int M, int G>
constexpr int score_lds_extra() {
  return (G * (2 * D + (M > 0 ? M : 1)) + (1 << BITS) + 4 * G) * 4 + 256;
}

// Threads per workgroup: tables that leave room for one workgroup per CU take 1024 threads;
// where two fit, 512 (the same 16 wavefronts per CU, twice the registers each); smaller
// tables 256.
template <int D, int BITS, int M, int G>
constexpr int score_threads() {
  constexpr int base = Lut<D, BITS, M, G>::BYTES + score_lds_extra<D, BITS, M, G>();
  return base > 80 * 1024 ? 1024 : (Lut<D, BITS, M, G>::BYTES > 48 * 1024 ? 512 : 256);
}

// The half-table builder's scratch, where it costs no workgroups per CU.
template <int D, int BITS, int M, int G>
constexpr bool score_half_scratch() {
  constexpr int base = Lut<D, BITS, M, G>::BYTES + score_lds_extra<D, BITS, M, G>();
  constexpr int with = base + lut_half_bytes<D, BITS, M, G>();
  constexpr int lds = 160 * 1024;
  return with <= lds && lds / with == lds / base;
}

// Error units of a 16-bit-table score (tq_lut.h): em per unit of nbar, eq per unit of rq =
// rnbar sqrt(pi/2)/m.  Each of the NG index entries and NQ sign entries is rounded to the
// nearest multiple of its table's unit (inv_m, inv_q), at most half a unit off; the integer sums
// are exact and convert to fp32 exactly (|sum| < NG 32767 < 2^24), and the fp32 conversion by
// the unit, the products with the norms and the final sum add at most 2^-21 of the largest
// possible |sum| (NG 32767 units, NQ 32767 units) -- 0.0157 units per entry.
template <int D, int BITS, int M>
__device__ __forceinline__ void i16_error_units(float inv_m, float inv_q, float &em, float &eq) {
  using C = Lut<D, BITS, M, 4>;
  em = (float)C::NG * inv_m * 0.5157f;
  eq = (float)C::NQ * inv_q * 0.5157f;
}

// Score keys t0 .. t1 - 1 of a kv block again for one query head with fp32 tables (the G = 1
// layout, built over the 16-bit tables' LDS) and overwrite its logits: the 16-bit tables' error
// guard's way back to fp32 accuracy.  qt [D] and qh [M] are the head's rotated query and sketch
// in LDS; one points to {1, 1} in LDS (the fp32 tables' scales).  All threads call it; it ends
// synchronised.
template <int D, int BITS, int M, int NT>
__device__ void rescore_fp32(const ScoreArgs &a, uint8_t *tabs, const float *qt, const float *qh, const float *cb,
                             const float *one, int64_t row, int64_t vbase, int64_t t0, int64_t t1, float kappa) {
  using C1 = Lut<D, BITS, M, 1>;
  constexpr int SWN = C1::SW > 0 ? C1::SW : 1;
  build_luts<D, BITS, M, 1, NT>(tabs, tabs + C1::MSE_BYTES, qt, qh, cb, one, one, nullptr);
  __syncthreads();
  HeadScales<1> hs1;
  hs1.inv_m[0] = hs1.inv_q[0] = 1.0f;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += NT) {
    const int64_t v = vbase + t;
    uint32_t iw[C1::IW];
    uint32_t sw[SWN];
    load_words<C1::IW>(a.idx + v * a.idx_stride, iw);
    if constexpr (M > 0) load_words<C1::SW>(a.sign + v * a.sign_stride, sw);
    const uint32_t nw = a.norms[v];
    float am[1], aq[1];
    lut_score<D, BITS, M, 1>(iw, sw, tabs, tabs + C1::MSE_BYTES, hs1, am, aq);
    float sc = f16_bits_to_float(nw & 0xFFFFu) * am[0];
    if constexpr (M > 0) sc = fmaf(f16_bits_to_float(nw >> 16) * kappa, aq[0], sc);
    a.logits[row * a.n_keys + t] = sc;
  }
  __syncthreads();  // the tables are rebuilt by the next call
}

template <int D, int BITS, int M, int G, int NT>
__global__ __launch_bounds__(NT) void score_kernel(ScoreArgs a) {
  using C = Lut<D, BITS, M, G>;
  constexpr int SWN = C::SW > 0 ? C::SW : 1;
  __shared__ __align__(16) uint8_t tabs[C::BYTES];
  __shared__ float qs[G * D];
  __shared__ float qt[G * D];
  __shared__ float qh[G * (M > 0 ? M : 1)];
  __shared__ float cb[C::L];
  __shared__ float sc[4 * G + 2];  // table scales (block_table_scales), then {1, 1} for fp32 tables
  // scratch of the half-table builder where LDS has room for it
  constexpr bool HALF = score_half_scratch<D, BITS, M, G>();
  __shared__ __align__(16) float halfs[HALF ? lut_half_bytes<D, BITS, M, G>() / 4 : 4];

  const int64_t b = blockIdx.x;
  const int chunk = (int)(b % a.n_chunks);
  const int64_t rest = b / a.n_chunks;
  const int sub = (int)(rest % a.nsub);
  const int64_t blk = rest / a.nsub;  // s * hkv + kvh
  const int64_t s = blk / a.hkv;
  const int kvh = (int)(blk % a.hkv);
  const int g = a.hq / a.hkv;
  const int h0 = kvh * g + sub * G;  // first query head of this group
  const int64_t qrow = s * a.hq + h0;

  int64_t rid = 0;  // the rotation of this kv block
  if (a.n_rot > 1 && a.vecs_per_rot > 0) {
    rid = (blk * a.n_keys) / a.vecs_per_rot;
    if (rid > a.n_rot - 1) rid = a.n_rot - 1;
  }
  QueryPrep<D, M, G, NT> prep;
  prep.issue(a.q + qrow * D, a.rot + rid * (int64_t)D * D, a.sketch);
  if (threadIdx.x < C::L) cb[threadIdx.x] = a.centroids[threadIdx.x];
  if (threadIdx.x < 2) sc[4 * G + threadIdx.x] = 1.0f;
  prep.finish(qs, qt, qh);
  HeadScales<G> hs;
  block_table_scales<D, BITS, M, G>(qt, qh, cb, sc, hs);
  build_luts<D, BITS, M, G, NT>(tabs, tabs + C::MSE_BYTES, qt, qh, cb, sc, sc + G, HALF ? halfs : nullptr);
  __syncthreads();

  const float kappa = M > 0 ? 1.2533141373155003f / (float)(M > 0 ? M : 1) : 0.0f;  // sqrt(pi/2)/m
  const uint8_t *qjl_tabs = tabs + opaque_offset(C::MSE_BYTES);
  const int64_t t0 = (int64_t)chunk * a.chunk;
  int64_t t1 = t0 + a.chunk;
  if (t1 > a.n_keys) t1 = a.n_keys;
  const int64_t vbase = blk * a.n_keys;
  // 16-bit tables: the chunk's largest |logit| per head and largest norms, for the error guard
  float smax[G], nmax = 0.0f, rmax = 0.0f;
#pragma unroll
  for (int h = 0; h < G; ++h) smax[h] = 0.0f;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += NT) {
    const int64_t v = vbase + t;
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
      float sc = nbar * am[h];
      if constexpr (M > 0) sc = fmaf(rq, aq[h], sc);
      a.logits[(qrow + h) * a.n_keys + t] = sc;
      if constexpr (C::I16) smax[h] = fmaxf(smax[h], fabsf(sc));
    }
    if constexpr (C::I16) {
      nmax = fmaxf(nmax, nbar);
      rmax = fmaxf(rmax, rq);
    }
  }
  if constexpr (C::I16) {
    // Error guard of the 16-bit tables.  A key's logit misses the exact table sums by at most
    // E = nbar Em + rq Eq (i16_error_units), so every logit of the chunk is within
    // Emax = nmax Em + rmax Eq of its fp32-table value.  The row's largest |logit| is at least
    // the chunk's, so Emax <= tau (max |logit| - Emax) with tau = 8e-4 keeps the chunk's errors
    // within 8e-4 of the row's largest |logit| (the fp32 parts add below 1e-5 of it, inside the
    // 1e-3 row-relative tolerance); a head of the chunk that fails it (a short row, or a query
    // nearly orthogonal to every key) is scored again with fp32 tables.
    float *red = reinterpret_cast<float *>(tabs);  // [NT / kWave][G + 2], after the barrier below
    constexpr int NW = NT / kWave;
#pragma unroll
    for (int h = 0; h < G; ++h) smax[h] = wave_max_dpp(smax[h]);
    nmax = wave_max_dpp(nmax);
    rmax = wave_max_dpp(rmax);
    __syncthreads();  // every wavefront is done with the tables
    const int wid = threadIdx.x / kWave;
    if (lane_id() == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) red[wid * (G + 2) + h] = smax[h];
      red[wid * (G + 2) + G] = nmax;
      red[wid * (G + 2) + G + 1] = rmax;
    }
    __syncthreads();
    float mx[G + 2];
#pragma unroll
    for (int k = 0; k < G + 2; ++k) {
      mx[k] = 0.0f;
      for (int w = 0; w < NW; ++w) mx[k] = fmaxf(mx[k], red[w * (G + 2) + k]);
    }
    unsigned redo = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float em, eq;
      i16_error_units<D, BITS, M>(hs.inv_m[h], hs.inv_q[h], em, eq);
      const float emax = mx[G] * em + mx[G + 1] * eq;
      if (!(emax <= 8e-4f * (mx[h] - emax))) redo |= 1u << h;
    }
    __syncthreads();  // every thread has read red (it aliases the tables rebuilt below)
    if (redo != 0u) {  // uniform: every thread computed it from the same LDS values
      for (int h = 0; h < G; ++h)
        if (redo & (1u << h))
          rescore_fp32<D, BITS, M, NT>(a, tabs, qt + h * D, qh + h * (M > 0 ? M : 1), cb, sc + 4 * G,
                                       qrow + h, vbase, t0, t1, kappa);
    }
  }
}

// ------------------------------------------------------------------ many query heads per kv head
//
// score_planes (tq_planes.h): with 32 or more query heads per kv head (every token of a sequence
// querying every cached key, say), the logits of 64 query heads x a chunk of the kv head's keys
// come from one workgroup whose four wavefronts walk the same keys.  Queries are prepared once
// (qprep: q~, q^ with the key block's rotation; planes_limbs: int8 limbs) in the workspace.
// Launched twice, ASYM false and true, as search_planes.
struct ScorePlanesArgs {
  const uint8_t *limbs;  // [n_seq * hq] limb records
  const float *centroids;
  int64_t n_seq, n;      // sequences; keys per (sequence, kv head)
  int hq, hkv, q_groups, n_chunks;
  int64_t chunk;         // keys per workgroup (a multiple of 16)
  const uint8_t *idx;
  int64_t idx_stride;
  const uint8_t *sign;
  int64_t sign_stride;
  const uint32_t *norms;
  float *logits;         // [n_seq][hq][n]
};

template <int D, int BITS, int M, bool ASYM>
__global__ __launch_bounds__(kSpW * kWave) void score_planes(ScorePlanesArgs a) {
  constexpr int NK = (D + 63) / 64;
  constexpr int NKM = (M + 63) / 64;
  constexpr int NKM1 = NKM > 0 ? NKM : 1;
  constexpr int NP = n_planes<BITS, ASYM>();

  double wd[1 << BITS];
  if (walsh_weights<BITS>(a.centroids, wd) != ASYM) return;

  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int g = lane >> 4, col = lane & 15;
  int64_t bid = blockIdx.x;
  const int j = (int)(bid % a.q_groups);  // workgroups next to each other share the keys
  bid /= a.q_groups;
  const int c = (int)(bid % a.n_chunks);
  const int64_t b = bid / a.n_chunks;     // key block: sequence * hkv + kv head
  const int G = a.hq / a.hkv;
  const int qg = 64 * j + 16 * wid;       // this wavefront's first query head within the group
  if (qg >= G) return;
  const int64_t rec = (b / a.hkv) * a.hq + (int64_t)(b % a.hkv) * G + qg + col;  // query head record
  const bool ok = qg + col < G;

  PlaneQuery<NK, NKM1, NP> pq;
  load_plane_query<D, BITS, M, ASYM>(a.limbs, rec, ok, wd, pq);

  const int64_t v0 = (int64_t)c * a.chunk;
  const int64_t v1 = v0 + a.chunk < a.n ? v0 + a.chunk : a.n;
  const RowPlanes rp{a.idx + b * a.n * a.idx_stride, a.idx_stride, M > 0 ? a.sign + b * a.n * a.sign_stride : a.idx,
                     a.sign_stride, a.norms + b * a.n};
  float *out = a.logits + (ok ? rec : 0) * a.n + 4 * g;
  const bool vec4 = (a.n & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
  planes_rows<D, BITS, M, ASYM>(rp, pq, v0, v1, [&](int64_t t0, int left, const float(&sc)[4]) {
    if (!ok) return;
    float *o = out + t0;
    if (vec4 && left == 16) {
      *reinterpret_cast<float4 *>(o) = make_float4(sc[0], sc[1], sc[2], sc[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < left) o[i] = sc[i];
    }
  });
}

// query heads per kv head from which the logits come from score_planes
constexpr int kScorePlanesMinG = 32;

static bool planes_config(const CodecView &kc) {
  return (kc.d == 64 || kc.d == 128 || kc.d == 200) && (kc.bits == 2 || kc.bits == 3) && (kc.m == 0 || kc.m == kc.d);
}

static bool use_planes(const CodecView &kc, const ScoreShape &s) {
  return s.hkv > 0 && s.hq / s.hkv >= kScorePlanesMinG && planes_config(kc);
}

size_t scores_workspace(const CodecView &kc, const ScoreShape &s) {
  if (!use_planes(kc, s)) return 0;
  const size_t heads = (size_t)s.n_seq * (size_t)s.hq;
  const size_t qf = heads * (size_t)(kc.d + kc.m) * sizeof(float);
  return (qf + 255) / 256 * 256 + heads * (size_t)limb_record_bytes(kc.d, kc.m);
}

template <int D, int M>
static int launch_qprep(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh,
                        hipStream_t st, const int32_t *pos, float rope_base, uint8_t *limbs = nullptr) {
  QprepArgs a{q, s.n_seq * s.hq, s.hq, s.hkv, s.n, kc.rot, kc.n_rot, kc.vecs_per_rot, kc.sketch, qt, qh, pos,
              rope_base, nullptr, kc.bits};
  const bool one_rot = kc.n_rot == 1 || kc.vecs_per_rot == 0;
  const int G = s.hq / s.hkv;
  if (one_rot || G % kQpHeads == 0) {
    a.limbs = limbs;  // the tiled kernel writes the limb records itself
    // 64 heads per block when that still leaves a thousand blocks (each block reads Pi and S once)
    // (d <= 128: at d = 200 the 64 heads a thread would carry do not fit its registers)
    if (D <= 128 && (one_rot || G % kQpHeadsMany == 0) && a.n_heads >= 1024 * kQpHeadsMany) {
      const int64_t blocks = (a.n_heads + kQpHeadsMany - 1) / kQpHeadsMany;
      if (!grid_fits(blocks)) return TQ_EUNSUPPORTED;
      hipLaunchKernelGGL((qprep_tiled<D, M, D <= 128 ? kQpHeadsMany : kQpHeads>), dim3((unsigned)blocks), dim3(256),
                         0, st, a);
    } else {
      const int64_t blocks = (a.n_heads + kQpHeads - 1) / kQpHeads;
      if (!grid_fits(blocks)) return TQ_EUNSUPPORTED;
      hipLaunchKernelGGL((qprep_tiled<D, M, kQpHeads>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
  }
  const int64_t blocks = (a.n_heads + 3) / 4;
  if (!grid_fits(blocks)) return TQ_EUNSUPPORTED;
  hipLaunchKernelGGL((qprep_kernel<D, M>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  if (limbs != nullptr) {
    hipLaunchKernelGGL((planes_limbs<D, M>), dim3((unsigned)((a.n_heads + 3) / 4)), dim3(256), 0, st, qt, qh,
                       a.n_heads, kc.bits, limbs);
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  }
  return TQ_OK;
}

int qprep(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh, hipStream_t st,
          const int32_t *pos, float rope_base) {
  const int D = kc.d, M = kc.m;
#define TQ_QP(DD, MM) if (D == DD && M == MM) return launch_qprep<DD, MM>(kc, q, s, qt, qh, st, pos, rope_base);
  TQ_QP(64, 0) TQ_QP(64, 64) TQ_QP(128, 0) TQ_QP(128, 128) TQ_QP(200, 0) TQ_QP(200, 200)
#undef TQ_QP
  return TQ_EUNSUPPORTED;
}

int qprep_limbs(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh, uint8_t *limbs,
                hipStream_t st) {
  const int D = kc.d, M = kc.m;
#define TQ_QP(DD, MM) \
  if (D == DD && M == MM) return launch_qprep<DD, MM>(kc, q, s, qt, qh, st, nullptr, 0.0f, limbs);
  TQ_QP(64, 0) TQ_QP(64, 64) TQ_QP(128, 0) TQ_QP(128, 128) TQ_QP(200, 0) TQ_QP(200, 200)
#undef TQ_QP
  return TQ_EUNSUPPORTED;
}

// heads per lookup entry for a GQA group of g heads
static int pick_g(int g) {
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

template <int D, int BITS, int M, int G>
static int launch_score_g(const ScoreArgs &a0, const ScoreShape &s, hipStream_t st) {
  constexpr int NT = score_threads<D, BITS, M, G>();
  ScoreArgs a = a0;
  a.nsub = (s.hq / s.hkv) / G;
  a.chunk = 32768;
  if (s.n < a.chunk) a.chunk = (int)((s.n + NT - 1) / NT * NT);
  if (a.chunk < NT) a.chunk = NT;
  a.n_chunks = (int)((s.n + a.chunk - 1) / a.chunk);
  const int64_t blocks = s.n_seq * s.hkv * a.nsub * a.n_chunks;
  if (!grid_fits(blocks)) return TQ_EUNSUPPORTED;
  hipLaunchKernelGGL((score_kernel<D, BITS, M, G, NT>), dim3((unsigned)blocks), dim3(NT), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

template <int D, int BITS, int M, int G>
constexpr bool lut_fits() {
  return Lut<D, BITS, M, G>::BYTES + G * (2 * D + M) * 4 + 512 <= 160 * 1024;
}

template <int D, int BITS, int M>
static int launch_score_dbm(const ScoreArgs &a, const ScoreShape &s, hipStream_t st) {
  const int want = pick_g(s.hq / s.hkv);
  if (want >= 4) {
    if constexpr (lut_fits<D, BITS, M, 4>()) return launch_score_g<D, BITS, M, 4>(a, s, st);
  }
  if (want >= 2) {
    if constexpr (lut_fits<D, BITS, M, 2>()) return launch_score_g<D, BITS, M, 2>(a, s, st);
  }
  return launch_score_g<D, BITS, M, 1>(a, s, st);
}

template <int D, int BITS, int M>
static int launch_score_planes(const CodecView &kc, const float *q, const ScoreShape &s, const CodesView &k,
                               float *logits, void *ws, hipStream_t st) {
  const size_t heads = (size_t)s.n_seq * (size_t)s.hq;
  float *qt = reinterpret_cast<float *>(ws);
  float *qh = qt + heads * D;
  const size_t qf = heads * (size_t)(D + M) * sizeof(float);
  uint8_t *limbs = reinterpret_cast<uint8_t *>(ws) + (qf + 255) / 256 * 256;
  int rc = qprep_limbs(kc, q, s, qt, qh, limbs, st);
  if (rc != TQ_OK) return rc;
  ScorePlanesArgs a{limbs, kc.centroids, s.n_seq, s.n, s.hq, s.hkv, 0, 1, 0,
                    k.idx, k.idx_stride, k.sign, k.sign_stride, k.norms, logits};
  const int G = s.hq / s.hkv;
  a.q_groups = (G + 16 * kSpW - 1) / (16 * kSpW);
  // about 4096 workgroups, chunks of at least kSpMinRows keys (a multiple of 16), each chunk's
  // bytes in every plane below 2^31 (32-bit buffer offsets)
  const int64_t base = s.n_seq * s.hkv * a.q_groups;
  int64_t want = (4096 + base - 1) / base;
  const int64_t max_chunks = (s.n + kSpMinRows - 1) / kSpMinRows;
  if (want > max_chunks) want = max_chunks;
  if (want < 1) want = 1;
  const int64_t stride = k.idx_stride > k.sign_stride ? k.idx_stride : k.sign_stride;
  const int64_t max_rows = ((int64_t)0x7FFFFFFF - 64 * stride) / (stride > 4 ? stride : 4);
  int64_t chunk = (s.n + want - 1) / want;
  if (chunk > max_rows) chunk = max_rows;
  chunk = (chunk + 15) / 16 * 16;
  a.chunk = chunk;
  a.n_chunks = (int)((s.n + chunk - 1) / chunk);
  if (!grid_fits(base * a.n_chunks)) return TQ_EUNSUPPORTED;
  const unsigned blocks = (unsigned)(base * a.n_chunks);
  hipLaunchKernelGGL((score_planes<D, BITS, M, false>), dim3(blocks), dim3(kSpW * kWave), 0, st, a);
  if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  hipLaunchKernelGGL((score_planes<D, BITS, M, true>), dim3(blocks), dim3(kSpW * kWave), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

int launch_scores(const CodecView &kc, const float *q, const ScoreShape &s, const CodesView &k, float *logits,
                  void *ws, size_t ws_bytes, void *stream) {
  if (s.n == 0 || s.n_seq == 0) return TQ_OK;
  (void)ws_bytes;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (use_planes(kc, s)) {
    const int D = kc.d, B = kc.bits, M = kc.m;
#define TQ_SP(DD, BB, MM) if (D == DD && B == BB && M == MM) return launch_score_planes<DD, BB, MM>(kc, q, s, k, logits, ws, st);
    TQ_SP(64, 2, 64) TQ_SP(64, 3, 64) TQ_SP(64, 2, 0) TQ_SP(64, 3, 0)
    TQ_SP(128, 2, 128) TQ_SP(128, 3, 128) TQ_SP(128, 2, 0) TQ_SP(128, 3, 0)
    TQ_SP(200, 2, 200) TQ_SP(200, 3, 200) TQ_SP(200, 2, 0) TQ_SP(200, 3, 0)
#undef TQ_SP
    return TQ_EUNSUPPORTED;
  }
  ScoreArgs a{q, kc.rot, kc.sketch, kc.centroids, kc.n_rot, kc.vecs_per_rot, s.n_seq, s.n, s.hq, s.hkv, 1, 1, 1,
              k.idx, k.idx_stride, k.sign, k.sign_stride, k.norms, logits};
  const int D = kc.d, B = kc.bits, M = kc.m;
#define TQ_SC(DD, BB, MM) if (D == DD && B == BB && M == MM) return launch_score_dbm<DD, BB, MM>(a, s, st);
  TQ_SC(64, 2, 64) TQ_SC(64, 3, 64) TQ_SC(64, 4, 64) TQ_SC(64, 2, 0) TQ_SC(64, 3, 0) TQ_SC(64, 4, 0)
  TQ_SC(128, 2, 128) TQ_SC(128, 3, 128) TQ_SC(128, 4, 128) TQ_SC(128, 2, 0) TQ_SC(128, 3, 0) TQ_SC(128, 4, 0)
  TQ_SC(200, 2, 200) TQ_SC(200, 3, 200) TQ_SC(200, 2, 0) TQ_SC(200, 3, 0)
#undef TQ_SC
  return TQ_EUNSUPPORTED;
}

}  // namespace tq
