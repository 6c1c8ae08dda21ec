// One decode step of attention over the compressed K/V cache.
//
// Sources: TurboESM summary (gist.science), section 2.E: a single fused decode kernel loads
// the compressed cache, unpacks the indices, applies the QJL correction and the inverse
// rotation Pi^T, and runs attention with an online softmax, with no dequantised fp16 copy;
// 7minutos.es TurboQuant walkthrough, "Etapa 2 (Corrección Residual)": the dequantised value
// is v~ = Pi^T (nbar c[idx] + sqrt(pi/2)/m rnbar S^T (2 bits - 1)).
//
// Split over the context (flash-decoding): attend_partial runs one workgroup per (sequence,
// kv head, head subgroup, context chunk).  It scores each tile of tokens with the key lookup
// tables (tq_lut.h), keeps a running max and sum per query head, and accumulates the
// softmax-weighted values in the rotated space -- nbar_n c_V[idx_n] per coordinate and, when
// V carries QJL bits, rnbar_n sqrt(pi/2)/m (2 bits - 1) per sketch row -- so no rotation is
// applied per token.  attend_combine merges the chunks of each query head and applies S_V^T
// and Pi_V^T once.

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_lut.h"

namespace tq {

int qprep(const CodecView &kc, const float *q, const ScoreShape &s, float *qt, float *qh, hipStream_t st,
          const int32_t *pos = nullptr, float rope_base = 0.0f);

constexpr float kLog2e = 1.4426950408889634f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct AttArgs {
  const float *qt, *qh, *kcent, *vcent;
  int64_t n_seq, n_ctx;
  int hq, hkv, nsub, n_chunks, chunk;
  float scale_log2;  // softmax scale * log2(e)
  const uint8_t *kidx;
  int64_t kidx_stride;
  const uint8_t *ksign;
  int64_t ksign_stride;
  const uint32_t *knorms;
  const uint8_t *vidx;
  int64_t vidx_stride;
  const uint8_t *vsign;
  int64_t vsign_stride;
  const uint32_t *vnorms;
  float *part;  // [n_seq * hq][n_chunks][2 + d + m_V]
  const int32_t *pos;  // decode step: sequence s attends over tokens 0 .. pos[s] (nullptr: all n_ctx)
  // logits given (attend_partial with LIN): [n_seq][hq][n_ctx] fp32, unscaled, in place of the
  // key codes (keys of another codec, scored by their own kernel)
  const float *lg_in;
};

// The value sum runs on the matrix cores (attend_partial, MV) for four query heads per kv head,
// d = 128, value codes of at most 3 bits and no value sketch, with keys that carry a sketch or
// logits given (3-bit keys without one keep the VALU value sum, which needs fewer registers
// beside their larger key tables).
constexpr bool att_mv(int d, int km, int vb, int vm, int g, bool lin) {
  return g == 4 && vm == 0 && d == 128 && vb <= 3 && (lin || km > 0);
}

// LIN: the logits come from a.lg_in (no key tables, no key records); KB and KM then only size
// unused parts.
template <int D, int KB, int KM, int VB, int VM, int G, int NT, bool LIN = false>
__global__ __launch_bounds__(NT) void attend_partial(AttArgs a) {
  using CK = Lut<D, KB, KM, G>;
  constexpr int KSW = CK::SW > 0 ? CK::SW : 1;
  constexpr int IWV = (D * VB + 31) / 32;
  constexpr int SWV = (VM + 31) / 32;
  constexpr int NOUT = D + VM;
  constexpr int NW = NT / kWave;
  // consecutive output coordinates per lane in the value phase: 16 where their codes fit one
  // 64-bit window of the record and the accumulators leave room (at most 128 outputs), else 8
  constexpr int CPT = (D % 16 == 0 && VM % 16 == 0 && VB * 16 <= 48 && D + VM <= 128) ? 16 : 8;
  constexpr int NCG = NOUT / CPT;    // coordinate groups
  constexpr int TPO = kWave / NCG;   // lanes of a wavefront sharing one coordinate group
  constexpr int TOK = kWave / TPO;   // tokens of a wavefront tile per lane in the value phase
  static_assert(D % CPT == 0 && VM % CPT == 0 && kWave % NCG == 0, "lanes must cover the outputs evenly");
  // MV: the value sum on the matrix cores.  With four query heads, no value sketch and d = 128,
  // the weighted sum over a tile's tokens is a [4 heads x 64 tokens] x [64 tokens x 128] product,
  // run as fp32 4x4x1 blocks.  Block b (lanes 4b .. 4b + 3) takes token TS q + (b mod TS) of the
  // tile and coordinate part b / TS (of 16 / TS): lane 4b + j supplies the weight of head j as
  // its A operand and, for g = 0 .. CPL - 1, the centroid of coordinate (4 (b / TS) + j) CPL + g
  // as its B operand, so a lane's value operands are one contiguous CPL-code slice of the
  // record.  Each block keeps its own partial sums (head i in element i of a lane's
  // accumulator), which the lanes add up once at the end of the chunk.
  constexpr bool MV = att_mv(D, KM, VB, VM, G, LIN);
  constexpr int TS = 8;                  // token slots per block instruction
  constexpr int CPL = D * TS / 64;       // coordinates per lane
  constexpr int LV = 1 << VB;
  constexpr int LP = LV * LV;        // entries of the two-code value table
  // One LDS arena with fixed offsets: the value table and the per-wavefront tiles at the bottom
  // (immediate ds offsets), the lookup tables at the top; the final merge reuses the tables.
  constexpr int WT_V = kWave * IWV;                 // words per wavefront: value index records
  constexpr int WT_S = VM > 0 ? kWave * SWV : 0;    // value sign records
  constexpr int O_CBV2 = 0;
  constexpr int O_WAVE = O_CBV2 + LP * 8;
  constexpr int WAVE_BYTES = ((WT_V + WT_S) * 4 + kWave * G * 4 * (VM > 0 ? 2 : 1) + 15) / 16 * 16;
  constexpr int O_CBK = O_WAVE + NW * WAVE_BYTES;
  constexpr int O_CBV = O_CBK + (1 << KB) * 4;
  constexpr int O_SC = O_CBV + LV * 4;
  constexpr int O_QT = O_SC + 4 * G * 4;
  constexpr int O_QH = O_QT + G * D * 4;
  constexpr int O_TABS = (O_QH + G * (KM > 0 ? KM : 1) * 4 + 15) / 16 * 16;
  constexpr int MERGE_BYTES = NW * (NOUT + 2) * G * 4;
  constexpr int TAB_BYTES = LIN ? 0 : CK::BYTES;
  constexpr int ARENA = O_TABS + (TAB_BYTES > MERGE_BYTES ? TAB_BYTES : MERGE_BYTES);
  static_assert(ARENA <= 160 * 1024, "LDS arena");
  __shared__ __align__(16) uint8_t arena[ARENA];
  float2 *cbv2 = reinterpret_cast<float2 *>(arena + O_CBV2);  // (c[a], c[b]) for (b << VB) | a
  float *cbk = reinterpret_cast<float *>(arena + O_CBK);
  float *cbv = reinterpret_cast<float *>(arena + O_CBV);
  float *sc = reinterpret_cast<float *>(arena + O_SC);  // table scales (block_table_scales)
  float *qt = reinterpret_cast<float *>(arena + O_QT);
  float *qh = reinterpret_cast<float *>(arena + O_QH);
  uint8_t *tabs = arena + O_TABS;

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  uint8_t *wbase = arena + O_WAVE + wid * WAVE_BYTES;
  uint32_t *vtile = reinterpret_cast<uint32_t *>(wbase);             // [64][IWV]
  uint32_t *vstile = vtile + WT_V;                                   // [64][SWV]
  float *wt = reinterpret_cast<float *>(vtile + WT_V + WT_S);        // [64][G]: p * nbar_V
  float *wq = wt + kWave * G;                                        // [64][G]: p * rnbar_V * kappa_V

  const int64_t b = blockIdx.x;
  const int chunk = (int)(b % a.n_chunks);
  const int64_t rest = b / a.n_chunks;
  const int sub = (int)(rest % a.nsub);
  const int64_t blk = rest / a.nsub;
  const int64_t s = blk / a.hkv;
  const int kvh = (int)(blk % a.hkv);
  const int h0 = kvh * (a.hq / a.hkv) + sub * G;
  const int64_t qrow = s * a.hq + h0;

  // Tokens of this sequence: all n_ctx, or 0 .. pos[s] in a decode step (none when pos[s] is
  // outside the cache).  A chunk past them holds an empty state: max -inf, sum 0, outputs 0.
  int64_t len = a.n_ctx;
  if (a.pos != nullptr) {
    const int64_t p = a.pos[s];
    len = (p >= 0 && p < a.n_ctx) ? p + 1 : 0;
  }
  if ((int64_t)chunk * a.chunk >= len) {
    for (int e = tid; e < G * (2 + NOUT); e += NT) {
      const int h = e / (2 + NOUT), o = e % (2 + NOUT);
      a.part[((qrow + h) * a.n_chunks + chunk) * (int64_t)(2 + NOUT) + o] = o == 0 ? -INFINITY : 0.0f;
    }
    return;  // uniform over the workgroup
  }

  if constexpr (!LIN) {
    for (int i = tid; i < G * D; i += NT) qt[i] = a.qt[qrow * D + i];
    if constexpr (KM > 0)
      for (int i = tid; i < G * KM; i += NT) qh[i] = a.qh[qrow * KM + i];
    if (tid < (1 << KB)) cbk[tid] = a.kcent[tid];
  }
  if (tid < LV) cbv[tid] = a.vcent[tid];
  for (int e = tid; e < LP; e += NT) cbv2[e] = make_float2(a.vcent[e & (LV - 1)], a.vcent[e >> VB]);
  __syncthreads();
  HeadScales<G> hs;
  if constexpr (!LIN) {
    block_table_scales<D, KB, KM, G>(qt, qh, cbk, sc, hs);
    // the half-table builder's scratch aliases the wavefronts' tile area, unused until the tiles
    constexpr bool HALF = lut_half_bytes<D, KB, KM, G>() <= NW * WAVE_BYTES;
    build_luts<D, KB, KM, G, NT>(tabs, tabs + CK::MSE_BYTES, qt, qh, cbk, sc, sc + G,
                                 HALF ? reinterpret_cast<float *>(arena + O_WAVE) : nullptr);
    __syncthreads();
  }

  const float kappa_k = KM > 0 ? 1.2533141373155003f / (float)(KM > 0 ? KM : 1) : 0.0f;
  const float kappa_v = VM > 0 ? 1.2533141373155003f / (float)(VM > 0 ? VM : 1) : 0.0f;
  const int64_t t0 = (int64_t)chunk * a.chunk;
  int64_t t1 = t0 + a.chunk;
  if (t1 > len) t1 = len;
  const int64_t vbase = blk * a.n_ctx;

  // value-phase role of this lane: outputs o0 .. o0 + CPT - 1 for tokens part*TOK .. + TOK - 1
  // of the wavefront's tile
  const int o0 = (lane % NCG) * CPT;
  const int part = lane / NCG;
  const bool is_val = o0 < D;
  const int vw0 = is_val ? (o0 * VB) >> 5 : 0;
  const int vsh = is_val ? (o0 * VB) & 31 : 0;
  const int vw1i = (vw0 + 1 < IWV) ? vw0 + 1 : vw0;  // a clamped second word: its bits are masked off when unused
  const int sj = is_val ? 0 : o0 - D;                 // first sketch row (value QJL part)

  // Wavefront-local online softmax: mrun is uniform over the wavefront; lpart is this lane's
  // share of the running sum (the tokens it scored), acc its share of the outputs.
  float mrun[G], lpart[G], acc[MV ? 1 : CPT][G];
  f32x4 macc[MV ? CPL : 1];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mrun[h] = -INFINITY;
    lpart[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < (MV ? 1 : CPT); ++c) acc[c][h] = 0.0f;
  }
#pragma unroll
  for (int g = 0; g < (MV ? CPL : 1); ++g) macc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // MV: the lane's slice (coordinates mc0 .. mc0 + CPL - 1) starts at bit mbit of the record:
  // word mw0, bit msh of that word
  const int mslot = (lane >> 2) % TS;             // token slot
  const int mc0 = (4 * (lane / (4 * TS)) + (lane & 3)) * CPL;
  const int mbit = VB * mc0;
  const int mw0 = mbit >> 5, msh = mbit & 31;
  const int mw1 = mw0 + 1 < IWV ? mw0 + 1 : mw0;  // a clamped second word (its bits unused when past the slice)

  // the records of the lane's token (LIN: its logits in place of its key record)
  struct Rec {
    uint32_t iw[CK::IW];
    uint32_t sw[KSW];
    uint32_t nw;
    uint32_t vw[IWV];
    uint32_t vs[VM > 0 ? SWV : 1];
    uint32_t vnw;
    float lgi[LIN ? G : 1];
  };
  auto load_rec = [&](int64_t t, Rec &r) {
    if (t < t1) {
      const int64_t v = vbase + t;
      if constexpr (LIN) {
#pragma unroll
        for (int h = 0; h < G; ++h) r.lgi[h] = a.lg_in[(qrow + h) * a.n_ctx + t];
      } else {
        load_words<CK::IW>(a.kidx + v * a.kidx_stride, r.iw);
        if constexpr (KM > 0) load_words<CK::SW>(a.ksign + v * a.ksign_stride, r.sw);
        r.nw = a.knorms[v];
      }
      load_words<IWV>(a.vidx + v * a.vidx_stride, r.vw);
      if constexpr (VM > 0) load_words<SWV>(a.vsign + v * a.vsign_stride, r.vs);
      r.vnw = a.vnorms[v];
    }
  };
  // Tiles of 64 tokens, wavefront w taking tiles w, w + NW, ...; no workgroup barrier until the
  // final merge, so wavefronts in the lookup phase overlap wavefronts in the value phase.
  Rec cur;
  load_rec(t0 + (int64_t)wid * kWave + lane, cur);
  // both table bases opaque (one scalar register each): the group offsets within them fit the
  // 16-bit immediate of the LDS reads, with no per-group base held in a vector register
  const uint8_t *mse_tabs = arena + opaque_offset(O_TABS);
  const uint8_t *qjl_tabs = arena + opaque_offset(O_TABS + CK::MSE_BYTES);

  for (int64_t tile = t0 + (int64_t)wid * kWave; tile < t1; tile += (int64_t)NW * kWave) {
    // ---- phase A: one token per lane: logits, value records to the wavefront's tile
    const int64_t t = tile + lane;
    const bool valid = t < t1;
    float lg[G];
    float vn = 0.0f, vr = 0.0f;
    if (valid) {
#pragma unroll
      for (int i = 0; i < IWV; ++i) vtile[lane * IWV + i] = cur.vw[i];
      if constexpr (VM > 0) {
#pragma unroll
        for (int i = 0; i < SWV; ++i) vstile[lane * SWV + i] = cur.vs[i];
      }
      vn = f16_bits_to_float(cur.vnw & 0xFFFFu);
      vr = f16_bits_to_float(cur.vnw >> 16) * kappa_v;
      if constexpr (LIN) {
#pragma unroll
        for (int h = 0; h < G; ++h) lg[h] = cur.lgi[h] * a.scale_log2;
      } else {
        float am[G], aq[G];
        lut_score<D, KB, KM, G>(cur.iw, cur.sw, mse_tabs, qjl_tabs, hs, am, aq);
        const float nbar = f16_bits_to_float(cur.nw & 0xFFFFu);
        const float rq = f16_bits_to_float(cur.nw >> 16) * kappa_k;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float sc = nbar * am[h];
          if constexpr (KM > 0) sc = fmaf(rq, aq[h], sc);
          lg[h] = sc * a.scale_log2;
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) lg[h] = -INFINITY;
    }
    load_rec(tile + (int64_t)NW * kWave + lane, cur);  // the next tile's records
    // The running maxima change only when some lane's logit exceeds them, which is rare after
    // the first tiles: the wavefront reductions and the rescale run only then (a ballot), and
    // otherwise the maxima and alpha = 1 are exactly what the reductions would give.
    float alpha[G];
    bool up = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      alpha[h] = 1.0f;
      up |= lg[h] > mrun[h];
    }
    if (__ballot(up) != 0ull) {  // uniform over the wavefront
      bool rescale = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mnew = fmaxf(mrun[h], wave_max(lg[h]));
        alpha[h] = exp2f(mrun[h] - mnew);  // 0 on the first tile (mrun = -inf)
        rescale |= mnew != mrun[h];
        mrun[h] = mnew;
      }
      if (rescale) {
        if constexpr (MV) {
#pragma unroll
          for (int g = 0; g < CPL; ++g)
#pragma unroll
            for (int h = 0; h < 4; ++h) macc[g][h] *= alpha[h];
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < CPT; ++c) acc[c][h] *= alpha[h];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = valid ? exp2f(lg[h] - mrun[h]) : 0.0f;
      lpart[h] = fmaf(lpart[h], alpha[h], p);
      wt[lane * G + h] = p * vn;
      if constexpr (VM > 0) wq[lane * G + h] = p * vr;
    }
    wave_lds_fence();
    // ---- phase B: weighted values; tokens past the end carry weight 0
    const int n0 = part * TOK;
    if constexpr (MV) {
      constexpr int PB = 2 * VB;  // bits of a code pair
      static_assert(VB * CPL <= 64, "a lane's slice within two realigned words");
#pragma unroll 2
      for (int q = 0; q < kWave / TS; ++q) {
        const int n = TS * q + mslot;
        const float w = wt[4 * TS * q + (lane & (4 * TS - 1))];  // p * nbar_V of token n, head lane mod 4
        const uint32_t x0 = __builtin_amdgcn_alignbit(vtile[n * IWV + mw1], vtile[n * IWV + mw0], msh);
        const uint32_t x1 = vtile[n * IWV + mw1] >> msh;  // bits 32 .. of the slice
#pragma unroll
        for (int k = 0; k < CPL / 2; ++k) {  // coordinates 2k, 2k + 1 of the slice
          const int bit = PB * k;
          const uint32_t code =
              (bit + PB <= 32 ? x0 >> bit : (bit >= 32 ? x1 >> (bit - 32) : __builtin_amdgcn_alignbit(x1, x0, bit))) &
              (LP - 1);
          const float2 cv = cbv2[code];
          macc[2 * k] = __builtin_amdgcn_mfma_f32_4x4x1f32(w, cv.x, macc[2 * k], 0, 0, 0);
          macc[2 * k + 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(w, cv.y, macc[2 * k + 1], 0, 0, 0);
        }
      }
    } else if (is_val) {
#pragma unroll 4
      for (int n = n0; n < n0 + TOK; ++n) {
        const uint32_t w0 = vtile[n * IWV + vw0];
        const uint32_t w1 = vtile[n * IWV + vw1i];
        const uint64_t bits = ((((uint64_t)w1) << 32) | w0) >> vsh;
        float wv[G];
        if constexpr (G == 4) {
          const float4 t4 = *reinterpret_cast<const float4 *>(&wt[n * G]);
          wv[0] = t4.x; wv[1] = t4.y; wv[2] = t4.z; wv[3] = t4.w;
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) wv[h] = wt[n * G + h];
        }
#pragma unroll
        for (int c = 0; c < CPT; c += 2) {
          const float2 cv = cbv2[(uint32_t)(bits >> (VB * c)) & (LP - 1)];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[c][h] = fmaf(wv[h], cv.x, acc[c][h]);
            acc[c + 1][h] = fmaf(wv[h], cv.y, acc[c + 1][h]);
          }
        }
      }
    } else if constexpr (VM > 0) {
#pragma unroll 4
      for (int n = n0; n < n0 + TOK; ++n) {
        const uint32_t sb = vstile[n * SWV + (sj >> 5)] >> (sj & 31);  // CPT rows within one word
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const bool pos = (sb >> c) & 1u;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float x = wq[n * G + h];
            acc[c][h] += pos ? x : -x;
          }
        }
      }
    }
    wave_lds_fence();  // the next tile overwrites this wavefront's records and weights
  }

  // ---- merge: the lanes of a coordinate group, then the wavefronts, then write this chunk's
  // partial state (max, sum, outputs) per query head
  // MV: the TS token slots' partial sums, halved at each exchange over lane bits log2(TS) + 1
  // .. 2 (a lane keeps the half its bit selects and adds its partner's copy of it), end with
  // lane 4b + j holding e = 4g + i for e in [MR (b mod TS), MR (b mod TS) + MR)
  constexpr int MR = MV ? 4 * CPL / TS : 1;
  float mred[MV ? 4 * CPL : 1];
  if constexpr (MV) {
#pragma unroll
    for (int g = 0; g < CPL; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) mred[4 * g + i] = macc[g][i];
#pragma unroll
    for (int m = 2 * TS; m >= 4; m >>= 1) {
      const int hlf = CPL * m / TS;  // values kept after this exchange
      const bool up = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < hlf; ++e) {
        const float keep = up ? mred[e + hlf] : mred[e];
        const float send = up ? mred[e] : mred[e + hlf];
        mred[e] = keep + __shfl_xor(send, m, kWave);
      }
    }
  } else {
#pragma unroll
    for (int off = NCG; off < kWave; off *= 2)
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[c][h] += __shfl_xor(acc[c][h], off, kWave);
  }
  float lw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lw[h] = wave_sumf(lpart[h]);
  __syncthreads();  // every wavefront is done with the tables
  float *mg = reinterpret_cast<float *>(tabs);  // [NW][G] max, [NW][G] sum, [NW][NOUT][G] outputs
  float *lsum = mg + NW * G;
  float *outs = lsum + NW * G;
  if (lane < G) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (h == lane) {
        mg[wid * G + h] = mrun[h];
        lsum[wid * G + h] = lw[h];
      }
  }
  if constexpr (MV) {
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int e = MR * mslot + r;
      outs[(wid * NOUT + mc0 + (e >> 2)) * G + (e & 3)] = mred[r];
    }
  } else if (part == 0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int h = 0; h < G; ++h) outs[(wid * NOUT + o0 + c) * G + h] = acc[c][h];
  }
  __syncthreads();
  for (int e = tid; e < NOUT * G; e += NT) {
    const int o = e / G, h = e % G;
    float m = -INFINITY;
    for (int w = 0; w < NW; ++w) m = fmaxf(m, mg[w * G + h]);
    float sacc = 0.0f, lt = 0.0f;
    for (int w = 0; w < NW; ++w) {
      const float sc = mg[w * G + h] == -INFINITY ? 0.0f : exp2f(mg[w * G + h] - m);
      sacc = fmaf(sc, outs[(w * NOUT + o) * G + h], sacc);
      lt = fmaf(sc, lsum[w * G + h], lt);
    }
    float *dst = a.part + ((qrow + h) * a.n_chunks + chunk) * (int64_t)(2 + NOUT);
    dst[2 + o] = sacc;
    if (o == 0) {
      dst[0] = m;
      dst[1] = lt;
    }
  }
}

struct CombArgs {
  const float *part;
  int64_t n_heads;  // n_seq * hq
  int hq, hkv, n_chunks;
  int64_t n_ctx;
  const float *vrot;
  int n_rot;
  int64_t vecs_per_rot;
  const float *vsketch;
  float *out;
};

// sum_i W[i * ld + col] v[i] for i = 0 .. N - 1, i ascending (one fp32 FMA chain), with the
// column's elements requested 32 at a time so that a chain waits for one load latency per 32
// elements instead of one per few
template <int N>
__device__ __forceinline__ float column_dot(const float *W, int64_t ld, int col, const float *v, float acc) {
  constexpr int B = 32;
#pragma unroll 1
  for (int i0 = 0; i0 < N; i0 += B) {
    float w[B];
#pragma unroll
    for (int t = 0; t < B; ++t) w[t] = (i0 + t < N) ? W[(int64_t)(i0 + t) * ld + col] : 0.0f;
#pragma unroll
    for (int t = 0; t < B; ++t)
      if (i0 + t < N) acc = fmaf(w[t], v[i0 + t], acc);
  }
  return acc;
}

// column_dot for H vectors at once: acc[h] = sum_i W[i * ld + col] v_h[i], i ascending (one FMA
// chain per h, the same as column_dot's), each element of W requested once for all H.
template <int N, int H>
__device__ __forceinline__ void column_dot_n(const float *W, int64_t ld, int col, const float *const (&v)[H],
                                             float (&acc)[H]) {
  constexpr int B = 32;
#pragma unroll 1
  for (int i0 = 0; i0 < N; i0 += B) {
    float w[B];
#pragma unroll
    for (int t = 0; t < B; ++t) w[t] = (i0 + t < N) ? W[(int64_t)(i0 + t) * ld + col] : 0.0f;
#pragma unroll
    for (int t = 0; t < B; ++t)
#pragma unroll
      for (int h = 0; h < H; ++h)
        if (i0 + t < N) acc[h] = fmaf(w[t], v[h][i0 + t], acc[h]);
  }
}

// Four query heads per workgroup, one wavefront each: the chunks' states merged, S_V^T applied,
// then Pi_V^T.  With one rotation for every head the workgroup applies Pi_V^T together: after a
// barrier, wavefront w takes output columns w D/4 .. (w + 1) D/4 - 1 of all four heads, so each
// element of Pi_V is read once per workgroup instead of once per head.
template <int D, int VM>
__global__ __launch_bounds__(256) void attend_combine(CombArgs a) {
  constexpr int NOUT = D + VM;
  constexpr int CW = D / 4;         // output columns per wavefront in the shared product
  constexpr int HPL = 4 * CW / kWave;  // heads per lane there
  static_assert(D % 4 == 0 && kWave % CW == 0 && HPL >= 1, "columns over the lanes");
  __shared__ float av[4][NOUT];
  __shared__ float uv[4][D];
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int64_t hidx = (int64_t)blockIdx.x * 4 + wid;
  const bool shared_rot = !(a.n_rot > 1 && a.vecs_per_rot > 0);  // uniform over the grid
  bool have = hidx < a.n_heads;  // uniform over the wavefront
  const float *p = a.part + (have ? hidx : 0) * a.n_chunks * (int64_t)(2 + NOUT);
  float m = -INFINITY;
  if (have) {
    for (int c = lane; c < a.n_chunks; c += kWave) m = fmaxf(m, p[c * (2 + NOUT)]);
    m = wave_max(m);
  }
  have = have && m != -INFINITY;  // else no cached token for this sequence: zero output
  if (have) {
    float l = 0.0f;
    for (int c = lane; c < a.n_chunks; c += kWave) l += exp2f(p[c * (2 + NOUT)] - m) * p[c * (2 + NOUT) + 1];
    l = wave_sumf(l);
    const float inv = 1.0f / l;
    for (int o = lane; o < NOUT; o += kWave) {
      float sacc = 0.0f;
      for (int c = 0; c < a.n_chunks; ++c) sacc = fmaf(exp2f(p[c * (2 + NOUT)] - m), p[c * (2 + NOUT) + 2 + o], sacc);
      av[wid][o] = sacc * inv;
    }
    wave_lds_fence();
    // u = A_rot + S_V^T A_sk in the rotated space (A_sk already carries sqrt(pi/2)/m)
    for (int i = lane; i < D; i += kWave) {
      float u = av[wid][i];
      if constexpr (VM > 0) u = column_dot<VM>(a.vsketch, D, i, &av[wid][D], u);
      uv[wid][i] = u;
    }
  } else {
    for (int i = lane; i < D; i += kWave) uv[wid][i] = 0.0f;  // Pi^T 0 = +0
  }
  if (shared_rot) {
    __syncthreads();  // every wavefront's u is in LDS
    const int col = wid * CW + lane % CW;
    const int hg = lane / CW;  // heads hg HPL .. hg HPL + HPL - 1
    const float *v[HPL];
    float acc[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      v[j] = uv[hg * HPL + j];
      acc[j] = 0.0f;
    }
    column_dot_n<D, HPL>(a.vrot, D, col, v, acc);  // (Pi^T u)_col
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      const int64_t hj = (int64_t)blockIdx.x * 4 + hg * HPL + j;
      if (hj < a.n_heads) a.out[hj * D + col] = acc[j];
    }
    return;
  }
  if (hidx >= a.n_heads) return;  // uniform over the wavefront
  wave_lds_fence();
  const int64_t s = hidx / a.hq;
  const int h = (int)(hidx % a.hq);
  const int64_t blk = s * a.hkv + h / (a.hq / a.hkv);
  int64_t rid = 0;
  rid = (blk * a.n_ctx) / a.vecs_per_rot;
  if (rid > a.n_rot - 1) rid = a.n_rot - 1;
  const float *R = a.vrot + rid * (int64_t)D * D;
  for (int k = lane; k < D; k += kWave) a.out[hidx * D + k] = column_dot<D>(R, D, k, uv[wid], 0.0f);  // (Pi^T u)_k
}

// ------------------------------------------------------------------ host side

static int att_g(int g) { return g % 4 == 0 ? 4 : (g % 2 == 0 ? 2 : 1); }

// Tokens per workgroup: as many as possible (each workgroup builds the key tables once), as long
// as enough workgroups remain when the context allows it.  With four query heads per kv head the
// tables take most of the LDS, one workgroup per CU, and nothing overlaps a workgroup's table
// build: chunks of up to 131072 tokens while at least 256 workgroups (one per CU) remain.  With
// fewer heads per workgroup, where several workgroups share a CU: up to 16384 tokens while at
// least 512 remain.
static int att_chunk(const ScoreShape &s) {
  const int64_t pairs = s.n_seq * s.hkv;
  const bool one_per_cu = s.hkv > 0 && att_g(s.hq / s.hkv) == 4;
  const int64_t min_wg = one_per_cu ? 256 : 512;
  int ch = one_per_cu ? 131072 : 16384;
  while (ch > 512 && pairs * ((s.n + ch - 1) / ch) < min_wg) ch /= 2;
  return ch;
}

size_t attend_workspace(const CodecView &kc, const CodecView &vc, const ScoreShape &s) {
  const int64_t nch = (s.n + att_chunk(s) - 1) / att_chunk(s);
  const size_t q = (size_t)s.n_seq * s.hq * (size_t)(kc.d + kc.m) * sizeof(float);
  const size_t q_al = (q + 255) / 256 * 256;
  return q_al + (size_t)s.n_seq * s.hq * nch * (size_t)(2 + vc.d + vc.m) * sizeof(float);
}

template <int D, int KB, int KM, int VB, int VM, int G, bool LIN = false>
static int launch_att(const AttArgs &a0, const ScoreShape &s, hipStream_t st) {
  constexpr int NOUT = D + VM;
  constexpr int NT = (G == 4) ? 512 : (NOUT > 256 ? 512 : 256);
  AttArgs a = a0;
  a.nsub = (s.hq / s.hkv) / G;
  if (!grid_fits(s.n_seq * s.hkv * a.nsub * a.n_chunks)) return TQ_EUNSUPPORTED;
  hipLaunchKernelGGL((attend_partial<D, KB, KM, VB, VM, G, NT, LIN>), dim3((unsigned)(s.n_seq * s.hkv * a.nsub * a.n_chunks)),
                     dim3(NT), 0, st, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

template <int D, int KB, int KM, int VB, int VM, bool LIN = false>
static int launch_att_g(const AttArgs &a, const ScoreShape &s, hipStream_t st) {
  switch (att_g(s.hq / s.hkv)) {
    case 4: return launch_att<D, KB, KM, VB, VM, 4, LIN>(a, s, st);
    case 2: return launch_att<D, KB, KM, VB, VM, 2, LIN>(a, s, st);
    default: return launch_att<D, KB, KM, VB, VM, 1, LIN>(a, s, st);
  }
}

template <int D, int VM>
static int launch_comb(const CombArgs &c, hipStream_t st) {
  hipLaunchKernelGGL((attend_combine<D, VM>), dim3((unsigned)((c.n_heads + 3) / 4)), dim3(256), 0, st, c);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

// The (d, key bits, key m, value bits, value m) combinations built for attention over key codes,
// and the (d, value bits, value m) ones built for attention from given logits.
#define TQ_ATTEND_CONFIGS(X) \
  X(64, 2, 64, 2, 64) X(64, 3, 64, 3, 64) X(64, 2, 64, 3, 0) X(128, 2, 128, 3, 0) X(128, 3, 0, 3, 0) \
  X(128, 2, 128, 2, 128) X(128, 3, 128, 3, 128)
#define TQ_ATTEND_LOGITS_CONFIGS(X) X(64, 2, 64) X(64, 3, 64) X(64, 3, 0) X(128, 3, 0) X(128, 2, 128) X(128, 3, 128)

// Grids of the attention launches within the launch limit.
static bool attend_grids_fit(const ScoreShape &s) {
  const int64_t nch = (s.n + att_chunk(s) - 1) / att_chunk(s);
  const int g = s.hq / s.hkv;
  // attend_partial; the query prep and attend_combine take at most one workgroup per 4 heads
  return grid_fits(s.n_seq * s.hkv * (g / att_g(g)) * nch) && grid_fits((s.n_seq * s.hq + 3) / 4);
}

int attend_preflight(const CodecView &kc, const CodecView &vc, const ScoreShape &s) {
  bool ok = false;
#define TQ_AT_OK(DD, A, B, C, E) ok = ok || (kc.d == DD && kc.bits == A && kc.m == B && vc.bits == C && vc.m == E);
  TQ_ATTEND_CONFIGS(TQ_AT_OK)
#undef TQ_AT_OK
  return ok && attend_grids_fit(s) ? TQ_OK : TQ_EUNSUPPORTED;
}

int attend_logits_preflight(const CodecView &vc, const ScoreShape &s) {
  bool ok = false;
#define TQ_AL_OK(DD, C, E) ok = ok || (vc.d == DD && vc.bits == C && vc.m == E);
  TQ_ATTEND_LOGITS_CONFIGS(TQ_AL_OK)
#undef TQ_AL_OK
  return ok && attend_grids_fit(s) ? TQ_OK : TQ_EUNSUPPORTED;
}

int launch_attend(const CodecView &kc, const CodecView &vc, const float *q, const ScoreShape &s, const CodesView &k,
                  const CodesView &v, float scale, float *out, void *ws, size_t ws_bytes, void *stream,
                  const int32_t *pos, float rope_base) {
  if (s.n_seq == 0) return TQ_OK;
  (void)ws_bytes;
  if (attend_preflight(kc, vc, s) != TQ_OK) return TQ_EUNSUPPORTED;  // before any launch
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float *qt = reinterpret_cast<float *>(ws);
  float *qh = qt + (size_t)s.n_seq * s.hq * kc.d;
  const size_t qbytes = (size_t)s.n_seq * s.hq * (size_t)(kc.d + kc.m) * sizeof(float);
  float *part = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + (qbytes + 255) / 256 * 256);
  int rc = qprep(kc, q, s, qt, qh, st, pos, rope_base);
  if (rc != TQ_OK) return rc;
  const int ch = att_chunk(s);
  const int nch = (int)((s.n + ch - 1) / ch);
  AttArgs a{qt, qh, kc.centroids, vc.centroids, s.n_seq, s.n, s.hq, s.hkv, 1, nch, ch, scale * kLog2e,
            k.idx, k.idx_stride, k.sign, k.sign_stride, k.norms, v.idx, v.idx_stride, v.sign, v.sign_stride,
            v.norms, part, pos};
  const int D = kc.d, KB = kc.bits, KM = kc.m, VB = vc.bits, VM = vc.m;
  rc = TQ_EUNSUPPORTED;
#define TQ_AT(DD, A, B, C, E) \
  if (D == DD && KB == A && KM == B && VB == C && VM == E) rc = launch_att_g<DD, A, B, C, E>(a, s, st); else
  TQ_ATTEND_CONFIGS(TQ_AT) {}
#undef TQ_AT
  if (rc != TQ_OK) return rc;
  CombArgs c{part, s.n_seq * s.hq, s.hq, s.hkv, nch, s.n, vc.rot, vc.n_rot, vc.vecs_per_rot, vc.sketch, out};
  if (D == 64 && VM == 64) return launch_comb<64, 64>(c, st);
  if (D == 64 && VM == 0) return launch_comb<64, 0>(c, st);
  if (D == 128 && VM == 0) return launch_comb<128, 0>(c, st);
  if (D == 128 && VM == 128) return launch_comb<128, 128>(c, st);
  return TQ_EUNSUPPORTED;
}

size_t attend_logits_workspace(const CodecView &vc, const ScoreShape &s) {
  const int64_t nch = (s.n + att_chunk(s) - 1) / att_chunk(s);
  return (size_t)s.n_seq * s.hq * nch * (size_t)(2 + vc.d + vc.m) * sizeof(float);
}

// Attention from given logits: the same chunked pass (online softmax, values in the rotated
// space) and chunk merge, with the logits read instead of computed from key codes.
int launch_attend_logits(const CodecView &vc, const float *logits, const ScoreShape &s, const CodesView &v,
                         float scale, float *out, void *ws, void *stream, const int32_t *pos) {
  if (s.n_seq == 0) return TQ_OK;
  if (attend_logits_preflight(vc, s) != TQ_OK) return TQ_EUNSUPPORTED;  // before any launch
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float *part = reinterpret_cast<float *>(ws);
  const int ch = att_chunk(s);
  const int nch = (int)((s.n + ch - 1) / ch);
  AttArgs a{nullptr, nullptr, nullptr, vc.centroids, s.n_seq, s.n, s.hq, s.hkv, 1, nch, ch, scale * kLog2e,
            nullptr, 0, nullptr, 0, nullptr, v.idx, v.idx_stride, v.sign, v.sign_stride, v.norms, part, pos,
            logits};
  const int D = vc.d, VB = vc.bits, VM = vc.m;
  int rc = TQ_EUNSUPPORTED;
#define TQ_AL(DD, C, E) \
  if (D == DD && VB == C && VM == E) rc = launch_att_g<DD, 2, 0, C, E, true>(a, s, st); else
  TQ_ATTEND_LOGITS_CONFIGS(TQ_AL) {}
#undef TQ_AL
  if (rc != TQ_OK) return rc;
  CombArgs c{part, s.n_seq * s.hq, s.hq, s.hkv, nch, s.n, vc.rot, vc.n_rot, vc.vecs_per_rot, vc.sketch, out};
  if (D == 64 && VM == 64) return launch_comb<64, 64>(c, st);
  if (D == 64 && VM == 0) return launch_comb<64, 0>(c, st);
  if (D == 128 && VM == 0) return launch_comb<128, 0>(c, st);
  if (D == 128 && VM == 128) return launch_comb<128, 128>(c, st);
  return TQ_EUNSUPPORTED;
}

}  // namespace tq
