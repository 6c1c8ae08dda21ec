// Measurement aid, not part of libtq: the HBM traffic of the score stream (tq_scores with four
// query heads per kv head) without its arithmetic.  Same grid, workgroup size, key order and
// logit layout as score_kernel: per key the index record, the sign record and the norm word are
// read with the same loads, and four fp32 values are written to the four head planes
// [n_seq][hq][n_keys].  What it reaches is the practical HBM ceiling of that access pattern on
// the part, against which the score stream's own time is read.  Built into libtq_traffic.so,
// loaded by bench.py only.

#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr int kNT = 1024;
constexpr int kChunk = 32768;

struct TwinArgs {
  const uint8_t *idx, *sign;
  int64_t idx_stride, sign_stride;
  const uint32_t *norms;
  float *logits;
  int64_t n_keys;
  int hq, hkv, nsub, n_chunks;
};

template <int IW, int SW>
__global__ __launch_bounds__(kNT) void score_traffic(TwinArgs a) {
  const int64_t b = blockIdx.x;
  const int chunk = (int)(b % a.n_chunks);
  const int64_t rest = b / a.n_chunks;
  const int sub = (int)(rest % a.nsub);
  const int64_t blk = rest / a.nsub;
  const int64_t s = blk / a.hkv;
  const int kvh = (int)(blk % a.hkv);
  const int64_t qrow = s * a.hq + kvh * (a.hq / a.hkv) + sub * 4;
  const int64_t t0 = (int64_t)chunk * kChunk;
  int64_t t1 = t0 + kChunk;
  if (t1 > a.n_keys) t1 = a.n_keys;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kNT) {
    const int64_t v = blk * a.n_keys + t;
    const uint4 *ip = reinterpret_cast<const uint4 *>(a.idx + v * a.idx_stride);
    const uint4 *sp = reinterpret_cast<const uint4 *>(a.sign + v * a.sign_stride);
    uint32_t x = a.norms[v];
#pragma unroll
    for (int k = 0; k < IW; ++k) {
      const uint4 w = ip[k];
      x ^= w.x ^ w.y ^ w.z ^ w.w;
    }
#pragma unroll
    for (int k = 0; k < SW; ++k) {
      const uint4 w = sp[k];
      x ^= w.x ^ w.y ^ w.z ^ w.w;
    }
    const float f = (float)(x & 0xFFFFu);
#pragma unroll
    for (int h = 0; h < 4; ++h) a.logits[(qrow + h) * a.n_keys + t] = f + (float)h;
  }
}

}  // namespace

// idx_stride 32 and sign_stride 16 bytes (d = 128, 2 bits, m = 128), four query heads per
// kv head; every pointer 16-byte aligned.  Returns 0, -1 for shapes it does not take, -5 for a
// failed launch.
extern "C" int tq_traffic_score_twin(const void *idx, int64_t idx_stride, const void *sign, int64_t sign_stride,
                                     const uint32_t *norms, int64_t n_seq, int32_t hq, int32_t hkv, int64_t n_keys,
                                     float *logits, void *stream) {
  if (idx_stride != 32 || sign_stride != 16 || hkv < 1 || hq % (4 * hkv) != 0 || n_seq < 1 || n_keys < 1) return -1;
  TwinArgs a{static_cast<const uint8_t *>(idx), static_cast<const uint8_t *>(sign), idx_stride, sign_stride,
             norms, logits, n_keys, hq, hkv, hq / hkv / 4, (int)((n_keys + kChunk - 1) / kChunk)};
  const int64_t blocks = n_seq * hkv * a.nsub * a.n_chunks;
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL((score_traffic<2, 1>), dim3((unsigned)blocks), dim3(kNT), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
