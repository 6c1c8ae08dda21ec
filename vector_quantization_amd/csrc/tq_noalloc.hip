// tq_decode_step_noalloc: the decode step with its workspace in a static device array, for
// callers that cannot allocate device memory.  The array lives in this file; host code reaches it
// only through the address hipGetSymbolAddress returns for the current device.

#include <mutex>

#include "tq_device.h"
#include "tq_internal.h"

namespace {

// The workspace of tq_decode_step_noalloc: the rotated queries and the per-chunk partial states
// of the attention (every value written by the call before it is read).  One copy per GPU.
__device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// This device's copy of `scratch` (the calling thread's current device), looked up once per
// device with that device current.
int scratch_of_current_device(void **ws, size_t *bytes) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_EHIP;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr) return TQ_EHIP;
  *ws = g_ptr[dev];
  *bytes = TQ_NOALLOC_SCRATCH_BYTES;
  return TQ_OK;
}

}  // namespace

extern "C" int tq_decode_step_noalloc(const tq_codec *kc, const tq_codec *vc, const float *q, const void *k_new,
                                      const void *v_new, tq_dtype dt, int64_t n_seq, int32_t hq, int32_t hkv,
                                      int64_t cap, const int32_t *pos, float rope_base, tq_codes kcache,
                                      tq_codes vcache, float scale, float *out, void *stream) {
  return tq::decode_step_impl(kc, vc, q, k_new, v_new, dt, n_seq, hq, hkv, cap, pos, rope_base, kcache, vcache,
                              scale, out, nullptr, 0, stream, scratch_of_current_device);
}
