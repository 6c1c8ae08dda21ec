// Inner-product top-k search over encoded vectors (placeholder until the scan kernel lands).
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

size_t search_workspace(const CodecView &, int64_t, int, int64_t) { return 0; }

int launch_search(const CodecView &, const float *, int64_t, const CodesView &, int64_t, int, int64_t *, float *,
                  void *, size_t, void *) {
  return TQ_EUNSUPPORTED;
}

}  // namespace tq
