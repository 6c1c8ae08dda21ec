// Decode attention over the compressed cache (placeholder until the split-K kernel lands).
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

size_t attend_workspace(const CodecView &, const CodecView &, const ScoreShape &) { return 0; }

int launch_attend(const CodecView &, const CodecView &, const float *, const ScoreShape &, const CodesView &,
                  const CodesView &, float, float *, void *, size_t, void *) {
  return TQ_EUNSUPPORTED;
}

}  // namespace tq
