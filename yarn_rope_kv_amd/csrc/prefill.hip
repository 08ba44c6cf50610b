// Chunked causal prefill attention (placeholder until the MFMA kernel lands).
#include "yrk_internal.h"

namespace yrk {

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace yrk
