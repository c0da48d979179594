// Prefill attention (placeholder until the MFMA kernel lands).
#include "device_common.h"
#include "internal.h"

namespace lra {
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  (void)a;
  (void)stream;
  return hipErrorNotSupported;
}
}  // namespace lra
