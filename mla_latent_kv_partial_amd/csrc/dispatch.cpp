// Kernel selection between the generic VALU prefill and the MFMA prefill of
// the bf16 GLM geometry.
#include "launch.hpp"

namespace mla {

size_t prefill_generic_workspace_bytes(const PrefillParams& p);
hipError_t launch_prefill_generic(const PrefillParams& p, hipStream_t stream);
bool prefill_mfma_shape_ok(const PrefillParams& p);
bool prefill_mfma_supported(const PrefillParams& p);
size_t prefill_mfma_workspace_bytes(const PrefillParams& p);
hipError_t launch_prefill_mfma(const PrefillParams& p, hipStream_t stream);

size_t prefill_workspace_bytes(const PrefillParams& p) {
  return prefill_mfma_supported(p) ? prefill_mfma_workspace_bytes(p) : prefill_generic_workspace_bytes(p);
}

// The size query runs before the caller has its buffers, and the path taken
// also depends on their alignment: it reports the larger of the two sizes.
size_t prefill_workspace_bytes_any_path(const PrefillParams& p) {
  const size_t a = prefill_mfma_shape_ok(p) ? prefill_mfma_workspace_bytes(p) : 0;
  const size_t b = prefill_generic_workspace_bytes(p);
  return a > b ? a : b;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  return prefill_mfma_supported(p) ? launch_prefill_mfma(p, stream) : launch_prefill_generic(p, stream);
}

}  // namespace mla
