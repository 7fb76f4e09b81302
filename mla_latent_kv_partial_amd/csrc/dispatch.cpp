// Kernel selection between the generic VALU kernels and the MFMA kernels of
// the bf16 GLM geometry.
#include "launch.hpp"

namespace mla {

size_t prefill_generic_workspace_bytes(const PrefillParams& p);
hipError_t launch_prefill_generic(const PrefillParams& p, hipStream_t stream);

size_t prefill_workspace_bytes(const PrefillParams& p) { return prefill_generic_workspace_bytes(p); }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) { return launch_prefill_generic(p, stream); }

}  // namespace mla
