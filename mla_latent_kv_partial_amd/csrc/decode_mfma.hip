// MFMA latent decode attention for the bf16 GLM geometry (placeholder: the
// generic kernel serves every shape until this kernel lands).
#include "common.hpp"
#include "launch.hpp"

namespace mla {

bool decode_mfma_supported(int32_t, int32_t, int32_t, int32_t) { return false; }

hipError_t launch_decode_mfma(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
