// Matrix-core causal attention for prefill chunks (placeholder until the
// MFMA kernel lands: every chunk row takes the vector path).
#include "pa_internal.hpp"

namespace pa {

bool chunks_supported(int32_t, int32_t, int32_t) { return false; }

int32_t launch_chunks(const ChunkArgs&, hipStream_t) { return PA_ERR_UNSUPPORTED; }

}  // namespace pa
