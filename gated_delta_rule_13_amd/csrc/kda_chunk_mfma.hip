// bf16 matrix-core chunk kernel (placeholder until the MFMA path lands).
#include "kda_internal.h"

namespace kda {

bool chunk_mfma_supports(int, int) { return false; }

hipError_t launch_chunk_mfma(const ChunkArgs&, bool, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kda
