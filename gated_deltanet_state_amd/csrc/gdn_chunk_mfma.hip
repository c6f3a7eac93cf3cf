// gdn_chunk_mfma.hip -- matrix-core chunkwise prefill (placeholder until the kernel lands).
#include "gdn_internal.h"
namespace gdn {
bool chunk_mfma_supported(const ChunkArgs&) { return false; }
hipError_t launch_chunk_mfma(const ChunkArgs&, bool, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace gdn
