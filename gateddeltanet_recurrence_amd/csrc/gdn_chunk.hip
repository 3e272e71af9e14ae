// Chunked prefill: not built yet; the plan resolver never selects it.
#include "gdn_kernels.h"

namespace gdn {

size_t chunk_workspace_bytes(int64_t, int, int, int) { return 0; }

hipError_t launch_chunk(const ChunkArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
