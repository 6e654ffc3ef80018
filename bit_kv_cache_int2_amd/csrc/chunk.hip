// Chunk attention (multi-query) over the packed cache: not built yet.
#include "device.h"
#include "internal.h"

namespace kvq {

size_t chunk_workspace_bytes(const kvq_layout*, int, int, int) { return 0; }

hipError_t launch_chunk(const kvq_cache*, int, const void*, int, int, float, void*, int, float*,
                        void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kvq
