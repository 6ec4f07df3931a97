// Chunkwise backward of the Muir gated delta rule (gfx950).
#include "kernels.h"
#include "mma.h"

namespace muir {

hipError_t launch_bwd_scan(const ChunkShape&, const void*, const void*, const float*, float*, float*,
                           hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_bwd_chunk(const ChunkShape&, const void*, const void*, const void*, const void*,
                            const void*, const void*, const void*, const float*, const float*,
                            const void*, float*, float*, float*, float*, float*, float*, float*,
                            hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace muir
