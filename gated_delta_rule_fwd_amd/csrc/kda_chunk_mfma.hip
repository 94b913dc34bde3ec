// kda_chunk_mfma.hip -- matrix-core chunkwise path (bf16 inputs, d = 128).
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

bool chunk_mfma_supported(const ChunkArgs&) { return false; }

hipError_t launch_chunk_mfma(const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
