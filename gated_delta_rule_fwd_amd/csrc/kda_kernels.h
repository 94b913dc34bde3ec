// kda_kernels.h -- internal launch functions behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Problem description shared by the chunkwise launchers.
struct ChunkArgs {
    int B, T, H, dk, dv, num_seqs;
    bool in_bf16, out_bf16;
    float scale;
    int normalize;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* init_state;
    const int32_t* cu_seqlens;
    void* o;
    float* final_state;
};

hipError_t launch_decode(int dk, int dv, bool in_bf16, bool out_bf16, int chains, const void* q,
                         const void* k, const void* v, const float* g, const float* beta, float* state,
                         void* o, float scale, int normalize, hipStream_t stream);

// fp32 per-position-pair path: any supported head dims and dtypes.
hipError_t launch_chunk_fp32(const ChunkArgs& a, hipStream_t stream);

// Matrix-core path: bf16 inputs, d_k = d_v = 128, g >= -5.
bool chunk_mfma_supported(const ChunkArgs& a);
hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t stream);

// Device-side range checks for KDA_FLAG_VALIDATE; counts violations into
// counters[0..2] (g, beta, cu_seqlens); the launcher zeroes them first with
// a fill kernel (no memset node, so the call stays capturable).
hipError_t launch_validate(const ChunkArgs& a, unsigned int* counters, hipStream_t stream);

}  // namespace kda
