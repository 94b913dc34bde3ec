// kda_conv.hip -- conv states after a prefill with the short convolution.
//
// The convolution of q, k and v (width 4, per channel; "Kimi K3 の KDA ..."
// section 1.2.1) runs inside the forward kernels where each tensor is
// loaded.  What a later call needs to continue a sequence is the conv state:
// the last 3 raw inputs of every channel ("GDN, KDA の整理", the conv cache).
// This kernel writes it once the forward kernels have read the incoming
// state, so the outgoing state may overwrite it in place.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

// One thread per (sequence, channel): rows len-3 .. len-1 of the sequence,
// taken from the incoming state where they lie before its first token.
template <typename T>
__global__ void __launch_bounds__(256)
conv_final_kernel(const T* __restrict__ x, const T* init, T* fin, const int32_t* __restrict__ cu, int T_, int width,
                  int col_blocks)
{
    const int seq = blockIdx.x / col_blocks;
    const int col = (blockIdx.x % col_blocks) * 256 + threadIdx.x;
    if (col >= width) return;
    long tok0, tok1;
    if (cu) {
        int b0 = cu[seq], b1 = cu[seq + 1];
        b0 = min(max(b0, 0), T_);
        b1 = min(max(b1, b0), T_);
        tok0 = b0;
        tok1 = b1;
    } else {
        tok0 = static_cast<long>(seq) * T_;
        tok1 = tok0 + T_;
    }
    const long len = tok1 - tok0;
    T src[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const long pos = len - 3 + p;
        if (pos >= 0)
            src[p] = x[static_cast<size_t>(tok0 + pos) * width + col];
        else
            src[p] = init ? init[(static_cast<size_t>(seq) * 3 + static_cast<size_t>(3 + pos)) * width + col] : T(0);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) fin[(static_cast<size_t>(seq) * 3 + p) * width + col] = src[p];
}

}  // namespace

hipError_t launch_conv_final(const ChunkArgs& a, void* const final_state[3], hipStream_t stream)
{
    const int N = a.cu_seqlens ? a.num_seqs : a.B;
    const void* x[3] = {a.q, a.k, a.v};
    const int width[3] = {a.H * a.dk, a.H * a.dk, a.H * a.dv};
    for (int i = 0; i < 3; ++i) {
        if (!final_state[i] || N == 0) continue;
        const int cb = (width[i] + 255) / 256;
        const dim3 grid(static_cast<unsigned>(static_cast<long long>(N) * cb)), block(256);
        if (a.in_bf16)
            conv_final_kernel<uint16_t><<<grid, block, 0, stream>>>(
                static_cast<const uint16_t*>(x[i]), static_cast<const uint16_t*>(a.conv_init[i]),
                static_cast<uint16_t*>(final_state[i]), a.cu_seqlens, a.T, width[i], cb);
        else
            conv_final_kernel<float><<<grid, block, 0, stream>>>(
                static_cast<const float*>(x[i]), static_cast<const float*>(a.conv_init[i]),
                static_cast<float*>(final_state[i]), a.cu_seqlens, a.T, width[i], cb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
