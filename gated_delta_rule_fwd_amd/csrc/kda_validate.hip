// kda_validate.hip -- device-side input range checks behind KDA_FLAG_VALIDATE.
//
// The matrix-core path relies on the bounded decay: every log-decay g is in
// [-5, 0], so 16 consecutive tokens rescale by at most e^80, inside the bf16
// and fp32 range ("Kimi K3 模型结构（2）", Q&A on the -5 bound).  beta is a
// write strength in [0, 1] ("Kimi K3 の KDA ..." section 1.2.1).  Packed
// sequences must partition [0, T] monotonically.  Complex KDA (signed alpha)
// needs |alpha| in [e^-5, 1] and allows beta in [0, 2].  The gated entry point maps
// z into (-5, 0) itself, so only beta (or, for logits, finiteness) and the
// sequence partition are checked there.
#include "kda_kernels.h"

namespace kda {

namespace {

__global__ void zero_counters(unsigned int* c)
{
    if (threadIdx.x < 4) c[threadIdx.x] = 0u;
}

__global__ void __launch_bounds__(256)
validate_kernel(const float* __restrict__ g, size_t ng, int signed_alpha, const float* __restrict__ beta, size_t nb,
                int beta_logits, const int32_t* __restrict__ cu, int nseq, int T, unsigned int* counters)
{
    unsigned int bad_g = 0, bad_b = 0, bad_cu = 0;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < ng; i += stride) {
        const float x = g[i];
        // signed alpha: |alpha| in [e^-5, 1] (e^-5 = 0.006737947, rounded down)
        bad_g += signed_alpha ? !(fabsf(x) >= 0.0067379470f && fabsf(x) <= 1.0f) : !(x >= -5.0f && x <= 0.0f);
    }
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nb; i += stride) {
        const float x = beta[i];
        const float bmax = signed_alpha ? 2.0f : 1.0f;   // Complex KDA widens beta to [0, 2]
        bad_b += beta_logits ? !(x == x && fabsf(x) <= 3.4e38f) : !(x >= 0.0f && x <= bmax);
    }
    if (cu && blockIdx.x == 0) {
        for (int n = threadIdx.x; n <= nseq; n += blockDim.x) {
            const int x = cu[n];
            if (n == 0 && x != 0) ++bad_cu;
            if (n == nseq && x != T) ++bad_cu;
            if (n > 0 && x < cu[n - 1]) ++bad_cu;
        }
    }
    if (bad_g) atomicAdd(&counters[0], bad_g);
    if (bad_b) atomicAdd(&counters[1], bad_b);
    if (bad_cu) atomicAdd(&counters[2], bad_cu);
}

}  // namespace

hipError_t launch_validate(const ChunkArgs& a, unsigned int* counters, hipStream_t stream)
{
    zero_counters<<<1, 64, 0, stream>>>(counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t tokens = static_cast<size_t>(a.B) * a.T;
    const size_t ng = a.gated ? 0 : tokens * a.H * a.dk, nb = tokens * a.H;
    validate_kernel<<<1024, 256, 0, stream>>>(a.g, ng, a.signed_alpha, a.beta, nb, a.beta_logits, a.cu_seqlens,
                                              a.num_seqs, a.T, counters);
    return hipGetLastError();
}

}  // namespace kda
