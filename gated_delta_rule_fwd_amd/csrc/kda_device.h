// kda_device.h -- small device helpers shared by the KDA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr float kNormEps = 1e-6f;  // inside the square root of the per-head L2 norm

// bf16 storage: 16-bit pattern, round to nearest even on store.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Packed pair of bf16 in one dword, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Gate prologue of the gated entry points ("Kimi K3 模型结构（2）", Q&A on the
// lower bound; "Kimi K3 の KDA ..." section 1.2.1 on A_log, dt_bias and the
// in-kernel sigmoid of beta):
//   g    = -5 sigmoid(e^{A_h} (z + dt_bias[h, c]))   in (-5, 0)
//   beta = sigmoid(logit)
// g is evaluated as -5 / (1 + 2^y) with y = -e^{A_h} log2(e) (z + dt_bias):
// one multiply-add, one exp2 and one reciprocal (to 1 ulp) per element, the
// factor -e^{A_h} log2(e) being the same for a whole head.  2^y overflowing
// to +inf gives g = -0, and exp(-x) overflowing gives beta = 0: the right
// limits.
__device__ __forceinline__ float gate_log_decay(float z, float bias, float exp_a) {
    const float y = (z + bias) * (-exp_a * 1.44269504088896341f);
    return -5.f * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(y));
}
__device__ __forceinline__ float beta_from_logit(float b) { return 1.f / (1.f + __expf(-b)); }
// sigmoid(x) as a reciprocal (to 1 ulp) of 1 + 2^{-x log2(e)}: three
// instructions; 2^{...} overflowing to +inf gives 0, the limit
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

// Short convolution prologue ("Kimi K3 の KDA ..." section 1.2.1: causal and
// per channel over the current token and the 3 before it, then SiLU).  Taps
// w[4c .. 4c+3] of channel c run oldest token first; inputs before a
// sequence's first token come from its conv state (3 rows of `width`
// channels per sequence, oldest first) or are zero.
// x / (1 + e^{-x}) as x times a reciprocal (to 1 ulp) of 1 + 2^{-x log2(e)}:
// three instructions instead of a correctly rounded division; 2^{...}
// overflowing to +inf gives -0, the limit.
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

template <typename Tin>
__device__ __forceinline__ float conv_input(const Tin* x, const Tin* state, long tk, long tok0, size_t width,
                                            size_t state_row0, size_t col)
{
    if (tk >= tok0) return Elem<Tin>::load(x, static_cast<size_t>(tk) * width + col);
    if (!state) return 0.f;
    return Elem<Tin>::load(state, (state_row0 + static_cast<size_t>(3 + tk - tok0)) * width + col);
}

// silu(conv) at token tk (>= tok0) of channel col; state_row0 = 3 * sequence.
template <typename Tin>
__device__ __forceinline__ float conv_silu(const Tin* x, const Tin* state, const float* w, long tk, long tok0,
                                           size_t width, size_t state_row0, size_t col)
{
    const float4 wt = *reinterpret_cast<const float4*>(w + 4 * col);
    float acc = wt.w * conv_input(x, state, tk, tok0, width, state_row0, col);
    acc += wt.z * conv_input(x, state, tk - 1, tok0, width, state_row0, col);
    acc += wt.y * conv_input(x, state, tk - 2, tok0, width, state_row0, col);
    acc += wt.x * conv_input(x, state, tk - 3, tok0, width, state_row0, col);
    return silu(acc);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace kda
