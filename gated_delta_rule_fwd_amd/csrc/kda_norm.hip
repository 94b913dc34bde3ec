// kda_norm.hip -- the output norm of the prefill paths.
//
// The model follows the kernel with a gated RMSNorm per head ("Kimi K3 の KDA
// ..." section 1.2.1: RMSNorm over the head's value channels, a sigmoid on
// the output gate, their product; the norm first).  Per (token, head) row of
// d_v values:  o <- o / sqrt(mean(o^2) + eps) * w * sigmoid(gate).
//
// The prefill kernels split each row of o over workgroups (two 64-column
// slices in the matrix-core scan, 32-column slices in the fp32 path), so the
// row reduction runs here, as a pass over the forward pass's fp32 output (o
// itself, or a staging area when o is bf16): 32 lanes per row of 128, the
// values held in registers between the reduction and the write.  The decode
// step applies the same norm inside its own kernel.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

template <typename T> struct Quad;
template <> struct Quad<float> {
    __device__ __forceinline__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct Quad<uint16_t> {
    __device__ __forceinline__ static float4 load(const uint16_t* p)
    {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
    __device__ __forceinline__ static void store(uint16_t* p, float4 v)
    {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
};

// DV / 4 lanes per row, 4 consecutive values per lane (16-byte fp32 loads).
// x and o may be the same fp32 array: each lane holds its values in
// registers between the read and the write.
template <int DV, typename Tg, typename To>
__global__ void __launch_bounds__(256)
out_norm_kernel(const float* x, To* o, const Tg* __restrict__ gate, const float* __restrict__ w, float eps, long rows)
{
    constexpr int LPR = DV / 4;                 // lanes per row
    constexpr int RPB = 256 / LPR;              // rows per block and pass
    const int c = 4 * (threadIdx.x % LPR);
    const float4 wt = w ? *reinterpret_cast<const float4*>(w + c) : make_float4(1.f, 1.f, 1.f, 1.f);
    // grid-stride over row blocks: the grid is capped, so any row count fits one launch
    for (long row0 = static_cast<long>(blockIdx.x) * RPB; row0 < rows; row0 += static_cast<long>(gridDim.x) * RPB) {
        const long row = row0 + threadIdx.x / LPR;
        const bool live = row < rows;
        const size_t base = static_cast<size_t>(live ? row : 0) * DV + c;
        const float4 v = live ? *reinterpret_cast<const float4*>(x + base) : make_float4(0.f, 0.f, 0.f, 0.f);
        float ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
        if (live) {
            const float rs = rsqrtf(ss * (1.f / DV) + eps);
            const float4 gt = Quad<Tg>::load(gate + base);
            Quad<To>::store(o + base,
                            make_float4(v.x * rs * wt.x / (1.f + __expf(-gt.x)), v.y * rs * wt.y / (1.f + __expf(-gt.y)),
                                        v.z * rs * wt.z / (1.f + __expf(-gt.z)), v.w * rs * wt.w / (1.f + __expf(-gt.w))));
        }
    }
}

template <int DV>
hipError_t launch_dv(const ChunkArgs& a, const float* x, long rows, hipStream_t stream)
{
    constexpr long RPB = 256 / (DV / 4);
    constexpr long kMaxBlocks = 1L << 20;
    const long blocks = (rows + RPB - 1) / RPB;
    const dim3 grid(static_cast<unsigned>(blocks < kMaxBlocks ? blocks : kMaxBlocks)), block(256);
    if (a.in_bf16 && a.out_bf16)
        out_norm_kernel<DV, uint16_t, uint16_t><<<grid, block, 0, stream>>>(
            x, static_cast<uint16_t*>(a.o), static_cast<const uint16_t*>(a.out_gate), a.norm_w, a.norm_eps, rows);
    else if (a.in_bf16)
        out_norm_kernel<DV, uint16_t, float><<<grid, block, 0, stream>>>(
            x, static_cast<float*>(a.o), static_cast<const uint16_t*>(a.out_gate), a.norm_w, a.norm_eps, rows);
    else if (a.out_bf16)
        out_norm_kernel<DV, float, uint16_t><<<grid, block, 0, stream>>>(
            x, static_cast<uint16_t*>(a.o), static_cast<const float*>(a.out_gate), a.norm_w, a.norm_eps, rows);
    else
        out_norm_kernel<DV, float, float><<<grid, block, 0, stream>>>(
            x, static_cast<float*>(a.o), static_cast<const float*>(a.out_gate), a.norm_w, a.norm_eps, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_out_norm(const ChunkArgs& a, const float* x, hipStream_t stream)
{
    const long rows = static_cast<long>(a.B) * a.T * a.H;
    if (rows == 0) return hipSuccess;
    return a.dv == 128 ? launch_dv<128>(a, x, rows, stream) : launch_dv<64>(a, x, rows, stream);
}

}  // namespace kda
