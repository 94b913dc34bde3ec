// kda_mfma.h -- matrix-core building blocks shared by the chunkwise kernels
// (gfx950: v_mfma_f32_16x16x32_{bf16,f16} and v_mfma_f32_16x16x4f32).
//
// Operand layouts of v_mfma_f32_16x16x32_* (64 lanes, lane l):
//   A (16 x 32): row l%16, k = 8*(l/16) + e for element e = 0..7
//   B (32 x 16): column l%16, k = 8*(l/16) + e
//   D (16 x 16): rows 4*(l/16) + i (i = 0..3), column l%16
// and of v_mfma_f32_16x16x4f32: A[l%16][l/16], B[l/16][l%16], same D.
#pragma once

#include "kda_device.h"

namespace kda {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;       // chunk length
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NT = 256;     // threads per workgroup: 4 waves, one per 16-token sub-tile

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mmh(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// x = hi + lo to about 16 mantissa bits (bf16) / 22 bits (fp16)
__device__ __forceinline__ void split(float x, __bf16& hi, __bf16& lo)
{
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ void splith(float x, _Float16& hi, _Float16& lo)
{
    hi = static_cast<_Float16>(x);
    lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c)
{
    c = mma(ah, bh, c);
    c = mma(ah, bl, c);
    return mma(al, bh, c);
}

// 8 consecutive floats from LDS (16-byte aligned)
__device__ __forceinline__ void lds8(const float* p, float* out)
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Inclusive prefix sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row_scan16(float x)
{
    int v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));  // row_shr:1
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));  // row_shr:2
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));  // row_shr:4
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));  // row_shr:8
    return x;
}

// value of the lane with index ^1 / ^2 inside its quad (DPP quad_perm)
__device__ __forceinline__ float quad_swap1(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_swap2(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
}

// Word 3 of a gfx9 buffer descriptor for untyped raw loads (32-bit data
// format, no swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lower-triangular 64 x 64 operands are kept as their six non-zero 16 x 32
// A-fragment blocks (token tile mt, token block kb <= mt/2):
// p = 0..5 <-> (mt, kb) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
__host__ __device__ constexpr int tri_block(int mt, int kb) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + kb; }

// Chunk-local operands of one (chunk, head), written by the chunk-parallel
// pass and streamed by the sequential pass; every array is in the per-lane
// order of the MFMA operand it feeds, so both sides move whole 16-byte
// fragments.  Token orders are permuted as the consumers need (see the
// kernels): T' and A_qk use token 32kb + 16(e/4) + 4(l/16) + e%4 for
// element e of lane l; K' and the state use channel order
// 16mt + 4(l/16) + i (i = 0..3) per 16-channel tile.
struct alignas(16) ChunkRecord {
    bf16x8 tp[2][6][64];     // T' = T Diag(beta)              [hi/lo][tri block][lane]
    f16x8 aqk[2][6][64];     // A_qk                           [hi/lo][tri block][lane]
    f16x8 kgn[4][4][64];     // -K^ Gamma    A-frags [token tile][channel block][lane]
    f16x8 qg[4][4][64];      // Q^ Gamma     A-frags [token tile][channel block][lane]
    f16x8 kp[8][2][64];      // (K^ gamma/Gamma)^T A-frags [channel tile][token block][lane]
    float gam[DK];           // gamma = exp(b) at the chunk end
};

}  // namespace mfma
}  // namespace kda
