// kda_chunk_mfma.hip -- chunkwise KDA forward on the gfx950 matrix cores.
//
// Scope: bf16 q/k/v, d_k = d_v = 128, log-decay g in [-5, 0].  One workgroup
// (4 waves) owns one chain (sequence, head) and a 64-column slice of d_v; the
// d_v columns are independent affine systems sharing one transition ("Kimi K3
// の KDA ..." section 2.3.2), so the two slices of a chain never talk.  Each
// wave keeps a 128 x 16 fp32 strip of the state in MFMA accumulators for the
// whole chain and walks the 64-token chunks in order.
//
// Per chunk (C = 64, tokens r, s; "Kimi K3 模型结构（2）" Q&A on the chunkwise
// algorithm, on A[t] and O[t]; page 1 section 1.2.1 on the two paths):
//   b     = running sum of g inside the chunk (per key channel), Gamma = e^b
//   A_kk  = StrictTril(Diag(beta) (K^ Gamma)(K^ / Gamma)^T)
//   A_qk  = Tril((Q^ Gamma)(K^ / Gamma)^T)                (diagonal kept)
//   T'    = (I + A_kk)^-1 Diag(beta)                      (UT transform)
//   U~    = T' (V - (K^ Gamma) S)          (= U - W S with W = T' K^ Gamma, U = T' V)
//   O     = (Q^ Gamma) S + A_qk U~
//   S    <- Diag(gamma) S + (K^ gamma / Gamma)^T U~
//
// The ratios Gamma_r / Gamma_s are formed per 16-token sub-tile with a
// reference point between s and r ("Kimi K3 の KDA ..." section 1.2.1 on the
// lower-bounded decay; "Kimi K3 模型结构（2）" Q&A on the -5 bound): with
// ref_j the running decay at the end of sub-tile j, tile (i, j <= i) is
//   [X_r exp(b_r - ref_{j+1})] . [K_s exp(ref_{j+1} - b_s)]
// where the right factor is <= 1 and the left one is <= 1 off the diagonal and
// <= e^80 on it (16 steps of g >= -5): both are dense bf16 matrix products.
//
// Precision (fp32 accumulate everywhere).  Each product's operands are
// rounded only as far as the output tolerance allows; a pair "x3" is
// hi*hi + hi*lo + lo*hi with x = hi + lo:
//   A_kk                bf16                     (damped through T)
//   A_qk factors        bf16 x3                  (diagonal factor up to e^80)
//   T' (V - K Gamma S)  bf16 x3                  (T may be large; near a fixed
//                                                 point of the recurrence V and
//                                                 K Gamma S nearly cancel)
//   K Gamma S, Q Gamma S  fp16 operand x fp16 hi/lo state
//   A_qk U~             fp16 hi/lo x fp16
//   K'^T U~             fp16 x fp16              (|K'| <= 1, U~ bounded)
// fp16 carries 3 more mantissa bits than bf16 at the same MFMA rate; it is
// used only where both operands are bounded well inside its range.

// Data layout: every MFMA operand is staged in LDS in the exact per-lane
// order of v_mfma_f32_16x16x32_bf16 (A: lane = row + 16*kgroup, 8 consecutive
// k per lane; B: lane = column + 16*kgroup), so each operand fetch is one
// 16-byte LDS read per lane.  The contraction order over k is free, so the
// state's channel order and the U~ token order are permuted to match the
// accumulator layout they come from: the state never leaves registers and U~
// feeds the next products without an LDS round trip.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;       // chunk length
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVS = 64;     // value columns per workgroup: 4 waves x 16
constexpr int NSLICE = DV / DVS;
constexpr int NT = 256;

struct alignas(16) Smem {
    __bf16 vs[C][DVS];                   // V slice, plain [token][column]
    union {
        struct {
            bf16x8 kf[2][4][4][64];      // K^ e^(ref_{j+1}-b) B-frags [hi/lo][token tile j][chan kb][lane]
            bf16x8 kfx[2][3][4][64];     // the same rescaled to ref_i for tiles (i,j) = (2,0), (3,0), (3,1)
        } b;
        f16x8 kp[8][2][64];              // (K^ gamma/Gamma)^T A-frags [chan tile][token kb][lane]
    } u1;
    float tot[4][DK];                    // sum of g over each sub-tile
    float akk[C][C + 4];                 // A_kk (fp32), then T = (I + A_kk)^-1 in place; rows 16-byte aligned;
                                         // reused to stage the output tile of the state phase
    f16x8 aqk[2][4][2][64];              // A_qk       A-frags [hi/lo][token tile][token kb][lane]
    bf16x8 tp[2][4][2][64];              // T'         A-frags [hi/lo][token tile][token kb][lane]
    f16x8 qg[4][4][64];                  // Q^ Gamma   A-frags [token tile][chan kb][lane]
    f16x8 kgn[4][4][64];                 // -K^ Gamma  A-frags [token tile][chan kb][lane]
    float fac[4][4][DK];                 // per sub-tile w and channel: tot_w, exp(tot_w),
                                         //   exp(ref_w), exp(ref_4 - ref_{w+1})
    float dl12[2][DK];                   // exp(tot_1), exp(tot_2)
    float gam[DK];                       // gamma = exp(b at the chunk end)
    float beta[C];
};

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

// 8 consecutive floats from LDS (16-byte aligned)
__device__ __forceinline__ void lds8(const float* p, float* out)
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c)
{
    c = mma(ah, bh, c);
    c = mma(ah, bl, c);
    return mma(al, bh, c);
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

// output tile staging in LDS, [token][column] of the workgroup's 64 columns;
// bf16 is rounded to nearest even by the hardware conversion
__device__ __forceinline__ void stage_out(float* base, int r, int c, float x, const float*)
{
    base[r * DVS + c] = x;
}
__device__ __forceinline__ void stage_out(float* base, int r, int c, float x, const uint16_t*)
{
    reinterpret_cast<uint16_t*>(base)[r * DVS + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
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

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One chunk's raw inputs for the lane's token row r = 16*wave + (lane % 16):
// channels 32*kb + 8*(lane/16) + 0..7 of q, k, g, and value columns
// 16*(lane/16) + 0..15 of this workgroup's slice.
struct Raw {
    uint4 q[4], k[4];
    float4 g[8];
    uint4 v[2];
    float beta;
};

template <typename Tout>
__global__ void __launch_bounds__(NT, 1)
chunk_mfma_kernel(ChunkArgs a)
{
    __shared__ Smem s;

    const int t = threadIdx.x;
    // the wave index is uniform across the wave: keep it in a scalar register
    // so branches on it stay scalar
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l = t & 63, g = l >> 4, n = l & 15;
    const int H = a.H;
    // Workgroup -> (chain, slice).  Both slices of a chain get ids that are
    // equal mod 8, so they are dispatched to the same XCD and the second read
    // of the chain's q/k/g hits that XCD's L2.
    const int bid = blockIdx.x;
    const int slice = (bid >> 3) & (NSLICE - 1);
    const int chain = ((bid >> 4) << 3) | (bid & 7);
    const int nchains = (a.cu_seqlens ? a.num_seqs : a.B) * H;
    if (chain >= nchains) return;
    const int j0 = slice * DVS;
    const int seq = chain / H, h = chain % H;

    long tok0, tok1;
    if (a.cu_seqlens) {
        int b0 = a.cu_seqlens[seq], b1 = a.cu_seqlens[seq + 1];
        b0 = min(max(b0, 0), a.T);
        b1 = min(max(b1, b0), a.T);
        tok0 = b0;
        tok1 = b1;
    } else {
        tok0 = static_cast<long>(seq) * a.T;
        tok1 = tok0 + a.T;
    }

    const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v);
    const float* __restrict__ gp = a.g;
    const float* __restrict__ bp = a.beta;
    Tout* __restrict__ op = static_cast<Tout*>(a.o);

    const int row = 16 * w + n;   // this lane's token row inside the chunk
    // Rows past the end of the sequence load the last valid token instead
    // (no branch, no zero fill); their k, g and beta are masked to zero when
    // the chunk is unpacked, which makes them the identity of the recurrence.
    auto load_raw = [&](Raw& R, long c0) {
        const long tk = min(c0 + row, tok1 - 1);
        const size_t base = (static_cast<size_t>(tk) * H + h);
        const uint16_t* qr = qp + base * DK + 8 * g;
        const uint16_t* kr = kp + base * DK + 8 * g;
        const float* gr = gp + base * DK + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            R.q[kb] = *reinterpret_cast<const uint4*>(qr + 32 * kb);
            R.k[kb] = *reinterpret_cast<const uint4*>(kr + 32 * kb);
            R.g[2 * kb] = *reinterpret_cast<const float4*>(gr + 32 * kb);
            R.g[2 * kb + 1] = *reinterpret_cast<const float4*>(gr + 32 * kb + 4);
        }
        const uint16_t* vr = vp + base * DV + j0 + 16 * g;
        R.v[0] = *reinterpret_cast<const uint4*>(vr);
        R.v[1] = *reinterpret_cast<const uint4*>(vr + 8);
        R.beta = bp[base];
    };

    // ---- state strip: channels 16*mt + 4*g + i, column j0 + 16*w + n
    f32x4 sacc[8];
    {
        const size_t sbase = static_cast<size_t>(chain) * DK * DV + j0 + 16 * w + n;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sacc[mt][i] = a.init_state ? a.init_state[sbase + static_cast<size_t>(16 * mt + 4 * g + i) * DV] : 0.f;
    }

    Raw R;
    if (tok0 < tok1) load_raw(R, tok0);

    for (long c0 = tok0; c0 < tok1; c0 += C) {
        const int L = static_cast<int>(min(static_cast<long>(C), tok1 - c0));

        // ================= P: preprocess this lane's row ==================
        float qv[32], kv[32], bv[32];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint32_t qw[4] = {R.q[kb].x, R.q[kb].y, R.q[kb].z, R.q[kb].w};
            const uint32_t kw[4] = {R.k[kb].x, R.k[kb].y, R.k[kb].z, R.k[kb].w};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                qv[8 * kb + 2 * e2] = bf_lo(qw[e2]);
                qv[8 * kb + 2 * e2 + 1] = bf_hi(qw[e2]);
                kv[8 * kb + 2 * e2] = bf_lo(kw[e2]);
                kv[8 * kb + 2 * e2 + 1] = bf_hi(kw[e2]);
            }
            bv[8 * kb + 0] = R.g[2 * kb].x;
            bv[8 * kb + 1] = R.g[2 * kb].y;
            bv[8 * kb + 2] = R.g[2 * kb].z;
            bv[8 * kb + 3] = R.g[2 * kb].w;
            bv[8 * kb + 4] = R.g[2 * kb + 1].x;
            bv[8 * kb + 5] = R.g[2 * kb + 1].y;
            bv[8 * kb + 6] = R.g[2 * kb + 1].z;
            bv[8 * kb + 7] = R.g[2 * kb + 1].w;
        }
        const uint4 vraw0 = R.v[0], vraw1 = R.v[1];
        const float live = (row < L) ? 1.f : 0.f;
        const float beta_r = R.beta * live;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            kv[e] *= live;
            bv[e] *= live;
        }

        // L2 norm of q and k over d_k (row spread over the 4 lane groups)
        {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                sq += qv[e] * qv[e];
                sk += kv[e] * kv[e];
            }
            sq += __shfl_xor(sq, 16, 64);
            sq += __shfl_xor(sq, 32, 64);
            sk += __shfl_xor(sk, 16, 64);
            sk += __shfl_xor(sk, 32, 64);
            const float rq = a.normalize ? rsqrtf(sq + kNormEps) : 1.f;
            const float rk = a.normalize ? rsqrtf(sk + kNormEps) : 1.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                qv[e] *= rq;
                kv[e] *= rk;
            }
        }
        // running decay inside the 16-token sub-tile
#pragma unroll
        for (int e = 0; e < 32; ++e) bv[e] = row_scan16(bv[e]);
        if (n == 15) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) s.tot[w][32 * kb + 8 * g + e] = bv[8 * kb + e];
        }
        if (g == 0) s.beta[row] = beta_r;
        // V slice, plain layout
        *reinterpret_cast<uint4*>(&s.vs[row][16 * g]) = vraw0;
        *reinterpret_cast<uint4*>(&s.vs[row][16 * g + 8]) = vraw1;
        __syncthreads();

        // per-channel decay factors for every sub-tile; each factor is an
        // exp of a non-positive sum, so none overflows
        {
            const int c = t & (DK - 1);
            const float t0 = s.tot[0][c], t1 = s.tot[1][c], t2 = s.tot[2][c], t3 = s.tot[3][c];
            const float r1 = t0, r2 = t0 + t1, r3 = r2 + t2, r4 = r3 + t3;
            if (t < DK) {
                s.fac[0][0][c] = t0;
                s.fac[0][1][c] = __expf(t0);
                s.fac[0][2][c] = 1.f;
                s.fac[0][3][c] = __expf(r4 - r1);
                s.fac[1][0][c] = t1;
                s.fac[1][1][c] = __expf(t1);
                s.fac[1][2][c] = __expf(r1);
                s.fac[1][3][c] = __expf(r4 - r2);
                s.dl12[0][c] = __expf(t1);
                s.dl12[1][c] = __expf(t2);
            } else {
                s.fac[2][0][c] = t2;
                s.fac[2][1][c] = __expf(t2);
                s.fac[2][2][c] = __expf(r2);
                s.fac[2][3][c] = __expf(r4 - r3);
                s.fac[3][0][c] = t3;
                s.fac[3][1][c] = __expf(t3);
                s.fac[3][2][c] = __expf(r3);
                s.fac[3][3][c] = 1.f;
                s.gam[c] = __expf(r4);
            }
        }
        __syncthreads();

        // Per element: d = exp(b - ref_{w+1}) in [1, e^80], f = 1/d,
        // E = exp(b - ref_w) <= 1, Gamma = exp(b).  The diagonal tile (w, w)
        // is computed right here: both of its operands are in this lane.  The
        // off-diagonal tiles share one A-operand, X^ E; the extra factor
        // exp(ref_w - ref_{j+1}) of tiles two or three sub-tiles apart is folded
        // into their B-operands (kfx).
        bf16x8 kao[4], qoh[4], qol[4];
        f16x8 kq16[4];   // K^ gamma/Gamma of this row, channels 32kb + 8g + e
        f32x4 akd = {0.f, 0.f, 0.f, 0.f}, aqd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int cb = 32 * kb + 8 * g;
            float tw[8], dw[8], er[8], el[8];
            lds8(&s.fac[w][0][cb], tw);
            lds8(&s.fac[w][1][cb], dw);
            lds8(&s.fac[w][2][cb], er);
            lds8(&s.fac[w][3][cb], el);
            bf16x8 kfh, kfl, kad, qdh, qdl;
            float qgv[8], kgv[8], kfv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float bl = bv[8 * kb + e];         // running sum inside sub-tile w
                const float d = __expf(bl - tw[e]);      // b - ref_{w+1}
                const float f = __builtin_amdgcn_rcpf(d);  // exp(ref_{w+1} - b)
                const float E = d * dw[e];               // exp(b - ref_w)
                const float gm = E * er[e];              // exp(b)
                const float kx = kv[8 * kb + e], qx = qv[8 * kb + e];
                kfv[e] = kx * f;
                __bf16 hi, lo;
                split(kx * f, hi, lo);
                kfh[e] = hi;
                kfl[e] = lo;
                qgv[e] = qx * gm;
                kgv[e] = -kx * gm;
                kad[e] = static_cast<__bf16>(kx * d);
                split(qx * d, hi, lo);
                qdh[e] = hi;
                qdl[e] = lo;
                kao[kb][e] = static_cast<__bf16>(kx * E);
                split(qx * E, hi, lo);
                qoh[kb][e] = hi;
                qol[kb][e] = lo;
                kq16[kb][e] = static_cast<_Float16>(kx * f * el[e]);
            }
            akd = mma(kad, kfh, akd);
            aqd = mma3(qdh, qdl, kfh, kfl, aqd);
            s.u1.b.kf[0][w][kb][l] = kfh;
            s.u1.b.kf[1][w][kb][l] = kfl;
            // sub-tiles 0 and 1 also provide their B-operands rescaled to
            // ref_i for rows two or three sub-tiles below
            if (w < 2) {
                float x1[8], x2[8];
                lds8(&s.dl12[0][cb], x1);
                lds8(&s.dl12[1][cb], x2);
#pragma unroll
                for (int ver = 0; ver < 2; ++ver) {
                    if (w == 1 && ver == 1) break;
                    bf16x8 xh, xl;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        // (i,j) = (2,0): exp(tot_1); (3,0): exp(tot_1 + tot_2); (3,1): exp(tot_2)
                        const float sc = (w == 0) ? ((ver == 0) ? x1[e] : x1[e] * x2[e]) : x2[e];
                        __bf16 hi, lo;
                        split(kfv[e] * sc, hi, lo);
                        xh[e] = hi;
                        xl[e] = lo;
                    }
                    const int vi = (w == 0) ? ver : 2;
                    s.u1.b.kfx[0][vi][kb][l] = xh;
                    s.u1.b.kfx[1][vi][kb][l] = xl;
                }
            }
            // Q^ Gamma and -K^ Gamma into the state's channel order: channel
            // 32kb + 8g + e goes to lane (2(g&1) + e/4)*16 + n, element 4(g>>1) + e%4
            {
                const int eo = 4 * (g >> 1);
                const int l0 = (2 * (g & 1)) * 16 + n, l1 = l0 + 16;
                f16x4 q0, q1, k0, k1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    q0[e] = static_cast<_Float16>(qgv[e]);
                    q1[e] = static_cast<_Float16>(qgv[4 + e]);
                    k0[e] = static_cast<_Float16>(kgv[e]);
                    k1[e] = static_cast<_Float16>(kgv[4 + e]);
                }
                *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&s.qg[w][kb][l0]) + eo) = q0;
                *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&s.qg[w][kb][l1]) + eo) = q1;
                *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&s.kgn[w][kb][l0]) + eo) = k0;
                *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&s.kgn[w][kb][l1]) + eo) = k1;
            }
        }
        // diagonal tile (w, w): lane holds rows 16w + 4g + i, column 16w + n
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * g + i, sc = 16 * w + n;
            if (sc < r) s.akk[r][sc] = s.beta[r] * akd[i];
            _Float16 hi, lo;
            splith((sc <= r) ? aqd[i] : 0.f, hi, lo);
            const int lt = (n >> 2) * 16 + 4 * g + i, e = (n & 3) + 4 * (w & 1);
            reinterpret_cast<_Float16*>(&s.aqk[0][w][w >> 1][lt])[e] = hi;
            reinterpret_cast<_Float16*>(&s.aqk[1][w][w >> 1][lt])[e] = lo;
            if ((w & 1) == 0) {   // tile (w, w+1) shares this token kb: zero it
                reinterpret_cast<_Float16*>(&s.aqk[0][w][w >> 1][lt])[e + 4] = static_cast<_Float16>(0.f);
                reinterpret_cast<_Float16*>(&s.aqk[1][w][w >> 1][lt])[e + 4] = static_cast<_Float16>(0.f);
            }
        }
        __syncthreads();

        // ================= A: off-diagonal intra-chunk tiles (w, j < w) ==================
        for (int j = 0; j < w; ++j) {
            f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
            // B-operand: sub-tile j's own (j = w - 1), or its copy rescaled to ref_w
            const bf16x8* bsrc_h = (j + 2 <= w) ? &s.u1.b.kfx[0][(w == 2) ? 0 : j + 1][0][0] : &s.u1.b.kf[0][j][0][0];
            const bf16x8* bsrc_l = (j + 2 <= w) ? &s.u1.b.kfx[1][(w == 2) ? 0 : j + 1][0][0] : &s.u1.b.kf[1][j][0][0];
            bf16x8 bh[4], bl[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bh[kb] = bsrc_h[kb * 64 + l];
                bl[kb] = bsrc_l[kb * 64 + l];
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                akk = mma(kao[kb], bh[kb], akk);
                aqk = mma3(qoh[kb], qol[kb], bh[kb], bl[kb], aqk);
            }
            // lane holds rows r = 16w + 4g + i, column s = 16j + n (all s < r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * g + i, sc = 16 * j + n;
                s.akk[r][sc] = s.beta[r] * akk[i];
                _Float16 hi, lo;
                splith(aqk[i], hi, lo);
                const int lt = (n >> 2) * 16 + 4 * g + i, e = (n & 3) + 4 * (j & 1);
                reinterpret_cast<_Float16*>(&s.aqk[0][w][j >> 1][lt])[e] = hi;
                reinterpret_cast<_Float16*>(&s.aqk[1][w][j >> 1][lt])[e] = lo;
            }
        }
        __syncthreads();

        // ================= T: (I + A_kk)^-1, blocked, in place ==================
        // diagonal 16x16 blocks by forward substitution: lane owns column
        // l/4 of block w and the rows l%4 + 4m of it; the four partial sums of
        // a column sit in one lane quad and are reduced with DPP
        {
            const int col = l >> 2, pr = l & 3;
            float tv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) tv[m] = (pr + 4 * m == col) ? 1.f : 0.f;
            const int b0 = 16 * w;
            float av[16][4];   // the block's strictly-lower entries this lane needs
#pragma unroll
            for (int rr = 1; rr < 16; ++rr)
#pragma unroll
                for (int m = 0; m < 4; ++m) av[rr][m] = s.akk[b0 + rr][b0 + pr + 4 * m];
#pragma unroll
            for (int rr = 1; rr < 16; ++rr) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (pr + 4 * m < rr) acc += av[rr][m] * tv[m];
                acc += quad_swap1(acc);
                acc += quad_swap2(acc);
                const float tval = (rr > col) ? -acc : ((rr == col) ? 1.f : 0.f);
                if ((rr & 3) == pr) tv[rr >> 2] = tval;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) s.akk[b0 + pr + 4 * m][b0 + col] = tv[m];
        }
        __syncthreads();

        // (all waves) (K^ gamma/Gamma)^T A-frags, token order matching U~:
        // channel c -> frag [c/16][w/2], lane (n/4)*16 + c%16, element n%4 + 4(w%2)
        {
            const int e = (n & 3) + 4 * (w & 1);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int mt = 2 * kb + (g >> 1);
                const int lb = (n >> 2) * 16 + 8 * (g & 1);
                _Float16* dst = reinterpret_cast<_Float16*>(&s.u1.kp[mt][w >> 1][0]);
#pragma unroll
                for (int ee = 0; ee < 8; ++ee) dst[(lb + ee) * 8 + e] = kq16[kb][ee];
            }
        }
        // level 1: T_{w,w-1} = -T_ww A_{w,w-1} T_{w-1,w-1} for w = 1, 3 (fp32 MFMA)
        if (w & 1) {
            const int hi = 16 * w, lo = 16 * (w - 1);
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                p = mma32(s.akk[hi + n][lo + 4 * kk + g], s.akk[lo + 4 * kk + g][lo + n], p);
#pragma unroll
            for (int i = 0; i < 4; ++i) s.akk[hi + 4 * g + i][lo + n] = p[i];
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's P is in LDS
            __builtin_amdgcn_wave_barrier();
            f32x4 q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                q = mma32(s.akk[hi + n][hi + 4 * kk + g], s.akk[hi + 4 * kk + g][lo + n], q);
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 4; ++i) s.akk[hi + 4 * g + i][lo + n] = -q[i];
        }
        __syncthreads();
        // level 2: T_BA = -T_BB (A_BA T_AA) on 32x32 blocks; wave -> tile (2 + w/2, w%2)
        {
            const int ti = 2 + (w >> 1), tj = w & 1;
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                if (kt < tj) continue;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    p = mma32(s.akk[16 * ti + n][16 * kt + 4 * kk + g], s.akk[16 * kt + 4 * kk + g][16 * tj + n], p);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) s.akk[16 * ti + 4 * g + i][16 * tj + n] = p[i];
            __syncthreads();
            f32x4 q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 2; kt < 4; ++kt) {
                if (kt > ti) continue;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    q = mma32(s.akk[16 * ti + n][16 * kt + 4 * kk + g], s.akk[16 * kt + 4 * kk + g][16 * tj + n], q);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) s.akk[16 * ti + 4 * g + i][16 * tj + n] = -q[i];
        }
        __syncthreads();
        // T' = T Diag(beta) as A-frags whose token (k) order matches the
        // accumulator layout of V - K Gamma S: element e of lane group g
        // holds token 32kb + 16(e/4) + 4g + e%4
        {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                bf16x8 th, tl;
                const float4 t0 = *reinterpret_cast<const float4*>(&s.akk[row][32 * kb + 4 * g]);
                const float4 t1 = *reinterpret_cast<const float4*>(&s.akk[row][32 * kb + 16 + 4 * g]);
                const float4 b0 = *reinterpret_cast<const float4*>(&s.beta[32 * kb + 4 * g]);
                const float4 b1 = *reinterpret_cast<const float4*>(&s.beta[32 * kb + 16 + 4 * g]);
                const float tv8[8] = {t0.x * b0.x, t0.y * b0.y, t0.z * b0.z, t0.w * b0.w,
                                      t1.x * b1.x, t1.y * b1.y, t1.z * b1.z, t1.w * b1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sc = 32 * kb + 16 * (e >> 2) + 4 * g + (e & 3);
                    const float x = (sc <= row) ? tv8[e] : 0.f;
                    __bf16 hi, lo;
                    split(x, hi, lo);
                    th[e] = hi;
                    tl[e] = lo;
                }
                s.tp[0][w][kb][l] = th;
                s.tp[1][w][kb][l] = tl;
            }
        }
        __syncthreads();

        // prefetch the next chunk: its latency hides behind the state phase,
        // and the raw registers are not live during the phases above
        if (c0 + C < tok1) load_raw(R, c0 + C);

        // ================= S: state-dependent part ==================
        // state as fp16 hi/lo B-frags (channel order of the accumulators)
        f16x8 sh[4], sl[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                _Float16 hi, lo;
                splith(sacc[2 * kb][i], hi, lo);
                sh[kb][i] = hi;
                sl[kb][i] = lo;
                splith(sacc[2 * kb + 1][i], hi, lo);
                sh[kb][4 + i] = hi;
                sl[kb][4 + i] = lo;
            }
        }
        // R = V - (K^ Gamma) S  (rows = tokens 16mt + 4g + i, column n of the strip)
        // Operand fragments of each step are read from LDS in one batch ahead
        // of its MFMAs (one wave per SIMD: nothing else hides LDS latency).
        f32x4 ut[4];
        {
            f16x8 fa[4][4];
            float vv[4][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) fa[mt][kb] = s.kgn[mt][kb][l];
#pragma unroll
                for (int i = 0; i < 4; ++i) vv[mt][i] = static_cast<float>(s.vs[16 * mt + 4 * g + i][16 * w + n]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 acc = {vv[mt][0], vv[mt][1], vv[mt][2], vv[mt][3]};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    acc = mmh(fa[mt][kb], sh[kb], acc);
                    acc = mmh(fa[mt][kb], sl[kb], acc);
                }
                ut[mt] = acc;
            }
        }
        bf16x8 rbh[2], rbl[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __bf16 hi, lo;
                split(ut[2 * kb][i], hi, lo);
                rbh[kb][i] = hi;
                rbl[kb][i] = lo;
                split(ut[2 * kb + 1][i], hi, lo);
                rbh[kb][4 + i] = hi;
                rbl[kb][4 + i] = lo;
            }
        }
        // U~ = T' R
        {
            bf16x8 th[6], tl[6];   // (mt, kb) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const int mt = (p < 2) ? p : 2 + ((p - 2) >> 1), kb = (p < 2) ? 0 : ((p - 2) & 1);
                th[p] = s.tp[0][mt][kb][l];
                tl[p] = s.tp[1][mt][kb][l];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= (mt >> 1); ++kb) {
                    const int p = (mt < 2) ? mt : 2 + 2 * (mt - 2) + kb;
                    acc = mma3(th[p], tl[p], rbh[kb], rbl[kb], acc);
                }
                ut[mt] = acc;
            }
        }
        f16x8 ub[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ub[kb][i] = static_cast<_Float16>(ut[2 * kb][i]);
                ub[kb][4 + i] = static_cast<_Float16>(ut[2 * kb + 1][i]);
            }
        }
        // O = (Q^ Gamma) S + A_qk U~, two token tiles per batch
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f16x8 qa[2][4], ah[2][2], al[2][2];
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                const int mt = 2 * half + m2;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) qa[m2][kb] = s.qg[mt][kb][l];
#pragma unroll
                for (int kb = 0; kb <= half; ++kb) {
                    ah[m2][kb] = s.aqk[0][mt][kb][l];
                    al[m2][kb] = s.aqk[1][mt][kb][l];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                const int mt = 2 * half + m2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    acc = mmh(qa[m2][kb], sh[kb], acc);
                    acc = mmh(qa[m2][kb], sl[kb], acc);
                }
#pragma unroll
                for (int kb = 0; kb <= half; ++kb) {
                    acc = mmh(ah[m2][kb], ub[kb], acc);
                    acc = mmh(al[m2][kb], ub[kb], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // stage the output tile in LDS (the A_kk area is free now)
                    // so that the global stores below write whole rows
                    stage_out(&s.akk[0][0], 16 * mt + 4 * g + i, 16 * w + n, a.scale * acc[i],
                              static_cast<const Tout*>(nullptr));
                }
            }
        }
        // S <- Diag(gamma) S + (K^ gamma/Gamma)^T U~, four channel tiles per batch
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f16x8 ka[4][2];
            float4 gm4[4];
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const int mt = 4 * half + m4;
                ka[m4][0] = s.u1.kp[mt][0][l];
                ka[m4][1] = s.u1.kp[mt][1][l];
                gm4[m4] = *reinterpret_cast<const float4*>(&s.gam[16 * mt + 4 * g]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const int mt = 4 * half + m4;
                sacc[mt][0] *= gm4[m4].x;
                sacc[mt][1] *= gm4[m4].y;
                sacc[mt][2] *= gm4[m4].z;
                sacc[mt][3] *= gm4[m4].w;
                sacc[mt] = mmh(ka[m4][0], ub[0], sacc[mt]);
                sacc[mt] = mmh(ka[m4][1], ub[1], sacc[mt]);
            }
        }
        __syncthreads();
        // coalesced output rows: 64 tokens x 64 columns of this slice
        {
            constexpr int CH = 16 / sizeof(Tout);            // elements per 16-byte piece
            constexpr int PER_ROW = DVS / CH;
#pragma unroll
            for (int pc = t; pc < C * PER_ROW; pc += NT) {
                const int r = pc / PER_ROW, part = pc % PER_ROW;
                if (r < L) {
                    const uint4 val = *reinterpret_cast<const uint4*>(
                        reinterpret_cast<const char*>(&s.akk[0][0]) + (r * DVS + part * CH) * sizeof(Tout));
                    *reinterpret_cast<uint4*>(op + (static_cast<size_t>(c0 + r) * H + h) * DV + j0 + part * CH) = val;
                }
            }
        }
        __syncthreads();
    }

    if (a.final_state) {
        const size_t sbase = static_cast<size_t>(chain) * DK * DV + j0 + 16 * w + n;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.final_state[sbase + static_cast<size_t>(16 * mt + 4 * g + i) * DV] = sacc[mt][i];
    }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a)
{
    return a.in_bf16 && a.dk == DK && a.dv == DV;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t stream)
{
    const int chains = (a.cu_seqlens ? a.num_seqs : a.B) * a.H;
    // ids: chain = 8 * (bid >> 4) + (bid & 7), slice = (bid >> 3) & 1
    const int groups = (chains + 7) / 8;
    const dim3 grid(groups * 8 * NSLICE), block(NT);
    if (a.out_bf16)
        chunk_mfma_kernel<uint16_t><<<grid, block, 0, stream>>>(a);
    else
        chunk_mfma_kernel<float><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace kda
