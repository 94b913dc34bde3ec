// kda_chunk_two_pass.hip -- chunkwise KDA forward on the gfx950 matrix cores,
// split into a chunk-parallel pass and a sequential pass.
//
// Scope: bf16 q/k/v, d_k = d_v = 128, log-decay g in [-5, 0].
//
// Per chunk (C = 64, tokens r, s; "Kimi K3 模型结构（2）" Q&A on the chunkwise
// algorithm, on A[t] and O[t]; "Kimi K3 の KDA ..." section 1.2.1 on the two
// paths):
//   b     = running sum of g inside the chunk (per key channel), Gamma = e^b
//   A_kk  = StrictTril(Diag(beta) (K^ Gamma)(K^ / Gamma)^T)
//   A_qk  = Tril((Q^ Gamma)(K^ / Gamma)^T)                (diagonal kept)
//   T'    = (I + A_kk)^-1 Diag(beta)                      (UT transform)
//   U~    = T' (V - (K^ Gamma) S)          (= U - W S with W = T' K^ Gamma, U = T' V)
//   O     = (Q^ Gamma) S + A_qk U~
//   S    <- Diag(gamma) S + (K^ gamma / Gamma)^T U~
//
// Only the last three lines involve the carried state S.  Everything above
// them is local to one chunk, so it is computed for all chunks of all heads
// at once (pass 1, one workgroup per (chunk, head)) and stored as a
// ChunkRecord of ready-made MFMA operand fragments.  Pass 2 walks each chain
// (sequence, head) in chunk order, one workgroup per 64-column slice of d_v
// (the columns are independent affine systems sharing one transition,
// "Kimi K3 の KDA ..." section 2.3.2), streaming one record per chunk while
// the state stays in MFMA accumulators.
//
// The ratios Gamma_r / Gamma_s are formed per 16-token sub-tile with a
// reference point between s and r ("Kimi K3 の KDA ..." section 1.2.1 on the
// lower-bounded decay; "Kimi K3 模型结构（2）" Q&A on the -5 bound): with
// ref_j the running decay at the end of sub-tile j, tile (i, j <= i) is
//   [X_r exp(b_r - ref_i)] . [K_s exp(ref_i - b_s)]          (j < i)
//   [X_r exp(b_r - ref_{i+1})] . [K_s exp(ref_{i+1} - b_s)]  (j = i)
// where every factor is <= 1 except the diagonal tile's left one (<= e^80
// for 16 steps of g >= -5): all are dense bf16 matrix products.
//
// Precision (fp32 accumulate everywhere; "x3" = hi*hi + hi*lo + lo*hi with
// x = hi + lo):
//   A_kk                bf16 (x3 for Complex KDA: with |alpha| near 1 the
//                            chain is undamped and single-bf16 A_kk rounding
//                            accumulates)
//   A_qk                bf16 x3                  (diagonal factor up to e^80)
//   T' (V - K Gamma S)  bf16 x3                  (near a fixed point of the
//                                                 recurrence V and K Gamma S
//                                                 nearly cancel)
//   K Gamma S, Q Gamma S  fp16 operand x fp16 hi/lo state
//   A_qk U~             fp16 hi/lo x fp16
//   K'^T U~             fp16 x fp16 hi/lo        (|K'| <= 1; U~ split because
//                                                 the state can be small next
//                                                 to U~)
#include "kda_kernels.h"
#include "kda_mfma.h"
#include "kda_stage_plan.h"

namespace kda {

namespace {

using namespace mfma;

static_assert(sizeof(ChunkRecord) == kChunkRecordBytes, "ChunkRecord layout");


// ---------------------------------------------------------------------------
// Pass 1: chunk-local operands
// ---------------------------------------------------------------------------

struct alignas(16) PrepSmem {
    union {
        bf16x8 kf[2][4][4][64];      // K^ e^(ref_{j+1}-b) B-frags [hi/lo][token tile j][chan kb][lane]
        f16x8 kp[8][2][64];          // (K^ gamma/Gamma)^T A-frags, built once kf is dead
    } u;
    float akk[C][C + 4];             // A_kk (fp32), then T = (I + A_kk)^-1 in place
    f16x8 aqk[2][6][64];             // A_qk [hi/lo][tri block][lane]
    float tot[4][DK];                // sum of g over each sub-tile
    float fac[4][4][DK];             // per sub-tile w and channel: tot_w, exp(tot_w),
                                     //   exp(ref_w), exp(ref_4 - ref_{w+1})
    float dl12[2][DK];               // exp(tot_1), exp(tot_2)
    float beta[C];
    uint32_t tsg[4][4];              // Complex KDA: sign bits of the decay product over each
                                     //   sub-tile [sub-tile][lane group], bit 8kb + e <->
                                     //   channel 32kb + 8g + e
};

// Packed sequences: slot -> sequence (or -1 for a slot no sequence uses).
__global__ void slot_map_kernel(const int32_t* __restrict__ cu, int num_seqs, int T, int nslots, int* __restrict__ map)
{
    const int slot = blockIdx.x * blockDim.x + threadIdx.x;
    if (slot >= nslots) return;
    auto start = [&](int i) { return min(max(cu[i], 0), T); };
    // largest i with first slot i + start_i / C <= slot
    int lo = 0, hi = num_seqs - 1, found = -1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        if (mid + start(mid) / C <= slot) {
            found = mid;
            lo = mid + 1;
        } else {
            hi = mid - 1;
        }
    }
    int seq = -1;
    if (found >= 0) {
        const int b0 = start(found), b1 = min(max(cu[found + 1], b0), T);
        if (slot - (found + b0 / C) < (b1 - b0 + C - 1) / C) seq = found;
    }
    map[slot] = seq;
}

// Staging slots of the scattered fragment writes (A_qk, K'^T) are permuted
// inside groups of eight, so the lanes of one 2-byte write instruction fall
// into different LDS banks; the copy to the record undoes it.
__device__ __forceinline__ int swz(int slot) { return slot ^ ((slot >> 3) & 7); }

// Inclusive prefix XOR over the 16 lanes of a DPP row (lanes with no source
// read 0, the identity): 32 sign bits scanned at once.
__device__ __forceinline__ uint32_t row_xor_scan16(uint32_t x)
{
    const int v = static_cast<int>(x);
    int r = v ^ __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    r ^= __builtin_amdgcn_update_dpp(0, r, 0x112, 0xf, 0xf, true);          // row_shr:2
    r ^= __builtin_amdgcn_update_dpp(0, r, 0x114, 0xf, 0xf, true);          // row_shr:4
    r ^= __builtin_amdgcn_update_dpp(0, r, 0x118, 0xf, 0xf, true);          // row_shr:8
    return static_cast<uint32_t>(r);
}

// x with its sign flipped when bit i of mask is set (x * -1, exactly)
__device__ __forceinline__ float flip_sign(float x, uint32_t mask, int i)
{
    return __uint_as_float(__float_as_uint(x) ^ (((mask >> i) & 1u) << 31));
}

// SIGNED: Complex KDA, g holds the signed decay alpha.  With sigma_r the sign
// of alpha's running product, Gamma_r = sigma_r e^{b_r}; sigma_r is folded
// into q^ and k^ of row r, which gives every pair factor its sigma_r sigma_s,
// and the chunk-end sign sigma_L into gamma and K^ gamma/Gamma.  All the
// exponential factors stay those of b = sum log|alpha|.
constexpr int XS_LD = DK + 8;   // row stride (bf16) of the short convolution's staging

template <bool SIGNED, bool CONV>
__global__ void __launch_bounds__(NT, 2)
chunk_prep_kernel(ChunkArgs a, ChunkRecord* __restrict__ recs, const int* __restrict__ slot_seq, int nslots)
{
    __shared__ PrepSmem s;

    const int t = threadIdx.x;
    // the wave index is uniform across the wave: keep it in a scalar register
    // Sub-tile w of this wave.  The sub-tiles carry unequal work (tile rows
    // further down have more off-diagonal tiles), so the mapping rotates with
    // the workgroup id: two workgroups sharing a CU then rarely put their
    // heaviest waves on the same SIMD.
    const int w = (__builtin_amdgcn_readfirstlane(t >> 6) + static_cast<int>(blockIdx.x & 3)) & 3;
    const int l = t & 63, g = l >> 4, n = l & 15;
    const int H = a.H;
    // consecutive workgroups take consecutive heads of one chunk: their
    // q/k/g rows are adjacent in memory
    const int h = blockIdx.x % H;
    int slot = blockIdx.x / H;

    long c0, tok0, tok1;
    int seq;
    if (a.cu_seqlens && a.rec_stride == 0) {
        seq = slot_seq[slot];
        if (seq < 0) return;
        int b0 = a.cu_seqlens[seq], b1 = a.cu_seqlens[seq + 1];
        b0 = min(max(b0, 0), a.T);
        b1 = min(max(b1, b0), a.T);
        c0 = b0 + static_cast<long>(slot - (seq + b0 / C)) * C;
        tok0 = b0;
        tok1 = b1;
    } else {
        // this launch covers chunks chunk_lo .. chunk_lo + chunk_cnt - 1 of
        // every sequence; the record goes to slot seq * rec_stride + (j - rec_base)
        seq = slot / a.chunk_cnt;
        const int j = a.chunk_lo + (slot - seq * a.chunk_cnt);
        slot = seq * a.rec_stride + (j - a.rec_base);
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
        c0 = tok0 + static_cast<long>(j) * C;
    }
    if (c0 >= tok1) return;
    const int L = static_cast<int>(min(static_cast<long>(C), tok1 - c0));
    ChunkRecord* __restrict__ rg = recs + static_cast<size_t>(h) * nslots + slot;

    // ---- raw inputs of this lane's token row r = 16w + n: channels
    // 32kb + 8g + 0..7.  Rows past the end of the sequence read the last valid
    // token and are masked to the identity of the recurrence (k = g = beta = 0).
    const int row = 16 * w + n;
    float qv[32], kv[32], bv[32];
    uint32_t neg = 0;                // Complex KDA: bit e set <-> alpha of element e is negative
    float beta_r;
    {
        const long tk = min(c0 + row, tok1 - 1);
        const size_t base = static_cast<size_t>(tk) * H + h;
        const uint16_t* qr = static_cast<const uint16_t*>(a.q) + base * DK + 8 * g;
        const uint16_t* kr = static_cast<const uint16_t*>(a.k) + base * DK + 8 * g;
        uint4 rq[4], rk[4];
        float4 rgv[8];
        uint4 rz[4];
        float a_log = 0.f;
        // the decay inputs and beta are requested first: with the short
        // convolution their latency then overlaps the staging below
        if (a.gated) {
            const uint16_t* zr = static_cast<const uint16_t*>(a.z) + base * DK + 8 * g;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) rz[kb] = *reinterpret_cast<const uint4*>(zr + 32 * kb);
            a_log = a.A_log[h];
            // this lane's dt_bias channels, requested with z (rgv holds them
            // until the map below replaces them by g)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                rgv[2 * kb] = make_float4(0.f, 0.f, 0.f, 0.f);
                rgv[2 * kb + 1] = rgv[2 * kb];
                if (a.dt_bias) {
                    rgv[2 * kb] = *reinterpret_cast<const float4*>(a.dt_bias + h * DK + 32 * kb + 8 * g);
                    rgv[2 * kb + 1] = *reinterpret_cast<const float4*>(a.dt_bias + h * DK + 32 * kb + 8 * g + 4);
                }
            }
        } else {
            const float* gr = a.g + base * DK + 8 * g;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                rgv[2 * kb] = *reinterpret_cast<const float4*>(gr + 32 * kb);
                rgv[2 * kb + 1] = *reinterpret_cast<const float4*>(gr + 32 * kb + 4);
            }
        }
        const float beta_in = a.beta[base];
        if constexpr (CONV) {
            // Short convolution of q and k ("Kimi K3 の KDA ..." section 1.2.1:
            // per channel, the current token and the 3 before it, then SiLU).
            // The chunk's raw rows with the 3 before it, and this head's taps,
            // go to LDS (the space of the later phases); each lane then
            // convolves its own row and channels in fp32.  Rows before the
            // sequence start come from its conv state (or are zero); rows past
            // its end repeat the last token (masked later, like the plain path).
            // rows padded to XS_LD so the 16 lanes that read 16 consecutive rows
            // of the same channels hit distinct LDS banks
            uint16_t* xs = reinterpret_cast<uint16_t*>(&s.u);                        // [2][C + 3][XS_LD] raw
            float* wsm = reinterpret_cast<float*>(xs + 2 * (C + 3) * XS_LD);         // [2][DK][4] taps
            static_assert(2 * (C + 3) * XS_LD * 2 + 2 * DK * 4 * 4 <= sizeof(s.u) + sizeof(s.akk), "conv staging fits");
            const uint16_t* src[2] = {static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k)};
            const uint16_t* st[2] = {static_cast<const uint16_t*>(a.conv_init[0]),
                                     static_cast<const uint16_t*>(a.conv_init[1])};
            constexpr int PPR = DK / 8, PIECES = 2 * (C + 3) * PPR;
            constexpr int ITER = (PIECES + NT - 1) / NT;
            // three loads in flight per thread, then their LDS stores: one
            // load at a time left the global latency exposed 9 times (8.50 ms
            // against 7.99 ms for the 64K prefill with the convolution)
            constexpr int BATCH = 3;
#pragma unroll
            for (int i0 = 0; i0 < ITER; i0 += BATCH) {
                uint4 val[BATCH];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int i = t + NT * (i0 + u);
                    val[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (i0 + u < ITER && i < PIECES) {
                        const int x = i / ((C + 3) * PPR), rem = i % ((C + 3) * PPR), r = rem / PPR, part = rem % PPR;
                        const long tj = c0 - 3 + r;
                        const uint16_t* sp = nullptr;
                        if (tj >= tok0)
                            sp = src[x] + (static_cast<size_t>(min(tj, tok1 - 1)) * H + h) * DK + 8 * part;
                        else if (st[x])
                            sp = st[x] + ((static_cast<size_t>(seq) * 3 + static_cast<size_t>(3 + tj - tok0)) * H + h) * DK +
                                 8 * part;
                        if (sp) val[u] = *reinterpret_cast<const uint4*>(sp);
                    }
                }
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int i = t + NT * (i0 + u);
                    if (i0 + u < ITER && i < PIECES) {
                        const int x = i / ((C + 3) * PPR), rem = i % ((C + 3) * PPR), r = rem / PPR, part = rem % PPR;
                        *reinterpret_cast<uint4*>(xs + (x * (C + 3) + r) * XS_LD + 8 * part) = val[u];
                    }
                }
            }
            {
                static_assert(NT == 2 * DK, "one thread per (tensor, channel)");
                const int x = t / DK, c = t % DK;
                *reinterpret_cast<float4*>(wsm + 4 * t) =
                    *reinterpret_cast<const float4*>(a.conv_w[x] + 4 * (static_cast<size_t>(h) * DK + c));
            }
            __syncthreads();
            // silu(conv) in fp32 from the staged rows row .. row + 3 (tokens
            // tk - 3 .. tk) and taps; one group of 8 channels at a time keeps
            // the operands of a single group live
            auto conv_row = [&](int x, float (&dst)[32]) __attribute__((always_inline)) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int ch = 32 * kb + 8 * g;
                    uint4 raw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        raw[j] = *reinterpret_cast<const uint4*>(xs + (x * (C + 3) + row + j) * XS_LD + ch);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float4 wt = *reinterpret_cast<const float4*>(wsm + 4 * (x * DK + ch + e));
                        const float tw[4] = {wt.x, wt.y, wt.z, wt.w};
                        float acc = 0.f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t word = (e >> 1) == 0 ? raw[j].x : (e >> 1) == 1 ? raw[j].y
                                                : (e >> 1) == 2 ? raw[j].z : raw[j].w;
                            acc += tw[j] * ((e & 1) ? bf_hi(word) : bf_lo(word));
                        }
                        dst[8 * kb + e] = silu(acc);
                    }
                    // this group's results are produced before the next
                    // group's LDS reads issue, which bounds the live operands
                    __asm__ volatile("" : "+v"(dst[8 * kb + 0]), "+v"(dst[8 * kb + 1]), "+v"(dst[8 * kb + 2]),
                                     "+v"(dst[8 * kb + 3]), "+v"(dst[8 * kb + 4]), "+v"(dst[8 * kb + 5]),
                                     "+v"(dst[8 * kb + 6]), "+v"(dst[8 * kb + 7])::"memory");
                }
            };
            conv_row(0, qv);
            conv_row(1, kv);
        } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                rq[kb] = *reinterpret_cast<const uint4*>(qr + 32 * kb);
                rk[kb] = *reinterpret_cast<const uint4*>(kr + 32 * kb);
            }
        }
        if (a.gated) {
            // g = -5 sigmoid(e^{A_h} (z + dt_bias)) from bf16 z
            const float ea = __expf(a_log);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const uint4 z4 = rz[kb];
                const float4 b0 = rgv[2 * kb], b1 = rgv[2 * kb + 1];
                rgv[2 * kb] = make_float4(gate_log_decay(bf_lo(z4.x), b0.x, ea), gate_log_decay(bf_hi(z4.x), b0.y, ea),
                                          gate_log_decay(bf_lo(z4.y), b0.z, ea), gate_log_decay(bf_hi(z4.y), b0.w, ea));
                rgv[2 * kb + 1] = make_float4(gate_log_decay(bf_lo(z4.z), b1.x, ea), gate_log_decay(bf_hi(z4.z), b1.y, ea),
                                              gate_log_decay(bf_lo(z4.w), b1.z, ea), gate_log_decay(bf_hi(z4.w), b1.w, ea));
            }
        }
        const float braw = a.beta_logits ? beta_from_logit(beta_in) : beta_in;
        const float live = (row < L) ? 1.f : 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if constexpr (CONV) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[8 * kb + e] *= live;
            } else {
                const uint32_t qw[4] = {rq[kb].x, rq[kb].y, rq[kb].z, rq[kb].w};
                const uint32_t kw[4] = {rk[kb].x, rk[kb].y, rk[kb].z, rk[kb].w};
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    qv[8 * kb + 2 * e2] = bf_lo(qw[e2]);
                    qv[8 * kb + 2 * e2 + 1] = bf_hi(qw[e2]);
                    kv[8 * kb + 2 * e2] = bf_lo(kw[e2]) * live;
                    kv[8 * kb + 2 * e2 + 1] = bf_hi(kw[e2]) * live;
                }
            }
            bv[8 * kb + 0] = rgv[2 * kb].x;
            bv[8 * kb + 1] = rgv[2 * kb].y;
            bv[8 * kb + 2] = rgv[2 * kb].z;
            bv[8 * kb + 3] = rgv[2 * kb].w;
            bv[8 * kb + 4] = rgv[2 * kb + 1].x;
            bv[8 * kb + 5] = rgv[2 * kb + 1].y;
            bv[8 * kb + 6] = rgv[2 * kb + 1].z;
            bv[8 * kb + 7] = rgv[2 * kb + 1].w;
        }
        if constexpr (SIGNED) {
            // alpha -> (sign bit, log|alpha|); rows past the end act as alpha = 1
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float al = bv[e];
                neg |= (al < 0.f ? 1u : 0u) << e;
                bv[e] = (row < L) ? __logf(fabsf(al)) : 0.f;
            }
            if (row >= L) neg = 0u;
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) bv[e] *= live;
        }
        beta_r = braw * live;
    }

    // L2 norm of q and k over d_k (the row is spread over the 4 lane groups)
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
    if constexpr (SIGNED) {
        // running sign inside the sub-tile: a prefix XOR of the 32 sign bits
        // over the 16 rows (it is applied to q^ and k^ of this row with the
        // sign of the sub-tiles before, in the loop below)
        neg = row_xor_scan16(neg);
        if (n == 15) s.tsg[w][g] = neg;
    }
    if (g == 0) s.beta[row] = beta_r;
    __syncthreads();

    // per-channel decay factors for every sub-tile; each factor is an exp of
    // a non-positive sum, so none overflows
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
            rg->gam[c] = __expf(r4);
        }
        if constexpr (SIGNED) {
            // sign of the decay product over the whole chunk, channel c
            const int gc = (c >> 3) & 3, bc = ((c >> 5) << 3) | (c & 7);
            const uint32_t sLb = ((s.tsg[0][gc] ^ s.tsg[1][gc] ^ s.tsg[2][gc] ^ s.tsg[3][gc]) >> bc) & 1u;
            const float sL = sLb ? -1.f : 1.f;
            __syncthreads();   // every fac entry above is written before it is rescaled
            if (t < DK) {
                s.fac[0][3][c] *= sL;
                s.fac[1][3][c] *= sL;
            } else {
                s.fac[2][3][c] *= sL;
                s.fac[3][3][c] = sL;
                rg->gam[c] *= sL;
            }
        }
    }
    __syncthreads();

    // Per element: d = exp(b - ref_{w+1}) in [1, e^80], f = 1/d,
    // E = exp(b - ref_w) <= 1, Gamma = exp(b).  The diagonal tile (w, w) is
    // computed right here: both of its operands are in this lane.  The
    // off-diagonal tiles share one A-operand, X^ E.
    // Complex KDA also keeps the low half of the A_kk operands: with |alpha|
    // near 1 nothing damps the rounding of single-bf16 A_kk over a long chain
    // Complex KDA: the sign of this row's decay product per channel = the
    // running sign inside sub-tile w XOR the sign over the sub-tiles before it
    uint32_t sgnb = 0u;
    if constexpr (SIGNED) {
        sgnb = neg;
        for (int v = 0; v < w; ++v) sgnb ^= s.tsg[v][g];
    }
    bf16x8 kao[4], qoh[4], qol[4], kaol[SIGNED ? 4 : 1];
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
        bf16x8 kfh, kfl, kad, kadl, qdh, qdl;
        float qgv[8], kgv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float bl = bv[8 * kb + e];         // running sum inside sub-tile w
            const float d = __expf(bl - tw[e]);      // b - ref_{w+1}
            const float f = __builtin_amdgcn_rcpf(d);  // exp(ref_{w+1} - b)
            const float E = d * dw[e];               // exp(b - ref_w)
            const float gm = E * er[e];              // exp(b)
            const float kx = SIGNED ? flip_sign(kv[8 * kb + e], sgnb, 8 * kb + e) : kv[8 * kb + e];
            const float qx = SIGNED ? flip_sign(qv[8 * kb + e], sgnb, 8 * kb + e) : qv[8 * kb + e];
            __bf16 hi, lo;
            split(kx * f, hi, lo);
            kfh[e] = hi;
            kfl[e] = lo;
            qgv[e] = qx * gm;
            kgv[e] = -kx * gm;
            if constexpr (SIGNED) {
                split(kx * d, hi, lo);
                kad[e] = hi;
                kadl[e] = lo;
            } else {
                kad[e] = static_cast<__bf16>(kx * d);
            }
            split(qx * d, hi, lo);
            qdh[e] = hi;
            qdl[e] = lo;
            if constexpr (SIGNED) {
                split(kx * E, hi, lo);
                kao[kb][e] = hi;
                kaol[kb][e] = lo;
            } else {
                kao[kb][e] = static_cast<__bf16>(kx * E);
            }
            split(qx * E, hi, lo);
            qoh[kb][e] = hi;
            qol[kb][e] = lo;
            kq16[kb][e] = static_cast<_Float16>(kx * f * el[e]);
        }
        if constexpr (SIGNED)
            akd = mma3(kad, kadl, kfh, kfl, akd);
        else
            akd = mma(kad, kfh, akd);
        aqd = mma3(qdh, qdl, kfh, kfl, aqd);
        s.u.kf[0][w][kb][l] = kfh;
        s.u.kf[1][w][kb][l] = kfl;
        // Q^ Gamma and -K^ Gamma, in the state's channel order, straight to
        // the record: channel 32kb + 8g + e goes to lane (2(g&1) + e/4)*16 + n,
        // element 4(g>>1) + e%4
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
            *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&rg->qg[w][kb][l0]) + eo) = q0;
            *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&rg->qg[w][kb][l1]) + eo) = q1;
            *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&rg->kgn[w][kb][l0]) + eo) = k0;
            *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(&rg->kgn[w][kb][l1]) + eo) = k1;
        }
    }
    // diagonal tile (w, w): lane holds rows 16w + 4g + i, column 16w + n.
    // A_qk goes to the A-fragment of U~'s token order: column token
    // 16j + n of tile (w, j) is element (n&3) + 4(j&1) of lane (n/4)*16 + row%16
    // in block (w, j/2).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * g + i, sc = 16 * w + n;
        if (sc < r) s.akk[r][sc] = s.beta[r] * akd[i];
        _Float16 hi, lo;
        splith((sc <= r) ? aqd[i] : 0.f, hi, lo);
        const int lt = (n >> 2) * 16 + 4 * g + i, e = (n & 3) + 4 * (w & 1);
        const int p = tri_block(w, w >> 1);
        reinterpret_cast<_Float16*>(&s.aqk[0][p][swz(lt)])[e] = hi;
        reinterpret_cast<_Float16*>(&s.aqk[1][p][swz(lt)])[e] = lo;
        if ((w & 1) == 0) {   // tile (w, w+1) shares this token block: zero it
            reinterpret_cast<_Float16*>(&s.aqk[0][p][swz(lt)])[e + 4] = static_cast<_Float16>(0.f);
            reinterpret_cast<_Float16*>(&s.aqk[1][p][swz(lt)])[e + 4] = static_cast<_Float16>(0.f);
        }
    }
    __syncthreads();

    // ---- off-diagonal tiles (w, j < w).  The B-operand of sub-tile j is
    // referenced to ref_{j+1}; tiles two or three sub-tiles apart rescale it
    // to ref_w by exp(tot_{j+1} + ... + tot_{w-1}) <= 1.
    for (int j = 0; j < w; ++j) {
        f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            bh[kb] = s.u.kf[0][j][kb][l];
            bl[kb] = s.u.kf[1][j][kb][l];
        }
        if (j + 2 <= w) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float x1[8], x2[8];
                lds8(&s.dl12[0][32 * kb + 8 * g], x1);
                lds8(&s.dl12[1][32 * kb + 8 * g], x2);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // (w, j) = (2,0): exp(tot_1); (3,0): exp(tot_1 + tot_2); (3,1): exp(tot_2)
                    const float sc = (w == 2) ? x1[e] : ((j == 0) ? x1[e] * x2[e] : x2[e]);
                    const float kf = (static_cast<float>(bh[kb][e]) + static_cast<float>(bl[kb][e])) * sc;
                    __bf16 hi, lo;
                    split(kf, hi, lo);
                    bh[kb][e] = hi;
                    bl[kb][e] = lo;
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if constexpr (SIGNED)
                akk = mma3(kao[kb], kaol[kb], bh[kb], bl[kb], akk);
            else
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
            const int p = tri_block(w, j >> 1);
            reinterpret_cast<_Float16*>(&s.aqk[0][p][swz(lt)])[e] = hi;
            reinterpret_cast<_Float16*>(&s.aqk[1][p][swz(lt)])[e] = lo;
        }
    }
    __syncthreads();

    // ---- T = (I + A_kk)^-1, blocked, in place.  Diagonal 16x16 blocks by
    // forward substitution: lane owns column l/4 of block w and the rows
    // l%4 + 4m of it; the four partial sums of a column sit in one lane quad
    // and are reduced with DPP.
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
            _Float16* dst = reinterpret_cast<_Float16*>(&s.u.kp[mt][w >> 1][0]);
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) dst[swz(lb + ee) * 8 + e] = kq16[kb][ee];
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
    // accumulator layout of V - K Gamma S: element e of lane group g holds
    // token 32kb + 16(e/4) + 4g + e%4.  Blocks above the diagonal are zero
    // and not stored.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb > (w >> 1)) continue;
        const float4 t0 = *reinterpret_cast<const float4*>(&s.akk[row][32 * kb + 4 * g]);
        const float4 t1 = *reinterpret_cast<const float4*>(&s.akk[row][32 * kb + 16 + 4 * g]);
        const float4 b0 = *reinterpret_cast<const float4*>(&s.beta[32 * kb + 4 * g]);
        const float4 b1 = *reinterpret_cast<const float4*>(&s.beta[32 * kb + 16 + 4 * g]);
        const float tv8[8] = {t0.x * b0.x, t0.y * b0.y, t0.z * b0.z, t0.w * b0.w,
                              t1.x * b1.x, t1.y * b1.y, t1.z * b1.z, t1.w * b1.w};
        bf16x8 th, tl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sc = 32 * kb + 16 * (e >> 2) + 4 * g + (e & 3);
            const float x = (sc <= row) ? tv8[e] : 0.f;
            __bf16 hi, lo;
            split(x, hi, lo);
            th[e] = hi;
            tl[e] = lo;
        }
        const int p = tri_block(w, kb);
        rg->tp[0][p][l] = th;
        rg->tp[1][p][l] = tl;
    }

    // A_qk and K'^T fragments: LDS -> record, whole 16-byte pieces
    {
        const uint4* src = reinterpret_cast<const uint4*>(&s.aqk[0][0][0]);
        uint4* dst = reinterpret_cast<uint4*>(&rg->aqk[0][0][0]);
        constexpr int NA = static_cast<int>(sizeof(s.aqk) / 16);
#pragma unroll
        for (int i = t; i < NA; i += NT) dst[i] = src[(i & ~63) | swz(i & 63)];
        const uint4* src2 = reinterpret_cast<const uint4*>(&s.u.kp[0][0][0]);
        uint4* dst2 = reinterpret_cast<uint4*>(&rg->kp[0][0][0]);
        constexpr int NK = static_cast<int>(sizeof(s.u.kp) / 16);
#pragma unroll
        for (int i = t; i < NK; i += NT) dst2[i] = src2[(i & ~63) | swz(i & 63)];
    }
}

// ---------------------------------------------------------------------------
// Pass 2: the state recurrence over the records
// ---------------------------------------------------------------------------

constexpr int DVS = 64;     // value columns per pass-2 workgroup: 4 waves x 16
constexpr int NSLICE = DV / DVS;

// Row stride (floats) of the fp32 output staging of the output norm: padded
// so that the 16 rows one wave instruction touches fall into distinct banks.
constexpr int OSTRIDE_NORM = DVS + 4;

// What the output-free summary launch of the segmented order reads of a
// record: T', -K^ Gamma, (K^ gamma/Gamma)^T and gamma, without A_qk and
// Q^ Gamma.  Each array keeps its place in whole 4 KB blocks of the record
// (16-byte piece t + 256 i), so block i of this struct is block
// summary_block(i) of the record.
struct alignas(16) SummaryRecord {
    bf16x8 tp[2][6][64];
    f16x8 kgn[4][4][64];
    f16x8 kp[8][2][64];
    float gam[DK];
};
__host__ __device__ constexpr int summary_block(int i) { return i < 3 ? i : (i < 7 ? i + 3 : (i < 11 ? i + 7 : 18)); }
static_assert(offsetof(ChunkRecord, kgn) == 6 * 4096 && offsetof(ChunkRecord, kp) == 14 * 4096 &&
                  offsetof(ChunkRecord, gam) == 18 * 4096 && offsetof(SummaryRecord, kgn) == 3 * 4096 &&
                  offsetof(SummaryRecord, kp) == 7 * 4096 && offsetof(SummaryRecord, gam) == 11 * 4096,
              "summary blocks");

// V staging: bf16 as loaded, or fp32 when it is the short convolution's output
template <bool CONV, bool NORM, bool OUT>
struct alignas(16) ScanSmem {
    typename std::conditional<OUT, ChunkRecord, SummaryRecord>::type r;   // this chunk's operands
    typename std::conditional<CONV, float, __bf16>::type vs[C][DVS];   // V slice [token][column]
    // output tile staging ([token][column], bf16 or fp32), two chunks; with
    // the output norm fp32 and three chunks (a tile waits one chunk for the
    // other slice's row sums before it is normalised and stored)
    float obuf[OUT ? (NORM ? 3 : 2) : 1][OUT ? C * (NORM ? OSTRIDE_NORM : DVS) : 4];
    float nw[NORM ? DVS : 4];        // output norm: gain of this slice's columns
};

// Output norm across the two value slices of a chain: per chunk, each slice
// publishes its 64 per-row sums of o^2 (taken from the unrounded fp32 o) as
// 64-bit words (chunk index + 1) << 32 | float bits, written and read with
// device-scope atomics, so a word is either the value of the expected chunk
// or recognisably stale; no other memory ordering is needed.  Four words per
// row and slice cycle with the chunk index.  A reader polls with a bounded
// number of retries (the other slice runs the same chunk sequence and
// publishes before it waits, so the bound is never reached unless that
// workgroup cannot run; it keeps the kernel finite in any case).
constexpr int kNormSlotsPerRow = 4;
constexpr int kNormSpinLimit = 1 << 20;
__host__ __device__ constexpr size_t norm_slot_words(long long chains)
{
    return static_cast<size_t>(chains) * NSLICE * kNormSlotsPerRow * C;
}

__global__ void zero_words_kernel(unsigned long long* __restrict__ p, size_t n)
{
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0ull;
}

// output tile staging; bf16 is rounded to nearest even by the hardware conversion
__device__ __forceinline__ void stage_out(float* base, int r, int c, float x, const float*)
{
    base[r * DVS + c] = x;
}
__device__ __forceinline__ void stage_out(float* base, int r, int c, float x, const uint16_t*)
{
    reinterpret_cast<uint16_t*>(base)[r * DVS + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// fp32 staging of the output norm (padded rows)
struct NormStage {};
__device__ __forceinline__ void stage_out(float* base, int r, int c, float x, const NormStage*)
{
    base[r * OSTRIDE_NORM + c] = x;
}

// The state update K'^T U~ takes U~ as fp16 hi + lo (two products) rather
// than one fp16 rounding: with the keys the model produces (SiLU'd, sharing a
// common direction) the state stays small next to what each chunk writes,
// and U~'s single fp16 rounding alone costs ~3e-2 of RMS(S).
// The output-free instantiation (OUT = false) holds less in LDS and in
// registers and runs two workgroups per CU (without the short convolution,
// whose registers do not fit half a CU).
template <typename Tout, bool CONV, bool NORM, bool SPLIT = true, bool OUT = true>
__global__ void __launch_bounds__(NT, (OUT || CONV) ? 1 : 2)
chunk_scan_kernel(ChunkArgs a, const ChunkRecord* __restrict__ recs, int nslots, unsigned long long* norm_slots)
{
    static_assert(OUT || !NORM, "the output norm needs the outputs");
    __shared__ ScanSmem<CONV, NORM, OUT> s;

    const int t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l = t & 63, g = l >> 4, n = l & 15;
    const int H = a.H;
    // Workgroup -> (chain, slice).  Both slices of a chain get ids that are
    // equal mod 8, so they are dispatched to the same XCD and the second read
    // of each record hits that XCD's L2.
    const int bid = blockIdx.x;
    const int slice = (bid >> 3) & (NSLICE - 1);
    // unit of work: a chain, or with the segmented pass a (chain, unit) pair
    const int vc = ((bid >> 4) << 3) | (bid & 7);
    const int nchains = (a.cu_seqlens ? a.num_seqs : a.B) * H;
    const int units = a.seg_phase == 1 ? seg_units_a(a.seg_count) : (a.seg_phase == 2 ? seg_units_c(a.seg_count) : 1);
    if (vc >= nchains * units) return;
    const int chain = vc / units, unit = vc - chain * units;
    const int j0 = slice * DVS;
    const int seq = chain / H, h = chain % H;

    long tok0, tok1;
    int slot0, rbase = 0;   // the record of chunk j is slot slot0 + j - rbase
    if (a.cu_seqlens) {
        int b0 = a.cu_seqlens[seq], b1 = a.cu_seqlens[seq + 1];
        b0 = min(max(b0, 0), a.T);
        b1 = min(max(b1, b0), a.T);
        tok0 = b0;
        tok1 = b1;
        slot0 = seq + b0 / C;
    } else {
        tok0 = static_cast<long>(seq) * a.T;
        tok1 = tok0 + a.T;
    }
    if (!a.cu_seqlens || a.rec_stride > 0) {
        slot0 = seq * a.rec_stride;
        rbase = a.rec_base;
    }
    const int nch = static_cast<int>((tok1 - tok0 + C - 1) / C);
    // this launch runs chunks jb .. je - 1 of the chain, from init_state (the
    // chain's initial state, or the state a launch over the chunks before
    // left) to final_state
    int jb = min(a.chunk_lo, nch);
    int je = static_cast<int>(min(static_cast<long>(nch), static_cast<long>(a.chunk_lo) + a.chunk_cnt));
    // per unit: where the state comes from and goes, whether o is written,
    // whether the values are taken as zero (the transition of a segment)
    const float* sinit = a.init_state ? a.init_state + static_cast<size_t>(chain) * DK * DV : nullptr;
    float* sfinal = a.final_state ? a.final_state + static_cast<size_t>(chain) * DK * DV : nullptr;
    // (OUT = false: the summary launch of the segmented order, no outputs)
    constexpr bool with_out = OUT;
    bool identity = false, zero_v = false;
    float* scopy = nullptr;   // where phase A keeps a copy of the chain's initial state
    if (a.seg_phase) {
        const int P = a.seg_count;
        float* blocks = a.seg_states + static_cast<size_t>(chain) * seg_state_blocks(P) * DK * DV;
        auto block = [&](int k) { return blocks + static_cast<size_t>(k) * DK * DV; };
        int sg;
        if (a.seg_phase == 1) {
            sg = (unit + 1) >> 1;
            if (unit == 0) {
                sfinal = block(0);
                scopy = block(seg_block_init(P));
            } else if (unit & 1) {
                sinit = nullptr;
                sfinal = block(seg_block_b(P, sg));
            } else {
                sinit = nullptr;
                identity = zero_v = true;
                sfinal = block(seg_block_m(P, sg));
            }
        } else {
            sg = unit;
            sinit = block(sg > 0 ? seg_block_in(P, sg) : seg_block_init(P));
            if (sg + 1 < P) sfinal = nullptr;
        }
        // segments of this chain's chunk range in the launch (the whole
        // chain, or a window): P pieces of ceil(range / P) chunks
        const int end = je, len = (end - jb + P - 1) / P;
        jb = min(jb + sg * len, end);
        je = min(jb + len, end);
    }
    const ChunkRecord* __restrict__ rc = recs + static_cast<size_t>(h) * nslots + slot0;
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v);
    Tout* __restrict__ op = static_cast<Tout*>(a.o);

    // ---- state strip: channels 16*mt + 4*g + i, column j0 + 16*w + n
    f32x4 sacc[8];
    {
        const size_t sbase = j0 + 16 * w + n;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * mt + 4 * g + i;
                sacc[mt][i] = sinit ? sinit[sbase + static_cast<size_t>(ch) * DV]
                                    : ((identity && ch == static_cast<int>(sbase)) ? 1.f : 0.f);
                if (scopy) scopy[sbase + static_cast<size_t>(ch) * DV] = sacc[mt][i];
            }
    }

    // The next chunk's record and V slice travel in registers while the
    // current chunk is computed (issued in pieces between the compute steps
    // so the loads overlap them), then go to LDS between two barriers.
    constexpr int RV = static_cast<int>(sizeof(s.r) / 16);
    constexpr int RFULL = RV / NT;
    constexpr int RTAIL = RV - RFULL * NT;
    // the four batches of pieces issued during a chunk: [0, F1) [F1, F2) [F2, F3) [F3, RFULL]
    constexpr int F1 = OUT ? 5 : 3, F2 = OUT ? 10 : 6, F3 = OUT ? 15 : 9;
    constexpr int PPR = DVS / 8;                   // 16-byte pieces per V row
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 P[RFULL + 1], PV[2];
    // Short convolution of v ("Kimi K3 の KDA ..." section 1.2.1): the 4 raw
    // rows under each output row travel in registers and are convolved (in
    // fp32, staged in fp32) when they are committed to LDS; this thread's 8
    // columns are the same for both of its rows.
    u32x4 PVc[CONV ? 2 : 1][CONV ? 4 : 1];
    float4 WV[CONV ? 8 : 1];
    const uint16_t* __restrict__ vst = static_cast<const uint16_t*>(a.conv_init[2]);
    if constexpr (CONV) {
        const size_t chv = static_cast<size_t>(h) * DV + j0 + 8 * (t % PPR);
#pragma unroll
        for (int e = 0; e < 8; ++e) WV[e] = *reinterpret_cast<const float4*>(a.conv_w[2] + 4 * (chv + e));
    }
    // record pieces i in [i0, i1) of chunk j; piece RFULL is the partial one
    // (the summary launch: pieces of the summary's blocks)
    // Pieces are read as raw buffer loads: the record's address in a
    // workgroup-uniform descriptor (scalar registers), the block's offset as
    // a scalar offset and this thread's fixed 16-byte offset, so issuing a
    // piece needs no vector address arithmetic.
    const int toff = 16 * t;
    auto fetch = [&](int j, int i0, int i1) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<ChunkRecord*>(rc + (j - rbase)), 0, static_cast<int>(sizeof(ChunkRecord)), kBufferWord3);
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            const int blk = OUT ? i : summary_block(i);
            if (i < RFULL || t < RTAIL) P[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, toff, 4096 * blk, 0);
        }
    };
    auto fetch_v = [&](int j) __attribute__((always_inline)) {
        const long cb = tok0 + static_cast<long>(j) * C;
        if (zero_v) {   // the transition of a segment: values taken as zero (a zero conv input gives silu(0) = 0)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if constexpr (CONV) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) PVc[u][jj] = u32x4{0u, 0u, 0u, 0u};
                } else {
                    PV[u] = u32x4{0u, 0u, 0u, 0u};
                }
            }
            return;
        }
        if constexpr (!CONV && OUT) {
            // rows past the end read the last valid token (T' has zero
            // columns for them, so only finiteness matters); raw buffer
            // loads from the chunk's first row of this slice, a uniform base
            // (the summary launch keeps the plain loads: under its register
            // bound the offsets' registers would wait on loads in flight)
            const int lim = static_cast<int>(min(static_cast<long>(C - 1), tok1 - 1 - cb));
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(vp + (static_cast<size_t>(cb) * H + h) * DV + j0), 0,
                (lim * H * DV + DVS) * 2, kBufferWord3);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int idx = t + NT * u, r = idx / PPR, part = idx % PPR;
                PV[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (min(r, lim) * H * DV + 8 * part) * 2, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = t + NT * u, r = idx / PPR, part = idx % PPR;
            // rows past the end read the last valid token: T' has zero
            // columns for them, so only finiteness matters
            const long tk = min(cb + r, tok1 - 1);
            if constexpr (CONV) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const long tj = tk - 3 + jj;
                    if (tj >= tok0)
                        PVc[u][jj] = *reinterpret_cast<const u32x4*>(vp + (static_cast<size_t>(tj) * H + h) * DV + j0 +
                                                                     8 * part);
                    else if (vst)
                        PVc[u][jj] = *reinterpret_cast<const u32x4*>(
                            vst + ((static_cast<size_t>(seq) * 3 + static_cast<size_t>(3 + tj - tok0)) * H + h) * DV +
                            j0 + 8 * part);
                    else
                        PVc[u][jj] = u32x4{0u, 0u, 0u, 0u};
                }
            } else {
                PV[u] = *reinterpret_cast<const u32x4*>(vp + (static_cast<size_t>(tk) * H + h) * DV + j0 + 8 * part);
            }
        }
    };
    // silu(conv) of the 8 columns of fetched row u, written to LDS in fp32
    auto commit_conv_v = [&](int u, float* dst) __attribute__((always_inline)) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float tw[4] = {WV[e].x, WV[e].y, WV[e].z, WV[e].w};
            float acc = 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t word = PVc[u][jj][e >> 1];
                acc += tw[jj] * ((e & 1) ? bf_hi(word) : bf_lo(word));
            }
            y[e] = silu(acc);
        }
        *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(y[4], y[5], y[6], y[7]);
    };
    auto commit = [&]() __attribute__((always_inline)) {
        u32x4* dst = reinterpret_cast<u32x4*>(&s.r);
#pragma unroll
        for (int i = 0; i < RFULL; ++i) dst[t + NT * i] = P[i];
        if (t < RTAIL) dst[t + NT * RFULL] = P[RFULL];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = t + NT * u, r = idx / PPR, part = idx % PPR;
            if constexpr (CONV)
                commit_conv_v(u, &s.vs[r][8 * part]);
            else
                *reinterpret_cast<u32x4*>(&s.vs[r][8 * part]) = PV[u];
        }
    };

    if constexpr (NORM) {
        if (t < DVS) s.nw[t] = a.norm_w ? a.norm_w[j0 + t] : 1.f;
    }
    if (je > jb) {
        fetch(jb, 0, RFULL + 1);
        fetch_v(jb);
        commit();
    }
    __syncthreads();

    // Output tiles are staged in LDS (alternating buffers) and written out as
    // whole rows during the next chunk, or after the loop for the last one.
    // (raw buffer stores from the tile's first row of this slice, a uniform base)
    auto store_tile = [&](int buf, long cbase, int rows) __attribute__((always_inline)) {
        constexpr int CH = 16 / sizeof(Tout);            // elements per 16-byte piece
        constexpr int PER_ROW = DVS / CH;
        const char* src = reinterpret_cast<const char*>(s.obuf[buf]);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            op + (static_cast<size_t>(cbase) * H + h) * DV + j0, 0,
            static_cast<int>(((rows - 1) * H * DV + DVS) * sizeof(Tout)), kBufferWord3);
#pragma unroll
        for (int pc = t; pc < C * PER_ROW; pc += NT) {
            const int r = pc / PER_ROW, part = pc % PER_ROW;
            if (r < rows) {
                const u32x4 val = *reinterpret_cast<const u32x4*>(src + (r * DVS + part * CH) * sizeof(Tout));
                __builtin_amdgcn_raw_buffer_store_b128(val, rs, static_cast<int>((r * H * DV + part * CH) * sizeof(Tout)),
                                                       0, 0);
            }
        }
    };
    // ---- output norm ("Kimi K3 の KDA ..." section 1.2.1: RMSNorm over the
    // head's d_v values, then the sigmoid gate): thread t handles row t/4 of a
    // staged fp32 tile and 16 of its 64 columns; the 4 threads of a row are
    // adjacent lanes.  publish: this slice's sum of o^2 per row of chunk m,
    // kept in a register and written to the row's word for the other slice.
    // finish: the other slice's sum for chunk m (polled), then
    // o = x / sqrt(mean(x^2) + eps) * w * sigmoid(gate) stored once.
    const int nrow = t >> 2, nq = t & 3;
    unsigned long long* __restrict__ my_words =
        NORM ? norm_slots + static_cast<size_t>(vc * NSLICE + slice) * kNormSlotsPerRow * C + nrow : nullptr;
    const unsigned long long* __restrict__ other_words =
        NORM ? norm_slots + static_cast<size_t>(vc * NSLICE + (slice ^ 1)) * kNormSlotsPerRow * C + nrow : nullptr;
    const uint16_t* __restrict__ gp = static_cast<const uint16_t*>(a.out_gate);
    auto row_sum = [&](int b) __attribute__((always_inline)) {
        const float* src = s.obuf[b] + nrow * OSTRIDE_NORM + 16 * nq;
        float ps = 0.f;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4 x = *reinterpret_cast<const float4*>(src + 4 * e4);
            ps += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
        }
        ps += __shfl_xor(ps, 1, 64);
        ps += __shfl_xor(ps, 2, 64);
        return ps;
    };
    auto publish = [&](int m, int b, bool live) __attribute__((always_inline)) {
        const float ps = row_sum(b);
        if (live && nq == 0)
            __hip_atomic_store(my_words + (m & (kNormSlotsPerRow - 1)) * C,
                               (static_cast<unsigned long long>(m + 1) << 32) | __float_as_uint(ps), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        return ps;
    };
    auto poll = [&](int m) __attribute__((always_inline)) {
        return __hip_atomic_load(other_words + (m & (kNormSlotsPerRow - 1)) * C, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    };
    // (raw buffer loads from the tile's first gate row of this slice, a
    // uniform base; rows past the end read the last valid one)
    auto load_gate = [&](long cbase, int rows, uint4 (&gt)[2]) __attribute__((always_inline)) {
        const int last = max(rows - 1, 0);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(gp + (static_cast<size_t>(cbase) * H + h) * DV + j0), 0,
            (last * H * DV + DVS) * 2, kBufferWord3);
        const int off = (min(nrow, last) * H * DV + 16 * nq) * 2;
        const u32x4 g0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        const u32x4 g1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
        gt[0] = make_uint4(g0[0], g0[1], g0[2], g0[3]);
        gt[1] = make_uint4(g1[0], g1[1], g1[2], g1[3]);
    };
    // w * sigmoid(gate) of the 16 values this thread finishes in a tile, from
    // the tile's gate rows (independent of o: computed a chunk ahead, beside
    // matrix products)
    auto gate_scale = [&](const uint4 (&gt)[2], float (&sw)[16]) __attribute__((always_inline)) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4 wt = *reinterpret_cast<const float4*>(&s.nw[16 * nq + 4 * e4]);
            const uint4 g4 = gt[e4 >> 1];
            const uint32_t w0 = (e4 & 1) ? g4.z : g4.x, w1 = (e4 & 1) ? g4.w : g4.y;
            sw[4 * e4 + 0] = wt.x * sigmoid_fast(bf_lo(w0));
            sw[4 * e4 + 1] = wt.y * sigmoid_fast(bf_hi(w0));
            sw[4 * e4 + 2] = wt.z * sigmoid_fast(bf_lo(w1));
            sw[4 * e4 + 3] = wt.w * sigmoid_fast(bf_hi(w1));
        }
    };
    // (live = false: nothing is waited for or stored; the loop calls these
    // unconditionally so that no branch around a load leaves the register
    // bookkeeping of later waits uncertain)
    auto finish = [&](int m, int b, long cbase, int rows, float own, unsigned long long word, const float (&sw)[16],
                      bool live) __attribute__((always_inline)) {
        for (int it = 0;
             live && static_cast<unsigned>(word >> 32) != static_cast<unsigned>(m + 1) && it < kNormSpinLimit; ++it) {
            __builtin_amdgcn_s_sleep(1);
            word = poll(m);
        }
        // a word still stale after the bound (the other slice never ran)
        // makes the row NaN, not silently mis-scaled
        const bool got = static_cast<unsigned>(word >> 32) == static_cast<unsigned>(m + 1);
        const float inv = got ? rsqrtf((own + __uint_as_float(static_cast<unsigned>(word))) * (1.f / DV) + a.norm_eps)
                              : __builtin_nanf("");
        const float* src = s.obuf[b] + nrow * OSTRIDE_NORM + 16 * nq;
        float y[16];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4 x = *reinterpret_cast<const float4*>(src + 4 * e4);
            y[4 * e4 + 0] = x.x * inv * sw[4 * e4 + 0];
            y[4 * e4 + 1] = x.y * inv * sw[4 * e4 + 1];
            y[4 * e4 + 2] = x.z * inv * sw[4 * e4 + 2];
            y[4 * e4 + 3] = x.w * inv * sw[4 * e4 + 3];
        }
        if (live && nrow < rows) {
            // raw buffer stores from the tile's first row of this slice
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                op + (static_cast<size_t>(cbase) * H + h) * DV + j0, 0,
                static_cast<int>(((rows - 1) * H * DV + DVS) * sizeof(Tout)), kBufferWord3);
            const int off = static_cast<int>((nrow * H * DV + 16 * nq) * sizeof(Tout));
            if constexpr (std::is_same<Tout, float>::value) {
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4{__float_as_uint(y[4 * e4]), __float_as_uint(y[4 * e4 + 1]), __float_as_uint(y[4 * e4 + 2]),
                              __float_as_uint(y[4 * e4 + 3])},
                        rs, off + 16 * e4, 0, 0);
            } else {
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4{pack_bf16x2(y[8 * h8], y[8 * h8 + 1]), pack_bf16x2(y[8 * h8 + 2], y[8 * h8 + 3]),
                              pack_bf16x2(y[8 * h8 + 4], y[8 * h8 + 5]), pack_bf16x2(y[8 * h8 + 6], y[8 * h8 + 7])},
                        rs, off + 16 * h8, 0, 0);
            }
        }
    };

    // operand fragments of the R step for token tiles 2mh, 2mh + 1
    auto load_r = [&](int mh, f16x8 (&fa)[2][4], float (&vv)[2][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            const int mt = 2 * mh + m2;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) fa[m2][kb] = s.r.kgn[mt][kb][l];
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[m2][i] = static_cast<float>(s.vs[16 * mt + 4 * g + i][16 * w + n]);
        }
    };
    // Q^ Gamma fragments for token tiles 2mh, 2mh + 1
    // (the summary launch's record has neither Q^ Gamma nor A_qk)
    auto load_q = [&](int mh, f16x8 (&qa)[2][4]) __attribute__((always_inline)) {
        if constexpr (OUT) {
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) qa[m2][kb] = s.r.qg[2 * mh + m2][kb][l];
        }
    };
    // R = V - (K^ Gamma) S and the first term of O, (Q^ Gamma) S, for token
    // tiles 2mh, 2mh + 1: four independent accumulation chains share the
    // state operand, so the matrix core has work while each chain waits on
    // its previous product
    auto step_rq = [&](int mh, const f16x8 (&fa)[2][4], const f16x8 (&qa)[2][4], const float (&vv)[2][4],
                       const f16x8 (&sh)[4], const f16x8 (&sl)[4], f32x4 (&ut)[4], f32x4 (&oq)[4])
        __attribute__((always_inline)) {
        f32x4 ar[2], aq[2];
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            ar[m2] = f32x4{vv[m2][0], vv[m2][1], vv[m2][2], vv[m2][3]};
            aq[m2] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                ar[m2] = mmh(fa[m2][kb], sh[kb], ar[m2]);
                if constexpr (OUT) aq[m2] = mmh(qa[m2][kb], sh[kb], aq[m2]);
            }
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                ar[m2] = mmh(fa[m2][kb], sl[kb], ar[m2]);
                if constexpr (OUT) aq[m2] = mmh(qa[m2][kb], sl[kb], aq[m2]);
            }
        }
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            ut[2 * mh + m2] = ar[m2];
            oq[2 * mh + m2] = aq[m2];
        }
    };
    // A_qk fragments for token tiles 2half, 2half + 1
    auto load_a = [&](int half, f16x8 (&ah)[2][2], f16x8 (&al)[2][2]) __attribute__((always_inline)) {
        if constexpr (OUT) {
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                const int mt = 2 * half + m2;
#pragma unroll
                for (int kb = 0; kb <= half; ++kb) {
                    ah[m2][kb] = s.r.aqk[0][tri_block(mt, kb)][l];
                    al[m2][kb] = s.r.aqk[1][tri_block(mt, kb)][l];
                }
            }
        }
    };
    // O = (Q^ Gamma) S + A_qk U~ for token tiles 2half, 2half + 1, staged in LDS
    auto step_oa = [&](int half, int buf, const f32x4 (&oq)[4], const f16x8 (&ah)[2][2], const f16x8 (&al)[2][2],
                       const f16x8 (&ub)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            const int mt = 2 * half + m2;
            f32x4 acc = oq[mt];
#pragma unroll
            for (int kb = 0; kb <= half; ++kb) {
                acc = mmh(ah[m2][kb], ub[kb], acc);
                acc = mmh(al[m2][kb], ub[kb], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                stage_out(s.obuf[buf], 16 * mt + 4 * g + i, 16 * w + n, a.scale * acc[i],
                          static_cast<const typename std::conditional<NORM, NormStage, Tout>::type*>(nullptr));
        }
    };
    // operand fragments of the state update for channel tiles 4half .. 4half + 3
    auto load_k = [&](int half, f16x8 (&ka)[4][2], float4 (&gm4)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const int mt = 4 * half + m4;
            ka[m4][0] = s.r.kp[mt][0][l];
            ka[m4][1] = s.r.kp[mt][1][l];
            gm4[m4] = *reinterpret_cast<const float4*>(&s.r.gam[16 * mt + 4 * g]);
        }
    };
    // S <- Diag(gamma) S + (K^ gamma/Gamma)^T U~ for channel tiles 4half .. 4half + 3
    auto step_k = [&](int half, const f16x8 (&ka)[4][2], const float4 (&gm4)[4], const f16x8 (&ub)[2],
                      const f16x8 (&ubl)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const int mt = 4 * half + m4;
            sacc[mt][0] *= gm4[m4].x;
            sacc[mt][1] *= gm4[m4].y;
            sacc[mt][2] *= gm4[m4].z;
            sacc[mt][3] *= gm4[m4].w;
            sacc[mt] = mmh(ka[m4][0], ub[0], sacc[mt]);
            sacc[mt] = mmh(ka[m4][1], ub[1], sacc[mt]);
            if constexpr (SPLIT) {
                sacc[mt] = mmh(ka[m4][0], ubl[0], sacc[mt]);
                sacc[mt] = mmh(ka[m4][1], ubl[1], sacc[mt]);
            }
        }
    };
    // state as fp16 hi/lo B-frags (channel order of the accumulators)
    auto split_state = [&](f16x8 (&sh)[4], f16x8 (&sl)[4]) __attribute__((always_inline)) {
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
    };
    auto load_t = [&](bf16x8 (&th)[6], bf16x8 (&tl)[6]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            th[p] = s.r.tp[0][p][l];
            tl[p] = s.r.tp[1][p][l];
        }
    };
    // U~ = T' R with R as bf16 hi/lo B-frags (token order of the
    // accumulators); the result goes out as fp16 B-frags
    auto step_t = [&](const bf16x8 (&th)[6], const bf16x8 (&tl)[6], f32x4 (&ut)[4], f16x8 (&ub)[2],
                      f16x8 (&ubl)[2]) __attribute__((always_inline)) {
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
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb <= (mt >> 1); ++kb) {
                const int p = tri_block(mt, kb);
                acc = mma3(th[p], tl[p], rbh[kb], rbl[kb], acc);
            }
            ut[mt] = acc;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (SPLIT) {
                    _Float16 hi, lo;
                    splith(ut[2 * kb][i], hi, lo);
                    ub[kb][i] = hi;
                    ubl[kb][i] = lo;
                    splith(ut[2 * kb + 1][i], hi, lo);
                    ub[kb][4 + i] = hi;
                    ubl[kb][4 + i] = lo;
                } else {
                    ub[kb][i] = static_cast<_Float16>(ut[2 * kb][i]);
                    ub[kb][4 + i] = static_cast<_Float16>(ut[2 * kb + 1][i]);
                }
            }
        }
    };

    // Each chunk is software-pipelined inside the wave: the LDS fragments of
    // the next step are requested before the matrix products of the current
    // one, so the LDS and the matrix cores work at the same time (one wave
    // per SIMD: nothing else would hide the LDS latency).  (Q^ Gamma) S rides
    // along with R's dependent chains, and the O and state-update products
    // are left to the scheduler to interleave.
    long prev_c0 = 0, prev2_c0 = 0;
    int prev_L = 0, prev2_L = 0;
    int cur = 0;                          // output norm: obuf buffer of chunk j, (j - jb) mod 3
    float own1 = 0.f, own2 = 0.f;         // output norm: this slice's row sums of chunks j-1, j-2
    // output norm: the other slice's row sum of chunk j-2, requested during
    // the previous iteration (with its record prefetch, so the wait at its
    // commit covers it and nothing waits on it here); the gate rows of chunk
    // j-1, requested the same way; w * sigmoid(gate) of chunk j-2, computed
    // from its rows during the previous iteration
    unsigned long long word2 = 0ull;
    uint4 gcur[2] = {};
    float sw[16] = {};
    for (int j = jb; j < je; ++j) {
        const long c0 = tok0 + static_cast<long>(j) * C;
        const int L = static_cast<int>(min(static_cast<long>(C), tok1 - c0));
        const bool more = j + 1 < je;
        const int buf = NORM ? cur : (j & 1);

        if constexpr (NORM) {
            // first, before this iteration issues any load: chunk j-2 is
            // normalised and stored, chunk j-1's row sums go out (in this
            // order: the other slice reads a word before it can be reused)
            finish(j - 2, cur == 2 ? 0 : cur + 1, prev2_c0, prev2_L, own2, word2, sw, with_out && j >= jb + 2);
            own1 = publish(j - 1, cur == 0 ? 2 : cur - 1, with_out && j > jb);
        }
        f16x8 fa0[2][4], fa1[2][4], qa0[2][4], qa1[2][4];
        float vv0[2][4], vv1[2][4];
        load_r(0, fa0, vv0);
        if constexpr (OUT) load_q(0, qa0);
        if (more) {
            fetch_v(j + 1);
            fetch(j + 1, 0, F1);
        }
        if constexpr (!NORM) {
            if (with_out && j > jb) store_tile(buf ^ 1, prev_c0, prev_L);
        }
        f16x8 sh[4], sl[4];
        split_state(sh, sl);
        __builtin_amdgcn_sched_barrier(0);
        load_r(1, fa1, vv1);
        if constexpr (OUT) load_q(1, qa1);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 ut[4], oq[4];
        step_rq(0, fa0, qa0, vv0, sh, sl, ut, oq);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 th[6], tl[6];
        load_t(th, tl);
        if (more) fetch(j + 1, F1, F2);
        if constexpr (NORM) {
            // the other slice published chunk j-1's sums at the start of its
            // iteration j; they are used at the start of the next iteration
            word2 = poll(j - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // (chunk j-1's gate factors, for the start of the next iteration)
        if constexpr (NORM) gate_scale(gcur, sw);
        step_rq(1, fa1, qa1, vv1, sh, sl, ut, oq);
        __builtin_amdgcn_sched_barrier(0);
        f16x8 ah0[2][2], al0[2][2], ah1[2][2], al1[2][2];
        if constexpr (OUT) {
            load_a(0, ah0, al0);
            load_a(1, ah1, al1);
        }
        __builtin_amdgcn_sched_barrier(0);
        f16x8 ub[2], ubl[2];
        step_t(th, tl, ut, ub, ubl);
        if (more) fetch(j + 1, F2, F3);
        if constexpr (NORM) load_gate(c0, L, gcur);
        __builtin_amdgcn_sched_barrier(0);
        f16x8 ka0[4][2];
        float4 gm0[4];
        load_k(0, ka0, gm0);
        __builtin_amdgcn_sched_barrier(0);
        f16x8 ka1[4][2];
        float4 gm1[4];
        // (the summary launch, two workgroups per CU, keeps fewer
        // fragments in flight)
        if constexpr (OUT) load_k(1, ka1, gm1);
        if (more) fetch(j + 1, F3, RFULL + 1);
        if constexpr (OUT) step_oa(0, buf, oq, ah0, al0, ub);
        step_k(0, ka0, gm0, ub, ubl);
        if constexpr (!OUT) load_k(1, ka1, gm1);
        if constexpr (OUT) step_oa(1, buf, oq, ah1, al1, ub);
        step_k(1, ka1, gm1, ub, ubl);
        __syncthreads();
        // every read of this chunk's record is done: the next one moves in
        if (more) commit();
        prev2_c0 = prev_c0;
        prev2_L = prev_L;
        prev_c0 = c0;
        prev_L = L;
        own2 = own1;
        cur = cur == 2 ? 0 : cur + 1;
        __syncthreads();
    }
    if constexpr (NORM) {
        // the last two chunks: je - 2 (its sums went out and the other
        // slice's were requested in the last iteration), then je - 1
        const int n_run = with_out ? je - jb : 0;
        if (n_run >= 2)
            finish(je - 2, cur == 0 ? 1 : (cur == 1 ? 2 : 0), prev2_c0, prev2_L, own2, word2, sw, true);
        if (n_run >= 1) {
            const int b = cur == 0 ? 2 : cur - 1;
            const float own = publish(je - 1, b, true);
            float sl1[16];
            gate_scale(gcur, sl1);
            finish(je - 1, b, prev_c0, prev_L, own, poll(je - 1), sl1, true);
        }
    } else {
        if (with_out && je > jb) store_tile((je - 1) & 1, prev_c0, prev_L);
    }

    if (sfinal) {
        const size_t sbase = j0 + 16 * w + n;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sfinal[sbase + static_cast<size_t>(16 * mt + 4 * g + i) * DV] = sacc[mt][i];
    }
}

// Phase B of the segmented sequential pass: every segment's initial state,
// in order, from the segments' summaries: S_1 = the state after segment 0,
// S_{s+1} = M_s S_s + B_s ("Kimi K3 の KDA ..." section 2.3.4.1: (A2, b2)
// after (A1, b1) is (A2 A1, A2 b1 + b2)).  One workgroup per (chain,
// 16-column strip of the state): the columns are independent affine systems
// (section 2.3.2).  The products run on the fp32 matrix cores (16x16x4, fp32
// operands and accumulation); wave w computes rows 32w .. 32w + 31.  The
// A operand (M_s) goes from memory straight into registers in the operand
// layout, one segment ahead: product (kk, i) takes channel 16 kk + 4 g + i
// for operand row g, so each lane's 8 values of a row tile are one 16-byte
// load.  The strip S_s is the B operand, from LDS; four independent
// accumulators per wave (row tile x halves of the channels) keep the chain
// of dependent products short.
__global__ void __launch_bounds__(256) seg_combine_kernel(float* __restrict__ seg_states, int P, int nchains)
{
    static_assert(DK == DV, "M_s is stored in a state-shaped block");
    constexpr int SW = 16;                       // columns per workgroup
    constexpr int XLD = SW + 4;                  // LDS row stride of the strip (floats)
    const int chain = blockIdx.x / (DV / SW), c0 = SW * (blockIdx.x % (DV / SW));
    if (chain >= nchains) return;
    float* blocks = seg_states + static_cast<size_t>(chain) * seg_state_blocks(P) * DK * DV;
    auto block = [&](int k) { return blocks + static_cast<size_t>(k) * DK * DV; };
    __shared__ float sx[DK][XLD];
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63, g = l >> 4, n = l & 15;
    // this lane's operand values of M_s: row 32w + 16tt + n, channels
    // 16kk + 4g .. + 3; and its accumulator values of B_s
    float4 ma[2][8];
    f32x4 bq[2];
    auto load = [&](int sg, float4 (&m)[2][8], f32x4 (&b)[2]) __attribute__((always_inline)) {
        const float* Ms = block(seg_block_m(P, sg));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                m[tt][kk] = *reinterpret_cast<const float4*>(Ms + static_cast<size_t>(32 * w + 16 * tt + n) * DV +
                                                             16 * kk + 4 * g);
        const float* Bs = block(seg_block_b(P, sg));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b[tt][i] = Bs[static_cast<size_t>(32 * w + 16 * tt + 4 * g + i) * DV + c0 + n];
    };
    if (P > 2) load(1, ma, bq);
    {
        // S_1: this thread's 8 values of the strip, all loads before the stores
        float x[DK * SW / 256];
#pragma unroll
        for (int u = 0; u < DK * SW / 256; ++u) {
            const int e = t + 256 * u;
            x[u] = block(0)[static_cast<size_t>(e / SW) * DV + c0 + e % SW];
        }
#pragma unroll
        for (int u = 0; u < DK * SW / 256; ++u) {
            const int e = t + 256 * u;
            sx[e / SW][e % SW] = x[u];
            block(seg_block_in(P, 1))[static_cast<size_t>(e / SW) * DV + c0 + e % SW] = x[u];
        }
    }
    for (int sg = 1; sg + 1 < P; ++sg) {
        __syncthreads();   // S_s in LDS
        float4 mn[2][8];
        f32x4 bn[2];
        if (sg + 2 < P) load(sg + 1, mn, bn);
        f32x4 acc[2][2] = {{bq[0], f32x4{0.f, 0.f, 0.f, 0.f}}, {bq[1], f32x4{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float b = sx[16 * kk + 4 * g + i][n];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) acc[tt][kk & 1] = mma32(ma[tt][kk][i], b, acc[tt][kk & 1]);
            }
        __syncthreads();   // every wave has read S_s
        float* out = block(seg_block_in(P, sg + 1));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * w + 16 * tt + 4 * g + i;
                const float y = acc[tt][0][i] + acc[tt][1][i];
                sx[r][n] = y;
                out[static_cast<size_t>(r) * DV + c0 + n] = y;
            }
        if (sg + 2 < P) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                bq[tt] = bn[tt];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) ma[tt][kk] = mn[tt][kk];
            }
        }
    }
}

// Workspace of the matrix-core path: the records, then the packed slot map
// or the state carried between stages (dense), then the output norm's
// row-sum words, then the segment states (dense batches that may take the
// segmented pass).  The sizes cover the largest plan the call can take.
struct TwoPassLayout {
    size_t norm_off, seg_off, total;
};

TwoPassLayout two_pass_layout(int B, int T, int H, int num_seqs, bool packed, bool norm)
{
    const long long slots = chunk_record_slots(B, T, num_seqs, packed);
    const long long chains = static_cast<long long>(packed ? num_seqs : B) * H;
    const int nck = packed ? 0 : (T + C - 1) / C;
    // packed sequences: ceil(T / 64) bounds the chunks of the longest one
    const int nck_max = packed ? (T + C - 1) / C : nck;
    const bool may_segment = plan_segments(nck_max, static_cast<int>(chains), 1 << 20, true) > 1;
    const int pcap = may_segment ? segment_cap(nck_max, static_cast<int>(chains)) : 1;
    TwoPassLayout L;
    L.norm_off = static_cast<size_t>(slots) * H * kChunkRecordBytes;
    L.norm_off += packed ? (static_cast<size_t>(slots) * sizeof(int) + 255) / 256 * 256
                         : static_cast<size_t>(B) * H * DK * DV * sizeof(float);
    const long long units = may_segment ? seg_units_c(pcap) : 1;   // phase C writes o
    L.seg_off = L.norm_off + (norm ? norm_slot_words(chains * units) * sizeof(unsigned long long) : 0);
    L.seg_off = (L.seg_off + 255) / 256 * 256;
    L.total = L.seg_off + (may_segment ? static_cast<size_t>(chains) * seg_state_blocks(pcap) * DK * DV * sizeof(float)
                                       : 0);
    return L;
}

// Workspace of the windowed order: a ring of records for `window` chunks of
// every sequence, the state carried between windows, the output norm's
// row-sum words.
// With seg_p > 0, room for the segmented order inside each window, up to
// seg_p segments: row-sum words for its segment units and the segment states.
struct WindowLayout {
    size_t carry_off, norm_off, seg_off, total;
};

WindowLayout window_layout(int B, int H, int num_seqs, bool packed, bool norm, long long window, int seg_p = 0)
{
    const long long chains = static_cast<long long>(packed ? num_seqs : B) * H;
    WindowLayout L;
    L.carry_off = static_cast<size_t>(window) * chains * kChunkRecordBytes;
    L.norm_off = L.carry_off + static_cast<size_t>(chains) * DK * DV * sizeof(float);
    const long long units = seg_p > 0 ? seg_units_c(seg_p) : 1;
    L.seg_off = L.norm_off + (norm ? norm_slot_words(chains * units) * sizeof(unsigned long long) : 0);
    L.seg_off = (L.seg_off + 255) / 256 * 256;
    L.total = L.seg_off + (seg_p > 0 ? static_cast<size_t>(chains) * seg_state_blocks(seg_p) * DK * DV * sizeof(float)
                                     : 0);
    return L;
}

// Largest window (chunks of every sequence per launch) that fits `bytes`,
// at most `nck` and below 2^24 pass-1 workgroups per launch; 0: none fits.
// With `seg`, room for the segmented order over windows of up to nck chunks.
long long window_chunks(int B, int H, int num_seqs, bool packed, bool norm, int nck, size_t bytes, bool seg = false)
{
    const long long chains = static_cast<long long>(packed ? num_seqs : B) * H;
    const int seg_p = seg && chains <= kMaxSegChains ? segment_cap(nck, static_cast<int>(chains)) : 0;
    const size_t fixed = window_layout(B, H, num_seqs, packed, norm, 0, seg_p).total;
    if (chains <= 0 || bytes < fixed) return 0;
    long long w = static_cast<long long>((bytes - fixed) / (static_cast<size_t>(chains) * kChunkRecordBytes));
    if (w > nck) w = nck;
    const long long cap = ((1LL << 24) - 1) / chains;
    return w < cap ? w : cap;
}

}  // namespace

long long chunk_record_slots(int B, int T, int num_seqs, bool packed)
{
    if (packed) return static_cast<long long>(num_seqs) + T / C;
    return static_cast<long long>(B) * ((T + C - 1) / C);
}

size_t two_pass_workspace_bytes(int B, int T, int H, int num_seqs, bool packed, bool norm)
{
    return two_pass_layout(B, T, H, num_seqs, packed, norm).total;
}

size_t two_pass_min_workspace_bytes(int B, int T, int H, int num_seqs, bool packed, bool norm)
{
    const size_t one = window_layout(B, H, num_seqs, packed, norm, T > 0 ? 1 : 0).total;
    const size_t full = two_pass_workspace_bytes(B, T, H, num_seqs, packed, norm);
    return one < full ? one : full;
}

namespace {

// A short idle gap on the pass-1 stream: the sequential pass of the stage
// that becomes ready together with the next pass-1 launch then takes its CUs
// first (its workgroups need a whole CU each, which the small pass-1
// workgroups would otherwise keep refilling).  About 20 us; always ends.
__global__ void stage_gap_kernel(int naps)
{
    for (int i = 0; i < naps; ++i) __builtin_amdgcn_s_sleep(127);
}

// Whether the staged order may use the context's stream for a call on
// `stream`: same device, and the context's stream is not part of a graph
// capture other than the one `stream` belongs to (a stream that joined a
// capture stays in it until the capture ends; work of an eager call, or of
// another capture, must not land there).  Under capture the fork and the
// join are recorded into the caller's graph.
bool context_usable(kda_context_s* ctx, hipStream_t stream, int dev)
{
    if (!ctx || ctx->device != dev) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone, ss = hipStreamCaptureStatusNone;
    unsigned long long cid = 0, sid = 0;
    if (hipStreamGetCaptureInfo(stream, &cs, &cid) != hipSuccess) return false;
    if (hipStreamGetCaptureInfo(ctx->side, &ss, &sid) != hipSuccess) return false;
    if (cs == hipStreamCaptureStatusInvalidated || ss == hipStreamCaptureStatusInvalidated) return false;
    if (ss == hipStreamCaptureStatusNone) return true;
    return cs == hipStreamCaptureStatusActive && cid == sid;
}

template <bool SIGNED, bool CONV>
void launch_prep(const ChunkArgs& a, ChunkRecord* recs, const int* map, int slots, unsigned groups,
                 hipStream_t stream)
{
    chunk_prep_kernel<SIGNED, CONV><<<groups, NT, 0, stream>>>(a, recs, map, slots);
}

void prep(const ChunkArgs& a, ChunkRecord* recs, const int* map, int slots, unsigned groups, hipStream_t stream)
{
    if (a.signed_alpha && a.conv)
        launch_prep<true, true>(a, recs, map, slots, groups, stream);
    else if (a.signed_alpha)
        launch_prep<true, false>(a, recs, map, slots, groups, stream);
    else if (a.conv)
        launch_prep<false, true>(a, recs, map, slots, groups, stream);
    else
        launch_prep<false, false>(a, recs, map, slots, groups, stream);
}

template <typename Tout, bool CONV>
void launch_scan(const ChunkArgs& a, const ChunkRecord* recs, int slots, unsigned long long* norm_slots, dim3 grid,
                 hipStream_t stream)
{
    if (a.out_norm)
        chunk_scan_kernel<Tout, CONV, true><<<grid, NT, 0, stream>>>(a, recs, slots, norm_slots);
    else
        chunk_scan_kernel<Tout, CONV, false><<<grid, NT, 0, stream>>>(a, recs, slots, nullptr);
}

void scan(const ChunkArgs& a, const ChunkRecord* recs, int slots, int chains, unsigned long long* norm_slots,
          hipStream_t stream)
{
    // ids: chain = 8 * (bid >> 4) + (bid & 7), slice = (bid >> 3) & 1
    const int groups = (chains + 7) / 8;
    const dim3 grid(groups * 8 * NSLICE);
    if (a.seg_phase == 1) {   // summaries of the segmented order: no outputs
        if (a.conv)
            chunk_scan_kernel<uint16_t, true, false, true, false><<<grid, NT, 0, stream>>>(a, recs, slots, nullptr);
        else
            chunk_scan_kernel<uint16_t, false, false, true, false><<<grid, NT, 0, stream>>>(a, recs, slots, nullptr);
        return;
    }
    if (a.conv) {
        if (a.out_bf16)
            launch_scan<uint16_t, true>(a, recs, slots, norm_slots, grid, stream);
        else
            launch_scan<float, true>(a, recs, slots, norm_slots, grid, stream);
    } else {
        if (a.out_bf16)
            launch_scan<uint16_t, false>(a, recs, slots, norm_slots, grid, stream);
        else
            launch_scan<float, false>(a, recs, slots, norm_slots, grid, stream);
    }
}

// The segmented order over the chunk range b.chunk_lo .. + b.chunk_cnt of
// every chain, whose records are in place: phase A, without outputs
// (segment 0 from b.init_state to its end state, the middle segments'
// summaries), phase B (the initial states of segments 1 .. P-1), phase C
// (every segment from its initial state with outputs; the last one ends in
// b.final_state), all on `stream`.
hipError_t run_segments(ChunkArgs b, const ChunkRecord* recs, int slots, int chains, int nseg, float* seg_states,
                        unsigned long long* norm_slots, hipStream_t stream, hipEvent_t before_c = nullptr)
{
    b.seg_count = nseg;
    b.seg_states = seg_states;
    b.seg_phase = 1;
    scan(b, recs, slots, chains * seg_units_a(nseg), norm_slots, stream);
    seg_combine_kernel<<<static_cast<unsigned>(chains * (DV / 16)), 256, 0, stream>>>(seg_states, nseg, chains);
    // phase C also needs what `before_c` marks (the last segment's records)
    if (before_c) {
        const hipError_t e = hipStreamWaitEvent(stream, before_c, 0);
        if (e != hipSuccess) return e;
    }
    b.seg_phase = 2;
    scan(b, recs, slots, chains * seg_units_c(nseg), norm_slots, stream);
    return hipGetLastError();
}

// Segments for a dense range of `nck` chunks per chain on the device of
// `stream` (phase A paired on a CU unless the short convolution runs).
int segments_for(int nck, int chains, bool conv, hipStream_t stream)
{
    if (plan_segments(nck, chains, 1 << 20, true) <= 1) return 1;
    int dev = 0, cus = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 1;
    return plan_segments(nck, chains, cus, !conv);
}

// The overlapped order over stages s = 0 .. n-1 (chunks lo(s) .. lo(s+1)-1
// of every sequence, records at recs_of(s) + h * slots + slot, slots
// addressed with a.rec_stride / a.rec_base as set here or by the caller):
// pass 1 on `stream`, pass 2 on the context's stream, pass 1 of stage s+1
// after pass 2 of stage s-1 (so a ring of two record areas suffices) and
// behind a short gap, so that pass 2 of stage s takes its CUs first.  The
// calling stream joins the context's stream before this returns.  Events
// are reused modulo kMaxStages: each wait is enqueued before its event is
// recorded again.
template <typename Lo, typename RecsOf>
hipError_t run_stages(const ChunkArgs& a, int stages, Lo lo, RecsOf recs_of, int slots, float* carried,
                      unsigned long long* norm_slots, kda_context_s* ctx, hipStream_t stream, bool capturing,
                      bool ring = false)
{
    const int chains = a.B * a.H;
    auto stage_args = [&](int k) {
        ChunkArgs b = a;
        b.chunk_lo = lo(k);
        b.chunk_cnt = lo(k + 1) - lo(k);
        if (ring) b.rec_base = b.chunk_lo;
        b.init_state = k == 0 ? a.init_state : carried;
        b.final_state = k + 1 == stages ? a.final_state : carried;
        return b;
    };
    auto ev1 = [&](int k) { return ctx->p1[k % kMaxStages]; };
    auto ev2 = [&](int k) { return ctx->p2[k % kMaxStages]; };
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t r) { if (e == hipSuccess && r != hipSuccess) e = r; return e == hipSuccess; };
    int launched = -1;   // last stage whose pass 2 is enqueued on the context's stream
    int recorded = -1;   // last stage whose pass-2 completion event is recorded behind it
    {
        const ChunkArgs b = stage_args(0);
        prep(b, recs_of(0), nullptr, slots, static_cast<unsigned>(a.B * b.chunk_cnt * a.H), stream);
    }
    ok(hipGetLastError());
    ok(hipEventRecord(ev1(0), stream));
    for (int k = 0; k < stages && e == hipSuccess; ++k) {
        if (!ok(hipStreamWaitEvent(ctx->side, ev1(k), 0))) break;
        scan(stage_args(k), recs_of(k), slots, chains, norm_slots, ctx->side);
        const hipError_t lr = hipGetLastError();
        if (lr == hipSuccess) launched = k;
        if (!ok(lr)) break;
        if (ok(hipEventRecord(ev2(k), ctx->side))) recorded = k;
        if (k + 1 < stages && e == hipSuccess) {
            // pass 1 of stage k+1 starts with pass 2 of stage k, behind a short gap
            if (k >= 1) ok(hipStreamWaitEvent(stream, ev2(k - 1), 0));
            stage_gap_kernel<<<1, 64, 0, stream>>>(6);
            const ChunkArgs b = stage_args(k + 1);
            prep(b, recs_of(k + 1), nullptr, slots, static_cast<unsigned>(a.B * b.chunk_cnt * a.H), stream);
            ok(hipGetLastError());
            ok(hipEventRecord(ev1(k + 1), stream));
        }
    }
    // join: later work on the caller's stream sees every stage, after an
    // error too, so that nothing on the second stream escapes the caller's
    // stream order
    const StageJoin jn = plan_join(launched, recorded, capturing);
    if (jn.wait_stage >= 0) ok(hipStreamWaitEvent(stream, ev2(jn.wait_stage), 0));
    if (jn.sync_side) ok(hipStreamSynchronize(ctx->side));
    return e;
}

// Whether a dense batch may overlap its two passes on the context's stream,
// and whether `stream` is being captured.
bool overlap_usable(kda_context_s* ctx, hipStream_t stream, int* cus, bool* capturing)
{
    int dev = 0;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (!ctx || hipStreamGetDevice(stream, &dev) != hipSuccess || !context_usable(ctx, stream, dev) ||
        hipStreamIsCapturing(stream, &cap) != hipSuccess ||
        hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    *capturing = cap != hipStreamCaptureStatusNone;
    return true;
}

// The windowed order, for a workspace below the full record area: windows of
// `w` chunks of every sequence, one after the other on `stream` -- pass 1
// writes the window's records into a ring of w chunks per sequence, pass 2
// runs the window's chunks from the state the previous window left (the
// chain's initial state for the first, a 64 KB-per-chain area in between,
// the final state after the last).  The state goes through memory in fp32,
// so the result is bit-identical to the unwindowed two-pass order; memory
// use is independent of T.
hipError_t launch_windowed(const ChunkArgs& args, void* workspace, size_t ws_bytes, hipStream_t stream,
                           kda_context_s* ctx)
{
    const bool packed = args.cu_seqlens != nullptr;
    const int nseq = packed ? args.num_seqs : args.B;
    const int chains = nseq * args.H;
    const int nck = (args.T + C - 1) / C;   // chunks of the longest possible sequence
    const bool norm = args.out_norm != 0;
    // a dense batch of few chains keeps the segmented order inside windows
    // that hold enough chunks for it (and the segment area next to them)
    long long w = 0;
    bool seg = false;
    if (!packed) {
        w = window_chunks(args.B, args.H, args.num_seqs, packed, norm, nck, ws_bytes, true);
        seg = w > 0 && segments_for(static_cast<int>(w), chains, args.conv != 0, stream) > 1;
    }
    if (!seg) w = window_chunks(args.B, args.H, args.num_seqs, packed, norm, nck, ws_bytes);
    if (w < 1) return hipErrorInvalidValue;   // below two_pass_min_workspace_bytes
    const int seg_p = seg ? segment_cap(nck, static_cast<int>(chains)) : 0;
    const WindowLayout lay = window_layout(args.B, args.H, args.num_seqs, packed, norm, w, seg_p);
    char* base = static_cast<char*>(workspace);
    ChunkRecord* recs = reinterpret_cast<ChunkRecord*>(base);
    float* carried = reinterpret_cast<float*>(base + lay.carry_off);
    float* seg_states = seg ? reinterpret_cast<float*>(base + lay.seg_off) : nullptr;
    const int ring = static_cast<int>(nseq * w);   // record slots per head
    unsigned long long* norm_slots = nullptr;
    if (norm) {
        norm_slots = reinterpret_cast<unsigned long long*>(base + lay.norm_off);
        const size_t words = norm_slot_words(static_cast<long long>(chains) * (seg_p > 0 ? seg_units_c(seg_p) : 1));
        const size_t blocks = (words + 255) / 256;
        zero_words_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(norm_slots, words);
    }
    // a dense batch whose sequential pass leaves CUs idle overlaps the two
    // passes as the staged order does, with the ring split in two halves
    // (stage k in half k mod 2)
    int cus = 0;
    bool capturing = false;
    const int half = static_cast<int>(w / 2);
    if (!packed && !seg && half >= kMinRingHalf && stages_may_pay(nck, chains) &&
        overlap_usable(ctx, stream, &cus, &capturing) && cus - 16 * ((chains + 7) / 8) >= 32) {
        ChunkArgs a = args;
        a.rec_stride = half;
        const size_t per_half = static_cast<size_t>(args.H) * nseq * half;   // records
        const int stages = (nck + half - 1) / half;
        return run_stages(a, stages, [&](int k) { return k * half < nck ? k * half : nck; },
                          [&](int k) { return recs + (k & 1) * per_half; }, nseq * half, carried, norm_slots, ctx,
                          stream, capturing, true);
    }
    for (int lo = 0; lo < nck; lo += static_cast<int>(w)) {
        ChunkArgs b = args;
        b.chunk_lo = lo;
        b.chunk_cnt = static_cast<int>(nck - lo < w ? nck - lo : w);
        b.rec_base = lo;
        b.rec_stride = static_cast<int>(w);
        b.init_state = lo == 0 ? args.init_state : carried;
        b.final_state = lo + b.chunk_cnt >= nck ? args.final_state : carried;
        prep(b, recs, nullptr, ring, static_cast<unsigned>(nseq * b.chunk_cnt * args.H), stream);
        const int nseg = seg ? segments_for(b.chunk_cnt, chains, args.conv != 0, stream) : 1;
        if (nseg > 1)
            run_segments(b, recs, ring, chains, nseg, seg_states, norm_slots, stream);
        else
            scan(b, recs, ring, chains, norm_slots, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_chunk_two_pass(const ChunkArgs& args, void* workspace, size_t ws_bytes, hipStream_t stream,
                                 kda_context_s* ctx)
{
    const bool packed = args.cu_seqlens != nullptr;
    const int chains = (packed ? args.num_seqs : args.B) * args.H;
    if (chains == 0) return hipSuccess;
    const long long slots = chunk_record_slots(args.B, args.T, args.num_seqs, packed);
    const TwoPassLayout lay = two_pass_layout(args.B, args.T, args.H, args.num_seqs, packed, args.out_norm != 0);
    if (args.T > 0 && (ws_bytes < lay.total || slots * args.H >= (1LL << 24)))
        return launch_windowed(args, workspace, ws_bytes, stream, ctx);
    const int ns = static_cast<int>(slots);
    ChunkRecord* recs = static_cast<ChunkRecord*>(workspace);
    char* after = static_cast<char*>(workspace) + static_cast<size_t>(slots) * args.H * kChunkRecordBytes;
    const int nck = packed ? 0 : (args.T + C - 1) / C;

    // the segmented order for a batch with few chains (packed sequences:
    // by the longest a sequence can be; each chain splits its own range)
    const int nseg = segments_for(packed ? (args.T + C - 1) / C : nck, chains, args.conv != 0, stream);
    const long long units = nseg > 1 ? seg_units_c(nseg) : 1;

    // output norm: the row-sum words the two value slices of a chain (or of a
    // segment unit) exchange, zeroed by a kernel (no memset node) before any
    // pass 2 of this call
    unsigned long long* norm_slots = nullptr;
    if (args.out_norm) {
        norm_slots = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + lay.norm_off);
        const size_t words = norm_slot_words(chains * units);
        const size_t blocks = (words + 255) / 256;
        zero_words_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(norm_slots, words);
    }

    if (nseg > 1) {
        // pass 1 over every chunk, then the three phases of run_segments
        ChunkArgs b = args;
        int* map = nullptr;
        b.chunk_lo = 0;
        if (packed) {
            map = reinterpret_cast<int*>(after);
            slot_map_kernel<<<static_cast<unsigned>((slots + 255) / 256), 256, 0, stream>>>(
                b.cu_seqlens, b.num_seqs, b.T, ns, map);
            b.chunk_cnt = ns;
        } else {
            b.chunk_cnt = nck;
            b.rec_stride = nck;
            b.rec_base = 0;
        }
        float* seg_states = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.seg_off);
        // Phase A reads the records of segments 0 .. P-2 only: with a
        // usable context, a long dense batch's pass 1 for the last segment
        // runs on the context's stream beside phase A (on the CUs its
        // 2 chains (2P - 3) workgroups leave idle, behind a short gap so that
        // phase A takes its CUs first), and phase C waits for it (64K tokens
        // x 32 heads: 2.82 against 2.98 ms; with less pass-1 work than the
        // staged order needs the gap and the events cost more than it gains:
        // 4096 x 32 heads 0.263 against 0.252 ms).
        const int len = (nck + nseg - 1) / nseg, lo_last = (nseg - 1) * len;
        int cus = 0;
        bool capturing = false;
        if (!packed && lo_last < nck && stages_may_pay(nck, chains) && overlap_usable(ctx, stream, &cus, &capturing) &&
            cus - (args.conv ? 2 : 1) * chains * seg_units_a(nseg) >= 32) {
            ChunkArgs head = b, tail = b;
            head.chunk_cnt = lo_last;
            tail.chunk_lo = lo_last;
            tail.chunk_cnt = nck - lo_last;
            prep(head, recs, nullptr, ns, static_cast<unsigned>(args.B * lo_last * args.H), stream);
            hipError_t e = hipGetLastError();
            if (e == hipSuccess) e = hipEventRecord(ctx->p1[0], stream);
            if (e == hipSuccess) e = hipStreamWaitEvent(ctx->side, ctx->p1[0], 0);
            if (e != hipSuccess) return e;   // nothing of the call is on the context's stream
            stage_gap_kernel<<<1, 64, 0, ctx->side>>>(6);
            prep(tail, recs, nullptr, ns, static_cast<unsigned>(args.B * tail.chunk_cnt * args.H), ctx->side);
            e = hipGetLastError();
            if (e == hipSuccess) e = hipEventRecord(ctx->p2[0], ctx->side);
            if (e != hipSuccess) {
                // no event covers the context's stream: drain it on the host
                // (outside a capture) so nothing of the call outlives it
                if (!capturing) hipStreamSynchronize(ctx->side);
                return e;
            }
            e = run_segments(b, recs, ns, chains, nseg, seg_states, norm_slots, stream, ctx->p2[0]);
            if (e != hipSuccess && !capturing) hipStreamSynchronize(ctx->side);
            return e;
        }
        prep(b, recs, map, ns, static_cast<unsigned>(slots * args.H), stream);
        return run_segments(b, recs, ns, chains, nseg, seg_states, norm_slots, stream);
    }

    // the overlapped schedule for a dense batch, when it pays and the
    // caller's context can carry it
    int bounds[kMaxStages + 1];
    int stages = 1;
    bool capturing = false;
    int cus = 0;
    if (!packed && stages_may_pay(nck, chains) && overlap_usable(ctx, stream, &cus, &capturing))
        stages = plan_stages(nck, chains, cus, bounds);

    ChunkArgs a = args;
    if (!packed) {
        a.rec_stride = nck;
        a.rec_base = 0;
    }
    if (stages == 1) {
        int* map = nullptr;
        if (slots > 0) {
            if (packed) {
                map = reinterpret_cast<int*>(after);
                slot_map_kernel<<<static_cast<unsigned>((slots + 255) / 256), 256, 0, stream>>>(
                    a.cu_seqlens, a.num_seqs, a.T, ns, map);
            }
            a.chunk_lo = 0;
            a.chunk_cnt = packed ? ns : nck;
            prep(a, recs, map, ns, static_cast<unsigned>(slots * a.H), stream);
        }
        a.chunk_lo = 0;
        a.chunk_cnt = packed ? ns : nck;
        scan(a, recs, ns, chains, norm_slots, stream);
        return hipGetLastError();
    }

    // stage s covers chunks bounds[s] .. bounds[s+1] - 1 of every sequence,
    // records in their absolute slots; the state between stages goes
    // through the workspace
    float* carried = reinterpret_cast<float*>(after);
    return run_stages(a, stages, [&](int k) { return bounds[k]; }, [&](int) { return recs; }, ns, carried,
                      norm_slots, ctx, stream, capturing);
}

}  // namespace kda
