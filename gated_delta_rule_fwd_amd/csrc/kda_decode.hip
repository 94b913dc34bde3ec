// kda_decode.hip -- fused single-token recurrent step (decode) for gfx950.
//
// Per chain (n, h), with the state S (d_k x d_v fp32, row i = key channel i):
//   q^, k^ = L2-normalised q, k ("Kimi K3 の KDA ..." section 1.2.1)
//   S~ = Diag(exp g) S                              (decay first)
//   p  = S~^T k^,  r = S~^T q^                      (two reductions over d_k)
//   u  = beta (v - p)                               (innovation times rate)
//   S  <- S~ + k^ u^T                               (erase + write, in place)
//   o  = scale * (r + (k^ . q^) u)  == scale * S_new^T q^  (read after write)
//   optional output norm: o <- o / sqrt(mean(o^2) + eps) * w * sigmoid(gate)
//   optional short convolution: q, k, v = silu(causal width-4 conv) of the
//   raw inputs with the 3 cached ones, the cache shifting by one token
// ("Kimi K3 模型结构（2）", Q&A: decode runs this recurrent form one token at a
// time.)
//
// The step is a pure stream over the state: 2 * 4 * d_k * d_v bytes per
// chain against ~7 d_k d_v flops, so it is HBM-bound.  One workgroup of 256
// threads owns one chain; each thread keeps RPT rows x 4 columns of S in
// registers between the reductions and the store, so S is read once and
// written once with 16-byte accesses, and both reductions share the one pass
// (o is rebuilt from S~^T q^ instead of re-reading S_new).
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {

// One token of the short convolution for channel col of sequence n: the 3
// cached inputs (rows 3n .. 3n + 2 of a [N, 3, width] state, oldest first;
// zero without a state) and x; the state shifts by one, written by the same
// thread that read it, so it may be updated in place.
template <typename Tin>
__device__ __forceinline__ float decode_conv(float x, const Tin* init, Tin* fin, const float* w, size_t row0,
                                             size_t width, size_t col)
{
    float c0 = 0.f, c1 = 0.f, c2 = 0.f;
    if (init) {
        c0 = Elem<Tin>::load(init, row0 * width + col);
        c1 = Elem<Tin>::load(init, (row0 + 1) * width + col);
        c2 = Elem<Tin>::load(init, (row0 + 2) * width + col);
    }
    const float4 wt = *reinterpret_cast<const float4*>(w + 4 * col);
    const float y = silu(wt.x * c0 + wt.y * c1 + wt.z * c2 + wt.w * x);
    if (fin) {
        Elem<Tin>::store(fin, row0 * width + col, c1);
        Elem<Tin>::store(fin, (row0 + 1) * width + col, c2);
        Elem<Tin>::store(fin, (row0 + 2) * width + col, x);
    }
    return y;
}

template <int DK, int DV, typename Tin, typename Tout>
__global__ void __launch_bounds__(256)
decode_step_kernel(DecodeArgs a)
{
    const Tin* __restrict__ q = static_cast<const Tin*>(a.q);
    const Tin* __restrict__ k = static_cast<const Tin*>(a.k);
    const Tin* __restrict__ v = static_cast<const Tin*>(a.v);
    const float* __restrict__ g = a.g;
    const float* __restrict__ beta = a.beta;
    float* __restrict__ state = a.state;
    Tout* __restrict__ o = static_cast<Tout*>(a.o);
    const float scale = a.scale;
    const int normalize = a.normalize;
    constexpr int CG = DV / 4;        // float4 column groups
    constexpr int RG = 256 / CG;      // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(RPT >= 1 && DK % RG == 0, "shape");

    const int c = blockIdx.x;         // chain = n * H + h
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const int lane = t & 63, wave = t >> 6;

    float4* S4 = reinterpret_cast<float4*>(state + static_cast<size_t>(c) * DK * DV);

    // Issue the state loads first so their latency overlaps the vector work.
    // The state streams through once per step: non-temporal loads and stores
    // keep it from displacing other data in the caches (-6 % per step).
    float4 s[RPT];
    typedef float nf4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const nf4 x = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(&S4[(rg + RG * m) * CG + cg]));
        s[m] = make_float4(x.x, x.y, x.z, x.w);
    }

    __shared__ float sq[DK], sk[DK], sa[DK], sv[DV];
    __shared__ float red[2][4][DV];
    __shared__ float sdot;

    if (wave == 0) {
        constexpr int PER = DK / 64;
        float qv[PER], kv[PER], ss_q = 0.f, ss_k = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int i = lane + 64 * e;
            qv[e] = Elem<Tin>::load(q, static_cast<size_t>(c) * DK + i);
            kv[e] = Elem<Tin>::load(k, static_cast<size_t>(c) * DK + i);
            if (a.conv) {   // silu(causal width-4 conv) with the cached inputs
                const int n = c / a.H, h = c % a.H;
                const size_t col = static_cast<size_t>(h) * DK + i, width = static_cast<size_t>(a.H) * DK;
                qv[e] = decode_conv(qv[e], static_cast<const Tin*>(a.conv_init[0]), static_cast<Tin*>(a.conv_final[0]),
                                    a.conv_w[0], 3 * static_cast<size_t>(n), width, col);
                kv[e] = decode_conv(kv[e], static_cast<const Tin*>(a.conv_init[1]), static_cast<Tin*>(a.conv_final[1]),
                                    a.conv_w[1], 3 * static_cast<size_t>(n), width, col);
            }
            float gi;
            if (a.gated) {   // bounded decay map of the gated entry point
                const int h = c % a.H;
                gi = gate_log_decay(Elem<Tin>::load(static_cast<const Tin*>(a.z), static_cast<size_t>(c) * DK + i),
                                    a.dt_bias ? a.dt_bias[h * DK + i] : 0.f, __expf(a.A_log[h]));
            } else {
                gi = g[static_cast<size_t>(c) * DK + i];
            }
            // Complex KDA passes the signed decay alpha itself
            sa[i] = a.signed_alpha ? gi : __expf(gi);
            ss_q += qv[e] * qv[e];
            ss_k += kv[e] * kv[e];
        }
        float rq = 1.f, rk = 1.f;
        if (normalize) {
            rq = rsqrtf(wave_sum(ss_q) + kNormEps);
            rk = rsqrtf(wave_sum(ss_k) + kNormEps);
        }
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int i = lane + 64 * e;
            sq[i] = qv[e] * rq;
            sk[i] = kv[e] * rk;
            dot += (qv[e] * rq) * (kv[e] * rk);
        }
        dot = wave_sum(dot);
        if (lane == 0) sdot = dot;
#pragma unroll
        for (int e = 0; e < DV / 64; ++e) {
            const int j = lane + 64 * e;
            float vj = Elem<Tin>::load(v, static_cast<size_t>(c) * DV + j);
            if (a.conv) {
                const int n = c / a.H, h = c % a.H;
                vj = decode_conv(vj, static_cast<const Tin*>(a.conv_init[2]), static_cast<Tin*>(a.conv_final[2]),
                                 a.conv_w[2], 3 * static_cast<size_t>(n), static_cast<size_t>(a.H) * DV,
                                 static_cast<size_t>(h) * DV + j);
            }
            sv[j] = vj;
        }
    }
    __syncthreads();

    // decay in registers, then partial reductions over this thread's rows
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const float a = sa[i], kk = sk[i], qq = sq[i];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        p[0] += kk * s[m].x; p[1] += kk * s[m].y; p[2] += kk * s[m].z; p[3] += kk * s[m].w;
        r[0] += qq * s[m].x; r[1] += qq * s[m].y; r[2] += qq * s[m].z; r[3] += qq * s[m].w;
    }
    // reduce across the row groups that share this wave
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] += __shfl_xor(p[e], off, 64);
            r[e] += __shfl_xor(r[e], off, 64);
        }
    }
    if (lane < CG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            red[0][wave][4 * cg + e] = p[e];
            red[1][wave][4 * cg + e] = r[e];
        }
    }
    __syncthreads();

    const float b = a.beta_logits ? beta_from_logit(beta[c]) : beta[c];
    const float dot = sdot;
    float u[4], ov[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * cg + e;
        const float pj = red[0][0][j] + red[0][1][j] + red[0][2][j] + red[0][3][j];
        const float rj = red[1][0][j] + red[1][1][j] + red[1][2][j] + red[1][3][j];
        const float vj = sv[j];
        u[e] = b * (vj - pj);
        ov[e] = scale * (rj + dot * u[e]);
    }

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const float kk = sk[i];
        float4 w;
        w.x = s[m].x + kk * u[0];
        w.y = s[m].y + kk * u[1];
        w.z = s[m].z + kk * u[2];
        w.w = s[m].w + kk * u[3];
        const nf4 wv = {w.x, w.y, w.z, w.w};
        __builtin_nontemporal_store(wv, reinterpret_cast<nf4*>(&S4[i * CG + cg]));
    }
    if (rg == 0) {
        if (a.out_norm) {
            // output norm over the d_v columns, held by the CG lanes of wave 0
            float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
            for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off, 64);
            const float rs = rsqrtf(ss * (1.f / DV) + a.norm_eps);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * cg + e;
                const float gt = Elem<Tin>::load(static_cast<const Tin*>(a.out_gate), static_cast<size_t>(c) * DV + j);
                ov[e] = ov[e] * rs * (a.norm_w ? a.norm_w[j] : 1.f) / (1.f + __expf(-gt));
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) Elem<Tout>::store(o, static_cast<size_t>(c) * DV + 4 * cg + e, ov[e]);
    }
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream)
{
    decode_step_kernel<DK, DV, Tin, Tout><<<dim3(a.chains), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream)
{
    if (a.in_bf16 && a.out_bf16) return launch_decode_t<DK, DV, uint16_t, uint16_t>(a, stream);
    if (a.in_bf16) return launch_decode_t<DK, DV, uint16_t, float>(a, stream);
    if (a.out_bf16) return launch_decode_t<DK, DV, float, uint16_t>(a, stream);
    return launch_decode_t<DK, DV, float, float>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    if (a.dk == 128 && a.dv == 128) return launch_decode_d<128, 128>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch_decode_d<128, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch_decode_d<64, 128>(a, stream);
    return launch_decode_d<64, 64>(a, stream);
}

}  // namespace kda
