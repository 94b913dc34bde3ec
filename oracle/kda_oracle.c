/*
 * kda_oracle.c -- CPU reference for the Kimi Delta Attention (KDA) forward
 * pass.  TEST INFRASTRUCTURE ONLY: nothing on the product path may link,
 * load or call this file.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.
 *
 * It is the plain definition, written token by token in double precision,
 * with no chunking, blocking or reordering:
 *
 *   per chain (sequence n, head h), S <- S0[n,h] (or 0), for each token t:
 *     q^ = q / sqrt(sum q^2 + eps),  k^ = k / sqrt(sum k^2 + eps)
 *        ("Kimi K3 の KDA ..." page, section 1.2.1: q and k are L2-normalised
 *         per head inside the kernel)
 *     alpha = exp(g)                       (g is the natural-log decay per key
 *        channel: "GDN, KDA の整理", section "Kimi Delta Attention")
 *     S~ = Diag(alpha) S                   (decay first: "Kimi K3 の KDA ..."
 *        section 1.2.1, decay then erase then write; "GDN, KDA の整理"
 *        applies the decay before the gradient step, section "Online learning")
 *     e  = v - S~^T k^                     (innovation: value minus the
 *        decayed state's prediction for k^)
 *     S  = S~ + beta k^ e^T                (erase + write, one gradient step
 *        of rate beta on 1/2 ||S^T k - v||^2)
 *     o_t = scale * S^T q^                 (read AFTER the write: "Kimi K3 の KDA ..."
 *        section 1.2.1: each token reads S_t, not S_{t-1})
 *   final_state[n,h] = S
 *
 * Inputs are fp32 arrays (bf16 tensors widened exactly by the caller) and
 * are widened to double here; outputs are double.
 *
 * Layouts (row-major, contiguous):
 *   q, k, g  [B, T, H, dk]      v, o  [B, T, H, dv]      beta [B, T, H]
 *   init_state (double, nullable => zeros), final_state (double, nullable)
 *              [N, H, dk, dv]
 *   cu_seqlens (nullable): int32 [N+1]; when given, B must be 1 and chain n
 *   covers tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed axis.
 *
 * kda_oracle_forward_signed is the same recurrence with the per-channel
 * decay given directly as alpha (any sign) in place of g, for the Complex KDA
 * range alpha in [-1, 1], beta in [0, 2] ("[논문리뷰] Complex KDA ..." page:
 * the gate range widened to [-1, 1] and beta to [0, 2]; the transition is
 * still (I - beta k^ k^T) Diag(alpha)).
 *
 * Returns 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static void run_chain(int len, int H, int dk, int dv, size_t tok_stride_h,
                      const float* q, const float* k, const float* v, const float* g, int alpha_given,
                      const float* beta, const double* s0, double scale, double eps,
                      int normalize, double* o, double* sT, double* S, double* work)
{
    double* qh = work;
    double* kh = qh + dk;
    double* e  = kh + dk;
    const size_t nS = (size_t)dk * dv;

    if (s0) memcpy(S, s0, nS * sizeof(double));
    else    memset(S, 0, nS * sizeof(double));

    for (int t = 0; t < len; ++t) {
        const float* qt = q + (size_t)t * tok_stride_h * dk;
        const float* kt = k + (size_t)t * tok_stride_h * dk;
        const float* gt = g + (size_t)t * tok_stride_h * dk;
        const float* vt = v + (size_t)t * tok_stride_h * dv;
        const double bt = (double)beta[(size_t)t * tok_stride_h];
        double* ot = o ? o + (size_t)t * tok_stride_h * dv : NULL;

        /* per-head L2 normalisation of q and k */
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; ++i) { sq += (double)qt[i] * qt[i]; sk += (double)kt[i] * kt[i]; }
        const double rq = normalize ? 1.0 / sqrt(sq + eps) : 1.0;
        const double rk = normalize ? 1.0 / sqrt(sk + eps) : 1.0;
        for (int i = 0; i < dk; ++i) { qh[i] = qt[i] * rq; kh[i] = kt[i] * rk; }

        /* decay: row i of S (key channel i) scaled by alpha_i = exp(g_i),
           or by the given signed alpha_i */
        for (int i = 0; i < dk; ++i) {
            const double a = alpha_given ? (double)gt[i] : exp((double)gt[i]);
            double* Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) Si[j] *= a;
        }
        /* innovation e = v - S~^T k^ */
        for (int j = 0; j < dv; ++j) e[j] = (double)vt[j];
        for (int i = 0; i < dk; ++i) {
            const double* Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) e[j] -= Si[j] * kh[i];
        }
        /* erase + write: S = S~ + beta k^ e^T */
        for (int i = 0; i < dk; ++i) {
            double* Si = S + (size_t)i * dv;
            const double c = bt * kh[i];
            for (int j = 0; j < dv; ++j) Si[j] += c * e[j];
        }
        /* read after write: o = scale * S^T q^ */
        if (ot) {
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                const double* Si = S + (size_t)i * dv;
                for (int j = 0; j < dv; ++j) ot[j] += Si[j] * qh[i];
            }
            for (int j = 0; j < dv; ++j) ot[j] *= scale;
        }
    }
    if (sT) memcpy(sT, S, nS * sizeof(double));
}

static int forward(int B, int T, int H, int dk, int dv,
                   int num_seqs, const int32_t* cu_seqlens,
                   const float* q, const float* k, const float* v,
                   const float* g, int alpha_given, const float* beta,
                   const double* init_state, double scale, double eps, int normalize,
                   double* o, double* final_state, int num_threads)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !beta) return -1;
    const int N = cu_seqlens ? num_seqs : B;
    if (cu_seqlens) {
        if (B != 1 || num_seqs < 0) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    }
    const long nchains = (long)N * H;
    const size_t nS = (size_t)dk * dv;
    int ok = 1;

#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel
#endif
    {
        double* S = (double*)malloc(nS * sizeof(double));
        double* work = (double*)malloc((size_t)(2 * dk + dv) * sizeof(double));
        if (!S || !work) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            ok = 0;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (long c = 0; c < nchains; ++c) {
                const int n = (int)(c / H), h = (int)(c % H);
                size_t tok0;   /* first token on the (b, t) axes, flattened */
                int len;
                if (cu_seqlens) { tok0 = (size_t)cu_seqlens[n]; len = cu_seqlens[n + 1] - cu_seqlens[n]; }
                else            { tok0 = (size_t)n * T;         len = T; }
                const size_t base = tok0 * H + h;   /* token-head index */
                run_chain(len, H, dk, dv, (size_t)H,
                          q + base * dk, k + base * dk, v + base * dv, g + base * dk, alpha_given, beta + base,
                          init_state ? init_state + (size_t)c * nS : NULL,
                          scale, eps, normalize,
                          o ? o + base * dv : NULL,
                          final_state ? final_state + (size_t)c * nS : NULL, S, work);
            }
        }
        free(S);
        free(work);
    }
    return ok ? 0 : -1;
}

int kda_oracle_forward(int B, int T, int H, int dk, int dv,
                       int num_seqs, const int32_t* cu_seqlens,
                       const float* q, const float* k, const float* v,
                       const float* g, const float* beta,
                       const double* init_state, double scale, double eps, int normalize,
                       double* o, double* final_state, int num_threads)
{
    return forward(B, T, H, dk, dv, num_seqs, cu_seqlens, q, k, v, g, 0, beta, init_state, scale, eps,
                   normalize, o, final_state, num_threads);
}

int kda_oracle_forward_signed(int B, int T, int H, int dk, int dv,
                              int num_seqs, const int32_t* cu_seqlens,
                              const float* q, const float* k, const float* v,
                              const float* alpha, const float* beta,
                              const double* init_state, double scale, double eps, int normalize,
                              double* o, double* final_state, int num_threads)
{
    return forward(B, T, H, dk, dv, num_seqs, cu_seqlens, q, k, v, alpha, 1, beta, init_state, scale, eps,
                   normalize, o, final_state, num_threads);
}

int kda_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
