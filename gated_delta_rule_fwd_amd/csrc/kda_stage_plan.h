// kda_stage_plan.h -- the chunk stages of the overlapped two-pass prefill
// (host code only; included by kda_chunk_two_pass.hip and by a host test).
//
// Pass 2 runs one workgroup per CU on 16 * ceil(chains / 8) CUs and is bound
// by the latency of its per-chunk steps; pass 1 of the next stage can run on
// the CUs it leaves idle.  These functions choose the stages.
#pragma once

namespace kda {

constexpr int kMaxStages = 6;
constexpr int kMinStageChunks = 16;

// With less pass-1 work than ~8K (chunk, chain) pairs the extra launches and
// the gaps cost more than the overlap gains (+5 % on 4096-token prefills at
// 24 and 32 heads, +2 % at 16K tokens and 16 heads).
inline bool stages_may_pay(int nck, int chains)
{
    return nck >= 256 && static_cast<long>(nck) * chains >= 8192;
}

// Chunk ranges of the overlapped schedule: bounds[0] = 0 < ... < bounds[n] =
// nck; returns n (1 = no overlap).  Stage s+1's pass 1 runs on the CUs that
// stage s's pass 2 leaves idle and should take no longer than it, so stage
// sizes follow n_{s+1} = n_s / rho with rho = (pass-1 time of one chunk of
// every chain on the idle CUs) / (pass-2 time of one chunk).  The unit costs
// are measured on the 64K-token, 96-head prefill: ~6.3 us of one CU per
// (chunk, head) for pass 1 on CUs it has to itself, ~3.4 us per chunk for
// pass 2 while pass 1 runs beside it.
inline int plan_stages(int nck, int chains, int cus, int* bounds)
{
    bounds[0] = 0;
    bounds[1] = nck;
    const int wg2 = 16 * ((chains + 7) / 8);       // pass-2 workgroups, one CU each
    const int idle = cus - wg2;
    if (!stages_may_pay(nck, chains) || idle < 32) return 1;
    const double rho = chains * 6.3 / idle / 3.4;
    const double grow = 1.0 / rho;
    double sum = 0.0, term = 1.0;
    for (int k = 0; k < kMaxStages; ++k, term *= grow) sum += term;
    int n = 0, done = 0;
    double size = static_cast<double>(nck) / sum;
    while (done < nck) {
        int take = static_cast<int>((size < nck ? size : nck) + 0.5);
        if (take < kMinStageChunks) take = kMinStageChunks;
        const int left = nck - done;
        if (take > left || left - take < kMinStageChunks || n + 1 == kMaxStages) take = left;
        done += take;
        bounds[++n] = done;
        size = take * grow;
    }
    return n;
}

}  // namespace kda
