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
// The overlapped windowed order needs ring halves of at least this many
// chunks: with smaller stages the gaps and events cost more than the overlap
// gains (the 64K-token, 96-head prefill in a 0.25 GB workspace, halves of 18
// chunks: 7.33 ms overlapped against 7.03 ms one window after the other).
constexpr int kMinRingHalf = 32;

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

// Segmented sequential pass ("Kimi K3 の KDA ..." sections 2.3.4.2-2.3.4.5:
// the map of a sequence is the composition of the affine maps of its
// segments, S -> M S + B, so segments can be summarised apart and combined in
// order).  For a dense batch with few chains the sequential pass occupies few
// CUs; splitting every chain into P segments runs (A), without outputs,
// segment 0 from the initial state and every middle segment 1 .. P-2 twice
// in parallel -- from a zero state with the values (its B) and from the
// identity with zero values (its M) -- then (B) chains the segments' initial
// states S_{s+1} = M_s S_s + B_s, then (C) runs all P segments from their
// initial states with outputs: about 2 segment lengths of sequential chunks
// instead of P.  Phase C needs 2 * chains * P workgroups of one CU each,
// phase A 2 * chains * (2P - 3) output-free ones, which run two per CU
// (`paired`; one per CU with the short convolution, whose registers do not
// fit half a CU), so P = min(floor(cus / (2 chains)),
// floor((w / (2 chains) + 3) / 2)) with w = 2 cus paired or cus, capped by
// segment_cap.  Returns P, or 1 when fewer than 3 segments fit (2 segments
// take as long as the plain pass).
constexpr int kMaxSegments = 32;
constexpr int kMinSegChunks = 16;
constexpr int kMaxSegChains = 42;   // 3 segments of more chains never fit 256 CUs
// segments x chains at most: the segment states a call reserves (3P - 3
// state-sized blocks per chain) stay below 3 * kSegBudget blocks, ~24 MB
constexpr int kSegBudget = 128;

// The most segments `chains` chains of `nck` chunks may take on any device:
// at most kMaxSegments, kSegBudget / chains and segments of at least
// kMinSegChunks chunks.  The workspace reserves for this many.
inline int segment_cap(int nck, int chains)
{
    if (chains <= 0) return 1;
    int p = kMaxSegments;
    if (p > kSegBudget / chains) p = kSegBudget / chains;
    if (p > nck / kMinSegChunks) p = nck / kMinSegChunks;
    return p < 1 ? 1 : p;
}

inline int plan_segments(int nck, int chains, int cus, bool paired)
{
    if (chains <= 0 || chains > kMaxSegChains || nck < 3 * kMinSegChunks) return 1;
    int p = cus / (2 * chains);
    const int pa = ((paired ? 2 * cus : cus) / (2 * chains) + 3) / 2;
    if (p > pa) p = pa;
    const int cap = segment_cap(nck, chains);
    if (p > cap) p = cap;
    return p >= 3 ? p : 1;
}

// Joining the second stream back to the calling stream at the end of a
// staged call.  `launched` is the last stage whose sequential kernel was
// enqueued on the second stream (-1: none), `recorded` the last stage whose
// completion event was recorded right behind it (recorded <= launched).
// When every launched stage has its event, the calling stream waits on the
// last one.  When the event after the last launched stage could not be
// recorded, no event covers that stage: the calling stream still waits on
// the last recorded one, and the second stream is drained on the host
// (outside a graph capture; inside one the capture fails with the error
// anyway), so no kernel of the call outlives it unordered.
struct StageJoin {
    int wait_stage;    // stage whose event the calling stream waits on, -1: none
    bool sync_side;    // synchronise the second stream on the host
};

inline StageJoin plan_join(int launched, int recorded, bool capturing)
{
    StageJoin j{-1, false};
    if (launched < 0) return j;
    j.wait_stage = recorded;
    if (recorded < launched && !capturing) j.sync_side = true;
    return j;
}

}  // namespace kda
