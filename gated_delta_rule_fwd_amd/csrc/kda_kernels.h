// kda_kernels.h -- internal launch functions behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_stage_plan.h"

// The objects behind a kda_context (include/kda.h): made by
// kda_context_create, released by kda_context_destroy, owned by the caller.
struct kda_context_s {
    int device;                          // device the stream and events belong to
    hipStream_t side;                    // second stream of the staged prefill (default priority)
    hipEvent_t p1[kda::kMaxStages];      // chunk-parallel kernel of stage s done (calling stream)
    hipEvent_t p2[kda::kMaxStages];      // sequential kernel of stage s done (second stream)
};

namespace kda {

// Problem description shared by the chunkwise launchers.
struct ChunkArgs {
    int B, T, H, dk, dv, num_seqs;
    bool in_bf16, out_bf16;
    float scale;
    int normalize;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* init_state;
    const int32_t* cu_seqlens;
    void* o;
    float* final_state;
    // gated entry point: g is computed from z (in_dtype, [tokens, H, d_k]),
    // A_log [H] and dt_bias [H, d_k] (nullable) instead of being read
    const void* z;
    const float* A_log;
    const float* dt_bias;
    int gated;
    int beta_logits;    // beta holds logits; the kernels apply the sigmoid
    int signed_alpha;   // g holds the signed decay alpha (Complex KDA), not its log
    // output norm: o <- o / sqrt(mean(o^2) + norm_eps) * norm_w * sigmoid(out_gate)
    // per (token, head) over d_v; out_gate in in_dtype [tokens, H, d_v],
    // norm_w [d_v] fp32 (nullable: ones)
    const void* out_gate;
    const float* norm_w;
    float norm_eps;
    int out_norm;
    // short convolution + SiLU on q, k, v (index 0, 1, 2): taps [H*d, 4]
    // fp32 and conv states [N, 3, H*d] in in_dtype (nullable: zeros)
    const float* conv_w[3];
    const void* conv_init[3];
    int conv;
    // matrix-core path: the chunks each launch covers in every chain
    // (chunk_lo .. chunk_lo + chunk_cnt - 1; set by launch_chunk_two_pass)
    int chunk_lo, chunk_cnt;
    // record of chunk j of sequence n: slot n * rec_stride + (j - rec_base)
    // (dense batches always; packed sequences when rec_stride > 0, the
    // windowed order); packed sequences with rec_stride == 0 start at slot
    // n + cu_seqlens[n]/64 and pass 1 finds its sequence in the slot map
    int rec_stride, rec_base;
    // segmented sequential pass (plan_segments in kda_stage_plan.h): 0 = off;
    // 1 = phase A, no outputs, 2P - 3 units per chain: (chain, 0) = segment 0
    // from the initial state, (chain, 2s - 1) / (chain, 2s) = segment s
    // (1 .. P-2) from zero with the values / from the identity with zero
    // values; 2 = phase C, P units: (chain, s) = segment s from its initial
    // state with outputs.  seg_states holds per chain
    // seg_state_blocks(seg_count) blocks of d_k x d_v fp32 (see there).
    int seg_phase, seg_count;
    float* seg_states;
};

// Blocks of a chain's segment states: 0 = state after segment 0, 1 .. P-2 =
// B_s, P-1 .. 2P-4 = M_s (s = 1 .. P-2), 2P-3 .. 3P-5 = initial state of
// segment s = 1 .. P-1, 3P-4 = a copy of the chain's initial state, taken by
// phase A, from which phase C starts segment 0: phase C's last segment writes
// the final state in the same launch, and the caller's initial state may
// alias its final state (a window's carried state always does).
constexpr int seg_state_blocks(int P) { return 3 * P - 3; }
constexpr int seg_block_b(int P, int s) { return s; }
constexpr int seg_block_m(int P, int s) { return P - 2 + s; }
constexpr int seg_block_in(int P, int s) { return 2 * P - 4 + s; }
constexpr int seg_block_init(int P) { return 3 * P - 4; }
constexpr int seg_units_a(int P) { return 2 * P - 3; }
constexpr int seg_units_c(int P) { return P; }

// Inputs of one decode step; z/A_log/dt_bias replace g when gated.
struct DecodeArgs {
    int dk, dv, chains, H;
    bool in_bf16, out_bf16;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* o;
    float scale;
    int normalize;
    const void* z;
    const float* A_log;
    const float* dt_bias;
    int gated;
    int beta_logits;
    int signed_alpha;
    const void* out_gate;   // output norm, as in ChunkArgs ([chains, d_v])
    const float* norm_w;
    float norm_eps;
    int out_norm;
    // short convolution: taps, the conv states read ([N, 3, H*d], nullable:
    // zeros) and where the shifted states go (nullable: not kept; may alias)
    const float* conv_w[3];
    const void* conv_init[3];
    void* conv_final[3];
    int conv;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// fp32 per-position-pair path: any supported head dims and dtypes.
hipError_t launch_chunk_fp32(const ChunkArgs& a, hipStream_t stream);

// Output norm, one wave per (token, head) row of d_v: a.o <- x / sqrt(mean(x^2)
// + a.norm_eps) * a.norm_w * sigmoid(a.out_gate) with x the fp32 output of the
// forward pass (a.o itself when a.o is fp32).  The prefill paths run it after
// the forward pass, since their workgroups hold only a slice of each row.
hipError_t launch_out_norm(const ChunkArgs& a, const float* x, hipStream_t stream);

// Matrix-core path: bf16 inputs, d_k = d_v = 128, g >= -5, in two passes.
//   pass 1 (chunk-parallel): every (chunk, head) writes one ChunkRecord of
//          chunk-local operands to the workspace;
//   pass 2 (sequential over chunks): carries the state through the records.
// Record slots: a dense batch uses B * ceil(T/64) slots per head (sequence b,
// chunk j -> slot b * ceil(T/64) + j); packed sequences use num_seqs + T/64
// slots, sequence n starting at slot n + cu_seqlens[n]/64 (a chunk count of
// ceil(len/64) never reaches the next sequence's first slot).
constexpr size_t kChunkRecordBytes = 74240;
long long chunk_record_slots(int B, int T, int num_seqs, bool packed);
// workspace: records (h * slots + slot), then one int32 per slot naming its
// sequence or -1 (packed sequences) or the fp32 state of every chain
// [B*H, 128, 128] carried between the overlapped launches (dense batch).
// With the output norm (`norm`), the pass-2 workgroups of the two value
// slices of a chain exchange per-row sums of o^2 through 2 KB per chain after
// that, and o is normalised as it is stored.
size_t two_pass_workspace_bytes(int B, int T, int H, int num_seqs, bool packed, bool norm);
// The least workspace the path runs with: records for one chunk of every
// sequence, the carried state and the norm's words (the windowed order;
// independent of T).  Any size from this up works: below
// two_pass_workspace_bytes() the chunks go in windows as large as fit.
size_t two_pass_min_workspace_bytes(int B, int T, int H, int num_seqs, bool packed, bool norm);
// With a context (nullable), a dense batch whose sequential pass leaves CUs
// idle runs in stages: pass 1 of stage s+1 on the idle CUs while pass 2 of
// stage s runs, pass 2 on the context's stream, joined to `stream` before
// returning.  A batch of at most 42 chains with at least 48 chunks per
// sequence (packed: ceil(T/64)) takes the segmented order instead
// (plan_segments).  Otherwise (no
// context, a context of another device or one whose stream belongs to
// another graph capture, packed sequences, short chains, many chains) pass 1
// then pass 2 on `stream`.  With ws_bytes below two_pass_workspace_bytes()
// (or more (chunk, head) records than one launch takes) the windowed order
// runs instead, on `stream`.  The staged, windowed and plain orders give the
// same bits; the segmented order differs from them by rounding.
hipError_t launch_chunk_two_pass(const ChunkArgs& a, void* workspace, size_t ws_bytes, hipStream_t stream,
                                 kda_context_s* ctx);

// Conv states after a prefill: the last 3 raw inputs of every sequence for
// q, k, v (rows from a.conv_init where a sequence is shorter than 3); each
// thread reads all three source rows of its (sequence, channel) before
// writing, so final may alias a.conv_init.
hipError_t launch_conv_final(const ChunkArgs& a, void* const final_state[3], hipStream_t stream);

// Device-side range checks for KDA_FLAG_VALIDATE; counts violations into
// counters[0..2] (g, beta, cu_seqlens); the launcher zeroes them first with
// a fill kernel (no memset node, so the call stays capturable).
hipError_t launch_validate(const ChunkArgs& a, unsigned int* counters, hipStream_t stream);

}  // namespace kda
