/*
 * kda.h -- C ABI of libkda.so: the Kimi Delta Attention (KDA) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (one chain per (sequence n, head h), state S in R^{d_k x d_v}):
 *
 *   q^_t = scale-free L2 normalisation of q_t over d_k, likewise k^_t
 *   S_t  = (I - beta_t k^_t k^_t^T) Diag(exp g_t) S_{t-1} + beta_t k^_t v_t^T
 *   o_t  = scale * S_t^T q^_t
 *
 * Sources (cited by page title and section):
 *   - "Kimi K3 の KDA が Gated MLA と AttnRes との連携を解説", section 1.2.1:
 *     q and k are L2-normalised per head inside the kernel; the recurrence is
 *     decay -> erase -> write; each token reads the state after its own
 *     write; beta is a per-head fp32 scalar; recurrence quantities stay fp32.
 *   - "GDN, KDA の整理", section "Kimi Delta Attention": the update rule with
 *     D_t = Diag(alpha_t) and S_t in R^{d_k x d_v}, o_t = S_t^T q_t; the
 *     bounded log-decay -5 < g < 0.
 *   - "Kimi K3 模型结构（2）：序列维度（下）", Q&A: the chunkwise form (C = 64,
 *     WY representation + UT transform) serves training and prefill, the
 *     recurrent form serves one-token decode; the caller picks the mode.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous in
 *     the layouts given below; beta and cu_seqlens must be 4-byte aligned,
 *     every other tensor 16-byte aligned.  The caller owns every buffer;
 *     the library allocates no device memory.  HIP streams and events are
 *     created only by kda_context_create (and released by
 *     kda_context_destroy); the caller owns the context and passes it in
 *     the prefill descriptor.  The only state the library keeps between
 *     calls is each calling thread's last HIP error code
 *     (kda_last_hip_error).  Entry points are thread-safe; one context
 *     serves one call at a time (use one per thread).
 *   - Work is enqueued on `stream` and runs asynchronously; there is no host
 *     synchronisation except under KDA_FLAG_VALIDATE (and after a failed
 *     event record, see kda_chunk_fwd).  Work a call puts on the context's
 *     stream is joined back to `stream` (an event wait) before the call
 *     returns, so later work on `stream` sees every output.  Without
 *     KDA_FLAG_VALIDATE a call only launches kernels and records or waits
 *     on events (no memset, copy or allocation), so it may be captured into
 *     a HIP graph and replayed; a staged prefill's fork to the context's
 *     stream and its join are then recorded into the graph.
 *   - Every argument is checked on the host before anything is launched, so a
 *     call that returns an error other than KDA_ERR_HIP / KDA_ERR_RANGE has had
 *     no side effect.
 *   - bf16 is stored as its 16-bit pattern; outputs are rounded to bf16 with
 *     round-to-nearest-even.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_API __attribute__((visibility("default")))

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, misaligned pointer, bad layout,
                                 size above the limits below */
    KDA_ERR_UNSUPPORTED = 2,  /* head dims other than 64/128, unknown dtype or flag */
    KDA_ERR_WORKSPACE = 3,    /* workspace smaller than kda_chunk_fwd_min_workspace_bytes() */
    KDA_ERR_RANGE = 4,        /* only with KDA_FLAG_VALIDATE: g outside [-5, 0], beta outside
                                 [0, 1], or cu_seqlens not a monotone partition of [0, T] */
    KDA_ERR_HIP = 5,          /* a HIP launch/runtime error; see kda_last_hip_error() */
    KDA_ERR_SCRATCH = 6       /* kda_chunk_fwd_noalloc only: the call needs more device scratch
                                 than its fixed area of KDA_NOALLOC_SCRATCH_BYTES, even in
                                 the windowed order */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* q and k are L2-normalised over d_k inside the kernel (eps = 1e-6 under the
 * square root).  Mirrors the model's use_qk_l2norm_in_kernel switch ("Kimi K3
 * の KDA ..." section 1.2.1).  Without it q and k are used as given. */
#define KDA_FLAG_QK_L2NORM 0x1u
/* Debug: before the forward pass, check on the device that every g is in
 * [-5, 0], every beta in [0, 1] and that cu_seqlens is monotone from 0 to T;
 * synchronises the stream and returns KDA_ERR_RANGE on failure (nothing else
 * is written then).  Needs kda_chunk_fwd_workspace_bytes() bytes of workspace. */
#define KDA_FLAG_VALIDATE 0x2u
/* Use the fp32 (per-position-pair) arithmetic path even for bf16 inputs. */
#define KDA_FLAG_FP32_PATH 0x4u
/* beta holds write-strength logits; the kernel applies the sigmoid, as the
 * model does in-kernel ("Kimi K3 の KDA ..." section 1.2.1: beta is a per-head
 * fp32 scalar passed through a sigmoid inside the kernel).  Accepted by every prefill and
 * decode entry point. */
#define KDA_FLAG_BETA_LOGITS 0x8u
/* Complex KDA ("[논문리뷰] Complex KDA ..." page: the gate range widened to
 * [-1, 1] and beta to [0, 2]): the g argument holds the signed per-channel
 * decay alpha itself instead of its logarithm, and beta may lie in [0, 2].
 * The transition stays (I - beta k^ k^T) Diag(alpha).  Prefill requires
 * exp(-5) <= |alpha| <= 1 (the bounded-decay range of the chunk kernels;
 * checked under KDA_FLAG_VALIDATE).  Not combinable with the gated entry
 * points. */
#define KDA_FLAG_SIGNED_ALPHA 0x10u
/* The call carries an output norm (kda_out_norm below).  Must be set exactly
 * when a norm is passed to kda_chunk_fwd_fused / kda_recurrent_step_fused.
 * It is part of the descriptor so that kda_chunk_fwd_workspace_bytes() can
 * size what the norm needs: on the matrix-core path 8 bytes per (row of a
 * 64-token chunk, value slice, slot) for the row sums the two value slices
 * of a chain exchange; on the fp32 path with a bf16 o the fp32 staging of o,
 * since the norm runs as a second kernel there and must see o before it is
 * rounded. */
#define KDA_FLAG_OUT_NORM 0x20u


/* Size limits (a larger call returns KDA_ERR_INVALID_ARG before any launch):
 * prefill B*T*H <= 2^31 token-heads and N*H <= 2^22 chains; decode N*H
 * <= 2^24 - 1 chains.  They come from the 2^32 work items one grid dimension
 * takes; every device index is 64-bit.  A matrix-core prefill with 2^24 or
 * more (64-token chunk, head) pairs runs in the windowed order (see
 * kda_chunk_fwd_min_workspace_bytes), whatever its workspace. */

/*
 * Caller-owned objects with which a long dense prefill overlaps its two
 * kernels: one HIP stream (non-blocking, default priority) and twelve events
 * (timing disabled) on the device that was current when it was created.
 * Nothing else in the library creates a stream or an event.
 */
typedef struct kda_context_s* kda_context;

/* Creates a context on the calling thread's current device.  Returns
 * KDA_ERR_INVALID_ARG for a null `ctx`, KDA_ERR_HIP when the runtime fails
 * (then nothing is left allocated and *ctx is NULL). */
KDA_API kda_status kda_context_create(kda_context* ctx);

/* Releases a context (NULL is a no-op).  No call that uses it may still be
 * running on the host; work it enqueued may still be pending on the device
 * (HIP releases the stream and events once it completes). */
KDA_API kda_status kda_context_destroy(kda_context ctx);

typedef struct kda_chunk_desc {
    int B;              /* batch (must be 1 when cu_seqlens is given) */
    int T;              /* tokens per batch row, or total packed tokens when varlen */
    int H;              /* heads */
    int d_k;            /* key/query head dim: 64 or 128 */
    int d_v;            /* value head dim: 64 or 128 */
    int num_seqs;       /* number of packed sequences when cu_seqlens != NULL, else ignored */
    kda_dtype in_dtype;  /* dtype of q, k, v */
    kda_dtype out_dtype; /* dtype of o */
    float scale;        /* output scale (1.0 = the pages' form) */
    unsigned flags;     /* KDA_FLAG_* */
    kda_context context; /* nullable: a context lets a long dense prefill overlap its
                            two kernels on the context's stream (kda_chunk_fwd); NULL
                            runs them one after the other on `stream` */
} kda_chunk_desc;

/* Bytes of device workspace with which the chunkwise entry points run this
 * descriptor in their fastest order.  The matrix-core path (bf16 inputs,
 * d_k = d_v = 128, no KDA_FLAG_FP32_PATH) keeps one 74,240-byte record per
 * (64-token chunk, head) there, plus, for a dense batch, the fp32 state of
 * every (b, h) chain (64 KB each) carried between launches, or, for packed
 * sequences, one int32 per chunk slot (256-byte rounded); KDA_FLAG_OUT_NORM
 * adds 4 KB per chain of row-sum words; a batch of at most 42 chains and at
 * least 48 chunks per sequence (packed: ceil(T/64)), which may take the
 * segmented order,
 * adds 3P - 3 state-sized blocks (64 KB each) per chain and, with
 * KDA_FLAG_OUT_NORM, row-sum words for P segment units per chain, where
 * P = min(32, 128 / chains, chunks / 16) is the most segments the call may
 * take (at most ~23 MB in all).  The fp32 path needs none, except with
 * KDA_FLAG_OUT_NORM and a bf16 o: B*T*H*d_v fp32 values.  KDA_FLAG_VALIDATE
 * adds 256 bytes in front.  When num_seqs > 0 and B == 1 the figure covers
 * both the dense and the packed (cu_seqlens) layout.  Returns 0 for a
 * descriptor the entry points reject and (size_t)-1 for a null
 * descriptor. */
KDA_API size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_desc* desc);

/* The least workspace the chunkwise entry points accept for this descriptor
 * (constant-memory long context).  On the matrix-core path: records for one
 * 64-token chunk of every sequence, the carried states and the norm's words,
 * whatever T is.  A workspace from this size up to
 * kda_chunk_fwd_workspace_bytes() runs the windowed order: windows of as
 * many chunks of every sequence as the records of the workspace hold, pass 1
 * then pass 2 per window on `stream`, the state carried between windows in
 * fp32 ("Kimi K3 模型结构（2）", Q&A on the chunkwise algorithm: one state
 * per chain, updated once per chunk), bit-identical to the unwindowed
 * two-pass order.  Same return convention as kda_chunk_fwd_workspace_bytes. */
KDA_API size_t kda_chunk_fwd_min_workspace_bytes(const kda_chunk_desc* desc);

/*
 * Chunkwise forward for training/prefill ("Kimi K3 模型结构（2）", Q&A on the
 * chunkwise algorithm and on which form each phase uses).  Chunks of 64
 * tokens restart at every sequence start; the last chunk of a sequence may be
 * partial; a zero-length sequence passes its initial state through unchanged.
 *
 * The matrix-core path runs a chunk-parallel kernel and then a sequential
 * one, in one of four orders, picked on the host from the shapes, the
 * workspace size and the context:
 *  - segmented: a batch of at most 42 chains and at least 48 chunks per
 *    sequence (packed sequences: ceil(T/64) chunks), with the full
 *    workspace.  Each chain is cut into P segments of its own chunk range
 *    (3 <= P <= 32, as many as the device's CUs hold and at most 128
 *    segment-chains in all); the middle
 *    segments are summarised as affine maps S -> M S + B and combined
 *    ("Kimi K3 の KDA ..." sections 2.3.4.2-2.3.4.5), then the segments run
 *    again from their true initial states.  On `stream`; with a usable
 *    context a long dense batch runs the chunk-parallel kernel of its last
 *    segment on the context's stream beside the summaries (joined before the
 *    last kernel, same bits).  The results differ from the other orders by
 *    rounding only.
 *  - staged: when desc->context is given and usable (created on the device
 *    of `stream`, its stream not part of a graph capture other than the one
 *    `stream` belongs to), a dense batch of more chains, at least 256 chunks
 *    per sequence, whose sequential kernel leaves CUs idle, is split into up
 *    to six stages: the chunk-parallel kernel of stage s+1 runs on the idle
 *    CUs while the sequential kernel of stage s runs on the context's
 *    stream.  If an event cannot be recorded after a stage was enqueued on
 *    the context's stream, that stream is synchronised on the host before
 *    the error returns (outside a capture), so no kernel of the call
 *    outlives it unordered.
 *  - windowed: a workspace below kda_chunk_fwd_workspace_bytes() (see
 *    kda_chunk_fwd_min_workspace_bytes), on `stream`.
 *  - plain: otherwise, the two kernels one after the other on `stream`.
 * The staged, windowed and plain orders give bit-identical results.
 *
 *   q, k        [B, T, H, d_k]  in_dtype
 *   v           [B, T, H, d_v]  in_dtype
 *   g           [B, T, H, d_k]  fp32, natural-log decay per key channel; the
 *                               fast path requires g >= -5 (the bounded decay
 *                               map keeps 16-token rescaling factors below
 *                               e^80, inside bf16/fp32 range)
 *   beta        [B, T, H]       fp32 write strength (after the sigmoid)
 *   init_state  [N, H, d_k, d_v] fp32, nullable (zeros); N = B, or num_seqs
 *               when cu_seqlens is given; may alias final_state
 *   cu_seqlens  [num_seqs + 1]  int32 device array, nullable; sequence n is
 *               tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed axis.
 *               Values are clamped into [0, T] on the device.
 *   o           [B, T, H, d_v]  out_dtype, fully overwritten; must not alias
 *               any input
 *   final_state [N, H, d_k, d_v] fp32, nullable
 *   workspace   device buffer of ws_bytes >= kda_chunk_fwd_min_workspace_bytes()
 *               (the fastest order needs kda_chunk_fwd_workspace_bytes());
 *               16-byte aligned; its contents need not be initialised
 */
KDA_API kda_status kda_chunk_fwd(const kda_chunk_desc* desc,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* init_state, const int32_t* cu_seqlens,
                         void* o, float* final_state,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * One fused recurrent step for decode (one new token per sequence), updating
 * the state in place ("Kimi K3 模型结构（2）", Q&A: decode uses the recurrent
 * form).  Per (n, h): S~ = Diag(exp g) S; u = beta (v - S~^T k^);
 * S <- S~ + k^ u^T; o = scale * S^T q^.
 *
 *   q, k, g  [N, H, d_k]  (q, k in in_dtype; g fp32)
 *   v        [N, H, d_v]  in_dtype
 *   beta     [N, H]       fp32
 *   state    [N, H, d_k, d_v] fp32, read and overwritten in place
 *   o        [N, H, d_v]  out_dtype
 */
KDA_API kda_status kda_recurrent_step(int N, int H, int d_k, int d_v,
                              kda_dtype in_dtype, kda_dtype out_dtype,
                              float scale, unsigned flags,
                              const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              float* state, void* o, hipStream_t stream);

/*
 * Gate prologue fused into the forward pass ("Kimi K3 模型结构（2）", Q&A on
 * the scaled-sigmoid decay map with its -5 lower bound; "Kimi K3 の KDA ..."
 * section 1.2.1 on A_log and dt_bias).  Instead of g, these take the decay
 * logits z and compute, per token, head h and key channel c,
 *
 *   g = -5 * sigmoid(exp(A_log[h]) * (z + dt_bias[h, c]))      in (-5, 0)
 *
 * which saves the g tensor's traffic (bf16 z is half of fp32 g).  Where
 * dt_bias enters is not legible on the pages; adding it to z before the
 * scale is this library's reading.
 *
 *   z        [B, T, H, d_k] (prefill) / [N, H, d_k] (decode), in_dtype,
 *            16-byte aligned
 *   A_log    [H] fp32, 4-byte aligned, required
 *   dt_bias  [H, d_k] fp32, nullable (zero), 16-byte aligned
 *
 * Every other argument, layout, flag, workspace rule and error is that of
 * kda_chunk_fwd / kda_recurrent_step; with KDA_FLAG_VALIDATE the g range
 * check is skipped (the map cannot leave (-5, 0)) and beta logits are only
 * checked to be finite.
 */
KDA_API kda_status kda_chunk_fwd_gated(const kda_chunk_desc* desc,
                         const void* q, const void* k, const void* v,
                         const void* z, const float* A_log, const float* dt_bias,
                         const float* beta,
                         const float* init_state, const int32_t* cu_seqlens,
                         void* o, float* final_state,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

KDA_API kda_status kda_recurrent_step_gated(int N, int H, int d_k, int d_v,
                              kda_dtype in_dtype, kda_dtype out_dtype,
                              float scale, unsigned flags,
                              const void* q, const void* k, const void* v,
                              const void* z, const float* A_log, const float* dt_bias,
                              const float* beta,
                              float* state, void* o, hipStream_t stream);

/*
 * Decay-gate inputs of the fused entry points (the map of kda_chunk_fwd_gated:
 * g = -5 sigmoid(exp(A_log[h]) (z + dt_bias[h, c])); layouts as given there).
 */
typedef struct kda_decay_gate {
    const void* z;          /* [B, T, H, d_k] / [N, H, d_k], in_dtype */
    const float* A_log;     /* [H], required */
    const float* dt_bias;   /* [H, d_k], nullable (zero) */
} kda_decay_gate;

/*
 * Output norm ("Kimi K3 の KDA ..." section 1.2.1:
 * after the kernel, the model applies a per-head RMSNorm over the head's
 * value dimension, a sigmoid on the output gate, and their elementwise
 * product).  Per token (and sequence) t, head h and value channel c, with o
 * the forward pass's output (scale included):
 *
 *   o'[t,h,c] = o[t,h,c] / sqrt(mean_c' o[t,h,c']^2 + eps) * weight[c]
 *               * sigmoid(gate[t,h,c])
 *
 *   gate    same layout as o ([B, T, H, d_v] prefill, [N, H, d_v] decode),
 *           in_dtype, 16-byte aligned: the output-gate logits
 *   weight  [d_v] fp32 per-channel gain shared by all heads, nullable
 *           (ones), 16-byte aligned
 *   eps     >= 0, added to the mean square (the pages give no value)
 *
 * The decode step applies it in the kernel that computes o.  The matrix-core
 * prefill applies it in the sequential kernel that computes o: each row of o
 * is split over the two value-slice workgroups of a chain, which exchange
 * per-row sums of o^2 (taken before rounding) through words in the
 * workspace and normalise their own columns as they store them.  A slice
 * waits for its partner's word with a bounded number of retries; should the
 * partner not get a compute unit while it waits (the pair's workgroup ids
 * are 8 apart, so a device that holds fewer than 9 of them at once), the
 * rows it did not deliver come out NaN rather than wrongly scaled.  The
 * exact fp32 path runs the norm as a second kernel over fp32 o: in place
 * for an fp32 o, from the workspace (sized by KDA_FLAG_OUT_NORM) for a
 * bf16 o.
 */
typedef struct kda_out_norm {
    const void* gate;
    const float* weight;
    float eps;
} kda_out_norm;

/*
 * Short convolution fused at the load of q, k and v ("Kimi K3 の KDA ..."
 * section 1.2.1: three causal convolutions of width 4, each channel
 * independent, over the current token and the 3 before it, followed by a
 * SiLU; "GDN, KDA の整理", the conv cache of the previous 3 inputs).  With it
 * q, k and v passed to the entry point are the raw projections, and the
 * forward pass uses, per tensor x in (q, k, v), sequence token t and channel
 * c of the H*d channels (c = h*d + i),
 *
 *   x'[t, c] = silu(sum_{j<4} weight[c][j] * x[t - 3 + j, c])
 *
 * with x[t'] for t' before the sequence's first token taken from row
 * 3 + t' - first of init_state (zero when it is NULL).  On the matrix-core
 * path x' is rounded to bf16 before use, as a bf16 module would hand it over.
 *
 *   weight[i]       [H*d, 4] fp32 (d = d_k for q, k; d_v for v), 16-byte
 *                   aligned; taps of channel c at 4c .. 4c+3, oldest token
 *                   first.  Required.
 *   init_state[i]   [N, 3, H*d] in_dtype, 16-byte aligned: the 3 inputs that
 *                   precede each sequence, oldest first; NULL = zeros.
 *   final_state[i]  [N, 3, H*d] in_dtype, 16-byte aligned: receives each
 *                   sequence's last 3 raw inputs (taken from init_state where
 *                   the sequence is shorter than 3); NULL = not written.  May
 *                   alias init_state[i] (it is written after every read).
 *
 * For the decode step N sequences advance by one token: init_state is the
 * conv cache before the token and final_state receives it shifted by one.
 */
typedef struct kda_short_conv {
    const float* weight[3];
    const void* init_state[3];
    void* final_state[3];
} kda_short_conv;

/*
 * The forward pass with the model's adjacent steps: the short convolution
 * of q, k, v (when conv is given), the decay-gate prologue (when decay_gate
 * is given; g must then be NULL) and the output norm (when norm is given;
 * KDA_FLAG_OUT_NORM must then be set in the flags, and only then).  With all
 * three NULL this is kda_chunk_fwd / kda_recurrent_step.  Every other
 * argument, layout, flag, workspace rule and error is that of those entry
 * points; a norm with a null gate or a negative or non-finite eps is
 * KDA_ERR_INVALID_ARG, as is a mismatch between norm and KDA_FLAG_OUT_NORM,
 * a conv with a missing weight or a misaligned conv pointer.  o must not
 * alias the norm's gate.
 */
KDA_API kda_status kda_chunk_fwd_fused(const kda_chunk_desc* desc,
                         const void* q, const void* k, const void* v,
                         const float* g, const kda_decay_gate* decay_gate,
                         const float* beta,
                         const float* init_state, const int32_t* cu_seqlens,
                         const kda_short_conv* conv, const kda_out_norm* norm,
                         void* o, float* final_state,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

KDA_API kda_status kda_recurrent_step_fused(int N, int H, int d_k, int d_v,
                              kda_dtype in_dtype, kda_dtype out_dtype,
                              float scale, unsigned flags,
                              const void* q, const void* k, const void* v,
                              const float* g, const kda_decay_gate* decay_gate,
                              const float* beta, const kda_short_conv* conv,
                              const kda_out_norm* norm,
                              float* state, void* o, hipStream_t stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, layouts, flags and errors are those of kda_chunk_fwd, without
 * the workspace: the scratch the kernels need lives in a fixed device array
 * of KDA_NOALLOC_SCRATCH_BYTES that the library defines; each GPU it runs on
 * holds one copy until the process ends.  Its address is looked up once per
 * device, on the first call that runs there.  The call allocates nothing (no
 * hipMalloc, no allocating library routine).  A call whose
 * kda_chunk_fwd_workspace_bytes exceeds the array runs in the windowed order
 * within it; one whose kda_chunk_fwd_min_workspace_bytes exceeds it returns
 * KDA_ERR_SCRATCH before any launch, and KDA_FLAG_VALIDATE (which
 * reads its counters back to the host) is KDA_ERR_UNSUPPORTED.  Every call
 * on one GPU uses that GPU's array and leaves its contents behind: calls
 * that overlap on one GPU (on different streams, or from different threads,
 * without ordering between them) race on it and give undefined results.
 * Nothing in the array needs to start at zero.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
KDA_API kda_status kda_chunk_fwd_noalloc(const kda_chunk_desc* desc,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* init_state, const int32_t* cu_seqlens,
                         void* o, float* final_state, hipStream_t stream);

/* Static description of a status code. */
KDA_API const char* kda_status_str(kda_status status);

/* The hipError_t behind the calling thread's last KDA_ERR_HIP (0 if none). */
KDA_API int kda_last_hip_error(void);

/* Library version string. */
KDA_API const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
