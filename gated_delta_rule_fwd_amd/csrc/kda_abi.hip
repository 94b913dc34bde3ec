// kda_abi.hip -- the extern "C" boundary of libkda.so: argument checks,
// kernel selection and error reporting.  See include/kda.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <new>

#include "../../include/kda.h"
#include "kda_kernels.h"

// Device scratch of kda_chunk_fwd_noalloc: one copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is a stand-in, not a device address): it uses the address that
// hipGetSymbolAddress returns for the device, kept in g_scratch below.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

// Per device: the address of `scratch` there, looked up once with that
// device current (or the error of the lookup).
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

hipError_t scratch_on(int dev, void** out)
{
    *out = nullptr;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev]() {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        g_scratch[dev] = e == hipSuccess ? p : nullptr;
        g_scratch_err[dev] = e;
    });
    *out = g_scratch[dev];
    return g_scratch_err[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(kda_dtype t) { return t == KDA_F32 || t == KDA_BF16; }

constexpr unsigned kKnownFlags = KDA_FLAG_QK_L2NORM | KDA_FLAG_VALIDATE | KDA_FLAG_FP32_PATH | KDA_FLAG_BETA_LOGITS |
                                 KDA_FLAG_SIGNED_ALPHA | KDA_FLAG_OUT_NORM;
constexpr unsigned kDecodeFlags = KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_LOGITS | KDA_FLAG_SIGNED_ALPHA | KDA_FLAG_OUT_NORM;
constexpr size_t kValidateBytes = 256;
constexpr long long kMaxTokenHeads = 1LL << 31;      // B*T*H of a prefill call
constexpr long long kMaxPrefillChains = 1LL << 22;   // N*H of a prefill call
constexpr long long kMaxDecodeChains = (1LL << 24) - 1;

kda_status hip_fail(hipError_t e)
{
    g_last_hip_error = static_cast<int>(e);
    return KDA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kda_version(void) { return "kda-mi355x 0.1.0 (gfx950)"; }

int kda_last_hip_error(void) { return g_last_hip_error; }

kda_status kda_context_create(kda_context* out)
{
    if (!out) return KDA_ERR_INVALID_ARG;
    *out = nullptr;
    kda_context_s* c = new (std::nothrow) kda_context_s{};
    if (!c) return hip_fail(hipErrorOutOfMemory);
    hipError_t e = hipGetDevice(&c->device);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);   // default priority
    for (int s = 0; e == hipSuccess && s < kda::kMaxStages; ++s) {
        e = hipEventCreateWithFlags(&c->p1[s], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->p2[s], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        // give back what was made
        for (int s = 0; s < kda::kMaxStages; ++s) {
            if (c->p1[s]) (void)hipEventDestroy(c->p1[s]);
            if (c->p2[s]) (void)hipEventDestroy(c->p2[s]);
        }
        if (c->side) (void)hipStreamDestroy(c->side);
        delete c;
        return hip_fail(e);
    }
    *out = c;
    return KDA_OK;
}

kda_status kda_context_destroy(kda_context c)
{
    if (!c) return KDA_OK;
    hipError_t first = hipSuccess;
    auto keep = [&](hipError_t r) { if (first == hipSuccess) first = r; };
    int cur = -1;
    keep(hipGetDevice(&cur));
    const bool switched = cur >= 0 && cur != c->device && hipSetDevice(c->device) == hipSuccess;
    for (int s = 0; s < kda::kMaxStages; ++s) {
        keep(hipEventDestroy(c->p1[s]));
        keep(hipEventDestroy(c->p2[s]));
    }
    keep(hipStreamDestroy(c->side));
    if (switched) keep(hipSetDevice(cur));
    delete c;
    return first == hipSuccess ? KDA_OK : hip_fail(first);
}

const char* kda_status_str(kda_status s)
{
    switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or flag";
    case KDA_ERR_WORKSPACE: return "workspace too small";
    case KDA_ERR_RANGE: return "input out of range (g outside [-5,0], beta outside [0,1] or bad cu_seqlens)";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_SCRATCH: return "call needs more device scratch than the fixed no-allocation area";
    }
    return "unknown status";
}

namespace {

// The matrix-core path serves bf16 inputs with d_k = d_v = 128 unless the
// fp32 path is forced; it needs the two-pass record workspace.
bool uses_two_pass(const kda_chunk_desc* d)
{
    return d->in_dtype == KDA_BF16 && d->d_k == 128 && d->d_v == 128 && !(d->flags & KDA_FLAG_FP32_PATH);
}

// fp32 staging of o for the separate norm pass of the fp32 path (a bf16 o
// with KDA_FLAG_OUT_NORM); the matrix-core path normalises o in its
// sequential kernel instead
size_t norm_staging_bytes(const kda_chunk_desc* d)
{
    if (!(d->flags & KDA_FLAG_OUT_NORM) || d->out_dtype != KDA_BF16 || uses_two_pass(d)) return 0;
    return static_cast<size_t>(d->B) * d->T * d->H * d->d_v * sizeof(float);
}

// Workspace of one call: validation counters, the records (matrix-core
// path, with the norm's row-sum words), then the norm staging (fp32 path).
size_t workspace_need(const kda_chunk_desc* d, bool packed)
{
    size_t bytes = (d->flags & KDA_FLAG_VALIDATE) ? kValidateBytes : 0;
    if (uses_two_pass(d))
        bytes += kda::two_pass_workspace_bytes(d->B, d->T, d->H, d->num_seqs, packed,
                                               (d->flags & KDA_FLAG_OUT_NORM) != 0);
    return bytes + norm_staging_bytes(d);
}

// The least workspace of one call: as workspace_need, with the matrix-core
// path's records for one chunk of every sequence (the windowed order).
size_t workspace_min(const kda_chunk_desc* d, bool packed)
{
    size_t bytes = (d->flags & KDA_FLAG_VALIDATE) ? kValidateBytes : 0;
    if (uses_two_pass(d))
        bytes += kda::two_pass_min_workspace_bytes(d->B, d->T, d->H, d->num_seqs, packed,
                                                   (d->flags & KDA_FLAG_OUT_NORM) != 0);
    return bytes + norm_staging_bytes(d);
}

// Both queries: the descriptor does not say whether cu_seqlens will be
// passed, so the larger of the dense and the packed figure is reported.
size_t workspace_query(const kda_chunk_desc* d, size_t (*need)(const kda_chunk_desc*, bool))
{
    if (!d) return static_cast<size_t>(-1);
    if (d->B <= 0 || d->T < 0 || d->H <= 0 || d->num_seqs < 0) return 0;   // rejected by kda_chunk_fwd
    if (static_cast<long long>(d->B) * d->T * d->H > kMaxTokenHeads) return 0;
    const size_t dense = need(d, false);
    const size_t packed = (d->B == 1 && d->num_seqs > 0) ? need(d, true) : 0;
    return dense > packed ? dense : packed;
}

// Conv pointers: every weight present, everything 16-byte aligned.
bool conv_ok(const kda_short_conv* conv)
{
    if (!conv) return true;
    for (int i = 0; i < 3; ++i) {
        if (!conv->weight[i] || !aligned16(conv->weight[i])) return false;
        if (conv->init_state[i] && !aligned16(conv->init_state[i])) return false;
        if (conv->final_state[i] && !aligned16(conv->final_state[i])) return false;
    }
    return true;
}

// Checks shared by the prefill and decode entry points for the output norm.
bool out_norm_ok(const kda_out_norm* norm, unsigned flags, const void* o)
{
    if (!norm) return !(flags & KDA_FLAG_OUT_NORM);
    if (!(flags & KDA_FLAG_OUT_NORM)) return false;
    if (!(norm->eps >= 0.f) || norm->eps > 3.0e38f) return false;   // rejects NaN and inf too
    if (norm->gate && (!aligned16(norm->gate) || norm->gate == o)) return false;
    if (norm->weight && !aligned16(norm->weight)) return false;
    return true;
}

}  // namespace

size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_desc* d)
{
    return workspace_query(d, workspace_need);
}

size_t kda_chunk_fwd_min_workspace_bytes(const kda_chunk_desc* d)
{
    return workspace_query(d, workspace_min);
}

}  // extern "C"

namespace {

// Gate inputs of the gated entry points (all null for the plain ones).
struct Gate {
    const void* z;
    const float* A_log;
    const float* dt_bias;
};

kda_status chunk_fwd_impl(const kda_chunk_desc* d, const void* q, const void* k, const void* v, const float* g,
                          const Gate* gate, const float* beta, const float* init_state, const int32_t* cu_seqlens,
                          const kda_short_conv* conv, const kda_out_norm* norm, void* o, float* final_state,
                          void* workspace, size_t ws_bytes, hipStream_t stream)
{
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->flags & ~kKnownFlags) return KDA_ERR_UNSUPPORTED;
    if (gate && (d->flags & KDA_FLAG_SIGNED_ALPHA)) return KDA_ERR_UNSUPPORTED;
    if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_dim_ok(d->d_k) || !head_dim_ok(d->d_v)) return KDA_ERR_UNSUPPORTED;
    if (d->B <= 0 || d->T < 0 || d->H <= 0) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens && (d->B != 1 || d->num_seqs < 0)) return KDA_ERR_INVALID_ARG;
    const long long N = cu_seqlens ? d->num_seqs : d->B;
    const long long tokens = static_cast<long long>(d->B) * d->T;
    // size limits: one grid dimension takes at most 2^32 work items (the
    // sequential passes launch 512 per chain; the chunk-parallel pass, 256 per
    // (chunk, head), is checked below)
    if (tokens * d->H > kMaxTokenHeads || N * d->H > kMaxPrefillChains) return KDA_ERR_INVALID_ARG;
    const void* decay = gate ? gate->z : static_cast<const void*>(g);
    if (tokens > 0 && (!q || !k || !v || !decay || !beta || !o)) return KDA_ERR_INVALID_ARG;
    if (gate && tokens > 0 && !gate->A_log) return KDA_ERR_INVALID_ARG;
    if (!out_norm_ok(norm, d->flags, o)) return KDA_ERR_INVALID_ARG;
    if (norm && tokens > 0 && !norm->gate) return KDA_ERR_INVALID_ARG;
    if (!conv_ok(conv)) return KDA_ERR_INVALID_ARG;
    const void* rows[] = {q, k, v, decay, init_state, o, final_state, gate ? gate->dt_bias : nullptr};
    for (const void* p : rows)
        if (p && !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if ((beta && !aligned4(beta)) || (cu_seqlens && !aligned4(cu_seqlens))) return KDA_ERR_INVALID_ARG;
    if (gate && gate->A_log && !aligned4(gate->A_log)) return KDA_ERR_INVALID_ARG;
    const size_t need = workspace_min(d, cu_seqlens != nullptr);
    if (ws_bytes < need || (need > 0 && !workspace)) return KDA_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;

    kda::ChunkArgs a{};
    a.B = d->B;
    a.T = d->T;
    a.H = d->H;
    a.dk = d->d_k;
    a.dv = d->d_v;
    a.num_seqs = cu_seqlens ? d->num_seqs : d->B;
    a.in_bf16 = d->in_dtype == KDA_BF16;
    a.out_bf16 = d->out_dtype == KDA_BF16;
    a.scale = d->scale;
    a.normalize = (d->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.init_state = init_state;
    a.cu_seqlens = cu_seqlens;
    a.o = o;
    a.final_state = final_state;
    a.gated = gate ? 1 : 0;
    a.z = gate ? gate->z : nullptr;
    a.A_log = gate ? gate->A_log : nullptr;
    a.dt_bias = gate ? gate->dt_bias : nullptr;
    a.beta_logits = (d->flags & KDA_FLAG_BETA_LOGITS) ? 1 : 0;
    a.signed_alpha = (d->flags & KDA_FLAG_SIGNED_ALPHA) ? 1 : 0;
    a.out_norm = norm ? 1 : 0;
    a.out_gate = norm ? norm->gate : nullptr;
    a.norm_w = norm ? norm->weight : nullptr;
    a.norm_eps = norm ? norm->eps : 0.f;
    a.conv = conv ? 1 : 0;
    for (int i = 0; i < 3; ++i) {
        a.conv_w[i] = conv ? conv->weight[i] : nullptr;
        a.conv_init[i] = conv ? conv->init_state[i] : nullptr;
    }

    hipError_t e;
    if (d->flags & KDA_FLAG_VALIDATE) {
        unsigned int* counters = static_cast<unsigned int*>(workspace);
        e = kda::launch_validate(a, counters, stream);
        if (e != hipSuccess) return hip_fail(e);
        unsigned int host[4] = {0, 0, 0, 0};
        e = hipMemcpyAsync(host, counters, sizeof(host), hipMemcpyDeviceToHost, stream);
        if (e != hipSuccess) return hip_fail(e);
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e);
        if (host[0] || host[1] || host[2]) return KDA_ERR_RANGE;
    }

    const size_t off = (d->flags & KDA_FLAG_VALIDATE) ? kValidateBytes : 0;
    if (uses_two_pass(d)) {
        // the sequential kernel applies the output norm as it stores o
        e = kda::launch_chunk_two_pass(a, static_cast<char*>(workspace) + off, ws_bytes - off, stream, d->context);
    } else {
        // with a norm, the fp32 path writes fp32 o (to the staging area when
        // o is bf16), then the norm pass writes o
        kda::ChunkArgs fw = a;
        if (norm) {
            fw.out_norm = 0;
            fw.out_bf16 = false;
            if (a.out_bf16) fw.o = static_cast<char*>(workspace) + off;
        }
        e = kda::launch_chunk_fp32(fw, stream);
        if (e == hipSuccess && norm) e = kda::launch_out_norm(a, static_cast<const float*>(fw.o), stream);
    }
    if (e != hipSuccess) return hip_fail(e);
    if (conv) {
        // after every kernel that reads the incoming conv state
        e = kda::launch_conv_final(a, conv->final_state, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return KDA_OK;
}

kda_status recurrent_step_impl(int N, int H, int d_k, int d_v, kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                               unsigned flags, const void* q, const void* k, const void* v, const float* g,
                               const Gate* gate, const float* beta, const kda_short_conv* conv,
                               const kda_out_norm* norm, float* state, void* o, hipStream_t stream)
{
    if (flags & ~kDecodeFlags) return KDA_ERR_UNSUPPORTED;
    if (gate && (flags & KDA_FLAG_SIGNED_ALPHA)) return KDA_ERR_UNSUPPORTED;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
    if (static_cast<long long>(N) * H > kMaxDecodeChains) return KDA_ERR_INVALID_ARG;   // one 256-thread group per chain
    if (!out_norm_ok(norm, flags, o)) return KDA_ERR_INVALID_ARG;
    if (!conv_ok(conv)) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;
    if (norm && !norm->gate) return KDA_ERR_INVALID_ARG;
    const void* decay = gate ? gate->z : static_cast<const void*>(g);
    if (!q || !k || !v || !decay || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    if (gate && !gate->A_log) return KDA_ERR_INVALID_ARG;
    const void* rows[] = {q, k, v, decay, state, o};
    for (const void* p : rows)
        if (!aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (!aligned4(beta)) return KDA_ERR_INVALID_ARG;
    if (gate && (!aligned4(gate->A_log) || (gate->dt_bias && !aligned4(gate->dt_bias)))) return KDA_ERR_INVALID_ARG;
    kda::DecodeArgs a{};
    a.dk = d_k;
    a.dv = d_v;
    a.chains = N * H;
    a.H = H;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.scale = scale;
    a.normalize = (flags & KDA_FLAG_QK_L2NORM) ? 1 : 0;
    a.gated = gate ? 1 : 0;
    a.z = gate ? gate->z : nullptr;
    a.A_log = gate ? gate->A_log : nullptr;
    a.dt_bias = gate ? gate->dt_bias : nullptr;
    a.beta_logits = (flags & KDA_FLAG_BETA_LOGITS) ? 1 : 0;
    a.signed_alpha = (flags & KDA_FLAG_SIGNED_ALPHA) ? 1 : 0;
    a.out_norm = norm ? 1 : 0;
    a.out_gate = norm ? norm->gate : nullptr;
    a.norm_w = norm ? norm->weight : nullptr;
    a.norm_eps = norm ? norm->eps : 0.f;
    a.conv = conv ? 1 : 0;
    for (int i = 0; i < 3; ++i) {
        a.conv_w[i] = conv ? conv->weight[i] : nullptr;
        a.conv_init[i] = conv ? conv->init_state[i] : nullptr;
        a.conv_final[i] = conv ? conv->final_state[i] : nullptr;
    }
    hipError_t e = kda::launch_decode(a, stream);
    if (e != hipSuccess) return hip_fail(e);
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const kda_chunk_desc* d, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* init_state, const int32_t* cu_seqlens, void* o,
                         float* final_state, void* workspace, size_t ws_bytes, hipStream_t stream)
{
    return chunk_fwd_impl(d, q, k, v, g, nullptr, beta, init_state, cu_seqlens, nullptr, nullptr, o, final_state,
                          workspace, ws_bytes, stream);
}

kda_status kda_chunk_fwd_noalloc(const kda_chunk_desc* d, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* init_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state, hipStream_t stream)
{
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->flags & KDA_FLAG_VALIDATE) return KDA_ERR_UNSUPPORTED;
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e);
    void* ws = nullptr;
    e = scratch_on(dev, &ws);
    if (e != hipSuccess) return hip_fail(e);
    const kda_status st = chunk_fwd_impl(d, q, k, v, g, nullptr, beta, init_state, cu_seqlens, nullptr, nullptr, o,
                                         final_state, ws, KDA_NOALLOC_SCRATCH_BYTES, stream);
    return st == KDA_ERR_WORKSPACE ? KDA_ERR_SCRATCH : st;
}

kda_status kda_chunk_fwd_gated(const kda_chunk_desc* d, const void* q, const void* k, const void* v, const void* z,
                               const float* A_log, const float* dt_bias, const float* beta, const float* init_state,
                               const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                               size_t ws_bytes, hipStream_t stream)
{
    const Gate gate{z, A_log, dt_bias};
    return chunk_fwd_impl(d, q, k, v, nullptr, &gate, beta, init_state, cu_seqlens, nullptr, nullptr, o, final_state,
                          workspace, ws_bytes, stream);
}

kda_status kda_chunk_fwd_fused(const kda_chunk_desc* d, const void* q, const void* k, const void* v, const float* g,
                               const kda_decay_gate* decay_gate, const float* beta, const float* init_state,
                               const int32_t* cu_seqlens, const kda_short_conv* conv, const kda_out_norm* norm,
                               void* o, float* final_state, void* workspace, size_t ws_bytes, hipStream_t stream)
{
    if (decay_gate && g) return KDA_ERR_INVALID_ARG;
    if (!decay_gate)
        return chunk_fwd_impl(d, q, k, v, g, nullptr, beta, init_state, cu_seqlens, conv, norm, o, final_state,
                              workspace, ws_bytes, stream);
    const Gate gate{decay_gate->z, decay_gate->A_log, decay_gate->dt_bias};
    return chunk_fwd_impl(d, q, k, v, nullptr, &gate, beta, init_state, cu_seqlens, conv, norm, o, final_state,
                          workspace, ws_bytes, stream);
}

kda_status kda_recurrent_step(int N, int H, int d_k, int d_v, kda_dtype in_dtype, kda_dtype out_dtype,
                              float scale, unsigned flags, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, float* state, void* o, hipStream_t stream)
{
    return recurrent_step_impl(N, H, d_k, d_v, in_dtype, out_dtype, scale, flags, q, k, v, g, nullptr, beta, nullptr,
                               nullptr, state, o, stream);
}

kda_status kda_recurrent_step_gated(int N, int H, int d_k, int d_v, kda_dtype in_dtype, kda_dtype out_dtype,
                                    float scale, unsigned flags, const void* q, const void* k, const void* v,
                                    const void* z, const float* A_log, const float* dt_bias, const float* beta,
                                    float* state, void* o, hipStream_t stream)
{
    const Gate gate{z, A_log, dt_bias};
    return recurrent_step_impl(N, H, d_k, d_v, in_dtype, out_dtype, scale, flags, q, k, v, nullptr, &gate, beta,
                               nullptr, nullptr, state, o, stream);
}

kda_status kda_recurrent_step_fused(int N, int H, int d_k, int d_v, kda_dtype in_dtype, kda_dtype out_dtype,
                                    float scale, unsigned flags, const void* q, const void* k, const void* v,
                                    const float* g, const kda_decay_gate* decay_gate, const float* beta,
                                    const kda_short_conv* conv, const kda_out_norm* norm, float* state, void* o,
                                    hipStream_t stream)
{
    if (decay_gate && g) return KDA_ERR_INVALID_ARG;
    if (!decay_gate)
        return recurrent_step_impl(N, H, d_k, d_v, in_dtype, out_dtype, scale, flags, q, k, v, g, nullptr, beta, conv,
                                   norm, state, o, stream);
    const Gate gate{decay_gate->z, decay_gate->A_log, decay_gate->dt_bias};
    return recurrent_step_impl(N, H, d_k, d_v, in_dtype, out_dtype, scale, flags, q, k, v, nullptr, &gate, beta, conv,
                               norm, state, o, stream);
}

}  // extern "C"
