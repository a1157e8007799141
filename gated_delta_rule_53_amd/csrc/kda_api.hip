// C ABI entry points: host-side validation, then one launch on the caller's stream.
// Nothing here allocates device memory or synchronises unless KDA_DEBUG=1.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_last_error[512] = "";

kda_status_t fail(kda_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("KDA_DEBUG");
        return e && e[0] && std::strcmp(e, "0") != 0;
    }();
    return on;
}

kda_status_t finish(hipError_t launch, hipStream_t stream, const char* what) {
    if (launch != hipSuccess)
        return fail(KDA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(launch));
    if (debug_sync()) {
        const hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: kernel failed: %s", what, hipGetErrorString(e));
    }
    g_last_error[0] = '\0';
    return KDA_OK;
}

// ---- workspace of kda_chunk_fwd_noalloc ----
// A file-scope device array: every GPU the library runs on holds its own copy,
// at its own address, until the process ends.  In host code `scratch` is only
// a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept in g_scratch_ptr.  Only those addresses are ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Vector loads and stores of 16 bytes: a null pointer passes (it is checked where it is required).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, size_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

// Largest token count of kda_short_conv, as its header states.  (The launch
// takes (run, channel block) pairs in turn from at most 2^20 workgroups, so
// the grid fits the hardware's limits for any count up to this one.)
constexpr int64_t kConvMaxTokens = (int64_t(1) << 27) - 1024;

// Alignment the kernels' vector accesses need: q, k, v, out, the states, the
// workspace and a per-channel g (or raw gate) move in 16-byte pieces; beta,
// a per-head g and the int32 arrays element by element.  elem: bytes of one
// g / beta element (4 for float32, 2 for a bf16 raw gate).
kda_status_t check_alignment(const char* what, const kda_problem_t* p, size_t elem, const void* q,
                             const void* k, const void* v, const void* g, const void* beta, const void* out,
                             std::initializer_list<const void*> blocks16,
                             std::initializer_list<const void*> ints = {}) {
    bool ok = aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned_to(beta, elem) &&
              (p->gate_per_head ? aligned_to(g, elem) : aligned16(g));
    for (const void* b : blocks16) ok = ok && aligned16(b);
    if (!ok)
        return fail(KDA_ERR_BAD_SHAPE, "%s: q, k, v, out, %sthe state and workspace buffers must be 16-byte "
                    "aligned, beta%s %zu-byte aligned", what, p->gate_per_head ? "" : "g, ",
                    p->gate_per_head ? " and g" : "", elem);
    for (const void* i : ints)
        if (!aligned_to(i, 4)) return fail(KDA_ERR_BAD_SHAPE, "%s: int32 index arrays must be 4-byte aligned", what);
    return KDA_OK;
}

// Checks shared by both entry points.  Returns KDA_OK or the first violation.
kda_status_t check_problem(const kda_problem_t* p, const char* what) {
    if (!p) return fail(KDA_ERR_NULL_POINTER, "%s: problem is NULL", what);
    if (p->num_seqs < 0) return fail(KDA_ERR_BAD_SHAPE, "%s: num_seqs = %d < 0", what, p->num_seqs);
    if (p->total_tokens < 0)
        return fail(KDA_ERR_BAD_SHAPE, "%s: total_tokens = %lld < 0", what, (long long)p->total_tokens);
    if (p->num_heads < 1) return fail(KDA_ERR_BAD_SHAPE, "%s: num_heads = %d < 1", what, p->num_heads);
    if (p->head_k < 1 || p->head_v < 1)
        return fail(KDA_ERR_BAD_SHAPE, "%s: head sizes %d, %d must be positive", what, p->head_k, p->head_v);
    if (p->head_k != p->head_v)
        return fail(KDA_ERR_UNSUPPORTED, "%s: head_k = %d != head_v = %d", what, p->head_k, p->head_v);
    if (p->head_k != 64 && p->head_k != 128)
        return fail(KDA_ERR_UNSUPPORTED, "%s: head size %d (supported: 64, 128)", what, p->head_k);
    if (p->qkv_dtype != KDA_F32 && p->qkv_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: qkv_dtype %d", what, p->qkv_dtype);
    if (p->out_dtype != KDA_F32 && p->out_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: out_dtype %d", what, p->out_dtype);
    if (p->qk_l2norm != 0 && p->qk_l2norm != 1)
        return fail(KDA_ERR_BAD_SHAPE, "%s: qk_l2norm must be 0 or 1", what);
    if (p->gate_per_head != 0 && p->gate_per_head != 1)
        return fail(KDA_ERR_BAD_SHAPE, "%s: gate_per_head must be 0 or 1", what);
    if (p->state_layout != KDA_STATE_DK_DV && p->state_layout != KDA_STATE_DV_DK)
        return fail(KDA_ERR_BAD_SHAPE, "%s: state_layout must be KDA_STATE_DK_DV (0) or KDA_STATE_DV_DK (1)", what);
    // Row counts that index int32 offsets inside kernels stay well within range.
    if (p->total_tokens > (int64_t(1) << 40) || int64_t(p->num_seqs) * p->num_heads > (int64_t(1) << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", what);
    return KDA_OK;
}

// Gate parameters of the *_gated entry points.
kda_status_t check_gate(const kda_gate_t* gate, const char* what, kda::GateParams& gp) {
    if (!gate) return fail(KDA_ERR_NULL_POINTER, "%s: gate is NULL", what);
    if (!gate->a_log || !gate->dt_bias) return fail(KDA_ERR_NULL_POINTER, "%s: gate a_log and dt_bias are required", what);
    if (gate->has_lower_bound != 0 && gate->has_lower_bound != 1)
        return fail(KDA_ERR_BAD_SHAPE, "%s: gate has_lower_bound must be 0 or 1", what);
    if (gate->has_lower_bound && !(gate->lower_bound <= 0.f && gate->lower_bound > -1e30f))
        return fail(KDA_ERR_BAD_SHAPE, "%s: gate lower_bound must be finite and <= 0", what);
    gp.a_log = gate->a_log;
    gp.dt_bias = gate->dt_bias;
    gp.has_lower_bound = gate->has_lower_bound;
    gp.lower_bound = gate->has_lower_bound ? gate->lower_bound : 0.f;
    return KDA_OK;
}

// Workspace of one prefill call: the caller's buffer, or (noalloc) the library's scratch array.
enum class Workspace { kCaller, kScratch };

kda_status_t chunk_fwd_impl(const char* what, const kda_problem_t* p, const kda::GateParams& gp,
                            const void* q, const void* k, const void* v, const void* g, const void* beta,
                            const int32_t* cu_seqlens, const float* initial_state, void* out,
                            float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                            const int32_t* slots = nullptr, int num_slots = 0,
                            Workspace ws_kind = Workspace::kCaller, const kda::ConvParams* conv = nullptr,
                            int64_t qkv_row = 0, void* conv_state_out = nullptr) {
    if (p->chunk_size != 0 && p->chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "%s: chunk_size %d (supported: 64)", what, p->chunk_size);
    if (p->num_seqs == 0) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    if (!cu_seqlens) return fail(KDA_ERR_NULL_POINTER, "%s: cu_seqlens is NULL", what);
    if (p->total_tokens > 0 && (!q || !k || !v || !g || !beta || !out))
        return fail(KDA_ERR_NULL_POINTER, "%s: q, k, v, g, beta and out are required", what);
    if (p->total_tokens == 0 && !final_state) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    {
        const size_t elem = gp.a_log && p->qkv_dtype == KDA_BF16 ? 2 : 4;
        const kda_status_t st = check_alignment(what, p, elem, q, k, v, g, beta, out,
                                                {initial_state, final_state, workspace}, {cu_seqlens, slots});
        if (st != KDA_OK) return st;
    }
    const size_t need = kda_chunk_fwd_workspace_bytes(p);
    if (ws_kind == Workspace::kScratch) {
        if (need > KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_UNSUPPORTED, "%s: the problem needs %zu bytes of workspace; the library's scratch "
                        "holds %zu (use kda_chunk_fwd with a workspace)", what, need,
                        static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES));
    } else {
        if (workspace_bytes < need)
            return fail(KDA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, workspace_bytes, need);
        if (need > 0 && !workspace) return fail(KDA_ERR_NULL_POINTER, "%s: workspace is NULL", what);
    }
    if (need > 0 && ((p->total_tokens + 63) / 64 + p->num_seqs) * int64_t(p->num_heads) > (int64_t(1) << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "%s: too many (chunk, head) pairs", what);
    if (ws_kind == Workspace::kScratch && need > 0) {
        // every argument is valid: only now touch the device
        const hipError_t e = scratch_address(&workspace);
        if (e != hipSuccess)
            return fail(KDA_ERR_HIP, "%s: address of the library's scratch: %s", what, hipGetErrorString(e));
    }
    kda::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.gate = gp;
    a.gate_per_head = p->gate_per_head;
    a.state_trans = p->state_layout == KDA_STATE_DV_DK;
    a.cu_seqlens = cu_seqlens;
    a.initial_state = initial_state;
    a.out = out;
    a.final_state = final_state;
    a.slots = slots;
    a.num_slots = num_slots;
    a.qkv_row = qkv_row > 0 ? qkv_row : int64_t(p->num_heads) * p->head_k;
    if (conv) a.conv = *conv;
    a.conv_state_out = conv ? conv_state_out : nullptr;
    a.total_tokens = p->total_tokens;
    a.num_seqs = p->num_seqs;
    a.num_heads = p->num_heads;
    a.head_dim = p->head_k;
    a.qkv_bf16 = p->qkv_dtype == KDA_BF16;
    a.out_bf16 = p->out_dtype == KDA_BF16;
    a.scale = p->scale;
    a.l2norm = p->qk_l2norm;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kda::split_prefill_applies(a)) return finish(kda::launch_prefill_split(a, workspace, s), s, what);
    return finish(kda::launch_prefill(a, s), s, what);
}

kda_status_t recurrent_step_impl(const char* what, const kda_problem_t* p, const kda::GateParams& gp,
                                 const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, float* state, void* out, void* stream,
                                 const kda::NormParams& norm = kda::NormParams{}) {
    if (p->total_tokens != p->num_seqs)
        return fail(KDA_ERR_BAD_SHAPE, "%s: total_tokens = %lld must equal num_seqs = %d (one token each)",
                    what, (long long)p->total_tokens, p->num_seqs);
    if (p->num_seqs == 0) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    if (!q || !k || !v || !g || !beta || !state || !out)
        return fail(KDA_ERR_NULL_POINTER, "%s: q, k, v, g, beta, state and out are required", what);
    {
        const size_t elem = gp.a_log && p->qkv_dtype == KDA_BF16 ? 2 : 4;
        const kda_status_t st = check_alignment(what, p, elem, q, k, v, g, beta, out,
                                                {state, norm.gate, norm.weight});
        if (st != KDA_OK) return st;
    }
    kda::DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.gate = gp;
    a.gate_per_head = p->gate_per_head;
    a.state_trans = p->state_layout == KDA_STATE_DV_DK;
    a.norm = norm;
    a.state = state;
    a.out = out;
    a.num_seqs = p->num_seqs;
    a.num_heads = p->num_heads;
    a.head_dim = p->head_k;
    a.qkv_bf16 = p->qkv_dtype == KDA_BF16;
    a.out_bf16 = p->out_dtype == KDA_BF16;
    a.scale = p->scale;
    a.l2norm = p->qk_l2norm;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(kda::launch_decode(a, s), s, what);
}

kda::GateParams optional_gate(const kda_gate_t* gate, const char* what, kda_status_t& st) {
    kda::GateParams gp{};
    st = gate ? check_gate(gate, what, gp) : KDA_OK;
    return gp;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_POINTER: return "null pointer";
        case KDA_ERR_BAD_SHAPE: return "bad shape";
        case KDA_ERR_UNSUPPORTED: return "unsupported";
        case KDA_ERR_WORKSPACE: return "workspace too small";
        case KDA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_last_error; }

size_t kda_chunk_fwd_workspace_bytes(const kda_problem_t* problem) {
    if (!problem || problem->num_seqs <= 0 || problem->num_heads < 1 || problem->total_tokens < 0) return 0;
    // bf16 inputs with 128-wide heads take the two-pass path, which stores the
    // per-chunk operands; every other configuration keeps them on chip.
    if (problem->qkv_dtype == KDA_BF16 && problem->head_k == 128 && problem->head_v == 128)
        return kda::split_workspace_bytes(problem->total_tokens, problem->num_seqs, problem->num_heads);
    return 0;
}

kda_status_t kda_chunk_fwd(const kda_problem_t* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const int32_t* cu_seqlens,
                           const float* initial_state, void* out, float* final_state,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* what = "kda_chunk_fwd";
    const kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    return chunk_fwd_impl(what, p, kda::GateParams{}, q, k, v, g, beta, cu_seqlens, initial_state, out,
                          final_state, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_noalloc(const kda_problem_t* p, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu_seqlens,
                                   const float* initial_state, void* out, float* final_state, void* stream) {
    const char* what = "kda_chunk_fwd_noalloc";
    const kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    return chunk_fwd_impl(what, p, kda::GateParams{}, q, k, v, g, beta, cu_seqlens, initial_state, out,
                          final_state, nullptr, 0, stream, nullptr, 0, Workspace::kScratch);
}

kda_status_t kda_chunk_fwd_gated(const kda_problem_t* p, const kda_gate_t* gate, const void* q, const void* k,
                                 const void* v, const void* raw_g, const void* raw_beta,
                                 const int32_t* cu_seqlens, const float* initial_state, void* out,
                                 float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    const char* what = "kda_chunk_fwd_gated";
    kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    kda::GateParams gp{};
    st = check_gate(gate, what, gp);
    if (st != KDA_OK) return st;
    return chunk_fwd_impl(what, p, gp, q, k, v, raw_g, raw_beta, cu_seqlens, initial_state, out, final_state,
                          workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_conv(const kda_problem_t* p, const kda_gate_t* gate, const kda_conv_t* conv,
                                const void* qkv, const void* g, const void* beta, const int32_t* cu_seqlens,
                                const float* initial_state, void* out, float* final_state, void* workspace,
                                size_t workspace_bytes, void* stream) {
    const char* what = "kda_chunk_fwd_conv";
    kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    const kda::GateParams gp = optional_gate(gate, what, st);
    if (st != KDA_OK) return st;
    if (!conv) return fail(KDA_ERR_NULL_POINTER, "%s: conv is NULL", what);
    if (conv->kernel_size < 1 || conv->kernel_size > 4)
        return fail(KDA_ERR_UNSUPPORTED, "%s: kernel_size %d (supported: 1 to 4)", what, conv->kernel_size);
    if (conv->silu != 0 && conv->silu != 1) return fail(KDA_ERR_BAD_SHAPE, "%s: silu must be 0 or 1", what);
    if (p->qkv_dtype != KDA_BF16 || p->head_k != 128)
        return fail(KDA_ERR_UNSUPPORTED, "%s: the convolution is fused into the bf16, d = 128 path only (use "
                    "kda_short_conv, then kda_chunk_fwd)", what);
    const int64_t channels = 3 * int64_t(p->num_heads) * p->head_k;
    if (channels > (1 << 26)) return fail(KDA_ERR_UNSUPPORTED, "%s: too many heads", what);
    if (!aligned16(conv->weight) || !aligned16(conv->state_in) || !aligned16(conv->state_out))
        return fail(KDA_ERR_BAD_SHAPE, "%s: the conv weight and states must be 16-byte aligned", what);
    if (p->num_seqs > 0 && !conv->weight) return fail(KDA_ERR_NULL_POINTER, "%s: conv->weight is NULL", what);
    if (p->total_tokens > 0 && !qkv) return fail(KDA_ERR_NULL_POINTER, "%s: qkv is NULL", what);
    const size_t hd = size_t(p->num_heads) * p->head_k;
    const kda::bf16_t* x = static_cast<const kda::bf16_t*>(qkv);
    kda::ConvParams cv{};
    cv.weight = static_cast<const kda::bf16_t*>(conv->weight);
    cv.state = static_cast<const kda::bf16_t*>(conv->state_in);
    cv.K = conv->kernel_size;
    cv.silu = conv->silu;
    cv.channels = static_cast<int>(channels);
    // The chain pass writes the new conv states (after its own reads of the old
    // ones); a call that launches nothing (no tokens, no final state) copies
    // them with a kernel of their own.
    const bool chain_runs = p->num_seqs > 0 && (p->total_tokens > 0 || final_state);
    st = chunk_fwd_impl(what, p, gp, x, x ? x + hd : nullptr, x ? x + 2 * hd : nullptr, g, beta, cu_seqlens,
                        initial_state, out, final_state, workspace, workspace_bytes, stream, nullptr, 0,
                        Workspace::kCaller, &cv, channels, conv->state_out);
    if (st != KDA_OK || chain_runs || !conv->state_out || p->num_seqs == 0 || conv->kernel_size < 2) return st;
    kda::ConvArgs a{};
    a.x = qkv;
    a.cu_seqlens = cu_seqlens;
    a.state_in = conv->state_in;
    a.state_out = conv->state_out;
    a.total_tokens = p->total_tokens;
    a.num_seqs = p->num_seqs;
    a.channels = static_cast<int>(channels);
    a.kernel_size = conv->kernel_size;
    a.bf16 = true;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(kda::launch_conv_state(a, s), s, what);
}

kda_status_t kda_recurrent_step(const kda_problem_t* p, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float* state, void* out,
                                void* stream) {
    const char* what = "kda_recurrent_step";
    const kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    return recurrent_step_impl(what, p, kda::GateParams{}, q, k, v, g, beta, state, out, stream);
}

kda_status_t kda_recurrent_step_gated(const kda_problem_t* p, const kda_gate_t* gate, const void* q,
                                      const void* k, const void* v, const void* raw_g, const void* raw_beta,
                                      float* state, void* out, void* stream) {
    const char* what = "kda_recurrent_step_gated";
    kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    kda::GateParams gp{};
    st = check_gate(gate, what, gp);
    if (st != KDA_OK) return st;
    return recurrent_step_impl(what, p, gp, q, k, v, raw_g, raw_beta, state, out, stream);
}

kda_status_t kda_recurrent_step_normed(const kda_problem_t* p, const kda_gate_t* gate, const void* q,
                                      const void* k, const void* v, const void* g, const void* beta, float* state,
                                      const void* out_gate, const float* norm_weight, float norm_eps, void* out,
                                      void* stream) {
    const char* what = "kda_recurrent_step_normed";
    kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    const kda::GateParams gp = optional_gate(gate, what, st);
    if (st != KDA_OK) return st;
    if (!(norm_eps >= 0.f && norm_eps < 1e30f))
        return fail(KDA_ERR_BAD_SHAPE, "%s: norm_eps must be finite and >= 0", what);
    if (p->num_seqs > 0 && (!out_gate || !norm_weight))
        return fail(KDA_ERR_NULL_POINTER, "%s: out_gate and norm_weight are required", what);
    return recurrent_step_impl(what, p, gp, q, k, v, g, beta, state, out, stream,
                               kda::NormParams{out_gate, norm_weight, norm_eps});
}

kda_status_t kda_chunk_fwd_pooled(const kda_problem_t* p, const kda_gate_t* gate, const void* q, const void* k,
                                  const void* v, const void* g, const void* beta, const int32_t* cu_seqlens,
                                  float* state_pool, int32_t num_slots, const int32_t* state_slots, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    const char* what = "kda_chunk_fwd_pooled";
    kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    const kda::GateParams gp = optional_gate(gate, what, st);
    if (st != KDA_OK) return st;
    if (num_slots < 0) return fail(KDA_ERR_BAD_SHAPE, "%s: num_slots = %d < 0", what, num_slots);
    if (p->num_seqs > 0 && (!state_pool || !state_slots))
        return fail(KDA_ERR_NULL_POINTER, "%s: state_pool and state_slots are required", what);
    if (int64_t(num_slots) * p->num_heads > (int64_t(1) << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "%s: state pool too large", what);
    return chunk_fwd_impl(what, p, gp, q, k, v, g, beta, cu_seqlens, state_pool, out, state_pool, workspace,
                          workspace_bytes, stream, state_slots, num_slots);
}

static kda_status_t verify_impl(const char* what, const kda_problem_t* p, int32_t width, const kda_gate_t* gate,
                                const void* q, const void* k, const void* v, const void* g, const void* beta,
                                float* state_pool, int32_t num_slots, const int32_t* state_indices,
                                const int32_t* num_accepted, void* out, void* stream,
                                const kda::NormParams& norm = kda::NormParams{}) {
    kda_status_t st = check_problem(p, what);
    if (st != KDA_OK) return st;
    const kda::GateParams gp = optional_gate(gate, what, st);
    if (st != KDA_OK) return st;
    if (width < 1) return fail(KDA_ERR_BAD_SHAPE, "%s: width = %d < 1", what, width);
    if (num_slots < 0) return fail(KDA_ERR_BAD_SHAPE, "%s: num_slots = %d < 0", what, num_slots);
    if (p->total_tokens != int64_t(p->num_seqs) * width)
        return fail(KDA_ERR_BAD_SHAPE, "%s: total_tokens = %lld must equal num_seqs * width = %lld", what,
                    (long long)p->total_tokens, (long long)(int64_t(p->num_seqs) * width));
    if (int64_t(num_slots) * p->num_heads > (int64_t(1) << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "%s: state pool too large", what);
    if (p->num_seqs == 0) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    if (!q || !k || !v || !g || !beta || !state_pool || !state_indices || !out)
        return fail(KDA_ERR_NULL_POINTER, "%s: q, k, v, g, beta, state_pool, state_indices and out are required",
                    what);
    {
        const size_t elem = gp.a_log && p->qkv_dtype == KDA_BF16 ? 2 : 4;
        st = check_alignment(what, p, elem, q, k, v, g, beta, out, {state_pool, norm.gate, norm.weight},
                             {state_indices, num_accepted});
        if (st != KDA_OK) return st;
    }
    kda::VerifyArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.gate = gp;
    a.gate_per_head = p->gate_per_head;
    a.state_trans = p->state_layout == KDA_STATE_DV_DK;
    a.pool = state_pool;
    a.num_slots = num_slots;
    a.indices = state_indices;
    a.accepted = num_accepted;
    a.norm = norm;
    a.out = out;
    a.num_seqs = p->num_seqs;
    a.width = width;
    a.num_heads = p->num_heads;
    a.head_dim = p->head_k;
    a.qkv_bf16 = p->qkv_dtype == KDA_BF16;
    a.out_bf16 = p->out_dtype == KDA_BF16;
    a.scale = p->scale;
    a.l2norm = p->qk_l2norm;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(kda::launch_verify(a, s), s, what);
}

kda_status_t kda_recurrent_verify(const kda_problem_t* p, int32_t width, const kda_gate_t* gate, const void* q,
                                  const void* k, const void* v, const void* g, const void* beta,
                                  float* state_pool, int32_t num_slots, const int32_t* state_indices,
                                  const int32_t* num_accepted, void* out, void* stream) {
    return verify_impl("kda_recurrent_verify", p, width, gate, q, k, v, g, beta, state_pool, num_slots,
                       state_indices, num_accepted, out, stream);
}

kda_status_t kda_recurrent_verify_normed(const kda_problem_t* p, int32_t width, const kda_gate_t* gate,
                                         const void* q, const void* k, const void* v, const void* g,
                                         const void* beta, float* state_pool, int32_t num_slots,
                                         const int32_t* state_indices, const int32_t* num_accepted,
                                         const void* out_gate, const float* norm_weight, float norm_eps, void* out,
                                         void* stream) {
    const char* what = "kda_recurrent_verify_normed";
    if (!(norm_eps >= 0.f && norm_eps < 1e30f))
        return fail(KDA_ERR_BAD_SHAPE, "%s: norm_eps must be finite and >= 0", what);
    if (p && p->num_seqs > 0 && (!out_gate || !norm_weight))
        return fail(KDA_ERR_NULL_POINTER, "%s: out_gate and norm_weight are required", what);
    return verify_impl(what, p, width, gate, q, k, v, g, beta, state_pool, num_slots, state_indices, num_accepted,
                       out, stream, kda::NormParams{out_gate, norm_weight, norm_eps});
}

kda_status_t kda_short_conv(int32_t num_seqs, int64_t total_tokens, int32_t channels, int32_t kernel_size,
                            int32_t dtype, int32_t silu, const void* x, const void* weight,
                            const int32_t* cu_seqlens, const void* state_in, void* state_out, void* y,
                            void* stream) {
    const char* what = "kda_short_conv";
    if (num_seqs < 0) return fail(KDA_ERR_BAD_SHAPE, "%s: num_seqs = %d < 0", what, num_seqs);
    if (total_tokens < 0) return fail(KDA_ERR_BAD_SHAPE, "%s: total_tokens = %lld < 0", what, (long long)total_tokens);
    if (channels < 8 || channels % 8 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: channels = %d (a positive multiple of 8)", what, channels);
    if (kernel_size < 1 || kernel_size > 4)
        return fail(KDA_ERR_UNSUPPORTED, "%s: kernel_size %d (supported: 1 to 4)", what, kernel_size);
    if (dtype != KDA_F32 && dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d", what, dtype);
    if (silu != 0 && silu != 1) return fail(KDA_ERR_BAD_SHAPE, "%s: silu must be 0 or 1", what);
    // in place the grid is one workgroup per request (x) and per 2048 channels (y)
    if (total_tokens > kConvMaxTokens || channels > (1 << 26) || num_seqs > (1 << 23))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large (at most %lld tokens, 2^23 requests, 2^26 "
                    "channels)", what, (long long)kConvMaxTokens);
    if (!aligned16(x) || !aligned16(weight) || !aligned16(state_in) || !aligned16(state_out) || !aligned16(y))
        return fail(KDA_ERR_BAD_SHAPE, "%s: x, weight, states and y must be 16-byte aligned", what);
    if (num_seqs == 0) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    if (!cu_seqlens || !weight || (total_tokens > 0 && (!x || !y)))
        return fail(KDA_ERR_NULL_POINTER, "%s: cu_seqlens, weight, x and y are required", what);
    if (total_tokens == 0 && !state_out) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    kda::ConvArgs a{};
    a.x = x;
    a.weight = weight;
    a.cu_seqlens = cu_seqlens;
    a.state_in = state_in;
    a.state_out = state_out;
    a.y = y;
    a.total_tokens = total_tokens;
    a.num_seqs = num_seqs;
    a.channels = channels;
    a.kernel_size = kernel_size;
    a.bf16 = dtype == KDA_BF16;
    a.silu = silu == 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(kda::launch_short_conv(a, s), s, what);
}

kda_status_t kda_gated_rmsnorm(int64_t rows, int32_t head_v, int32_t in_dtype, int32_t out_dtype, const void* o,
                               const void* gate, const float* weight, float eps, void* out, void* stream) {
    const char* what = "kda_gated_rmsnorm";
    if (rows < 0) return fail(KDA_ERR_BAD_SHAPE, "%s: rows = %lld < 0", what, (long long)rows);
    if (head_v != 64 && head_v != 128)
        return fail(KDA_ERR_UNSUPPORTED, "%s: head_v %d (supported: 64, 128)", what, head_v);
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "%s: in_dtype %d", what, in_dtype);
    if (out_dtype != KDA_F32 && out_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: out_dtype %d", what, out_dtype);
    if (!(eps >= 0.f && eps < 1e30f)) return fail(KDA_ERR_BAD_SHAPE, "%s: eps must be finite and >= 0", what);
    // grid: one workgroup per 64 rows (dv = 128) or 128 (dv = 64)
    if (rows > (int64_t(1) << 36)) return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", what);
    if (!aligned16(o) || !aligned16(gate) || !aligned16(weight) || !aligned16(out))
        return fail(KDA_ERR_BAD_SHAPE, "%s: o, gate, weight and out must be 16-byte aligned", what);
    if (rows == 0) {
        g_last_error[0] = '\0';
        return KDA_OK;
    }
    if (!o || !gate || !weight || !out)
        return fail(KDA_ERR_NULL_POINTER, "%s: o, gate, weight and out are required", what);
    if (out == o && in_dtype != out_dtype)
        return fail(KDA_ERR_BAD_SHAPE, "%s: out may be o only with out_dtype == in_dtype", what);
    kda::EpilogueArgs a{};
    a.o = o;
    a.gate = gate;
    a.weight = weight;
    a.eps = eps;
    a.out = out;
    a.rows = rows;
    a.head_v = head_v;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(kda::launch_gated_rmsnorm(a, s), s, what);
}

}  // extern "C"
