// Launch descriptors passed from the C ABI layer to the kernel launchers.
// Every pointer here has already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_common.h"

namespace kda {

// g and beta are float32 when gate.a_log is null; otherwise they are the raw
// gate [rows, H, dk] and raw beta [rows, H] in the q/k/v dtype, activated in
// the kernels.
// Output epilogue fused into decode: out = o / sqrt(mean(o^2) + eps) * weight
// * sigmoid(gate); gate null means none.
struct NormParams {
    const void* gate;      // [rows, H, dv] in the q/k/v dtype
    const float* weight;   // [dv]
    float eps;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    GateParams gate;
    int gate_per_head;  // g (or the raw gate) is [rows, H]: one decay per head
    int state_trans;    // state blocks are S^T [dv][dk]
    NormParams norm;
    float* state;
    void* out;
    int num_seqs;
    int num_heads;
    int head_dim;
    bool qkv_bf16;
    bool out_bf16;
    float scale;
    int l2norm;
};

// Multi-token verify decode over a slot pool [num_slots, H, dk, dv].
struct VerifyArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    GateParams gate;
    int gate_per_head;
    int state_trans;
    float* pool;
    int num_slots;
    const int32_t* indices;   // [num_seqs, width]
    const int32_t* accepted;  // [num_seqs] or null
    NormParams norm;          // fused output epilogue (norm.gate null: none)
    void* out;
    int num_seqs;
    int width;
    int num_heads;
    int head_dim;
    bool qkv_bf16;
    bool out_bf16;
    float scale;
    int l2norm;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    GateParams gate;
    int gate_per_head;
    int state_trans;
    const int32_t* cu_seqlens;
    const float* initial_state;
    void* out;
    float* final_state;
    // With slots (a state pool): sequence n's initial and final state are
    // slot slots[n] of initial_state / final_state (both the pool); a slot
    // outside [0, num_slots) starts from zero and is not written.
    const int32_t* slots;
    int num_slots;
    // Elements between consecutive tokens of q, k and v (H d for separate
    // [T, H, d] tensors; 3 H d when they are the column blocks of the fused
    // projection, as with conv).
    int64_t qkv_row;
    ConvParams conv;  // conv.weight null: q, k, v are used as given
    // With conv: the new conv states [N, K - 1, 3 H d], written by the chain
    // pass (may be conv.state itself), or null.
    void* conv_state_out;
    int64_t total_tokens;
    int num_seqs;
    int num_heads;
    int head_dim;
    bool qkv_bf16;
    bool out_bf16;
    float scale;
    int l2norm;
};

// Output epilogue: gated RMSNorm over rows of head_v values.
struct EpilogueArgs {
    const void* o;
    const void* gate;
    const float* weight;
    float eps;
    void* out;
    int64_t rows;
    int head_v;
    bool in_bf16;
    bool out_bf16;
};

// Short causal convolution over [total_tokens, channels] with per-request states.
struct ConvArgs {
    const void* x;
    const void* weight;       // [kernel_size, channels]
    const int32_t* cu_seqlens;
    const void* state_in;     // [num_seqs, kernel_size - 1, channels] or null (zeros)
    void* state_out;          // same shape, or null
    void* y;
    int64_t total_tokens;
    int num_seqs;
    int channels;
    int kernel_size;
    bool bf16;
    bool silu;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_short_conv(const ConvArgs& a, hipStream_t stream);
// The conv-state update alone (bf16): each request's last K - 1 inputs of x
// [T, channels] (its old state followed by its inputs when it is shorter)
// into state_out; state_out may be state_in.
hipError_t launch_conv_state(const ConvArgs& a, hipStream_t stream);
hipError_t launch_gated_rmsnorm(const EpilogueArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
// fp32 q/k/v, or dk = dv = 64: one workgroup per (sequence, head, 16-column
// tile) carries the state through the chunks with everything on chip.
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// bf16 q/k/v with dk = dv = 128: chunk-parallel preparation into a workspace of
// split_workspace_bytes() bytes, then the state scan.
bool split_prefill_applies(const PrefillArgs& a);
size_t split_workspace_bytes(int64_t total_tokens, int num_seqs, int num_heads);
hipError_t launch_prefill_split(const PrefillArgs& a, void* workspace, hipStream_t stream);

}  // namespace kda
