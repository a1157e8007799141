// Private helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNormEps = 1e-6f;

// bfloat16 is carried as its raw 16 bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

typedef float cfloatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 cbf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16, round to nearest even in hardware (a NaN stays a
// quiet NaN): a in the low half.  (Converting a four-wide vector and taking
// its elements apart is avoided: the compiler at hand keeps only element 0
// there.)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(cfloatx2{a, b}, cbf16x2));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return bf16_t{static_cast<uint16_t>(pack_bf16x2(f, 0.f))}; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Vector load of N contiguous elements (N * sizeof(T) a multiple of 8 bytes,
// source aligned to min(16, N * sizeof(T))).
template <int N, typename T>
__device__ __forceinline__ void load_vec(T (&dst)[N], const T* src) {
    constexpr int BYTES = N * static_cast<int>(sizeof(T));
    static_assert(BYTES % 8 == 0, "vector load size");
    if constexpr (BYTES == 8) {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else {
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Gate activation on raw inputs (the Ascend model file's gated prefill and
// decode paths, `_prefill_torch_kda` and the decode branch of the attention
// forward, with its `_softplus`): u = x + dt_bias[h][c], then
//   g = -e^{a_log[h]} softplus(u)             or, with a lower bound,
//   g = lower_bound * sigmoid(e^{a_log[h]} u),
// and beta = sigmoid(raw beta).
struct GateParams {
    const float* a_log;    // [H]; nullptr: g and beta arrive activated, in float32
    const float* dt_bias;  // [H, dk]
    float lower_bound;
    int has_lower_bound;
};

// Short causal convolution fused into the prefill's q/k/v loads (the Ascend
// model file's `KimiShortConvolution`, run on the fused q/k/v projection
// before the core).  Channels of the fused projection: q = [0, H d),
// k = [H d, 2 H d), v = [2 H d, 3 H d).  weight null: no convolution.
struct ConvParams {
    const bf16_t* weight;  // [K, channels], tap-major
    const bf16_t* state;   // [N, K - 1, channels] (oldest first), or null for zeros
    int K;                 // 1 .. 4
    int silu;              // 1: y * sigmoid(y)
    int channels;          // 3 H d
};

// The short convolution's arithmetic on bf16 inputs, shared by kda_short_conv
// and the prefill that fuses it, so both give the same bits.  Four taps (a
// filter of K < 4 taps is padded at the front with zero taps); per channel
// c, with x_m the input m steps back and w_t tap t (tap 3 meets x_0):
//   y = dot(x_0 w_3 + x_1 w_2, on top of x_2 w_1 + x_3 w_0)
// as two bf16 pair products with float32 accumulation (v_dot2_f32_bf16).

// (lo half of a, lo half of b) and (hi of a, hi of b) as packed pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// The tap pairs of eight channels: a[c] = (w_3, w_2), b[c] = (w_1, w_0).
struct ConvTaps8 {
    uint32_t a[8], b[8];
};

__device__ __forceinline__ uint32_t word_at(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// w[t]: tap t of eight channels (packed bf16, channel 2e in the low half of word e)
__device__ __forceinline__ ConvTaps8 conv_taps8(const uint4 (&w)[4]) {
    ConvTaps8 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        t.a[2 * e] = pair_lo(word_at(w[3], e), word_at(w[2], e));
        t.a[2 * e + 1] = pair_hi(word_at(w[3], e), word_at(w[2], e));
        t.b[2 * e] = pair_lo(word_at(w[1], e), word_at(w[0], e));
        t.b[2 * e + 1] = pair_hi(word_at(w[1], e), word_at(w[0], e));
    }
    return t;
}

// The convolution (before any activation) of eight channels from their
// inputs 0 .. 3 steps back: y[2e], y[2e + 1] for the words e in [E0, E1).
template <int E0 = 0, int E1 = 4>
__device__ __forceinline__ void conv8_bf16(const uint4& x0, const uint4& x1, const uint4& x2, const uint4& x3,
                                           const ConvTaps8& t, float (&y)[8]) {
#pragma unroll
    for (int e = E0; e < E1; ++e) {
        const uint32_t a0 = word_at(x0, e), a1 = word_at(x1, e), a2 = word_at(x2, e), a3 = word_at(x3, e);
        const uint32_t p01[2] = {pair_lo(a0, a1), pair_hi(a0, a1)};
        const uint32_t p23[2] = {pair_lo(a2, a3), pair_hi(a2, a3)};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(cbf16x2, p23[h]),
                                                            __builtin_bit_cast(cbf16x2, t.b[2 * e + h]), 0.f, false);
            y[2 * e + h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(cbf16x2, p01[h]),
                                                           __builtin_bit_cast(cbf16x2, t.a[2 * e + h]), s, false);
        }
    }
}

// e^x and 1/x through the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float gate_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float gate_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + gate_exp(-x)); }

// log(1 + y) for y >= 0 to a few ulp: with w = 1 + y rounded, log(w) * y / (w - 1)
// cancels the rounding of w (Goldberg's correction; w == 1 means log1p(y) = y to
// float precision).
__device__ __forceinline__ float gate_log1p(float y) {
    const float w = 1.f + y;
    const float d = w - 1.f;
    const float lw = __builtin_amdgcn_logf(w) * 0.69314718055994531f;  // log2 -> ln
    return d == 0.f ? y : lw * (y * __builtin_amdgcn_rcpf(d));
}

// softplus(u) = max(u, 0) + log(1 + e^{-|u|}): no overflow for any u.
__device__ __forceinline__ float gate_softplus(float u) { return fmaxf(u, 0.f) + gate_log1p(gate_exp(-fabsf(u))); }

// g for raw value x with bias b; a = e^{a_log[h]}.
__device__ __forceinline__ float gate_g(float x, float b, float a, float lower_bound, int has_lower_bound) {
    const float u = x + b;
    return has_lower_bound ? lower_bound * gate_sigmoid(a * u) : -a * gate_softplus(u);
}

// Sum over the lanes of a wave64 whose lane ids differ only in the bits of `mask_lo..32`.
__device__ __forceinline__ float wave_sum_from(float x, int first_offset) {
    for (int off = first_offset; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// 16x16x4 fp32 MFMA.  Lane l supplies A[l%16][l/16] and B[l/16][l%16]; the
// accumulator holds D[4*(l/16)+j][l%16] in element j.
__device__ __forceinline__ floatx4 mfma_f32_16x16x4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Offset of the (sequence n, head h) state block: sequence-major, or slot
// slots[n] of a state pool [num_slots, H, D, D].  False for a pool slot
// outside [0, num_slots): that sequence starts from zero and keeps no state.
__device__ inline bool state_block(const int32_t* slots, int num_slots, int n, int h, int num_heads, int d,
                                   size_t& off) {
    int row = n;
    if (slots) {
        row = slots[n];
        if (row < 0 || row >= num_slots) return false;
    }
    off = (static_cast<size_t>(row) * num_heads + h) * d * d;
    return true;
}

// Element (r, c) of a state block, r a key channel and c a value channel:
// S[dk][dv] (c contiguous), or its transpose S^T[dv][dk] (r contiguous).
__device__ __forceinline__ size_t state_elem(int r, int c, int d, int trans) {
    return trans ? static_cast<size_t>(c) * d + r : static_cast<size_t>(r) * d + c;
}

// Phase timing for kernel tuning.  Compiled out unless KDA_PHASE_TIMING is
// defined; then thread 0 of every workgroup accumulates clock64() deltas
// between consecutive marks into kda_phase_cycles[mark].
#ifdef KDA_PHASE_TIMING
#ifndef KDA_PHASE_TID
#define KDA_PHASE_TID 0  // the thread that records (its wave's timeline)
#endif
__device__ unsigned long long kda_phase_cycles[32];
#define KDA_PHASE_BEGIN long long kda_phase_t = clock64(); long long kda_phase_acc[32] = {0};
#define KDA_PHASE_MARK(i)                                  \
    do {                                                   \
        if (threadIdx.x == KDA_PHASE_TID) {                \
            const long long kda_now = clock64();           \
            kda_phase_acc[i] += kda_now - kda_phase_t;     \
            kda_phase_t = kda_now;                         \
        }                                                  \
    } while (0)
#define KDA_PHASE_END                                                          \
    do {                                                                       \
        if (threadIdx.x == KDA_PHASE_TID)                                      \
            for (int kda_i = 0; kda_i < 32; ++kda_i)                           \
                if (kda_phase_acc[kda_i])                                      \
                    atomicAdd(&kda_phase_cycles[kda_i], (unsigned long long)kda_phase_acc[kda_i]); \
    } while (0)
#else
#define KDA_PHASE_BEGIN
#define KDA_PHASE_MARK(i) \
    do {                  \
    } while (0)
#define KDA_PHASE_END \
    do {              \
    } while (0)
#endif

}  // namespace kda
