// Short causal convolution before the core (the Ascend model file's
// `KimiShortConvolution`): a depthwise causal convolution over the fused
// q/k/v projection, one filter of K taps per channel, run per request with a
// conv-state cache holding each request's last K - 1 inputs.  With the window
// w = [state (K - 1 inputs, oldest first), x of the request],
//
//   y[t, c] = sum_{j < K} W[j, c] * w[t + j, c],   then optionally y * sigmoid(y),
//
// and the request's last K - 1 inputs become its state.  Decode is the same
// call with one token per request.
//
// bf16 inputs go through the shared bf16 dot-product arithmetic
// (conv8_bf16: four taps, two pair products per channel), the same that the
// prefill applies when it fuses this convolution into its loads; float32
// inputs through float32 multiply-adds.
//
// HBM-bound: every input is read once and every output written once.  Launch:
// a thread owns eight consecutive channels (one 16-byte load of bf16) of a run
// of 16 tokens (8 in float32), issues the run's loads first and keeps the K - 1 previous
// inputs in registers; a run that crosses into the next request restarts its
// window from that request's state.  Workgroups take (run, 2048-channel
// block) pairs with the channel block varying fastest, so the workgroups in
// flight together read and write whole rows.  One extra run row writes the
// state of empty requests (their initial state, or zeros).
//
// In place (state_out == state_in, the decode case): a request's old state
// could be read by one run while another run writes its new state, so that
// case has its own launch, request-major: one thread per request and eight
// channels reads the old state, runs the request's tokens and only then
// writes the new state.  Empty requests keep their state untouched.
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

// Tokens per thread: 16 for bf16 (best of 4 / 8 / 16 / 32 on a 4096 x 12,288
// projection), 8 for float32 (twice the registers per token).
template <typename T>
constexpr int run_tokens() { return sizeof(T) == 2 ? 16 : 8; }
// Workgroups per launch at most; more (run, channel block) pairs are taken in turn.
constexpr int64_t kConvMaxGroups = int64_t(1) << 20;

template <typename T>
__device__ __forceinline__ void load8c(float (&v)[8], const T* p) {
    T r[8];
    load_vec<8>(r, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = to_f32(r[i]);
}

// Eight channels out, non-temporal: nothing here reads y back (measured
// 57.7 -> 48.3 us on the bench shape).  bf16: rounded by pairs in hardware.
template <typename T>
__device__ __forceinline__ void store8c(T* p, const float (&v)[8]) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(T) == 2) {
        __builtin_nontemporal_store(u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                          pack_bf16x2(v[6], v[7])},
                                    reinterpret_cast<u32x4*>(p));
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(v)[i], reinterpret_cast<u32x4*>(p) + i);
    }
}

// bf16: the eight channels' raw words, and their non-temporal store.
__device__ __forceinline__ uint4 load_raw8(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void store_raw8(bf16_t* p, const uint4& v) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// The tap rows of eight channels padded at the front to four (zero rows).
template <int K>
__device__ __forceinline__ ConvTaps8 load_taps8(const bf16_t* weight, size_t C, int c) {
    uint4 w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        w[t] = t < 4 - K ? uint4{0u, 0u, 0u, 0u} : load_raw8(weight + static_cast<size_t>(t - (4 - K)) * C + c);
    return conv_taps8(w);
}

// The request containing token t: the last n with cu[n] <= t < cu[n + 1] (empty requests skipped).
__device__ __forceinline__ int request_of(const int32_t* cu, int num_seqs, int64_t t) {
    int lo = 0, hi = num_seqs;  // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace

// One run of run_tokens<T>() tokens (run == run_rows: the states of empty requests) in
// channels c .. c + 7.
template <int K, typename T, bool SILU>
__device__ __forceinline__ void conv_run(const T* __restrict__ x, const T* __restrict__ weight,
                                         const int32_t* __restrict__ cu, int num_seqs, const T* state_in,
                                         T* state_out, T* __restrict__ y, int64_t total_tokens, int channels,
                                         int64_t run_rows, int64_t run, int c) {
    constexpr int TB = run_tokens<T>();
    const size_t C = static_cast<size_t>(channels);
    constexpr int S = K - 1;  // state length
    auto soff = [&](int n, int m) { return (static_cast<size_t>(n) * S + m) * C + c; };

    if (run == run_rows) {
        // empty requests keep their state
        if (!state_out) return;
        for (int n = 0; n < num_seqs; ++n) {
            if (cu[n + 1] != cu[n]) continue;
#pragma unroll
            for (int m = 0; m < S; ++m) {
                float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (state_in) load8c(v, state_in + soff(n, m));
                store8c(state_out + soff(n, m), v);
            }
        }
        return;
    }

    const int64_t t0 = run * TB;
    const int64_t t1 = min(t0 + TB, total_tokens);
    if (t0 >= t1) return;
    int n = request_of(cu, num_seqs, t0);
    int64_t start = cu[n], end = cu[n + 1];
    // the input p steps before token t is x[t - p], or, before the request,
    // its state row S - back (1 .. S steps before the request; clamped: cu_seqlens
    // is not checked on the device); zero without a state
    auto back_row = [&](int64_t p) {
        return static_cast<int>(min(max(start - p, static_cast<int64_t>(1)), static_cast<int64_t>(S)));
    };
    if constexpr (std::is_same<T, bf16_t>::value) {
        // bf16: the raw words, through the shared dot-product arithmetic
        const ConvTaps8 taps = load_taps8<K>(weight, C, c);
        uint4 win[3] = {};  // win[m]: the input m + 1 steps back (zero past S)
        auto fill_window = [&](int64_t t) {
#pragma unroll
            for (int m = 0; m < S; ++m) {
                const int64_t p = t - 1 - m;
                if (p >= start && p >= 0)
                    win[m] = load_raw8(x + static_cast<size_t>(p) * C + c);
                else
                    win[m] = state_in ? load_raw8(state_in + soff(n, S - back_row(p))) : uint4{0u, 0u, 0u, 0u};
            }
        };
        uint4 xin[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) xin[u] = load_raw8(x + static_cast<size_t>(min(t0 + u, t1 - 1)) * C + c);
        if (t1 <= end && t0 - S >= start) {
            // the run and the K - 1 rows before it lie inside one request
#pragma unroll
            for (int m = 0; m < S; ++m) win[m] = load_raw8(x + static_cast<size_t>(t0 - 1 - m) * C + c);
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                if (t0 + u >= t1) break;
                float acc[8];
                conv8_bf16(xin[u], win[0], win[1], win[2], taps, acc);
                if constexpr (SILU) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] *= gate_sigmoid(acc[i]);
                }
                store8c(y + static_cast<size_t>(t0 + u) * C + c, acc);
#pragma unroll
                for (int m = S - 1; m > 0; --m) win[m] = win[m - 1];
                if constexpr (S > 0) win[0] = xin[u];
            }
            if (t1 == end && state_out) {
#pragma unroll
                for (int m = 0; m < S; ++m) store_raw8(state_out + soff(n, m), win[S - 1 - m]);
            }
            return;
        }
        fill_window(t0);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int64_t t = t0 + u;
            if (t >= t1) break;
            if (t >= end) {
                n = request_of(cu, num_seqs, t);
                start = cu[n];
                end = cu[n + 1];
                fill_window(t);
            }
            float acc[8];
            conv8_bf16(xin[u], win[0], win[1], win[2], taps, acc);
            if constexpr (SILU) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= gate_sigmoid(acc[i]);
            }
            store8c(y + static_cast<size_t>(t) * C + c, acc);
#pragma unroll
            for (int m = S - 1; m > 0; --m) win[m] = win[m - 1];
            if constexpr (S > 0) win[0] = xin[u];
            if (t == end - 1 && state_out) {
#pragma unroll
                for (int m = 0; m < S; ++m) store_raw8(state_out + soff(n, m), win[S - 1 - m]);
            }
        }
        return;
    } else {
        float w[K][8];
#pragma unroll
        for (int j = 0; j < K; ++j) load8c(w[j], weight + static_cast<size_t>(j) * C + c);

        // win[m]: the input m + 1 steps before the current token (m < S)
        float win[S > 0 ? S : 1][8];
        auto fill_window = [&](int64_t t) {
#pragma unroll
            for (int m = 0; m < S; ++m) {
                const int64_t p = t - 1 - m;
                if (p >= start && p >= 0) {
                    load8c(win[m], x + static_cast<size_t>(p) * C + c);
                } else {
                    if (state_in) {
                        load8c(win[m], state_in + soff(n, S - back_row(p)));
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) win[m][i] = 0.f;
                    }
                }
            }
        };
        // the run's inputs, loaded raw before any arithmetic (rows past t1 repeat the last row)
        T xin[TB][8];
#pragma unroll
        for (int u = 0; u < TB; ++u) load_vec<8>(xin[u], x + static_cast<size_t>(min(t0 + u, t1 - 1)) * C + c);
        fill_window(t0);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int64_t t = t0 + u;
            if (t >= t1) break;
            if (t >= end) {
                // the run enters the next non-empty request
                n = request_of(cu, num_seqs, t);
                start = cu[n];
                end = cu[n + 1];
                fill_window(t);
            }
            float cur[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) cur[i] = to_f32(xin[u][i]);
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = w[K - 1][i] * cur[i];
#pragma unroll
            for (int m = 0; m < S; ++m)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += w[K - 2 - m][i] * win[m][i];
            if constexpr (SILU) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= gate_sigmoid(acc[i]);
            }
            store8c(y + static_cast<size_t>(t) * C + c, acc);
            // shift: the current input becomes one step back
#pragma unroll
            for (int m = S - 1; m > 0; --m)
#pragma unroll
                for (int i = 0; i < 8; ++i) win[m][i] = win[m - 1][i];
            if constexpr (S > 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) win[0][i] = cur[i];
            }
            if (t == end - 1 && state_out) {
                // the request's last S inputs, oldest first
#pragma unroll
                for (int m = 0; m < S; ++m) store8c(state_out + soff(n, m), win[S - 1 - m]);
            }
        }
    }
}

template <int K, typename T, bool SILU>
__global__ __launch_bounds__(256) void short_conv_kernel(const T* __restrict__ x, const T* __restrict__ weight,
                                                         const int32_t* __restrict__ cu, int num_seqs,
                                                         const T* state_in, T* state_out, T* __restrict__ y,
                                                         int64_t total_tokens, int channels, int64_t run_rows,
                                                         int cblocks) {
    const int64_t pairs = (run_rows + 1) * cblocks;
    for (int64_t id = blockIdx.x; id < pairs; id += gridDim.x) {
        const int64_t run = id / cblocks;
        const int c = (static_cast<int>(id - run * cblocks) * 256 + static_cast<int>(threadIdx.x)) * 8;
        if (c < channels)
            conv_run<K, T, SILU>(x, weight, cu, num_seqs, state_in, state_out, y, total_tokens, channels, run_rows,
                                 run, c);
    }
}

// In place: blockIdx.x is the request, blockIdx.y 2048 channels.
template <int K, typename T, bool SILU>
__global__ __launch_bounds__(256) void short_conv_inplace_kernel(const T* __restrict__ x, const T* __restrict__ weight,
                                                                 const int32_t* __restrict__ cu, T* state,
                                                                 T* __restrict__ y, int64_t total_tokens,
                                                                 int channels) {
    const int n = static_cast<int>(blockIdx.x);
    const int c = (static_cast<int>(blockIdx.y) * 256 + static_cast<int>(threadIdx.x)) * 8;
    if (c >= channels) return;
    int64_t start = cu[n], end = cu[n + 1];
    if (start < 0 || end > total_tokens || end < start) end = start;  // malformed: no tokens
    if (start == end) return;
    const size_t C = static_cast<size_t>(channels);
    constexpr int S = K - 1;
    auto soff = [&](int m) { return (static_cast<size_t>(n) * S + m) * C + c; };
    if constexpr (std::is_same<T, bf16_t>::value) {
        // bf16: the raw words, through the shared dot-product arithmetic
        const ConvTaps8 taps = load_taps8<K>(weight, C, c);
        uint4 win[3] = {};  // win[m]: the input m + 1 steps back (zero past S)
#pragma unroll
        for (int m = 0; m < S; ++m) win[m] = load_raw8(state + soff(S - 1 - m));
        for (int64_t t = start; t < end; ++t) {
            const uint4 cur = load_raw8(x + static_cast<size_t>(t) * C + c);
            float acc[8];
            conv8_bf16(cur, win[0], win[1], win[2], taps, acc);
            if constexpr (SILU) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= gate_sigmoid(acc[i]);
            }
            store8c(y + static_cast<size_t>(t) * C + c, acc);
#pragma unroll
            for (int m = S - 1; m > 0; --m) win[m] = win[m - 1];
            if constexpr (S > 0) win[0] = cur;
        }
#pragma unroll
        for (int m = 0; m < S; ++m) store_raw8(state + soff(m), win[S - 1 - m]);
        return;
    }
    float w[K][8];
#pragma unroll
    for (int j = 0; j < K; ++j) load8c(w[j], weight + static_cast<size_t>(j) * C + c);
    // win[m]: the input m + 1 steps back; the old state, newest last
    float win[S > 0 ? S : 1][8];
#pragma unroll
    for (int m = 0; m < S; ++m) load8c(win[m], state + soff(S - 1 - m));
    for (int64_t t = start; t < end; ++t) {
        float cur[8];
        load8c(cur, x + static_cast<size_t>(t) * C + c);
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = w[K - 1][i] * cur[i];
#pragma unroll
        for (int m = 0; m < S; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += w[K - 2 - m][i] * win[m][i];
        if constexpr (SILU) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] *= gate_sigmoid(acc[i]);
        }
        store8c(y + static_cast<size_t>(t) * C + c, acc);
#pragma unroll
        for (int m = S - 1; m > 0; --m)
#pragma unroll
            for (int i = 0; i < 8; ++i) win[m][i] = win[m - 1][i];
        if constexpr (S > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[0][i] = cur[i];
        }
    }
    // every read of this request's state is done: write the new one, oldest first
#pragma unroll
    for (int m = 0; m < S; ++m) store8c(state + soff(m), win[S - 1 - m]);
}

// The state update alone, for the prefill with the convolution fused into
// its loads (which writes no y): blockIdx.x is the request, blockIdx.y 2048
// channels.  With the window w = [old state, the request's inputs], the new
// state is w's last K - 1 entries; all of them are read before any is
// written, so state_out may be state_in.
template <typename T>
__global__ __launch_bounds__(256) void conv_state_kernel(const T* __restrict__ x, const int32_t* __restrict__ cu,
                                                         const T* state_in, T* state_out, int64_t total_tokens,
                                                         int channels, int K) {
    const int n = static_cast<int>(blockIdx.x);
    const int c = (static_cast<int>(blockIdx.y) * 256 + static_cast<int>(threadIdx.x)) * 8;
    if (c >= channels) return;
    int64_t start = cu[n], end = cu[n + 1];
    if (start < 0 || end > total_tokens || end < start) end = start;  // malformed: no tokens
    const int64_t len = end - start;
    const size_t C = static_cast<size_t>(channels);
    const int S = K - 1;
    float v[3][8];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        if (m >= S) break;
        const int64_t i = len + m;  // index into the window
        if (i >= S) {
            load8c(v[m], x + static_cast<size_t>(start + i - S) * C + c);
        } else if (state_in) {
            load8c(v[m], state_in + (static_cast<size_t>(n) * S + i) * C + c);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[m][e] = 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        if (m >= S) break;
        store8c(state_out + (static_cast<size_t>(n) * S + m) * C + c, v[m]);
    }
}

hipError_t launch_conv_state(const ConvArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.kernel_size < 2 || !a.state_out) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.num_seqs), static_cast<unsigned>((a.channels / 8 + 255) / 256));
    conv_state_kernel<bf16_t><<<grid, 256, 0, stream>>>(
        static_cast<const bf16_t*>(a.x), a.cu_seqlens, static_cast<const bf16_t*>(a.state_in),
        static_cast<bf16_t*>(a.state_out), a.total_tokens, a.channels, a.kernel_size);
    return hipGetLastError();
}

template <int K, typename T>
static hipError_t launch_conv_kt(const ConvArgs& a, hipStream_t stream) {
    if (a.state_out && a.state_out == a.state_in) {
        const dim3 grid(static_cast<unsigned>(a.num_seqs), static_cast<unsigned>((a.channels / 8 + 255) / 256));
        T* st = static_cast<T*>(a.state_out);
        if (a.silu)
            short_conv_inplace_kernel<K, T, true><<<grid, 256, 0, stream>>>(
                static_cast<const T*>(a.x), static_cast<const T*>(a.weight), a.cu_seqlens, st,
                static_cast<T*>(a.y), a.total_tokens, a.channels);
        else
            short_conv_inplace_kernel<K, T, false><<<grid, 256, 0, stream>>>(
                static_cast<const T*>(a.x), static_cast<const T*>(a.weight), a.cu_seqlens, st,
                static_cast<T*>(a.y), a.total_tokens, a.channels);
        return hipGetLastError();
    }
    constexpr int TB = run_tokens<T>();
    const int64_t run_rows = (a.total_tokens + TB - 1) / TB;
    const int cblocks = (a.channels / 8 + 255) / 256;
    const int64_t pairs = (run_rows + 1) * cblocks;
    const unsigned grid = static_cast<unsigned>(pairs < kConvMaxGroups ? pairs : kConvMaxGroups);
    const T* x = static_cast<const T*>(a.x);
    const T* w = static_cast<const T*>(a.weight);
    const T* si = static_cast<const T*>(a.state_in);
    T* so = static_cast<T*>(a.state_out);
    T* y = static_cast<T*>(a.y);
    if (a.silu)
        short_conv_kernel<K, T, true><<<grid, 256, 0, stream>>>(x, w, a.cu_seqlens, a.num_seqs, si, so, y,
                                                                 a.total_tokens, a.channels, run_rows, cblocks);
    else
        short_conv_kernel<K, T, false><<<grid, 256, 0, stream>>>(x, w, a.cu_seqlens, a.num_seqs, si, so, y,
                                                                  a.total_tokens, a.channels, run_rows, cblocks);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_conv_t(const ConvArgs& a, hipStream_t stream) {
    switch (a.kernel_size) {
        case 1: return launch_conv_kt<1, T>(a, stream);
        case 2: return launch_conv_kt<2, T>(a, stream);
        case 3: return launch_conv_kt<3, T>(a, stream);
        default: return launch_conv_kt<4, T>(a, stream);
    }
}

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_conv_t<bf16_t>(a, stream) : launch_conv_t<float>(a, stream);
}

}  // namespace kda
