// KDA decode step: one token per sequence, state updated in place.
//
// Per (sequence, head) the step is a read-modify-write of the fp32 state
// S[dk][dv] (the Ascend model file's decode paths update the recurrent cache in
// place with a per-channel decay; the nnterp Kimi-Linear page gives the
// decay-then-delta-rule order).  With S read once:
//
//   S_bar = diag(exp(g)) S
//   u     = S_bar^T k_hat,   p = S_bar^T q_hat          (one sweep over S_bar)
//   delta = beta (v - u)
//   o     = S_new^T q_hat = p + (k_hat . q_hat) delta
//   S_new = S_bar + k_hat delta^T                          (written back)
//
// so HBM sees exactly one read and one write of the state, 2*dk*dv*4 bytes
// per (sequence, head), which bounds the kernel.
//
// With GATED, g and beta are the raw gate and raw beta (q/k/v dtype),
// activated here as they are loaded.
//
// Launch: one 256-thread workgroup per (sequence, head).  Thread (cg, rg)
// owns value columns 4cg..4cg+3 of rows rg, rg+NRG, ...: every load and store
// of the state is a float4, and a wave touches whole 512-byte rows.
#include <type_traits>

#include "kda_bf16_mfma.h"
#include "kda_internal.h"

namespace kda {

// Sum over the lanes of a group of G consecutive lanes (G a power of two).
__device__ __forceinline__ float group_sum(float x, int G) {
    for (int off = 1; off < G; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// TRANS: the state block is S^T[dv][dk].  The thread then owns key rows
// 4cg..4cg+3 of value columns rg, rg+NRG, ...: the same float4 addresses, and
// each column's contraction over the key rows is a sum over the NCG lanes of
// one lane group, with no exchange between waves.
// NORM: the output epilogue is applied before anything is written: the
// step's output row (all dv values of one (sequence, head), which this
// workgroup holds) goes through LDS to wave 0, which writes
// o / sqrt(mean(o^2) + eps) * weight * sigmoid(out_gate) (the Ascend model
// file's `_project_out` norm and gate), so o itself never reaches HBM.
template <int D, typename TIn, typename TOut, bool GATED, bool TRANS, bool NORM>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta, GateParams gp, int gph, float* __restrict__ state,
    TOut* __restrict__ out, int num_heads, float scale, int l2norm, NormParams np) {
    constexpr int NCG = D / 4;      // column groups of four
    constexpr int NRG = 256 / NCG;  // row groups
    constexpr int RPT = D / NRG;    // rows per thread
    static_assert(NRG * NCG == 256 && RPT * NRG == D, "tiling");

    const int pair = blockIdx.x;  // n * H + h; also the token row of q/k/v/g/beta
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid % NCG, rg = tid / NCG;

    float* S = state + static_cast<size_t>(pair) * D * D;

    // Issue the state loads first; they are the bulk of the traffic.
    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = *reinterpret_cast<const floatx4*>(S + (rg + NRG * i) * D + 4 * cg);

    __shared__ float sq[D], sk[D], se[D];
    __shared__ float red[4][NCG][8];
    __shared__ float so[NORM ? D : 1];  // the output row on its way to the epilogue
    if (tid < D) {
        const size_t off = static_cast<size_t>(pair) * D + tid;
        sq[tid] = to_f32(q[off]);
        sk[tid] = to_f32(k[off]);
        // one decay per head: every channel reads the head's value
        const size_t goff = gph ? static_cast<size_t>(pair) : off;
        float gv;
        if constexpr (GATED) {
            const int h = pair % num_heads;
            gv = gate_g(to_f32(static_cast<const TIn*>(g)[goff]), gp.dt_bias[gph ? h : h * D + tid],
                        gate_exp(gp.a_log[h]), gp.lower_bound, gp.has_lower_bound);
        } else {
            gv = static_cast<const float*>(g)[goff];
        }
        se[tid] = fast_exp2(gv * kLog2e);
    }
    __syncthreads();

    // Norms and k.q, computed by every wave (no extra barrier needed).
    float aq = 0.f, ak = 0.f, aqk = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += 64) {
        const float qq = sq[c], kk = sk[c];
        aq += qq * qq;
        ak += kk * kk;
        aqk += qq * kk;
    }
    aq = wave_sum_from(aq, 1);
    ak = wave_sum_from(ak, 1);
    aqk = wave_sum_from(aqk, 1);
    const float rq = (l2norm ? rsqrtf(aq + kNormEps) : 1.f) * scale;
    const float rk = l2norm ? rsqrtf(ak + kNormEps) : 1.f;

    if constexpr (TRANS) {
        const floatx4 e4 = {se[4 * cg], se[4 * cg + 1], se[4 * cg + 2], se[4 * cg + 3]};
        const floatx4 k4 = {sk[4 * cg], sk[4 * cg + 1], sk[4 * cg + 2], sk[4 * cg + 3]};
        const floatx4 q4 = {sq[4 * cg], sq[4 * cg + 1], sq[4 * cg + 2], sq[4 * cg + 3]};
        float b;
        if constexpr (GATED)
            b = gate_sigmoid(to_f32(static_cast<const TIn*>(beta)[pair]));
        else
            b = static_cast<const float*>(beta)[pair];
        const float kq = rk * rq * aqk;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = rg + NRG * i;
            s[i] *= e4;
            const float u = group_sum(s[i][0] * k4[0] + s[i][1] * k4[1] + s[i][2] * k4[2] + s[i][3] * k4[3], NCG) * rk;
            const float p = group_sum(s[i][0] * q4[0] + s[i][1] * q4[1] + s[i][2] * q4[2] + s[i][3] * q4[3], NCG) * rq;
            const float delta = b * (to_f32(v[static_cast<size_t>(pair) * D + c]) - u);
            s[i] += (rk * delta) * k4;
            __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4*>(S + c * D + 4 * cg));
            if (cg == 0) {
                if constexpr (NORM)
                    so[c] = p + kq * delta;
                else
                    out[static_cast<size_t>(pair) * D + c] = from_f32<TOut>(p + kq * delta);
            }
        }
    } else {
        // Decay, then the two partial contractions over this thread's rows.
        floatx4 pu = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + NRG * i;
            s[i] *= se[r];
            pu += sk[r] * s[i];
            pp += sq[r] * s[i];
        }
        // Lanes of one wave that share cg differ by multiples of NCG.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pu[j] = wave_sum_from(pu[j], NCG);
            pp[j] = wave_sum_from(pp[j], NCG);
        }
        if (lane < NCG) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                red[wave][lane][j] = pu[j];
                red[wave][lane][4 + j] = pp[j];
            }
        }
        __syncthreads();
        floatx4 u, p;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] = (red[0][cg][j] + red[1][cg][j] + red[2][cg][j] + red[3][cg][j]) * rk;
            p[j] = (red[0][cg][4 + j] + red[1][cg][4 + j] + red[2][cg][4 + j] + red[3][cg][4 + j]) * rq;
        }

        const size_t voff = static_cast<size_t>(pair) * D + 4 * cg;
        float b;
        if constexpr (GATED)
            b = gate_sigmoid(to_f32(static_cast<const TIn*>(beta)[pair]));
        else
            b = static_cast<const float*>(beta)[pair];
        floatx4 delta;
#pragma unroll
        for (int j = 0; j < 4; ++j) delta[j] = b * (to_f32(v[voff + j]) - u[j]);

        // The state is not read again in this step: non-temporal stores stream it
        // out without keeping it in the caches (measured ~25 % more HBM throughput
        // than plain stores for this read-then-write pattern).
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + NRG * i;
            s[i] += (rk * sk[r]) * delta;
            __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4*>(S + r * D + 4 * cg));
        }
        if (rg == 0) {
            const float kq = rk * rq * aqk;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (NORM)
                    so[4 * cg + j] = p[j] + kq * delta[j];
                else
                    out[voff + j] = from_f32<TOut>(p[j] + kq * delta[j]);
            }
        }
    }
    if constexpr (NORM) {
        __syncthreads();
        if (wave == 0) {
            float ss = 0.f;
#pragma unroll
            for (int c = lane; c < D; c += 64) ss += so[c] * so[c];
            ss = wave_sum_from(ss, 1);
            const float r = rsqrtf(ss * (1.f / D) + np.eps);
            const TIn* og = static_cast<const TIn*>(np.gate) + static_cast<size_t>(pair) * D;
#pragma unroll
            for (int c = lane; c < D; c += 64)
                out[static_cast<size_t>(pair) * D + c] =
                    from_f32<TOut>(so[c] * r * np.weight[c] * gate_sigmoid(to_f32(og[c])));
        }
    }
}

// Element loads of 16- or 32-bit values, kept as raw bits until used (a
// conversion at the load would make the wave wait for it there).
template <typename T>
__device__ __forceinline__ uint32_t load_bits(__amdgpu_buffer_rsrc_t r, int off_bytes) {
    if constexpr (sizeof(T) == 2)
        return __builtin_amdgcn_raw_buffer_load_b16(r, off_bytes, 0, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b32(r, off_bytes, 0, 0);
}
template <typename T>
__device__ __forceinline__ float bits_f32(uint32_t u) {
    return sizeof(T) == 2 ? __uint_as_float(u << 16) : __uint_as_float(u);
}

// Four consecutive outputs at byte offset off of the resource.
template <typename TOut>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int off, const floatx4& x) {
    typedef int intx4 __attribute__((ext_vector_type(4)));
    typedef int intx2 __attribute__((ext_vector_type(2)));
    if constexpr (sizeof(TOut) == 4)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(intx4, x), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b64(
            intx2{static_cast<int>(pack_bf16x2(x[0], x[1])), static_cast<int>(pack_bf16x2(x[2], x[3]))}, r, off, 0, 0);
}
template <typename TOut>
__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, int off, float x) {
    if constexpr (sizeof(TOut) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(pack_bf16x2(x, 0.f)), r, off, 0, 0);
}

// Multi-token verify decode with state-slot indirection.  Sequence n has
// `width` tokens (rows n*width .. n*width+width-1) and one state slot per
// token, idx = indices[n*width ..]: it starts from the state in slot
// idx[a-1], a = accepted[n] clamped to [1, width] (a = 1 without accepted),
// and the state after its token t is written to slot idx[t].  A slot outside
// [0, num_slots) reads as the zero state and is not written.  The whole
// starting state is read before anything is written, so idx[a-1] may also
// appear among the destinations.  Each token is the decode step above.
// NORM: each token's output row gets the gated RMSNorm of decode_step_kernel
// before it is written, so o itself never reaches HBM.  With S[dk][dv] every
// row group holds the whole row and applies it in registers; with S^T the row
// goes through LDS and every wave applies it after the token's last barrier.
// The token's output-gate row is loaded with its q and k, and the norm weight
// once, both into LDS; the gate row alternates between two buffers, since the
// next token's is stored while this one's may still be read.
template <int D, typename TIn, typename TOut, bool GATED, bool TRANS, bool NORM>
__global__ __launch_bounds__(256) void verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const void* __restrict__ g, const void* __restrict__ beta, GateParams gp, int gph, float* __restrict__ pool,
    int num_slots, const int32_t* __restrict__ indices, const int32_t* __restrict__ accepted,
    TOut* __restrict__ out, int num_heads, int width, float scale, int l2norm, NormParams np) {
    constexpr int NCG = D / 4;
    constexpr int NRG = 256 / NCG;
    constexpr int RPT = D / NRG;
    static_assert(NRG * NCG == 256 && RPT * NRG == D, "tiling");
    constexpr int kNonTemporal = 2;  // buffer cache policy: the states are not read back here

    const int pair = blockIdx.x;  // n * H + h
    const int n = pair / num_heads, h = pair - n * num_heads;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cg = tid % NCG, rg = tid / NCG;
    const int32_t* idx = indices + static_cast<size_t>(n) * width;
    const size_t slot_stride = static_cast<size_t>(num_heads) * D * D;
    auto slot_ptr = [&](int slot) -> float* {
        return (slot >= 0 && slot < num_slots) ? pool + slot * slot_stride + static_cast<size_t>(h) * D * D
                                               : nullptr;
    };
    // The state block of a slot as a buffer resource: an invalid slot gets an
    // empty range, so its stores are dropped and no branch surrounds them.
    auto slot_rsrc = [&](int slot) {
        float* S = slot_ptr(slot);
        return buffer_rsrc(S ? S : pool, S ? D * D * 4 : 0);
    };
    // byte offset of this thread's row i of the block
    auto s_off = [&](int i) { return ((rg + NRG * i) * D + 4 * cg) * 4; };

    int a = accepted ? accepted[n] : 1;
    a = a < 1 ? 1 : (a > width ? width : a);
    floatx4 s[RPT];
    {
        const auto sr = slot_rsrc(idx[a - 1]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(sr, s_off(i), 0, 0));
    }

    // per-token rows, one entry per thread (threads >= D write entries that are never read)
    __shared__ float sq[256], sk[256], se[256], sv[256];
    __shared__ float red[4][NCG][8];
    __shared__ float so[TRANS ? D : 1];                  // TRANS: the token's output row
    __shared__ float sog[NORM ? 2 : 1][NORM ? 256 : 1];  // sigmoid of the output-gate row of token t in [t & 1]
    __shared__ float snw[NORM ? D : 1];                   // the norm weight
    if constexpr (NORM) {
        if (tid < D) snw[tid] = np.weight[tid];
    }
    // A token's inputs, loaded raw one token ahead (the last token's again
    // after the last), so their loads fly while the previous token is
    // computed and its state stored.  Thread c < D takes channel c of q, k, v,
    // g and the output gate; threads past D read past the row, which gives
    // zeros; every thread takes beta.  No branch surrounds a load or a store
    // in the token loop, so the wait for these loads counts exactly the
    // stores issued after them and never waits for those stores.
    typedef std::conditional_t<GATED, TIn, float> GIn;
    typedef std::conditional_t<GATED, TIn, float> BIn;
    const int ct = tid & (D - 1);  // the channel of this thread's LDS entries
    const int eo = tid < D ? tid : D;
    uint32_t nq, nk, nv, ngate = 0, ng, nb;
    auto fetch = [&](int t) {
        const size_t tok = (static_cast<size_t>(n) * width + t) * num_heads + h;
        nq = load_bits<TIn>(buffer_rsrc(q + tok * D, D * sizeof(TIn)), eo * sizeof(TIn));
        nk = load_bits<TIn>(buffer_rsrc(k + tok * D, D * sizeof(TIn)), eo * sizeof(TIn));
        nv = load_bits<TIn>(buffer_rsrc(v + tok * D, D * sizeof(TIn)), eo * sizeof(TIn));
        if constexpr (NORM)
            ngate = load_bits<TIn>(buffer_rsrc(static_cast<const TIn*>(np.gate) + tok * D, D * sizeof(TIn)),
                                   eo * sizeof(TIn));
        const GIn* gb = static_cast<const GIn*>(g) + (gph ? tok : tok * D);
        ng = load_bits<GIn>(buffer_rsrc(gb, (gph ? 1 : D) * sizeof(GIn)), (gph ? (tid < D ? 0 : 1) : eo) * sizeof(GIn));
        nb = load_bits<BIn>(buffer_rsrc(static_cast<const BIn*>(beta) + tok, sizeof(BIn)), 0);
    };
    fetch(0);
    // The first token needs the state and its inputs anyway; waiting here also
    // keeps the compiler's count at the loop head to what the loop issues (it
    // merges the entry path into every iteration).
    wait_vmcnt<0>();
    for (int t = 0; t < width; ++t) {
        const size_t row = static_cast<size_t>(n) * width + t;  // token row
        const size_t tok = row * num_heads + h;                  // (token, head)
        sq[tid] = bits_f32<TIn>(nq);
        sk[tid] = bits_f32<TIn>(nk);
        sv[tid] = bits_f32<TIn>(nv);
        if constexpr (NORM) sog[t & 1][tid] = gate_sigmoid(bits_f32<TIn>(ngate));
        float gv;
        if constexpr (GATED)
            gv = gate_g(bits_f32<GIn>(ng), gp.dt_bias[gph ? h : h * D + ct], gate_exp(gp.a_log[h]), gp.lower_bound,
                        gp.has_lower_bound);
        else
            gv = bits_f32<GIn>(ng);
        se[tid] = fast_exp2(gv * kLog2e);
        float b;
        if constexpr (GATED)
            b = gate_sigmoid(bits_f32<BIn>(nb));
        else
            b = bits_f32<BIn>(nb);
        fetch(t + 1 < width ? t + 1 : t);
        __syncthreads();
        float aq = 0.f, ak = 0.f, aqk = 0.f;
#pragma unroll
        for (int c = lane; c < D; c += 64) {
            const float qq = sq[c], kk = sk[c];
            aq += qq * qq;
            ak += kk * kk;
            aqk += qq * kk;
        }
        aq = wave_sum_from(aq, 1);
        ak = wave_sum_from(ak, 1);
        aqk = wave_sum_from(aqk, 1);
        const float rq = (l2norm ? rsqrtf(aq + kNormEps) : 1.f) * scale;
        const float rk = l2norm ? rsqrtf(ak + kNormEps) : 1.f;
        const float kq = rk * rq * aqk;
        const auto sr = slot_rsrc(idx[t]);
        const auto orr = buffer_rsrc(out + tok * D, D * sizeof(TOut));
        if constexpr (TRANS) {
            const floatx4 e4 = {se[4 * cg], se[4 * cg + 1], se[4 * cg + 2], se[4 * cg + 3]};
            const floatx4 k4 = {sk[4 * cg], sk[4 * cg + 1], sk[4 * cg + 2], sk[4 * cg + 3]};
            const floatx4 q4 = {sq[4 * cg], sq[4 * cg + 1], sq[4 * cg + 2], sq[4 * cg + 3]};
            typedef int intx4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int c = rg + NRG * i;
                s[i] *= e4;
                const float u =
                    group_sum(s[i][0] * k4[0] + s[i][1] * k4[1] + s[i][2] * k4[2] + s[i][3] * k4[3], NCG) * rk;
                const float p =
                    group_sum(s[i][0] * q4[0] + s[i][1] * q4[1] + s[i][2] * q4[2] + s[i][3] * q4[3], NCG) * rq;
                const float delta = b * (sv[c] - u);
                s[i] += (rk * delta) * k4;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(intx4, s[i]), sr, s_off(i), 0, kNonTemporal);
                if (cg == 0) so[c] = p + kq * delta;
            }
        } else {
            floatx4 pu = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg + NRG * i;
                s[i] *= se[r];
                pu += sk[r] * s[i];
                pp += sq[r] * s[i];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pu[j] = wave_sum_from(pu[j], NCG);
                pp[j] = wave_sum_from(pp[j], NCG);
            }
            if (lane < NCG) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    red[wave][lane][j] = pu[j];
                    red[wave][lane][4 + j] = pp[j];
                }
            }
            __syncthreads();
            // every thread gets its four columns' u and p (the same in each row group)
            floatx4 u, p;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u[j] = (red[0][cg][j] + red[1][cg][j] + red[2][cg][j] + red[3][cg][j]) * rk;
                p[j] = (red[0][cg][4 + j] + red[1][cg][4 + j] + red[2][cg][4 + j] + red[3][cg][4 + j]) * rq;
            }
            floatx4 delta;
#pragma unroll
            for (int j = 0; j < 4; ++j) delta[j] = b * (sv[4 * cg + j] - u[j]);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg + NRG * i;
                s[i] += (rk * sk[r]) * delta;
                typedef int intx4 __attribute__((ext_vector_type(4)));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(intx4, s[i]), sr, s_off(i), 0, kNonTemporal);
            }
            floatx4 ov;
#pragma unroll
            for (int j = 0; j < 4; ++j) ov[j] = p[j] + kq * delta[j];
            if constexpr (NORM) {
                // each row group holds the whole output row (four columns per
                // lane of its NCG lanes): the epilogue runs in registers
                float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
                for (int m = 1; m < NCG; m <<= 1) ss += __shfl_xor(ss, m, 64);
                const float r = rsqrtf(ss * (1.f / D) + np.eps);
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] *= r * snw[4 * cg + j] * sog[t & 1][4 * cg + j];
            }
            // row group 0 stores the row (the others aim past its end)
            store4<TOut>(orr, rg == 0 ? 4 * cg * static_cast<int>(sizeof(TOut)) : D * static_cast<int>(sizeof(TOut)),
                         ov);
        }
        // sq, sk, sv, se, red and so are rewritten by the next token
        __syncthreads();
        if constexpr (TRANS) {
            // the row from LDS, one element per thread c < D (so is rewritten
            // only after the next token's first barrier, which every wave
            // reaches after reading it here)
            float o = so[ct];
            if constexpr (NORM) {
                float ss = 0.f;
#pragma unroll
                for (int c = lane; c < D; c += 64) ss += so[c] * so[c];
                ss = wave_sum_from(ss, 1);
                o *= rsqrtf(ss * (1.f / D) + np.eps) * snw[ct] * sog[t & 1][ct];
            }
            store1<TOut>(orr, eo * static_cast<int>(sizeof(TOut)), o);
        }
    }
}

template <int D, typename TIn, typename TOut>
static hipError_t launch_verify_t(const VerifyArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads));
    const TIn* q = static_cast<const TIn*>(a.q);
    const TIn* k = static_cast<const TIn*>(a.k);
    const TIn* v = static_cast<const TIn*>(a.v);
    auto pick = [&](auto norm) {
        constexpr bool N = decltype(norm)::value;
        return a.gate.a_log ? (a.state_trans ? verify_kernel<D, TIn, TOut, true, true, N>
                                             : verify_kernel<D, TIn, TOut, true, false, N>)
                            : (a.state_trans ? verify_kernel<D, TIn, TOut, false, true, N>
                                             : verify_kernel<D, TIn, TOut, false, false, N>);
    };
    auto* kern = a.norm.gate ? pick(std::true_type{}) : pick(std::false_type{});
    kern<<<grid, 256, 0, stream>>>(q, k, v, a.g, a.beta, a.gate, a.gate_per_head, a.pool, a.num_slots, a.indices,
                                   a.accepted, static_cast<TOut*>(a.out), a.num_heads, a.width, a.scale, a.l2norm,
                                   a.norm);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_verify_d(const VerifyArgs& a, hipStream_t stream) {
    if (a.qkv_bf16)
        return a.out_bf16 ? launch_verify_t<D, bf16_t, bf16_t>(a, stream) : launch_verify_t<D, bf16_t, float>(a, stream);
    return a.out_bf16 ? launch_verify_t<D, float, bf16_t>(a, stream) : launch_verify_t<D, float, float>(a, stream);
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    return a.head_dim == 128 ? launch_verify_d<128>(a, stream) : launch_verify_d<64>(a, stream);
}

template <int D, typename TIn, typename TOut>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads));
    const TIn* q = static_cast<const TIn*>(a.q);
    const TIn* k = static_cast<const TIn*>(a.k);
    const TIn* v = static_cast<const TIn*>(a.v);
    auto pick = [&](auto norm) {
        constexpr bool N = decltype(norm)::value;
        return a.gate.a_log ? (a.state_trans ? decode_step_kernel<D, TIn, TOut, true, true, N>
                                             : decode_step_kernel<D, TIn, TOut, true, false, N>)
                            : (a.state_trans ? decode_step_kernel<D, TIn, TOut, false, true, N>
                                             : decode_step_kernel<D, TIn, TOut, false, false, N>);
    };
    auto* kern = a.norm.gate ? pick(std::true_type{}) : pick(std::false_type{});
    kern<<<grid, 256, 0, stream>>>(q, k, v, a.g, a.beta, a.gate, a.gate_per_head, a.state, static_cast<TOut*>(a.out),
                                   a.num_heads, a.scale, a.l2norm, a.norm);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    if (a.qkv_bf16) {
        return a.out_bf16 ? launch_decode_t<D, bf16_t, bf16_t>(a, stream)
                          : launch_decode_t<D, bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? launch_decode_t<D, float, bf16_t>(a, stream)
                      : launch_decode_t<D, float, float>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    return a.head_dim == 128 ? launch_decode_d<128>(a, stream) : launch_decode_d<64>(a, stream);
}

}  // namespace kda
