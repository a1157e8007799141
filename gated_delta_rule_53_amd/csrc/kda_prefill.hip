// KDA chunked prefill over packed variable-length sequences.
//
// The chunk algorithm is the one of the Ascend Kimi-Linear model file
// (`_torch_chunk_kda`): per chunk of C = 64 tokens with input state S
// (dk x dv), cumulative log-decay G[r] = sum_{s<=r} g[s] inside the chunk,
// Gamma[r] = exp(G[r]) and normalised q, k,
//
//   A[r,i] = beta_r sum_c k[r,c] k[i,c] exp(G[r,c]-G[i,c])       (i < r)
//   P[r,i] =        sum_c q[r,c] k[i,c] exp(G[r,c]-G[i,c])       (i <= r)
//   (I + A) Delta = diag(beta) (V - (Gamma*K) S)
//   O  = (Gamma*Q) S + P Delta
//   S' = diag(Gamma[last]) S + (K * exp(G[last]-G))^T Delta
//
// Design for gfx950 (what differs from the page's listing):
//   * One 256-thread workgroup owns one (sequence, head, 16-wide value tile).
//     The value columns of S evolve independently, so a head's state is split
//     over dv/16 workgroups that run the chunk chain side by side; their
//     linear ids are congruent mod 8 so they share one XCD and its L2 for the
//     common q/k/g reads.  Only the dv-dependent products are per tile.
//   * Delta is computed as (I+A)^{-1} [diag(beta)(V - (Gamma*K) S)]: the WY
//     matrices W = T Gamma K and U = T V of the listing are never formed.
//   * (I+A)^{-1} is built blockwise: 16x16 diagonal blocks by forward
//     substitution, off-diagonal blocks by X_RI = -X_RR sum_J L_RJ X_JI.
//   * exp(G[r]-G[i]) is factored through the start s_B of 16-token blocks:
//     row side k[r] exp(G[r]-G[s_R]) (<= 1), column side k[i] exp(G[s_I]-G[i])
//     (>= 1, bounded by one block's decay) and a per-channel block factor
//     exp(G[s_R]-G[s_I]) (<= 1).  All contractions then run on MFMA.  A chunk
//     in which some block's decay exceeds kRefSpan (the column side would
//     leave the float range) forms A and P exactly instead: for each column
//     i the vector k[i] exp(G[r]-G[i]) is carried down the rows by products
//     of exp(g[r]) <= 1, and the state update takes k exp(G[last]-G) directly.
//   * The state tile lives in MFMA accumulators across the whole chunk chain;
//     a copy in LDS feeds the (Gamma*K) S and (Gamma*Q) S products.
//   * A tail chunk is masked, not padded: rows past the sequence end read as
//     k = q = v = g = beta = 0, which makes them no-ops.
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kC = 64;     // chunk length
constexpr int kDVT = 16;   // value columns per workgroup
constexpr int kSC = kC + 2;  // LDS row stride of 64x64 matrices (floats)
// Largest decay (natural log) one 16-token block may span on the factored
// path: exp(60) is well inside the float32 range.
constexpr float kRefSpan = 60.f;

__device__ __forceinline__ int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }

}  // namespace

// With GATED, g and beta are the raw gate and raw beta (q/k/v dtype),
// activated as each chunk is staged; rows past a sequence's end get g = beta = 0.
template <int D, typename TIn, typename TOut, bool GATED>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const void* __restrict__ g_in, const void* __restrict__ beta_in, GateParams gp, int gph,
    const int32_t* __restrict__ cu_seqlens, const float* initial_state, TOut* __restrict__ out,
    float* final_state, const int32_t* __restrict__ slots, int num_slots, int64_t total_tokens, int num_seqs,
    int num_heads, float scale, int l2norm, int state_trans) {
    using GT = typename std::conditional<GATED, TIn, float>::type;  // element type of g and beta
    const GT* __restrict__ g = static_cast<const GT*>(g_in);
    const GT* __restrict__ beta = static_cast<const GT*>(beta_in);
    constexpr int SD = D + 2;           // LDS row stride of [64][D] buffers (floats)
    constexpr int NSEG = 256 / D;       // token segments per channel in the cumsum
    constexpr int SEGLEN = kC / NSEG;
    constexpr int CBW = D / 64;         // 16-row state blocks per wave

    const int chain = blockIdx.x;
    if (chain >= num_seqs * num_heads) return;
    const int n = chain / num_heads, h = chain % num_heads;
    const int col0 = blockIdx.y * kDVT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, l4 = lane >> 4;

    int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
    if (t0 < 0 || t1 > total_tokens || t1 < t0) t1 = t0;  // malformed: no tokens

    __shared__ float sKl[kC * SD];   // k_hat[r] exp(G[r]-G[s_R]); later X = (I+A)^{-1}
    __shared__ float sQl[kC * SD];   // q_hat[r] exp(G[r]-G[s_R]); later scratch
    __shared__ float sKi[kC * SD];   // k_hat[r] exp(G[s_R]-G[r])
    __shared__ float sL[kC * kSC];   // I + A
    __shared__ float sP[kC * kSC];   // P
    __shared__ float sS[D * kDVT];   // state tile at chunk start
    __shared__ float sY[kC * kDVT];  // diag(beta)(V - Gamma K S), then Delta
    __shared__ float sV[kC * kDVT];  // value tile of the chunk
    __shared__ float srk[kC], srq[kC], sbeta[kC];
    __shared__ float sB[4 * D];      // G at block starts (log2 units)
    __shared__ float sGam[4 * D];    // exp(G[s_R])
    __shared__ float sFL[4 * D];     // exp(G[last]-G[s_R])
    __shared__ float sFb[6 * D];     // exp(G[s_R]-G[s_I]), I < R
    __shared__ float sGLlog[D], sGL[D];
    __shared__ float sCarry[NSEG * D];
    float* sX = sKl;
    float* sT = sQl;

    size_t head_state = 0;
    const bool has_state = state_block(slots, num_slots, n, h, num_heads, D, head_state);
    const float* init = has_state ? initial_state : nullptr;
    float* fin = has_state ? final_state : nullptr;
    KDA_PHASE_BEGIN

    floatx4 Sacc[CBW];
#pragma unroll
    for (int b = 0; b < CBW; ++b) {
        const int cb = wave * CBW + b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 16 * cb + 4 * l4 + j;
            const float s = init ? init[head_state + state_elem(c, col0 + l16, D, state_trans)] : 0.f;
            Sacc[b][j] = s;
            sS[c * kDVT + l16] = s;
        }
    }
    __syncthreads();

    // Register prefetch of one chunk.  Thread (pq, pc) holds rows 4pq..4pq+3 and
    // channels CPT*pc .. CPT*pc+CPT-1 of k, q and g; threads < 128 hold half a row
    // of the value tile, threads < 64 one beta.
    constexpr int CPT = D / 16;
    const int pq = tid >> 4, pc = tid & 15;
    alignas(16) TIn pk[4][CPT];
    alignas(16) TIn pqv[4][CPT];
    alignas(16) GT pg[4][CPT];
    // gate parameters of this thread's channels (one head per workgroup)
    float gbias[CPT], ga = 0.f;
    if constexpr (GATED) {
        ga = gate_exp(gp.a_log[h]);
#pragma unroll
        for (int i = 0; i < CPT; ++i) gbias[i] = gp.dt_bias[gph ? h : h * D + CPT * pc + i];
    }
    int valid_rows = 0;  // rows of the prefetched chunk inside the sequence
    alignas(16) TIn pv[8];
    float pb = 0.f;
    auto fetch = [&](int64_t c0) {
        const int Ln = static_cast<int>(min<int64_t>(kC, t1 - c0));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * pq + j;
            if (r < Ln) {
                const size_t off = (static_cast<size_t>(c0 + r) * num_heads + h) * D + CPT * pc;
                load_vec(pk[j], k + off);
                load_vec(pqv[j], q + off);
                if (gph) {  // one decay per head, the same for every channel
                    const GT gs = g[static_cast<size_t>(c0 + r) * num_heads + h];
#pragma unroll
                    for (int i = 0; i < CPT; ++i) pg[j][i] = gs;
                } else {
                    load_vec(pg[j], g + off);
                }
            } else {
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    pk[j][i] = from_f32<TIn>(0.f);
                    pqv[j][i] = from_f32<TIn>(0.f);
                    pg[j][i] = from_f32<GT>(0.f);
                }
            }
        }
        if (tid < 2 * kC) {
            const int r = tid >> 1;
            if (r < Ln) {
                load_vec(pv, v + (static_cast<size_t>(c0 + r) * num_heads + h) * D + col0 + 8 * (tid & 1));
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = from_f32<TIn>(0.f);
            }
        }
        if (tid < kC) {
            if constexpr (GATED)
                pb = tid < Ln ? gate_sigmoid(to_f32(beta[static_cast<size_t>(c0 + tid) * num_heads + h])) : 0.f;
            else
                pb = tid < Ln ? beta[static_cast<size_t>(c0 + tid) * num_heads + h] : 0.f;
        }
        valid_rows = Ln;
    };
    if (t0 < t1) fetch(t0);

    for (int64_t cs = t0; cs < t1; cs += kC) {
        const int L = static_cast<int>(min<int64_t>(kC, t1 - cs));

        // ---- stage the prefetched chunk in LDS, then prefetch the next one ----
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * pq + j;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                sKl[r * SD + CPT * pc + i] = to_f32(pk[j][i]);
                sQl[r * SD + CPT * pc + i] = to_f32(pqv[j][i]);
                float gv = to_f32(pg[j][i]);
                if constexpr (GATED)
                    gv = r < valid_rows ? gate_g(gv, gbias[i], ga, gp.lower_bound, gp.has_lower_bound) : 0.f;
                sKi[r * SD + CPT * pc + i] = gv * kLog2e;
            }
        }
        if (tid < 2 * kC) {
#pragma unroll
            for (int i = 0; i < 8; ++i) sV[(tid >> 1) * kDVT + 8 * (tid & 1) + i] = to_f32(pv[i]);
        }
        if (tid < kC) sbeta[tid] = pb;
        __syncthreads();
        KDA_PHASE_MARK(1);
        if (cs + kC < t1) fetch(cs + kC);
        KDA_PHASE_MARK(2);

        // ---- row norms: four lanes per row ----
        {
            const int r = 16 * wave + (lane >> 2), part = lane & 3;
            float a = 0.f, b = 0.f;
            for (int c = part; c < D; c += 4) {
                const float kk = sKl[r * SD + c], qq = sQl[r * SD + c];
                a += kk * kk;
                b += qq * qq;
            }
            a += __shfl_xor(a, 1, 64);
            a += __shfl_xor(a, 2, 64);
            b += __shfl_xor(b, 1, 64);
            b += __shfl_xor(b, 2, 64);
            if (part == 0) {
                srk[r] = l2norm ? rsqrtf(a + kNormEps) : 1.f;
                srq[r] = (l2norm ? rsqrtf(b + kNormEps) : 1.f) * scale;
            }
        }

        // ---- cumulative log-decay per channel: local prefix, then carry ----
        const int c = tid % D, seg = tid / D;
        float Gv[SEGLEN];
        {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < SEGLEN; ++i) {
                acc += sKi[(seg * SEGLEN + i) * SD + c];
                Gv[i] = acc;
            }
            sCarry[seg * D + c] = acc;
        }
        __syncthreads();
        KDA_PHASE_MARK(4);
        int unsafe = 0;
        {
            float carry = 0.f;
            for (int s = 0; s < seg; ++s) carry += sCarry[s * D + c];
#pragma unroll
            for (int i = 0; i < SEGLEN; ++i) Gv[i] += carry;
#pragma unroll
            for (int i = 0; i < SEGLEN; ++i)
                if (((seg * SEGLEN + i) & 15) == 0) sB[((seg * SEGLEN + i) >> 4) * D + c] = Gv[i];
            if (seg == NSEG - 1) sGLlog[c] = Gv[SEGLEN - 1];
            // segments hold whole 16-token blocks: the column-side exponent
            // G[s_R] - G[r] of every row is known here (NaN counts as unsafe)
            static_assert(SEGLEN % 16 == 0, "segments of whole blocks");
#pragma unroll
            for (int i = 0; i < SEGLEN; ++i)
                unsafe |= !(Gv[i & ~15] - Gv[i] <= kRefSpan * kLog2e);
        }
        // every thread learns whether any channel of the chunk is out of range
        const bool exact = __syncthreads_or(unsafe) != 0;
        KDA_PHASE_MARK(5);
        if (exact) {
            // sKi holds g (log2 units): turn it into e^g in place
#pragma unroll
            for (int i = 0; i < SEGLEN; ++i) {
                float* p = &sKi[(seg * SEGLEN + i) * SD + c];
                *p = fast_exp2(*p);
            }
            __syncthreads();
            // thread (column i, part): channels part, part + 4, ...; z = k_hat[i]
            // exp(G[r] - G[i]) per channel, carried from row i down the rows.
            // With D = 128 the channels go in two passes of 16, to keep z in
            // registers next to the prefetched chunk; the first pass leaves
            // its partial sums in sL and sP.
            constexpr int CH = D / 4, CHP = CH > 16 ? 16 : CH, NP = CH / CHP;
            const int ic = tid >> 2, part = tid & 3;
            const float rki = srk[ic];
            for (int hp = 0; hp < NP; ++hp) {
                float z[CHP];
#pragma unroll
                for (int m = 0; m < CHP; ++m) z[m] = 0.f;
                for (int r = 0; r < kC; ++r) {
                    float a = 0.f, p = 0.f;
#pragma unroll
                    for (int m = 0; m < CHP; ++m) {
                        const int o = r * SD + 4 * (hp * CHP + m) + part;
                        const float kr = sKl[o];
                        z[m] = r == ic ? kr * rki : z[m] * sKi[o];
                        a += kr * z[m];
                        p += sQl[o] * z[m];
                    }
                    a += __shfl_xor(a, 1, 64);
                    a += __shfl_xor(a, 2, 64);
                    p += __shfl_xor(p, 1, 64);
                    p += __shfl_xor(p, 2, 64);
                    if (part == 0) {
                        const int o = r * kSC + ic;
                        if (hp > 0) {
                            a += sL[o];
                            p += sP[o];
                        }
                        if (hp + 1 < NP) {
                            sL[o] = a;
                            sP[o] = p;
                        } else {
                            sL[o] = ic < r ? sbeta[r] * srk[r] * a : (ic == r ? 1.f : 0.f);
                            sP[o] = ic <= r ? srq[r] * p : 0.f;
                        }
                    }
                }
            }
            __syncthreads();
        }

        // ---- scaled operands and per-channel block factors ----
#pragma unroll
        for (int i = 0; i < SEGLEN; ++i) {
            const int r = seg * SEGLEN + i;
            const float Bv = sB[(r >> 4) * D + c];
            const float kk = sKl[r * SD + c] * srk[r];
            const float qq = sQl[r * SD + c] * srq[r];
            const float e = fast_exp2(Gv[i] - Bv);
            // exact path: k exp(G[last] - G), for the state update only
            const float einv = fast_exp2(exact ? sGLlog[c] - Gv[i] : Bv - Gv[i]);
            sKl[r * SD + c] = kk * e;
            sQl[r * SD + c] = qq * e;
            sKi[r * SD + c] = kk * einv;
        }
        if (seg == 0) {
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                sGam[R * D + c] = fast_exp2(sB[R * D + c]);
                for (int I = 0; I < R; ++I)
                    sFb[pair_index(R, I) * D + c] = fast_exp2(sB[R * D + c] - sB[I * D + c]);
            }
        }
        if (seg == NSEG - 1) {
            const float gl = sGLlog[c];
#pragma unroll
            for (int R = 0; R < 4; ++R) sFL[R * D + c] = exact ? 1.f : fast_exp2(gl - sB[R * D + c]);
            sGL[c] = fast_exp2(gl);
        }
        __syncthreads();
        KDA_PHASE_MARK(6);

        // ---- Z = (Gamma K) S and Oq = (Gamma Q) S for row block R = wave ----
        floatx4 Z = {0.f, 0.f, 0.f, 0.f}, Oq = {0.f, 0.f, 0.f, 0.f};
        {
            const int R = wave, r = 16 * R + l16;
            for (int k0 = 0; k0 < D; k0 += 4) {
                const int cc = k0 + l4;
                const float gam = sGam[R * D + cc];
                const float bS = sS[cc * kDVT + l16];
                Z = mfma_f32_16x16x4(sKl[r * SD + cc] * gam, bS, Z);
                Oq = mfma_f32_16x16x4(sQl[r * SD + cc] * gam, bS, Oq);
            }
        }
        // ---- A and P, block pairs (R, I <= R) spread over the waves (exact path: done) ----
        for (int pi = exact ? 10 : wave; pi < 10; pi += 4) {
            const int R = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
            const int I = pi - R * (R + 1) / 2;
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            const int ra = 16 * R + l16, ib = 16 * I + l16;
            for (int k0 = 0; k0 < D; k0 += 4) {
                const int cc = k0 + l4;
                const float fb = I < R ? sFb[pair_index(R, I) * D + cc] : 1.f;
                const float bK = sKi[ib * SD + cc] * fb;
                accA = mfma_f32_16x16x4(sKl[ra * SD + cc], bK, accA);
                accP = mfma_f32_16x16x4(sQl[ra * SD + cc], bK, accP);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j, i = ib;
                float lv, pv;
                if (I < R) {
                    lv = sbeta[r] * accA[j];
                    pv = accP[j];
                } else {
                    lv = i < r ? sbeta[r] * accA[j] : (i == r ? 1.f : 0.f);
                    pv = i <= r ? accP[j] : 0.f;
                }
                sL[r * kSC + i] = lv;
                sP[r * kSC + i] = pv;
            }
        }
        __syncthreads();
        KDA_PHASE_MARK(7);

        // ---- diagonal blocks of X = (I+A)^{-1}; Y = diag(beta)(V - Z) ----
        {
            const int R = wave;
            if (lane < 16) {
                const int j = lane;
                float x[16];
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    float s = (m == j) ? 1.f : 0.f;
#pragma unroll
                    for (int p = 0; p < m; ++p) s -= sL[(16 * R + m) * kSC + 16 * R + p] * x[p];
                    x[m] = s;
                }
#pragma unroll
                for (int m = 0; m < 16; ++m) sX[(16 * R + m) * kSC + 16 * R + j] = x[m];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                sY[r * kDVT + l16] = sbeta[r] * (sV[r * kDVT + l16] - Z[j]);
            }
        }
        __syncthreads();
        KDA_PHASE_MARK(8);

        // ---- off-diagonal blocks of X, one block distance at a time ----
#pragma unroll
        for (int dist = 1; dist < 4; ++dist) {
            const bool active = wave < 4 - dist;
            const int I = wave, R = wave + dist;
            float* T = sT + wave * 16 * 17;
            if (active) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int J = I; J < R; ++J) {
#pragma unroll
                    for (int k0 = 0; k0 < 16; k0 += 4)
                        acc = mfma_f32_16x16x4(sL[(16 * R + l16) * kSC + 16 * J + k0 + l4],
                                               sX[(16 * J + k0 + l4) * kSC + 16 * I + l16], acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) T[(4 * l4 + j) * 17 + l16] = acc[j];
            }
            __syncthreads();
        KDA_PHASE_MARK(9);
            if (active) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    acc = mfma_f32_16x16x4(sX[(16 * R + l16) * kSC + 16 * R + k0 + l4],
                                           T[(k0 + l4) * 17 + l16], acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) sX[(16 * R + 4 * l4 + j) * kSC + 16 * I + l16] = -acc[j];
            }
            __syncthreads();
        KDA_PHASE_MARK(10);
        }

        // ---- Delta = X Y for row block R = wave ----
        floatx4 Dl = {0.f, 0.f, 0.f, 0.f};
        {
            const int R = wave;
            for (int I = 0; I <= R; ++I) {
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    Dl = mfma_f32_16x16x4(sX[(16 * R + l16) * kSC + 16 * I + k0 + l4],
                                          sY[(16 * I + k0 + l4) * kDVT + l16], Dl);
            }
        }
        __syncthreads();
        KDA_PHASE_MARK(11);
#pragma unroll
        for (int j = 0; j < 4; ++j) sY[(16 * wave + 4 * l4 + j) * kDVT + l16] = Dl[j];
        __syncthreads();
        KDA_PHASE_MARK(12);

        // ---- O = Oq + P Delta, written out ----
        {
            const int R = wave;
            floatx4 acc = Oq;
            for (int I = 0; I <= R; ++I) {
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    acc = mfma_f32_16x16x4(sP[(16 * R + l16) * kSC + 16 * I + k0 + l4],
                                           sY[(16 * I + k0 + l4) * kDVT + l16], acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                if (r < L)
                    out[(static_cast<size_t>(cs + r) * num_heads + h) * D + col0 + l16] =
                        from_f32<TOut>(acc[j]);
            }
        }
        // ---- S = diag(Gamma[last]) S + (K exp(G[last]-G))^T Delta ----
#pragma unroll
        for (int b = 0; b < CBW; ++b) {
            const int cb = wave * CBW + b;
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[b][j] *= sGL[16 * cb + 4 * l4 + j];
            const int cc = 16 * cb + l16;
            for (int r0 = 0; r0 < kC; r0 += 4) {
                const int r = r0 + l4;
                Sacc[b] = mfma_f32_16x16x4(sKi[r * SD + cc] * sFL[(r >> 4) * D + cc],
                                           sY[r * kDVT + l16], Sacc[b]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sS[(16 * cb + 4 * l4 + j) * kDVT + l16] = Sacc[b][j];
        }
        __syncthreads();
        KDA_PHASE_MARK(13);
    }

    if (fin) {
#pragma unroll
        for (int b = 0; b < CBW; ++b) {
            const int cb = wave * CBW + b;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fin[head_state + state_elem(16 * cb + 4 * l4 + j, col0 + l16, D, state_trans)] = Sacc[b][j];
        }
    }
    KDA_PHASE_END;
}

template <int D, typename TIn, typename TOut>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    const unsigned chains = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
    // Round the chain count up to a multiple of 8 so that the value tiles of one
    // chain (linear ids chain + k * grid.x) land on the same XCD.
    const dim3 grid((chains + 7u) & ~7u, D / kDVT);
    const TIn* q = static_cast<const TIn*>(a.q);
    const TIn* k = static_cast<const TIn*>(a.k);
    const TIn* v = static_cast<const TIn*>(a.v);
    if (a.gate.a_log)
        prefill_chunk_kernel<D, TIn, TOut, true><<<grid, 256, 0, stream>>>(
            q, k, v, a.g, a.beta, a.gate, a.gate_per_head, a.cu_seqlens, a.initial_state, static_cast<TOut*>(a.out),
            a.final_state, a.slots, a.num_slots, a.total_tokens, a.num_seqs, a.num_heads, a.scale, a.l2norm,
            a.state_trans);
    else
        prefill_chunk_kernel<D, TIn, TOut, false><<<grid, 256, 0, stream>>>(
            q, k, v, a.g, a.beta, a.gate, a.gate_per_head, a.cu_seqlens, a.initial_state, static_cast<TOut*>(a.out),
            a.final_state, a.slots, a.num_slots, a.total_tokens, a.num_seqs, a.num_heads, a.scale, a.l2norm,
            a.state_trans);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
    if (a.qkv_bf16) {
        return a.out_bf16 ? launch_prefill_t<D, bf16_t, bf16_t>(a, stream)
                          : launch_prefill_t<D, bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? launch_prefill_t<D, float, bf16_t>(a, stream)
                      : launch_prefill_t<D, float, float>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    return a.head_dim == 128 ? launch_prefill_d<128>(a, stream) : launch_prefill_d<64>(a, stream);
}

}  // namespace kda
