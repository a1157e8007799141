// KDA chunked prefill, bf16 inputs, dk = dv = 128: the bf16 MFMA path.
//
// Same chunk algebra as the fp32 kernel (the Ascend Kimi-Linear model file,
// `_torch_chunk_kda`): per chunk of 64 tokens with input state S,
//
//   A[r,i] = beta_r k_hat_r . (k_hat_i * exp(G_r - G_i))             (i < r)
//   P[r,i] =        q_hat_r . (k_hat_i * exp(G_r - G_i))             (i <= r)
//   Delta  = (I + A)^{-1} diag(beta) (V - (Gamma k_hat) S)
//   O      = (Gamma q_hat) S + P Delta
//   S'     = diag(Gamma_last) S + (k_hat * exp(G_last - G))^T Delta
//
// gfx950 design of this kernel:
//   * 512 threads (8 waves) per (sequence, head, 16-column value tile).
//   * One reference token m = 31 (end of the first half) per chunk: E = exp(G - G_m).  The operands
//     Kg = k E, Qg = q E and Ki = k / E are then fixed per chunk, so every
//     contraction is a plain MFMA: A = Kg Ki^T, P = Qg Ki^T, (Gamma K) S =
//     Kg (diag(exp G_m) S) and (K exp(G_last - G))^T = diag(exp(G_last - G_m)) Ki^T.
//     The factors stay within exp(+-|decay over 32 tokens|).
//   * The L2 norms of q and k never touch the operands: they are row/column
//     scalings of the 64x64 results, of Z, of Oq and of Delta.
//   * Every operand is stored in LDS as a bf16 hi/lo pair (x = hi + lo to
//     about 2^-17) and products use hi*hi + hi*lo + lo*hi on the bf16
//     16x16x32 MFMA (fp32 accumulate), except k.k in A, which is inverted
//     afterwards and tolerates plain bf16.  The inverse itself is fp32.
//   * LDS rows are padded by 16 bytes so the 16-byte operand reads of one
//     MFMA hit distinct banks.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int C = 64;       // chunk length
constexpr int D = 128;      // head size
constexpr int DVT = 16;     // value columns per workgroup
constexpr int NT = 512;     // threads per workgroup
constexpr int SW = D + 8;   // bf16 row stride of 128-wide planes
constexpr int SN = C + 8;   // bf16 row stride of 64-wide planes
constexpr int SF = C + 1;   // fp32 row stride of the inverse
constexpr int SL = C + 8;   // fp32 row stride of I + A

// LDS map (bytes).  Region A holds Kg/Qg during the contraction phase and
// Ki^T, P', Delta'^T and inverse scratch afterwards.
constexpr int PLANE_W = C * SW * 2;                  // 17408
constexpr int OFF_KGH = 0;
constexpr int OFF_KGL = OFF_KGH + PLANE_W;
constexpr int OFF_QGH = OFF_KGL + PLANE_W;
constexpr int OFF_QGL = OFF_QGH + PLANE_W;
constexpr int REGION_A = 4 * PLANE_W;                // 69632
constexpr int OFF_KTH = 0;                           // Ki^T [128][SN]
constexpr int OFF_KTL = OFF_KTH + D * SN * 2;
constexpr int OFF_PH = OFF_KTL + D * SN * 2;         // P' [64][SN]
constexpr int OFF_PL = OFF_PH + C * SN * 2;
constexpr int OFF_DH = OFF_PL + C * SN * 2;          // Delta'^T [16][SN]
constexpr int OFF_DL = OFF_DH + DVT * SN * 2;
constexpr int OFF_TS = OFF_DL + DVT * SN * 2;        // 4 x 16x17 fp32 scratch
static_assert(OFF_TS + 4 * 16 * 17 * 4 <= REGION_A, "region A overflow");
constexpr int OFF_KIH = REGION_A;                    // Ki [64][SW]
constexpr int OFF_KIL = OFF_KIH + PLANE_W;
constexpr int OFF_L = OFF_KIL + PLANE_W;             // I + A fp32 [64][SL], later X'
constexpr int OFF_XH = OFF_L;
constexpr int OFF_XL = OFF_XH + C * SN * 2;
constexpr int OFF_XF = OFF_L + C * SL * 4;           // X fp32 [64][SF]; early: wave totals
constexpr int OFF_SPH = OFF_XF + C * SF * 4;         // (e^{G_m} S)^T [16][SW]
constexpr int OFF_SPL = OFF_SPH + DVT * SW * 2;
constexpr int OFF_YH = OFF_SPL + DVT * SW * 2;       // Y^T [16][SN]
constexpr int OFF_YL = OFF_YH + DVT * SN * 2;
constexpr int OFF_RK = OFF_YL + DVT * SN * 2;        // fp32 [64]
constexpr int OFF_RQ = OFF_RK + C * 4;
constexpr int OFF_BETA = OFF_RQ + C * 4;
constexpr int OFF_EM = OFF_BETA + C * 4;             // fp32 [128] exp(G_m)
constexpr int OFF_EL = OFF_EM + D * 4;               // exp(G_last - G_m)
constexpr int OFF_GL = OFF_EL + D * 4;               // exp(G_last)
constexpr int LDS_BYTES = OFF_GL + D * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(C * SN * 4 <= C * SL * 4, "X' must fit in the I + A buffer");

__device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ floatx4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, floatx4 c) {
    c = mma(ah, bh, c);
    c = mma(ah, bl, c);
    return mma(al, bh, c);
}

__device__ __forceinline__ bf16x8 ld8(const unsigned char* smem, int off_bytes) {
    return *reinterpret_cast<const bf16x8*>(smem + off_bytes);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Split 8 floats into bf16 hi and lo parts.
__device__ __forceinline__ void split8(const floatx8& x, bf16x8& hi, bf16x8& lo) {
    hi = __builtin_convertvector(x, bf16x8);
    const floatx8 hf = __builtin_convertvector(hi, floatx8);
    lo = __builtin_convertvector(x - hf, bf16x8);
}

__device__ __forceinline__ void split4(const floatx4& x, bf16x4& hi, bf16x4& lo) {
    hi = __builtin_convertvector(x, bf16x4);
    const floatx4 hf = __builtin_convertvector(hi, floatx4);
    lo = __builtin_convertvector(x - hf, bf16x4);
}

// Row blocks and (row, column) block pairs of the 64x64 products, per wave.
// Units: Z_R (even waves) / Oq_R (odd waves) for R = wave / 2, plus up to two
// (R, I) blocks of A and P.  Balances MFMA work across the four SIMDs.
__constant__ int8_t kPairs[8][2][2] = {
    {{0, 0}, {-1, -1}}, {{3, 1}, {-1, -1}}, {{1, 0}, {-1, -1}}, {{1, 1}, {-1, -1}},
    {{2, 0}, {2, 1}},   {{2, 2}, {-1, -1}}, {{3, 0}, {-1, -1}}, {{3, 2}, {3, 3}},
};

}  // namespace

template <typename TOut>
__global__ __launch_bounds__(NT) void prefill_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu_seqlens, const float* initial_state, TOut* __restrict__ out,
    float* final_state, int64_t total_tokens, int num_seqs, int num_heads, float scale,
    int l2norm) {
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    float* sL = reinterpret_cast<float*>(smem + OFF_L);
    float* sXf = reinterpret_cast<float*>(smem + OFF_XF);
    float* sWT = sXf;  // wave totals of the log-decay, [8][128], before the inverse
    float* sTS = reinterpret_cast<float*>(smem + OFF_TS);
    float* srk = reinterpret_cast<float*>(smem + OFF_RK);
    float* srq = reinterpret_cast<float*>(smem + OFF_RQ);
    float* sbeta = reinterpret_cast<float*>(smem + OFF_BETA);
    float* sEm = reinterpret_cast<float*>(smem + OFF_EM);
    float* sEL = reinterpret_cast<float*>(smem + OFF_EL);
    float* sGL = reinterpret_cast<float*>(smem + OFF_GL);

    const int chain = blockIdx.x;
    if (chain >= num_seqs * num_heads) return;
    const int n = chain / num_heads, h = chain % num_heads;
    const int col0 = blockIdx.y * DVT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, l4 = lane >> 4;

    int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
    if (t0 < 0 || t1 > total_tokens || t1 < t0) t1 = t0;  // malformed: no tokens

    // State tile: wave w owns rows 16w..16w+15 (accumulator layout).
    const size_t head_state = (static_cast<size_t>(n) * num_heads + h) * D * D;
    floatx4 Sacc;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        Sacc[j] = initial_state ? initial_state[head_state + (16 * wave + 4 * l4 + j) * D + col0 + l16] : 0.f;

    // Prefetch mapping: thread (rp, cc) holds rows 2rp, 2rp+1 and channels
    // 8cc..8cc+7 of k, q, g.  Even waves also hold the value entries they
    // need for Y = beta (V - Z), threads < 64 one beta.
    const int rp = tid >> 4, cc = tid & 15;
    uint4 pk[2], pq[2];
    floatx4 pg[2][2];
    uint16_t pv[4];
    float pb = 0.f;
    const bool zwave = (wave & 1) == 0;
    const int zR = wave >> 1;
    auto fetch = [&](int64_t c0) {
        const int Ln = static_cast<int>(min<int64_t>(C, t1 - c0));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 2 * rp + j;
            if (r < Ln) {
                const size_t off = (static_cast<size_t>(c0 + r) * num_heads + h) * D + 8 * cc;
                pk[j] = *reinterpret_cast<const uint4*>(k + off);
                pq[j] = *reinterpret_cast<const uint4*>(q + off);
                pg[j][0] = *reinterpret_cast<const floatx4*>(g + off);
                pg[j][1] = *reinterpret_cast<const floatx4*>(g + off + 4);
            } else {
                pk[j] = uint4{0, 0, 0, 0};
                pq[j] = uint4{0, 0, 0, 0};
                pg[j][0] = floatx4{0.f, 0.f, 0.f, 0.f};
                pg[j][1] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (zwave) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * zR + 4 * l4 + j;
                pv[j] = r < Ln ? v[(static_cast<size_t>(c0 + r) * num_heads + h) * D + col0 + l16].bits
                               : uint16_t(0);
            }
        }
        if (tid < C) pb = tid < Ln ? beta[static_cast<size_t>(c0 + tid) * num_heads + h] : 0.f;
    };
    if (t0 < t1) fetch(t0);

    for (int64_t cs = t0; cs < t1; cs += C) {
        const int L = static_cast<int>(min<int64_t>(C, t1 - cs));

        // ================= phase 1: per-element operands =================
        floatx8 kf[2], qf[2], gf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t kw[4] = {pk[j].x, pk[j].y, pk[j].z, pk[j].w};
            const uint32_t qw[4] = {pq[j].x, pq[j].y, pq[j].z, pq[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kf[j][2 * i] = __uint_as_float(kw[i] << 16);
                kf[j][2 * i + 1] = __uint_as_float(kw[i] & 0xffff0000u);
                qf[j][2 * i] = __uint_as_float(qw[i] << 16);
                qf[j][2 * i + 1] = __uint_as_float(qw[i] & 0xffff0000u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gf[j][i] = pg[j][0][i];
                gf[j][4 + i] = pg[j][1][i];
            }
        }
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = bf2f(pv[j]);
        const float bcur = pb;

        // Row norms: the 16 lanes of a row pair share rows 2rp, 2rp+1.
        float rkr[2], rqr[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sk += kf[j][i] * kf[j][i];
                sq += qf[j][i] * qf[j][i];
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                sk += __shfl_xor(sk, off, 64);
                sq += __shfl_xor(sq, off, 64);
            }
            rkr[j] = l2norm ? rsqrtf(sk + kNormEps) : 1.f;
            rqr[j] = (l2norm ? rsqrtf(sq + kNormEps) : 1.f) * scale;
        }
        if (cc == 0) {
            srk[2 * rp] = rkr[0];
            srk[2 * rp + 1] = rkr[1];
            srq[2 * rp] = rqr[0];
            srq[2 * rp + 1] = rqr[1];
        }
        if (tid < C) sbeta[tid] = bcur;

        // Cumulative log-decay: pair sums, scan over the wave's four pairs,
        // then wave totals through LDS.
        floatx8 pair = gf[0] + gf[1];
        floatx8 incl = pair;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float t = __shfl_up(incl[i], 16, 64);
            if (l4 >= 1) incl[i] += t;
            t = __shfl_up(incl[i], 32, 64);
            if (l4 >= 2) incl[i] += t;
        }
        if (l4 == 3) {
            *reinterpret_cast<floatx4*>(sWT + wave * D + 8 * cc) = floatx4{incl[0], incl[1], incl[2], incl[3]};
            *reinterpret_cast<floatx4*>(sWT + wave * D + 8 * cc + 4) = floatx4{incl[4], incl[5], incl[6], incl[7]};
        }
        __syncthreads();

        floatx8 carry = {0, 0, 0, 0, 0, 0, 0, 0}, gm = carry, glast = carry;
#pragma unroll
        for (int w2 = 0; w2 < 8; ++w2) {
            const floatx4 a = *reinterpret_cast<const floatx4*>(sWT + w2 * D + 8 * cc);
            const floatx4 b = *reinterpret_cast<const floatx4*>(sWT + w2 * D + 8 * cc + 4);
            const floatx8 t = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            glast += t;
            if (w2 < 4) gm += t;
            if (w2 < wave) carry += t;
        }
        const floatx8 G0 = carry + (incl - pair) + gf[0];
        const floatx8 G1 = G0 + gf[1];
        bf16x8 kih[2], kil[2];  // Ki hi/lo kept for the transposed copy
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 2 * rp + j;
            const floatx8 d = ((j == 0 ? G0 : G1) - gm) * kLog2e;
            floatx8 e, ei;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = fast_exp2(d[i]);
                ei[i] = fast_exp2(-d[i]);
            }
            const int o = (r * SW + 8 * cc) * 2;
            bf16x8 hi, lo;
            split8(kf[j] * e, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + OFF_KGH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + OFF_KGL + o) = lo;
            split8(qf[j] * e, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + OFF_QGH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + OFF_QGL + o) = lo;
            split8(kf[j] * ei, kih[j], kil[j]);
            *reinterpret_cast<bf16x8*>(smem + OFF_KIH + o) = kih[j];
            *reinterpret_cast<bf16x8*>(smem + OFF_KIL + o) = kil[j];
        }
        if (rp == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = 8 * cc + i;
                sEm[c] = fast_exp2(gm[i] * kLog2e);
                sEL[c] = fast_exp2((glast[i] - gm[i]) * kLog2e);
                sGL[c] = fast_exp2(glast[i] * kLog2e);
            }
        }
        // (e^{G_m} S)^T for this wave's 16 state rows.
        {
            floatx4 gmr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) gmr += *reinterpret_cast<const floatx4*>(sWT + w2 * D + 16 * wave + 4 * l4);
            floatx4 sp;
#pragma unroll
            for (int j = 0; j < 4; ++j) sp[j] = Sacc[j] * fast_exp2(gmr[j] * kLog2e);
            bf16x4 hi, lo;
            split4(sp, hi, lo);
            *reinterpret_cast<bf16x4*>(smem + OFF_SPH + (l16 * SW + 16 * wave + 4 * l4) * 2) = hi;
            *reinterpret_cast<bf16x4*>(smem + OFF_SPL + (l16 * SW + 16 * wave + 4 * l4) * 2) = lo;
        }
        __syncthreads();

        // The next chunk's loads fly while this one is contracted.
        if (cs + C < t1) fetch(cs + C);

        // ================= phase 2: contractions over channels =================
        floatx4 Oq = {0.f, 0.f, 0.f, 0.f};
        floatx4 Pacc[2];
        {
            const int R = zR;
            const int ar = (16 * R + l16) * SW;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ah = zwave ? OFF_KGH : OFF_QGH, al = zwave ? OFF_KGL : OFF_QGL;
#pragma unroll 1
            for (int s = 0; s < 4; ++s) {
                const int ko = 32 * s + 8 * l4;
                acc = mma3(ld8(smem, ah + (ar + ko) * 2), ld8(smem, al + (ar + ko) * 2),
                           ld8(smem, OFF_SPH + (l16 * SW + ko) * 2), ld8(smem, OFF_SPL + (l16 * SW + ko) * 2), acc);
            }
            if (zwave) {
                // Y = beta (V - rk Z), stored transposed as bf16 hi/lo
                floatx4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * l4 + j;
                    y[j] = sbeta[r] * (vv[j] - srk[r] * acc[j]);
                }
                bf16x4 hi, lo;
                split4(y, hi, lo);
                *reinterpret_cast<bf16x4*>(smem + OFF_YH + (l16 * SN + 16 * R + 4 * l4) * 2) = hi;
                *reinterpret_cast<bf16x4*>(smem + OFF_YL + (l16 * SN + 16 * R + 4 * l4) * 2) = lo;
            } else {
                Oq = acc;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int R = kPairs[wave][u][0], I = kPairs[wave][u][1];
            Pacc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (R < 0) continue;
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            const int ar = (16 * R + l16) * SW, br = (16 * I + l16) * SW;
#pragma unroll 1
            for (int s = 0; s < 4; ++s) {
                const int ko = 32 * s + 8 * l4;
                const bf16x8 bh = ld8(smem, OFF_KIH + (br + ko) * 2);
                const bf16x8 bl = ld8(smem, OFF_KIL + (br + ko) * 2);
                accA = mma(ld8(smem, OFF_KGH + (ar + ko) * 2), bh, accA);
                accP = mma3(ld8(smem, OFF_QGH + (ar + ko) * 2), ld8(smem, OFF_QGL + (ar + ko) * 2), bh, bl, accP);
            }
            const int i = 16 * I + l16;
            const float rki = srk[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                const bool below = I < R || i < r;
                sL[r * SL + i] = below ? sbeta[r] * srk[r] * rki * accA[j] : (i == r ? 1.f : 0.f);
                Pacc[u][j] = (I < R || i <= r) ? srq[r] * accP[j] : 0.f;
            }
        }
        __syncthreads();

        // ================= phase 3: inverse of I + A; P', Ki^T =================
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int R = kPairs[wave][u][0], I = kPairs[wave][u][1];
            if (R < 0) continue;
            bf16x4 hi, lo;
            split4(Pacc[u], hi, lo);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                reinterpret_cast<__bf16*>(smem + OFF_PH)[r * SN + 16 * I + l16] = hi[j];
                reinterpret_cast<__bf16*>(smem + OFF_PL)[r * SN + 16 * I + l16] = lo[j];
            }
        }
        // Blocks (0,1) and (2,3) lie inside the K range of the 32-wide MFMA
        // steps of rows 0-15 and 32-47; they must read as zero.
        if (tid < 128) {
            const int blk = tid >> 6, row = (tid >> 2) & 15, part = tid & 3;
            const int r = (blk ? 32 : 0) + row, c0 = (blk ? 48 : 16) + 4 * part;
            const bf16x4 z = {0, 0, 0, 0};
            *reinterpret_cast<bf16x4*>(smem + OFF_PH + (r * SN + c0) * 2) = z;
            *reinterpret_cast<bf16x4*>(smem + OFF_PL + (r * SN + c0) * 2) = z;
        }
        // Ki^T [c][r] from this thread's two rows.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * cc + i;
            const bf16x2 hi = {kih[0][i], kih[1][i]};
            const bf16x2 lo = {kil[0][i], kil[1][i]};
            *reinterpret_cast<bf16x2*>(smem + OFF_KTH + (c * SN + 2 * rp) * 2) = hi;
            *reinterpret_cast<bf16x2*>(smem + OFF_KTL + (c * SN + 2 * rp) * 2) = lo;
        }
        // Diagonal 16x16 blocks by forward substitution: lane (block l4, column l16).
        if (wave == 0) {
            const int B = l4, jcol = l16;
            float x[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) x[m] = (m == jcol) ? 1.f : 0.f;
#pragma unroll
            for (int p = 0; p < 15; ++p) {
#pragma unroll
                for (int m = p + 1; m < 16; ++m) x[m] -= sL[(16 * B + m) * SL + 16 * B + p] * x[p];
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) sXf[(16 * B + m) * SF + 16 * B + jcol] = x[m];
        }
        __syncthreads();
        // Off-diagonal blocks: X_RI = -X_RR sum_{J=I}^{R-1} L_RJ X_JI, by block distance.
#pragma unroll
        for (int dist = 1; dist < 4; ++dist) {
            const bool active = wave < 4 - dist;
            const int I = wave, R = wave + dist;
            float* T = sTS + wave * 16 * 17;
            if (active) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int J = I; J < R; ++J) {
#pragma unroll
                    for (int k0 = 0; k0 < 16; k0 += 4)
                        acc = mfma_f32_16x16x4(sL[(16 * R + l16) * SL + 16 * J + k0 + l4],
                                               sXf[(16 * J + k0 + l4) * SF + 16 * I + l16], acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) T[(4 * l4 + j) * 17 + l16] = acc[j];
            }
            __syncthreads();
            if (active) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    acc = mfma_f32_16x16x4(sXf[(16 * R + l16) * SF + 16 * R + k0 + l4], T[(k0 + l4) * 17 + l16], acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) sXf[(16 * R + 4 * l4 + j) * SF + 16 * I + l16] = -acc[j];
            }
            __syncthreads();
        }
        // X' = diag(rk) X, lower triangle, as bf16 hi/lo (over the dead I + A buffer).
        {
            const int r = tid >> 3, c0 = 8 * (tid & 7);
            const float rk = srk[r];
            floatx8 xv;
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = (c0 + i <= r) ? rk * sXf[r * SF + c0 + i] : 0.f;
            bf16x8 hi, lo;
            split8(xv, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + OFF_XH + (r * SN + c0) * 2) = hi;
            *reinterpret_cast<bf16x8*>(smem + OFF_XL + (r * SN + c0) * 2) = lo;
        }
        __syncthreads();

        // ================= phase 4: Delta', O, state =================
        if (wave < 4) {
            const int R = wave, ns = R < 2 ? 1 : 2;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < ns; ++s) {
                const int ko = 32 * s + 8 * l4;
                acc = mma3(ld8(smem, OFF_XH + ((16 * R + l16) * SN + ko) * 2),
                           ld8(smem, OFF_XL + ((16 * R + l16) * SN + ko) * 2),
                           ld8(smem, OFF_YH + (l16 * SN + ko) * 2), ld8(smem, OFF_YL + (l16 * SN + ko) * 2), acc);
            }
            bf16x4 hi, lo;
            split4(acc, hi, lo);
            *reinterpret_cast<bf16x4*>(smem + OFF_DH + (l16 * SN + 16 * R + 4 * l4) * 2) = hi;
            *reinterpret_cast<bf16x4*>(smem + OFF_DL + (l16 * SN + 16 * R + 4 * l4) * 2) = lo;
        }
        __syncthreads();
        if (!zwave) {
            const int R = zR, ns = R < 2 ? 1 : 2;
            floatx4 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = srq[16 * R + 4 * l4 + j] * Oq[j];
            for (int s = 0; s < ns; ++s) {
                const int ko = 32 * s + 8 * l4;
                acc = mma3(ld8(smem, OFF_PH + ((16 * R + l16) * SN + ko) * 2),
                           ld8(smem, OFF_PL + ((16 * R + l16) * SN + ko) * 2),
                           ld8(smem, OFF_DH + (l16 * SN + ko) * 2), ld8(smem, OFF_DL + (l16 * SN + ko) * 2), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                if (r < L) out[(static_cast<size_t>(cs + r) * num_heads + h) * D + col0 + l16] = from_f32<TOut>(acc[j]);
            }
        }
        {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            const int cr = (16 * wave + l16) * SN;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ko = 32 * s + 8 * l4;
                acc = mma3(ld8(smem, OFF_KTH + (cr + ko) * 2), ld8(smem, OFF_KTL + (cr + ko) * 2),
                           ld8(smem, OFF_DH + (l16 * SN + ko) * 2), ld8(smem, OFF_DL + (l16 * SN + ko) * 2), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 16 * wave + 4 * l4 + j;
                Sacc[j] = sGL[c] * Sacc[j] + sEL[c] * acc[j];
            }
        }
        __syncthreads();
    }

    if (final_state) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            final_state[head_state + (16 * wave + 4 * l4 + j) * D + col0 + l16] = Sacc[j];
    }
}

template <typename TOut>
static hipError_t launch_bf16_t(const PrefillArgs& a, hipStream_t stream) {
    const unsigned chains = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
    const dim3 grid((chains + 7u) & ~7u, D / DVT);
    prefill_bf16_kernel<TOut><<<grid, NT, 0, stream>>>(
        static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v),
        a.g, a.beta, a.cu_seqlens, a.initial_state, static_cast<TOut*>(a.out), a.final_state,
        a.total_tokens, a.num_seqs, a.num_heads, a.scale, a.l2norm);
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    return a.out_bf16 ? launch_bf16_t<bf16_t>(a, stream) : launch_bf16_t<float>(a, stream);
}

}  // namespace kda
