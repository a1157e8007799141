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

// LDS map (bytes).  Region A holds Kg/Qg during the contraction phase and
// P', Delta'^T, the substitution operators and X Y' afterwards.
constexpr int PLANE_W = C * SW * 2;                  // 17408: [64][SW] bf16
constexpr int PLANE_N = C * SN * 2;                  // 9216:  [64][SN] bf16
constexpr int OFF_KGH = 0;
constexpr int OFF_KGL = OFF_KGH + PLANE_W;
constexpr int OFF_QGH = OFF_KGL + PLANE_W;
constexpr int OFF_QGL = OFF_QGH + PLANE_W;
constexpr int REGION_A = 4 * PLANE_W;                // 69632
constexpr int OFF_PH = 0;                            // P' [64][SN]
constexpr int OFF_PL = OFF_PH + PLANE_N;
constexpr int OFF_DH = OFF_PL + PLANE_N;             // Delta'^T [16][SN]
constexpr int OFF_DL = OFF_DH + DVT * SN * 2;
constexpr int OFF_WH = OFF_DL + DVT * SN * 2;        // -X_RR A'_RJ, [64][SN]
constexpr int OFF_WL = OFF_WH + PLANE_N;
constexpr int YS = DVT + 1;                          // fp32 row stride of X_RR Y'_R
constexpr int OFF_XY = OFF_WL + PLANE_N;             // X_RR Y'_R [64][17] fp32
static_assert(OFF_XY + C * YS * 4 <= REGION_A, "region A overflow");
constexpr int OFF_KIH = REGION_A;                    // Ki [64][SW]
constexpr int OFF_KIL = OFF_KIH + PLANE_W;
constexpr int OFF_ATH = OFF_KIL + PLANE_W;           // A' off-diagonal blocks, transposed [64][SN]
constexpr int OFF_ATL = OFF_ATH + PLANE_N;
constexpr int LD_STRIDE = 20;                        // fp32 row stride of the diagonal blocks
constexpr int OFF_LDT = OFF_ATL + PLANE_N;           // L' diagonal blocks, transposed: [4][16][20] fp32
constexpr int XD_STRIDE = 24;                        // bf16 row stride of the diagonal inverses
constexpr int OFF_XDH = OFF_LDT + 4 * 16 * LD_STRIDE * 4;   // [4][16][24] bf16
constexpr int OFF_XDL = OFF_XDH + 4 * 16 * XD_STRIDE * 2;
constexpr int OFF_SPH = OFF_XDL + 4 * 16 * XD_STRIDE * 2;   // (e^{G_m} S)^T [16][SW]
constexpr int OFF_SPL = OFF_SPH + DVT * SW * 2;
constexpr int OFF_YH = OFF_SPL + DVT * SW * 2;       // Y'^T [16][SN]
constexpr int OFF_YL = OFF_YH + DVT * SN * 2;
constexpr int OFF_WT = OFF_YL + DVT * SN * 2;        // wave totals of g [8][128] fp32
constexpr int OFF_RK = OFF_WT + 8 * D * 4;           // fp32 [64]
constexpr int OFF_RQ = OFF_RK + C * 4;
constexpr int OFF_BETA = OFF_RQ + C * 4;
constexpr int OFF_EM = OFF_BETA + C * 4;             // fp32 [128] exp(G_m)
constexpr int OFF_EL = OFF_EM + D * 4;               // exp(G_last - G_m)
constexpr int OFF_GL = OFF_EL + D * 4;               // exp(G_last)
constexpr int LDS_BYTES = OFF_GL + D * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

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

// Operand fragment or zeros (for K ranges that lie past the valid rows).
__device__ __forceinline__ bf16x8 ld8_if(const unsigned char* smem, int off_bytes, bool valid) {
    const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    return valid ? ld8(smem, off_bytes) : z;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would expose the full
// latency of the next chunk's prefetch at the first barrier after it; here
// only this wave's LDS operations are drained before s_barrier.  The memory
// clobber keeps the compiler from moving loads or stores across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum over the 16 lanes of a DPP row (all lanes receive the total).
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror 4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror 8
    return x;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

__device__ __forceinline__ floatx8 unpack8(const uint4& w) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    floatx8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
    return f;
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Split two floats into packed bf16 hi and lo words (x = hi + lo to about
// 2^-17 relative).  The high halves are recovered from the packed word with
// integer ops so the rounding conversion runs once per pair.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const floatx2 xv = {x0, x1};
    const uint32_t hu = __builtin_bit_cast(uint32_t, __builtin_convertvector(xv, bf16x2v));
    const floatx2 r = {x0 - __uint_as_float(hu << 16), x1 - __uint_as_float(hu & 0xffff0000u)};
    hi = hu;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2v));
}

__device__ __forceinline__ void split8(const floatx8& x, bf16x8& hi, bf16x8& lo) {
    uint4 h, l;
    split2(x[0], x[1], h.x, l.x);
    split2(x[2], x[3], h.y, l.y);
    split2(x[4], x[5], h.z, l.z);
    split2(x[6], x[7], h.w, l.w);
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ void split4(const floatx4& x, bf16x4& hi, bf16x4& lo) {
    uint2 h, l;
    split2(x[0], x[1], h.x, l.x);
    split2(x[2], x[3], h.y, l.y);
    hi = __builtin_bit_cast(bf16x4, h);
    lo = __builtin_bit_cast(bf16x4, l);
}

// Z_R = Kg_R (e^{G_m} S) (kg = true) or Oq_R = Qg_R (e^{G_m} S): one 16x16
// tile, K = 128 channels.  R is uniform across the wave.
__device__ __forceinline__ floatx4 unit_zo(const unsigned char* smem, int R, bool kg, int l16, int l4) {
    const int AH = kg ? OFF_KGH : OFF_QGH, AL = kg ? OFF_KGL : OFF_QGL;
    const int ar = (16 * R + l16) * SW;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int ko = 32 * s + 8 * l4;
        acc = mma3(ld8(smem, AH + (ar + ko) * 2), ld8(smem, AL + (ar + ko) * 2),
                   ld8(smem, OFF_SPH + (l16 * SW + ko) * 2), ld8(smem, OFF_SPL + (l16 * SW + ko) * 2), acc);
    }
    return acc;
}

// Block (R, I) of A' = diag(beta rk^2) (Kg Ki^T) and of P' = diag(rq) (Qg Ki^T).
// Off-diagonal A' blocks go to the transposed bf16 hi/lo planes, the diagonal ones
// (unit diagonal added, upper part zero) to the fp32 transposed store.
// Returns the P' block (masked to i <= r) in accumulator layout.
__device__ __forceinline__ floatx4 unit_ap(unsigned char* smem, int R, int I, int l16, int l4) {
    const float* srk = reinterpret_cast<const float*>(smem + OFF_RK);
    const float* srq = reinterpret_cast<const float*>(smem + OFF_RQ);
    const float* sbeta = reinterpret_cast<const float*>(smem + OFF_BETA);
    const int ar = (16 * R + l16) * SW, br = (16 * I + l16) * SW;
    floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int ko = 32 * s + 8 * l4;
        const bf16x8 bh = ld8(smem, OFF_KIH + (br + ko) * 2);
        const bf16x8 bl = ld8(smem, OFF_KIL + (br + ko) * 2);
        accA = mma(ld8(smem, OFF_KGH + (ar + ko) * 2), bh, accA);
        accP = mma3(ld8(smem, OFF_QGH + (ar + ko) * 2), ld8(smem, OFF_QGL + (ar + ko) * 2), bh, bl, accP);
    }
    floatx4 a, pv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * R + 4 * l4 + j;
        const float rk = srk[r];
        a[j] = sbeta[r] * rk * rk * accA[j];
        pv[j] = srq[r] * accP[j];
    }
    if (I < R) {
        // transposed: row = column i, four consecutive rows r per lane
        bf16x4 hi, lo;
        split4(a, hi, lo);
        const int o = ((16 * I + l16) * SN + 16 * R + 4 * l4) * 2;
        *reinterpret_cast<bf16x4*>(smem + OFF_ATH + o) = hi;
        *reinterpret_cast<bf16x4*>(smem + OFF_ATL + o) = lo;
    } else {
        // local row 4*l4 + j, local column l16
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int lr = 4 * l4 + j;
            a[j] = l16 < lr ? a[j] : (l16 == lr ? 1.f : 0.f);
            pv[j] = l16 <= lr ? pv[j] : 0.f;
        }
        *reinterpret_cast<floatx4*>(smem + OFF_LDT + ((R * 16 + l16) * LD_STRIDE + 4 * l4) * 4) = a;
    }
    return pv;
}

// (R, I) blocks whose P' each wave holds after the contraction phase.
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
        float* sWT = reinterpret_cast<float*>(smem + OFF_WT);
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
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: wave-uniform branches and loop bounds stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, l4 = lane >> 4;

    int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
    if (t0 < 0 || t1 > total_tokens || t1 < t0) t1 = t0;  // malformed: no tokens

    // State tile: wave w owns rows 16w..16w+15 (accumulator layout).
    const size_t head_state = (static_cast<size_t>(n) * num_heads + h) * D * D;
    KDA_PHASE_BEGIN
    floatx4 Sacc;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        Sacc[j] = initial_state ? initial_state[head_state + (16 * wave + 4 * l4 + j) * D + col0 + l16] : 0.f;

    // Prefetch mapping: thread (rp, cc) holds rows 2rp, 2rp+1 and channels
    // 8cc..8cc+7 of k, q, g.  Even waves also hold the value entries they
    // need for Y' (rows 16*(wave/2) + 4*l4 + j, column l16), threads < 64 one beta.
    uint4 pk[2], pq[2];
    floatx4 pg[4];
    uint16_t pv[4];
    float pb = 0.f;
    const bool zwave = (wave & 1) == 0;
    const int zR = wave >> 1;
    const int row_stride = num_heads * D;  // elements between consecutive tokens
    auto fetch = [&](int64_t c0, int rp, int cc, int l16, int l4, int tid) {
        const int Ln = static_cast<int>(min<int64_t>(C, t1 - c0));
        // chunk base (wave-uniform) plus 32-bit lane offsets
        const size_t base = (static_cast<size_t>(c0) * num_heads + h) * D;
        const bf16_t* kb = k + base;
        const bf16_t* qb = q + base;
        const float* gb = g + base;
        const bf16_t* vb = v + base + col0;
        const float* bb = beta + static_cast<size_t>(c0) * num_heads + h;
        if (Ln == C) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int off = (2 * rp + j) * row_stride + 8 * cc;
                pk[j] = *reinterpret_cast<const uint4*>(kb + off);
                pq[j] = *reinterpret_cast<const uint4*>(qb + off);
                pg[2 * j] = *reinterpret_cast<const floatx4*>(gb + off);
                pg[2 * j + 1] = *reinterpret_cast<const floatx4*>(gb + off + 4);
            }
            if (zwave) {
#pragma unroll
                for (int j = 0; j < 4; ++j) pv[j] = vb[(16 * zR + 4 * l4 + j) * row_stride + l16].bits;
            }
            if (tid < C) pb = bb[tid * num_heads];
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = 2 * rp + j;
                const int off = r * row_stride + 8 * cc;
                if (r < Ln) {
                    pk[j] = *reinterpret_cast<const uint4*>(kb + off);
                    pq[j] = *reinterpret_cast<const uint4*>(qb + off);
                    pg[2 * j] = *reinterpret_cast<const floatx4*>(gb + off);
                    pg[2 * j + 1] = *reinterpret_cast<const floatx4*>(gb + off + 4);
                } else {
                    pk[j] = uint4{0, 0, 0, 0};
                    pq[j] = uint4{0, 0, 0, 0};
                    pg[2 * j] = floatx4{0.f, 0.f, 0.f, 0.f};
                    pg[2 * j + 1] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
            }
            if (zwave) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * zR + 4 * l4 + j;
                    pv[j] = r < Ln ? vb[r * row_stride + l16].bits : uint16_t(0);
                }
            }
            if (tid < C) pb = tid < Ln ? bb[tid * num_heads] : 0.f;
        }
    };
    if (t0 < t1) fetch(t0, tid >> 4, tid & 15, l16, l4, tid);

    for (int64_t cs = t0; cs < t1; cs += C) {
        const int L = static_cast<int>(min<int64_t>(C, t1 - cs));
        // Lane indices are re-materialised opaquely every chunk so that the
        // compiler cannot hoist lane-dependent constants (masks, addresses,
        // unit vectors) out of the loop; kept live across it they would be
        // spilled to scratch.
        int lane_o;
        asm volatile("v_mov_b32 %0, %1" : "=v"(lane_o) : "v"(lane));
        const int l16 = lane_o & 15, l4 = lane_o >> 4;
        const int tid = wave * 64 + lane_o;
        const int rp = tid >> 4, cc = tid & 15;

        // ================= phase 1: per-element operands =================
        // Row norms: the 16 lanes of a row pair share rows 2rp, 2rp+1.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const floatx8 kf = unpack8(pk[j]), qf = unpack8(pq[j]);
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sk += kf[i] * kf[i];
                sq += qf[i] * qf[i];
            }
            sk = row16_sum(sk);
            sq = row16_sum(sq);
            if (cc == 0) {
                srk[2 * rp + j] = l2norm ? rsqrtf(sk + kNormEps) : 1.f;
                srq[2 * rp + j] = (l2norm ? rsqrtf(sq + kNormEps) : 1.f) * scale;
            }
        }
        if (tid < C) sbeta[tid] = pb;

        // Cumulative log-decay: pair sums, scan over the wave's four row
        // pairs, then wave totals through LDS.
        const floatx8 g0 = {pg[0][0], pg[0][1], pg[0][2], pg[0][3], pg[1][0], pg[1][1], pg[1][2], pg[1][3]};
        const floatx8 g1 = {pg[2][0], pg[2][1], pg[2][2], pg[2][3], pg[3][0], pg[3][1], pg[3][2], pg[3][3]};
        const floatx8 pair = g0 + g1;
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
        lds_barrier();

        // cm = (sum of the totals of earlier waves) - G_m, per channel; G_m is the
        // sum of the first four wave totals, so only waves between this one
        // and wave 4 contribute.
        floatx8 cm = {0, 0, 0, 0, 0, 0, 0, 0};
        {
            const int lo_w = wave < 4 ? wave : 4, hi_w = wave < 4 ? 4 : wave;
            const float sgn = wave < 4 ? -1.f : 1.f;
            for (int w2 = lo_w; w2 < hi_w; ++w2) {
                const floatx4 a = *reinterpret_cast<const floatx4*>(sWT + w2 * D + 8 * cc);
                const floatx4 b = *reinterpret_cast<const floatx4*>(sWT + w2 * D + 8 * cc + 4);
                const floatx8 t = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
                cm += t;
            }
            cm *= sgn;
        }
        // Exponents (log2 units) of E = exp(G - G_m) for rows 2rp and 2rp+1.
        const floatx8 d0 = (cm + (incl - pair) + g0) * kLog2e;
        const floatx8 d1 = d0 + g1 * kLog2e;
        if (tid < 3 * D) {
            // per-channel factors: thread t computes factor t / 128 of channel t % 128
            const int c = tid & (D - 1), which = tid >> 7;
            float gm = 0.f, gl = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 8; ++w2) {
                const float t = sWT[w2 * D + c];
                gl += t;
                if (w2 < 4) gm += t;
            }
            const float ex = which == 0 ? gm : (which == 1 ? gl - gm : gl);
            float* dst = which == 0 ? sEm : (which == 1 ? sEL : sGL);
            dst[c] = fast_exp2(ex * kLog2e);
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
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int o = ((2 * rp + j) * SW + 8 * cc) * 2;
            const floatx8 d = j == 0 ? d0 : d1;
            floatx8 e, ei;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = fast_exp2(d[i]);
                ei[i] = fast_exp2(-d[i]);
            }
            const floatx8 kf = unpack8(pk[j]), qf = unpack8(pq[j]);
            bf16x8 hi, lo;
            split8(kf * e, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + OFF_KGH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + OFF_KGL + o) = lo;
            split8(qf * e, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + OFF_QGH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + OFF_QGL + o) = lo;
            split8(kf * ei, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + OFF_KIH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + OFF_KIL + o) = lo;
            __builtin_amdgcn_sched_barrier(0);  // keep the two rows' temporaries apart
        }
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = bf2f(pv[j]);
        // The raw inputs are consumed: the next chunk's loads fly from here on.
        if (cs + C < t1) fetch(cs + C, rp, cc, l16, l4, tid);
        lds_barrier();
        KDA_PHASE_MARK(1);

        // ================= phase 2: contractions over channels =================
        floatx4 zo = {0.f, 0.f, 0.f, 0.f}, pa0 = zo, pa1 = zo;
        zo = unit_zo(smem, zR, zwave, l16, l4);
        {
            const int R0 = kPairs[wave][0][0], I0 = kPairs[wave][0][1];
            pa0 = unit_ap(smem, R0, I0, l16, l4);
            const int R1 = kPairs[wave][1][0], I1 = kPairs[wave][1][1];
            if (R1 >= 0) pa1 = unit_ap(smem, R1, I1, l16, l4);
        }
        if (zwave) {
            // Y' = rk beta (V - rk Z), stored transposed as bf16 hi/lo
            floatx4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * zR + 4 * l4 + j;
                const float rk = srk[r];
                y[j] = rk * sbeta[r] * (vv[j] - rk * zo[j]);
            }
            bf16x4 hi, lo;
            split4(y, hi, lo);
            *reinterpret_cast<bf16x4*>(smem + OFF_YH + (l16 * SN + 16 * zR + 4 * l4) * 2) = hi;
            *reinterpret_cast<bf16x4*>(smem + OFF_YL + (l16 * SN + 16 * zR + 4 * l4) * 2) = lo;
        }
        lds_barrier();
        KDA_PHASE_MARK(2);

        // ================= phase 3: P', diagonal inverses =================
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int R = kPairs[wave][u][0], I = kPairs[wave][u][1];
            if (R < 0) continue;
            bf16x4 hi, lo;
            split4(u == 0 ? pa0 : pa1, hi, lo);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                reinterpret_cast<__bf16*>(smem + OFF_PH)[r * SN + 16 * I + l16] = hi[j];
                reinterpret_cast<__bf16*>(smem + OFF_PL)[r * SN + 16 * I + l16] = lo[j];
            }
        }
        if (wave == 0) {
            // Lane (block l4, column l16): forward substitution L'_BB x = e_j.
            // Row p of the transposed store is column p of the block.
            const float* ldt = reinterpret_cast<const float*>(smem + OFF_LDT) + l4 * 16 * LD_STRIDE;
            float x[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) x[m] = (m == l16) ? 1.f : 0.f;
            // Four columns per step: finish x[p0..p0+3] inside their 4x4
            // block, then eliminate them from all later rows.
#pragma unroll
            for (int p0 = 0; p0 < 16; p0 += 4) {
                floatx4 col[4][4];  // col[t][qd]: column p0 + t of the block, rows 4qd..4qd+3
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int qd = p0 / 4; qd < 4; ++qd)
                        col[t][qd] = *reinterpret_cast<const floatx4*>(ldt + (p0 + t) * LD_STRIDE + 4 * qd);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int m = p0 + t + 1; m < p0 + 4; ++m) x[m] -= col[t][m >> 2][m & 3] * x[p0 + t];
#pragma unroll
                for (int m = p0 + 4; m < 16; ++m)
#pragma unroll
                    for (int t = 0; t < 4; ++t) x[m] -= col[t][m >> 2][m & 3] * x[p0 + t];
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const __bf16 hi = static_cast<__bf16>(x[m]);
                const __bf16 lo = static_cast<__bf16>(x[m] - static_cast<float>(hi));
                reinterpret_cast<__bf16*>(smem + OFF_XDH)[(l4 * 16 + m) * XD_STRIDE + l16] = hi;
                reinterpret_cast<__bf16*>(smem + OFF_XDL)[(l4 * 16 + m) * XD_STRIDE + l16] = lo;
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(3);

        // ================= phase 4: substitution operators =================
        // W_RJ = -X_RR A'_RJ (six blocks) and X_RR Y'_R (four blocks), K = 16.
        {
            const bool ok = l4 < 2;
            if (wave < 6) {
                const int R = wave < 1 ? 1 : wave < 3 ? 2 : 3;
                const int J = wave - (R * (R - 1)) / 2;
                const int xo = ((R * 16 + l16) * XD_STRIDE + 8 * l4) * 2;
                const int bo = ((16 * J + l16) * SN + 16 * R + 8 * l4) * 2;
                floatx4 w = {0.f, 0.f, 0.f, 0.f};
                w = mma3(ld8_if(smem, OFF_XDH + xo, ok), ld8_if(smem, OFF_XDL + xo, ok),
                         ld8_if(smem, OFF_ATH + bo, ok), ld8_if(smem, OFF_ATL + bo, ok), w);
                bf16x4 hi, lo;
                split4(-w, hi, lo);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * l4 + j;
                    reinterpret_cast<__bf16*>(smem + OFF_WH)[r * SN + 16 * J + l16] = hi[j];
                    reinterpret_cast<__bf16*>(smem + OFF_WL)[r * SN + 16 * J + l16] = lo[j];
                }
            } else {
                float* sXY = reinterpret_cast<float*>(smem + OFF_XY);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int R = 2 * (wave - 6) + u;
                    const int xo = ((R * 16 + l16) * XD_STRIDE + 8 * l4) * 2;
                    const int yo = (l16 * SN + 16 * R + 8 * l4) * 2;
                    floatx4 xy = {0.f, 0.f, 0.f, 0.f};
                    xy = mma3(ld8_if(smem, OFF_XDH + xo, ok), ld8_if(smem, OFF_XDL + xo, ok),
                              ld8_if(smem, OFF_YH + yo, ok), ld8_if(smem, OFF_YL + yo, ok), xy);
#pragma unroll
                    for (int j = 0; j < 4; ++j) sXY[(16 * R + 4 * l4 + j) * YS + l16] = xy[j];
                }
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(4);

        // ================= phase 5: Delta' by block forward substitution =================
        // Delta'_R = X_RR Y'_R + sum_{J<R} W_RJ Delta'_J; one wave, LDS hand-off within it.
        if (wave == 0) {
            const float* sXY = reinterpret_cast<const float*>(smem + OFF_XY);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                floatx4 acc;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = sXY[(16 * R + 4 * l4 + j) * YS + l16];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (32 * s >= 16 * R) continue;
                    const int ko = 32 * s + 8 * l4;
                    const bool ok = ko < 16 * R;
                    acc = mma3(ld8_if(smem, OFF_WH + ((16 * R + l16) * SN + ko) * 2, ok),
                               ld8_if(smem, OFF_WL + ((16 * R + l16) * SN + ko) * 2, ok),
                               ld8_if(smem, OFF_DH + (l16 * SN + ko) * 2, ok),
                               ld8_if(smem, OFF_DL + (l16 * SN + ko) * 2, ok), acc);
                }
                bf16x4 hi, lo;
                split4(acc, hi, lo);
                *reinterpret_cast<bf16x4*>(smem + OFF_DH + (l16 * SN + 16 * R + 4 * l4) * 2) = hi;
                *reinterpret_cast<bf16x4*>(smem + OFF_DL + (l16 * SN + 16 * R + 4 * l4) * 2) = lo;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(5);

        // ================= phase 6: output and state =================
        if (!zwave) {
            const int R = zR;
            floatx4 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = srq[16 * R + 4 * l4 + j] * zo[j];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (32 * s > 16 * R) continue;
                const int ko = 32 * s + 8 * l4;
                const bool ok = ko < 16 * R + 16;
                acc = mma3(ld8_if(smem, OFF_PH + ((16 * R + l16) * SN + ko) * 2, ok),
                           ld8_if(smem, OFF_PL + ((16 * R + l16) * SN + ko) * 2, ok),
                           ld8_if(smem, OFF_DH + (l16 * SN + ko) * 2, ok),
                           ld8_if(smem, OFF_DL + (l16 * SN + ko) * 2, ok), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * l4 + j;
                if (r < L) out[(static_cast<size_t>(cs + r) * num_heads + h) * D + col0 + l16] = from_f32<TOut>(acc[j]);
            }
        }
        {
            // U = Ki^T Delta' for state rows c = 16 wave + (0..15).  The A operand
            // (8 consecutive tokens of one channel) is gathered from the
            // row-major Ki planes.
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            const __bf16* kih = reinterpret_cast<const __bf16*>(smem + OFF_KIH);
            const __bf16* kil = reinterpret_cast<const __bf16*>(smem + OFF_KIL);
            const int cidx = 16 * wave + l16;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ko = 32 * s + 8 * l4;
                bf16x8 ah, al;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    ah[i] = kih[(ko + i) * SW + cidx];
                    al[i] = kil[(ko + i) * SW + cidx];
                }
                acc = mma3(ah, al, ld8(smem, OFF_DH + (l16 * SN + ko) * 2), ld8(smem, OFF_DL + (l16 * SN + ko) * 2), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 16 * wave + 4 * l4 + j;
                Sacc[j] = sGL[c] * Sacc[j] + sEL[c] * acc[j];
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(6);
    }

    if (final_state) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            final_state[head_state + (16 * wave + 4 * l4 + j) * D + col0 + l16] = Sacc[j];
    }
    KDA_PHASE_END;
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
