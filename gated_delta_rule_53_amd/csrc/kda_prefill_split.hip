// KDA chunked prefill for bf16 q/k/v with dk = dv = 128: chunk-parallel
// preparation followed by a short state scan.
//
// Algebra.  The chunk form of the Ascend Kimi-Linear model file
// (`_torch_chunk_kda`) computes, per chunk of 64 tokens with input state S,
//   Delta = (I + A)^{-1} diag(beta) (V - (Gamma k_hat) S),
//   O     = (Gamma q_hat) S + P Delta,
//   S'    = diag(Gamma_last) S + (k_hat exp(G_last - G))^T Delta.
// With E = exp(G - G_31) (G_31: cumulative log-decay at the chunk's token
// 31), Kg = k E, Qg = q E, Ki = k / E, L' = I + diag(beta rk^2) (Kg Ki^T)
// (strictly lower part), P' = diag(rq) (Qg Ki^T) (lower incl. diagonal) and
// X' = L'^{-1}, everything that does not involve S can be formed per chunk:
//   Psi' = X' diag(rk^2 beta) Kg diag(e^{G_31})          [64 x 128]
//   Qg'  = diag(rq) Qg diag(e^{G_31})                     [64 x 128]
//   Delta0 = X' diag(rk beta) V                           [64 x dv]
// and the chunk step becomes
//   D  = Delta0 - Psi' S          (D = diag(rk) Delta)
//   O  = Qg' S + P' D
//   S' = diag(e^{G_last}) S + diag(e^{G_last - G_31}) Ki^T D.
// rk, rq are the L2-norm factors of k and q (rq includes the scale).
//
// Kernels.
//   chunk_map_kernel  one workgroup: per-sequence chunk offsets from
//                     cu_seqlens (device side, no host synchronisation).
//   prep_kernel       persistent, fully parallel over (chunk, head): builds
//                     Kg/Qg/Ki, A and P on MFMA, the four 16x16 diagonal
//                     inverses, W_RJ = -X_RR A'_RJ, and solves for Psi' and X'
//                     by block forward substitution.  Writes Psi', Qg', Ki^T,
//                     X', P' and three vectors to a per-(chunk, head) record,
//                     in the lane order the scan's MFMA operands use.
//   scan_kernel       per (sequence, head, 16-column value tile): the chunk
//                     chain above; per chunk two barriers and 36 bf16 MFMAs
//                     on the dependent path.  The next chunk's record is
//                     prefetched into registers during the current one.
// All operands are bf16 hi/lo pairs (hi*hi + hi*lo + lo*hi), except k.k in
// A (inverted afterwards); the 16x16 diagonal inverses are fp32.
#include "kda_bf16_mfma.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;       // chunk length
constexpr int D = 128;      // head size
constexpr int DVT = 16;     // value columns of one MFMA tile in the scan
constexpr int NT = 512;     // threads per workgroup (both kernels)
constexpr int SW = D + 8;   // bf16 row stride of 128-wide LDS planes
constexpr int SN = C + 8;   // bf16 row stride of 64-wide LDS planes

// ---- per-(chunk, head) record written by prep_kernel ----
// A fragment is one wave-wide MFMA operand: 64 lanes x 16 bytes, lane l
// holding M[row0 + l%16][k0 + 8*(l/16) .. +7].
constexpr int FRAG = 1024;
// The operands the state meets (Psi', Qg', Ke^T, P') are single fp16; the
// state side (S, D) is an fp16 hi/lo pair.  fp16 keeps 11 significant bits,
// and every one of these operands is bounded: Qg' by |q_hat|, P' by
// |q_hat||k_hat|, Ke = k e^{G_last - G} by |k|, Psi' by the scaled inverse.
// X' diag(rk beta), which multiplies the bf16 values V, stays a bf16 hi/lo
// pair.
constexpr int REC_PSI = 0;                    // Psi' : [R 4][s 4] fragments, fp16
constexpr int REC_QG = REC_PSI + 16 * FRAG;   // Qg'  : [R 4][s 4], fp16
constexpr int REC_KE = REC_QG + 16 * FRAG;    // Ke^T : [c-block 8][s 2], fp16
constexpr int REC_X = REC_KE + 16 * FRAG;     // X' diag(rk beta) : [R 4][s 2][hi/lo], bf16
constexpr int REC_P = REC_X + 16 * FRAG;      // P'   : [R 4][s 2], fp16
constexpr int REC_VEC = REC_P + 8 * FRAG;     // fp32 e^{G_last}[128], unused[128]
constexpr int VEC_GL = 0;
constexpr int REC_BYTES = REC_VEC + 256 * 4;  // 74752

// ---- prep_kernel LDS map (bytes) ----
constexpr int PW = C * SW * 2;                 // 17408: [64][SW] bf16
constexpr int PN = C * SN * 2;                 // 9216:  [64][SN] bf16
constexpr int WSTR = 24;                       // bf16 row stride of 16x16 blocks
constexpr int BLK = 16 * WSTR * 2;             // 768: one 16x16 block
constexpr int LDS_STR = 20;                    // fp32 row stride of the diagonal blocks
constexpr int P_KGH = 0, P_KGL = PW;                           // region 1: Kg
constexpr int P_R2 = 2 * PW;                                    // region 2: Qg, later W and X'^T
constexpr int P_QGH = P_R2, P_QGL = P_R2 + PW;
constexpr int P_WH = P_R2, P_WL = P_R2 + 6 * BLK;               // W_RJ, six blocks [16][24]
constexpr int P_XTH = P_R2 + 12 * BLK, P_XTL = P_XTH + PN;      // X'^T [64][SN]
static_assert(P_XTL + PN <= P_R2 + 2 * PW, "region 2 overflow");
constexpr int P_R3 = P_R2 + 2 * PW;                             // region 3: Ki, later Psi'^T
constexpr int P_KIH = P_R3, P_KIL = P_R3 + PW;
constexpr int P_PTH = P_R3, P_PTL = P_R3 + D * SN * 2;          // Psi'^T [128][SN]
constexpr int P_R3_END = P_R3 + 2 * D * SN * 2;
static_assert(P_R3_END >= P_KIL + PW, "region 3 size");
constexpr int P_PH = P_R3_END, P_PL = P_PH + PN;                // P' [64][SN]
constexpr int P_ATH = P_PL + PN, P_ATL = P_ATH + 6 * BLK;       // A'^T blocks [16][24]
constexpr int P_LDT = P_ATL + 6 * BLK;                          // L' diagonal blocks, transposed, fp32
constexpr int P_XDH = P_LDT + 4 * 16 * LDS_STR * 4;             // X_RR [4][16][24] bf16
constexpr int P_XDL = P_XDH + 4 * BLK;
constexpr int P_XFH = P_XDL + 4 * BLK;                          // X_RR diag(rk^2 beta)
constexpr int P_XFL = P_XFH + 4 * BLK;
constexpr int P_RK = P_XFL + 4 * BLK;                           // fp32 [64]
constexpr int P_RQ = P_RK + C * 4;
constexpr int P_BETA = P_RQ + C * 4;
constexpr int P_EM = P_BETA + C * 4;                            // fp32 [128] e^{G_31}
constexpr int P_EL = P_EM + D * 4;                              // e^{G_last - G_31}
constexpr int P_GL = P_EL + D * 4;                              // e^{G_last}
constexpr int P_LDS = P_GL + D * 4;
static_assert(P_LDS <= 160 * 1024, "prep LDS budget");
static_assert(8 * D * 4 <= 4 * 16 * LDS_STR * 4, "wave totals alias the diagonal blocks");

// ---- scan_kernel LDS map (bytes), for NTL column tiles of 16 per workgroup ----
template <int NTL>
struct ScanLds {
    static constexpr int COLS = DVT * NTL;
    static constexpr int STH = 0, STL = COLS * SW * 2;                     // S^T [COLS][SW] fp16 hi, lo
    static constexpr int V = 2 * COLS * SW * 2;                            // V^T [COLS][SN] (bf16, exact)
    static constexpr int DH = V + COLS * SN * 2, DL = DH + COLS * SN * 2;  // D^T [COLS][SN] fp16 hi, lo
    static constexpr int VEC = DL + COLS * SN * 2;                         // two slots of the vector block
    static constexpr int BYTES = VEC + 2 * 256 * 4;
};

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }

// (R, I) blocks of A and P computed by each wave of prep_kernel.
__constant__ int8_t kPrepPairs[8][2][2] = {
    {{0, 0}, {3, 3}}, {{1, 0}, {3, 2}}, {{1, 1}, {3, 1}}, {{2, 0}, {3, 0}},
    {{2, 1}, {-1, -1}}, {{2, 2}, {-1, -1}}, {{-1, -1}, {-1, -1}}, {{-1, -1}, {-1, -1}},
};

__device__ __forceinline__ const unsigned char* frag_ptr(const unsigned char* rec, int base, int unit, int ns,
                                                         int s, int hl, int lane) {
    return rec + base + ((unit * ns + s) * 2 + hl) * FRAG + lane * 16;
}

// Sequence of chunk cg: the last n with offsets[n] <= cg (empty sequences are skipped).
__device__ __forceinline__ int find_seq(const int32_t* offsets, int num_seqs, int cg) {
    int lo = 0, hi = num_seqs;  // offsets[lo] <= cg < offsets[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= cg) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace

// --------------------------------------------------------------------------
// offsets[n] = number of 64-token chunks in sequences 0..n-1; offsets[N] = total.
// A sequence whose bounds are not 0 <= cu[n] <= cu[n+1] <= total_tokens gets
// no chunks, and offsets are clamped to max_chunks, the record capacity of the
// workspace, so later kernels never index past it.
__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                         int64_t total_tokens, int max_chunks,
                                                         int32_t* __restrict__ offsets) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int carry = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int i = base + tid;
        int nch = 0;
        if (i < num_seqs) {
            const int64_t a = cu[i], b = cu[i + 1];
            if (a >= 0 && b <= total_tokens && b >= a) nch = static_cast<int>((b - a + C - 1) / C);
        }
        int x = nch;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wv] = x;
        __syncthreads();
        int pre = 0, total = 0;
        for (int w2 = 0; w2 < 16; ++w2) {
            const int t = wsum[w2];
            if (w2 < wv) pre += t;
            total += t;
        }
        if (i < num_seqs) offsets[i] = min(carry + pre + x - nch, max_chunks);
        carry += total;
        __syncthreads();
    }
    if (tid == 0) offsets[num_seqs] = min(carry, max_chunks);
}

// --------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void prep_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ offsets, unsigned char* __restrict__ records, int num_seqs, int num_heads,
    float scale, int l2norm) {
    __shared__ __align__(16) unsigned char smem[P_LDS];
    float* sWT = reinterpret_cast<float*>(smem + P_LDT);
    float* srk = reinterpret_cast<float*>(smem + P_RK);
    float* srq = reinterpret_cast<float*>(smem + P_RQ);
    float* sbeta = reinterpret_cast<float*>(smem + P_BETA);
    float* sEm = reinterpret_cast<float*>(smem + P_EM);
    float* sEL = reinterpret_cast<float*>(smem + P_EL);
    float* sGL = reinterpret_cast<float*>(smem + P_GL);

    KDA_PHASE_BEGIN
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int n_chunks = offsets[num_seqs];
    const int items = n_chunks * num_heads;
    const int row_stride = num_heads * D;

    // Prefetch registers: rows 2rp, 2rp+1, channels 8cc..8cc+7 of k, q, g; beta.
    uint4 pk[2], pq[2];
    floatx4 pg[4];
    float pb = 0.f;
    auto fetch = [&](int item, int tid) {
        const int cg = item / num_heads, h = item - (item / num_heads) * num_heads;
        const int n = find_seq(offsets, num_seqs, cg);
        const int64_t start = cu_seqlens[n] + static_cast<int64_t>(C) * (cg - offsets[n]);
        const int L = static_cast<int>(min64(C, cu_seqlens[n + 1] - start));
        const size_t base = (static_cast<size_t>(start) * num_heads + h) * D;
        const int rp = tid >> 4, cc = tid & 15;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 2 * rp + j;
            const int off = r * row_stride + 8 * cc;
            if (r < L) {
                pk[j] = *reinterpret_cast<const uint4*>(k + base + off);
                pq[j] = *reinterpret_cast<const uint4*>(q + base + off);
                pg[2 * j] = *reinterpret_cast<const floatx4*>(g + base + off);
                pg[2 * j + 1] = *reinterpret_cast<const floatx4*>(g + base + off + 4);
            } else {
                pk[j] = uint4{0, 0, 0, 0};
                pq[j] = uint4{0, 0, 0, 0};
                pg[2 * j] = floatx4{0.f, 0.f, 0.f, 0.f};
                pg[2 * j + 1] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (tid < C) pb = tid < L ? beta[static_cast<size_t>(start + tid) * num_heads + h] : 0.f;
    };
    // Items run from the last chunk to the first: the records the state scan
    // reads first are the ones written last, still in the last-level cache.
    if (static_cast<int>(blockIdx.x) < items) fetch(items - 1 - static_cast<int>(blockIdx.x), threadIdx.x);

    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int item = items - 1 - it;
        const int lane = opaque(static_cast<int>(threadIdx.x) & 63);
        const int tid = wave * 64 + lane;
        const int l16 = lane & 15, l4 = lane >> 4;
        const int rp = tid >> 4, cc = tid & 15;
        const int cg = item / num_heads, h = item - cg * num_heads;
        unsigned char* rec = records + (static_cast<size_t>(cg) * num_heads + h) * REC_BYTES;

        // ======== phase 1: norms, cumulative log-decay, operand planes ========
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
        floatx8 cm = {0, 0, 0, 0, 0, 0, 0, 0};  // (totals of earlier waves) - G_31
        {
            const int lo_w = wave < 4 ? wave : 4, hi_w = wave < 4 ? 4 : wave;
            for (int w2 = lo_w; w2 < hi_w; ++w2) {
                const floatx4 a = *reinterpret_cast<const floatx4*>(sWT + w2 * D + 8 * cc);
                const floatx4 b = *reinterpret_cast<const floatx4*>(sWT + w2 * D + 8 * cc + 4);
                cm += floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            }
            if (wave < 4) cm = -cm;
        }
        const floatx8 d0 = (cm + (incl - pair) + g0) * kLog2e;
        const floatx8 d1 = d0 + g1 * kLog2e;
        if (tid < 3 * D) {
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
            *reinterpret_cast<bf16x8*>(smem + P_KGH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + P_KGL + o) = lo;
            split8(qf * e, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + P_QGH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + P_QGL + o) = lo;
            split8(kf * ei, hi, lo);
            *reinterpret_cast<bf16x8*>(smem + P_KIH + o) = hi;
            *reinterpret_cast<bf16x8*>(smem + P_KIL + o) = lo;
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next item's loads fly from here on
        if (it + static_cast<int>(gridDim.x) < items) fetch(items - 1 - (it + static_cast<int>(gridDim.x)), tid);
        lds_barrier();
        KDA_PHASE_MARK(0);

        // ======== phase 2: A' and P' blocks (K = 128 channels) ========
        floatx4 pacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            pacc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int R = kPrepPairs[wave][u][0], I = kPrepPairs[wave][u][1];
            if (R < 0) continue;
            const int ar = (16 * R + l16) * SW, br = (16 * I + l16) * SW;
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ko = 32 * s + 8 * l4;
                const bf16x8 bh = ld8(smem, P_KIH + (br + ko) * 2);
                const bf16x8 bl = ld8(smem, P_KIL + (br + ko) * 2);
                accA = mma(ld8(smem, P_KGH + (ar + ko) * 2), bh, accA);
                accP = mma3(ld8(smem, P_QGH + (ar + ko) * 2), ld8(smem, P_QGL + (ar + ko) * 2), bh, bl, accP);
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
                bf16x4 hi, lo;
                split4(a, hi, lo);
                const int o = ((pair_index(R, I) * 16 + l16) * WSTR + 4 * l4) * 2;
                *reinterpret_cast<bf16x4*>(smem + P_ATH + o) = hi;
                *reinterpret_cast<bf16x4*>(smem + P_ATL + o) = lo;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int lr = 4 * l4 + j;
                    a[j] = l16 < lr ? a[j] : (l16 == lr ? 1.f : 0.f);
                    pv[j] = l16 <= lr ? pv[j] : 0.f;
                }
                *reinterpret_cast<floatx4*>(smem + P_LDT + ((R * 16 + l16) * LDS_STR + 4 * l4) * 4) = a;
            }
            pacc[u] = pv;
        }
        lds_barrier();
        KDA_PHASE_MARK(1);

        // ======== phase 3: diagonal inverses (wave 0); P', Ki^T, Qg', vectors (waves 1-7) ========
        if (wave == 0) {
            const float* ldt = reinterpret_cast<const float*>(smem + P_LDT) + l4 * 16 * LDS_STR;
            float x[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) x[m] = (m == l16) ? 1.f : 0.f;
#pragma unroll
            for (int p0 = 0; p0 < 16; p0 += 4) {
                floatx4 col[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int qd = p0 / 4; qd < 4; ++qd)
                        col[t][qd] = *reinterpret_cast<const floatx4*>(ldt + (p0 + t) * LDS_STR + 4 * qd);
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
            const int r = 16 * l4 + l16;  // the column's own row in the chunk
            const float sphi = sbeta[r] * srk[r] * srk[r];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int o = ((l4 * 16 + m) * WSTR + l16) * 2;
                const float xv = x[m], xf = x[m] * sphi;
                const __bf16 hi = static_cast<__bf16>(xv), fh = static_cast<__bf16>(xf);
                *reinterpret_cast<__bf16*>(smem + P_XDH + o) = hi;
                *reinterpret_cast<__bf16*>(smem + P_XDL + o) = static_cast<__bf16>(xv - static_cast<float>(hi));
                *reinterpret_cast<__bf16*>(smem + P_XFH + o) = fh;
                *reinterpret_cast<__bf16*>(smem + P_XFL + o) = static_cast<__bf16>(xf - static_cast<float>(fh));
            }
        }
        // P' from the accumulators of phase 2 (any wave)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int R = kPrepPairs[wave][u][0], I = kPrepPairs[wave][u][1];
            if (R < 0) continue;
            bf16x4 hi, lo;
            split4(pacc[u], hi, lo);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int o = ((16 * R + 4 * l4 + j) * SN + 16 * I + l16) * 2;
                *reinterpret_cast<__bf16*>(smem + P_PH + o) = hi[j];
                *reinterpret_cast<__bf16*>(smem + P_PL + o) = lo[j];
            }
        }
        if (wave == 7) {
            // blocks (0,1) and (2,3) lie in the K range of 32-wide steps and read as zero
            const int blk = lane >> 5, row = (lane >> 1) & 15, part = lane & 1;
            const int r = (blk ? 32 : 0) + row, c0 = (blk ? 48 : 16) + 8 * part;
            const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
            *reinterpret_cast<bf16x8*>(smem + P_PH + (r * SN + c0) * 2) = z;
            *reinterpret_cast<bf16x8*>(smem + P_PL + (r * SN + c0) * 2) = z;
        }
        if (wave >= 1) {
            const int t1 = tid - 64;  // 0..447
            // Ke^T fragments: lane holds Ki[32s + 8(l/16) + i][16w + l%16] e^{G_last - G_31}[16w + l%16]
            //   = k e^{G_last - G} for 8 tokens of one channel (the decay to the chunk's end)
            for (int f = t1; f < 16 * 64; f += 448) {
                const int fr = f >> 6, ln = f & 63;
                const int w = fr >> 1, s = fr & 1;
                const int r0 = 32 * s + 8 * (ln >> 4), c = 16 * w + (ln & 15);
                floatx8 x = bf8_to_f(col8_tr(smem, P_KIH, SW, r0, 16 * w, ln & 15)) +
                            bf8_to_f(col8_tr(smem, P_KIL, SW, r0, 16 * w, ln & 15));
                x *= sEL[c];
                *reinterpret_cast<halfx8*>(rec + REC_KE + fr * FRAG + ln * 16) = __builtin_convertvector(x, halfx8);
            }
            // Qg' fragments: rq_r Qg[r][c] e^{G_31}[c]
            for (int f = t1; f < 16 * 64; f += 448) {
                const int fr = f >> 6, ln = f & 63;
                const int R = fr >> 2, s = fr & 3;
                const int r = 16 * R + (ln & 15), c0 = 32 * s + 8 * (ln >> 4);
                floatx8 x = bf8_to_f(ld8(smem, P_QGH + (r * SW + c0) * 2)) + bf8_to_f(ld8(smem, P_QGL + (r * SW + c0) * 2));
                const float rq = srq[r];
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] *= rq * sEm[c0 + i];
                *reinterpret_cast<halfx8*>(rec + REC_QG + fr * FRAG + ln * 16) = __builtin_convertvector(x, halfx8);
            }
            float* vec = reinterpret_cast<float*>(rec + REC_VEC);
            if (t1 < D) vec[VEC_GL + t1] = sGL[t1];
        }
        lds_barrier();
        KDA_PHASE_MARK(2);

        // ======== phase 4: W_RJ = -X_RR A'_RJ (six blocks, K = 16) ========
        if (wave < 6) {
            const int R = wave < 1 ? 1 : wave < 3 ? 2 : 3;
            const bool ok = l4 < 2;
            const int xo = ((R * 16 + l16) * WSTR + 8 * l4) * 2;
            const int bo = ((wave * 16 + l16) * WSTR + 8 * l4) * 2;
            floatx4 w = {0.f, 0.f, 0.f, 0.f};
            w = mma3(ld8_if(smem, P_XDH + xo, ok), ld8_if(smem, P_XDL + xo, ok), ld8_if(smem, P_ATH + bo, ok),
                     ld8_if(smem, P_ATL + bo, ok), w);
            bf16x4 hi, lo;
            split4(-w, hi, lo);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int o = ((wave * 16 + 4 * l4 + j) * WSTR + l16) * 2;
                *reinterpret_cast<__bf16*>(smem + P_WH + o) = hi[j];
                *reinterpret_cast<__bf16*>(smem + P_WL + o) = lo[j];
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(3);

        // ======== phase 5: Psi' and X' by block forward substitution ========
        // Column tile t of Psi' (wave t) and of X' (waves 0-3).  Step R:
        // out_R = rhs_R + sum_{J<R} W_RJ out_J, with out kept transposed in LDS.
        {
            const bool ok = l4 < 2;
            const int t = wave, c0 = 16 * t;
            const float em = sEm[c0 + l16];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                // rhs: (X_RR diag(rk^2 beta)) Kg_R[:, tile] e^{G_31}[col]
                const int xo = ((R * 16 + l16) * WSTR + 8 * l4) * 2;
                // rows past 16R + 15 (lanes with l4 >= 2) read other LDS data and are zeroed
                const bf16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
                const bf16x8 kgh8 = col8_tr(smem, P_KGH, SW, 16 * R + 8 * l4, c0, l16);
                const bf16x8 kgl8 = col8_tr(smem, P_KGL, SW, 16 * R + 8 * l4, c0, l16);
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma3(ld8_if(smem, P_XFH + xo, ok), ld8_if(smem, P_XFL + xo, ok), ok ? kgh8 : z8, ok ? kgl8 : z8,
                           acc);
                acc *= em;
#pragma unroll
                for (int J = 0; J < R; ++J) {
                    const int wo = ((pair_index(R, J) * 16 + l16) * WSTR + 8 * l4) * 2;
                    const int po = ((c0 + l16) * SN + 16 * J + 8 * l4) * 2;
                    acc = mma3(ld8_if(smem, P_WH + wo, ok), ld8_if(smem, P_WL + wo, ok), ld8_if(smem, P_PTH + po, ok),
                               ld8_if(smem, P_PTL + po, ok), acc);
                }
                bf16x4 hi, lo;
                split4(acc, hi, lo);
                const int oo = ((c0 + l16) * SN + 16 * R + 4 * l4) * 2;
                *reinterpret_cast<bf16x4*>(smem + P_PTH + oo) = hi;
                *reinterpret_cast<bf16x4*>(smem + P_PTL + oo) = lo;
                asm volatile("" ::: "memory");
            }
            if (wave < 4) {
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (R == t) {
                        // columns scaled by rk beta: the scan multiplies this X' by V directly
                        const float cs = srk[16 * t + l16] * sbeta[16 * t + l16];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int o = ((R * 16 + 4 * l4 + j) * WSTR + l16) * 2;
                            acc[j] = (static_cast<float>(*reinterpret_cast<const __bf16*>(smem + P_XDH + o)) +
                                      static_cast<float>(*reinterpret_cast<const __bf16*>(smem + P_XDL + o))) * cs;
                        }
                    }
                    for (int J = t; J < R; ++J) {
                        const int wo = ((pair_index(R, J) * 16 + l16) * WSTR + 8 * l4) * 2;
                        const int xo2 = ((16 * t + l16) * SN + 16 * J + 8 * l4) * 2;
                        acc = mma3(ld8_if(smem, P_WH + wo, ok), ld8_if(smem, P_WL + wo, ok),
                                   ld8_if(smem, P_XTH + xo2, ok), ld8_if(smem, P_XTL + xo2, ok), acc);
                    }
                    bf16x4 hi, lo;
                    split4(acc, hi, lo);
                    const int oo = ((16 * t + l16) * SN + 16 * R + 4 * l4) * 2;
                    *reinterpret_cast<bf16x4*>(smem + P_XTH + oo) = hi;
                    *reinterpret_cast<bf16x4*>(smem + P_XTL + oo) = lo;
                    asm volatile("" ::: "memory");
                }
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(4);

        // ======== phase 6: Psi', X', P' fragments out ========
        for (int f = tid; f < 40 * 64; f += NT) {
            const int fr = f >> 6, ln = f & 63;
            const int li = ln & 15, lk = 8 * (ln >> 4);
            if (fr < 16) {  // Psi' [R][s], fp16: lane holds Psi'[16R + li][32s + lk + i] = Psi'^T[..][..]
                const int R = fr >> 2, s = fr & 3;
                const floatx8 x = bf8_to_f(col8_tr(smem, P_PTH, SN, 32 * s + lk, 16 * R, li)) +
                                  bf8_to_f(col8_tr(smem, P_PTL, SN, 32 * s + lk, 16 * R, li));
                *reinterpret_cast<halfx8*>(rec + REC_PSI + fr * FRAG + ln * 16) = __builtin_convertvector(x, halfx8);
            } else if (fr < 32) {  // X' diag(rk beta) [R][s][hl], bf16
                const int f2 = fr - 16, R = f2 >> 2, s = (f2 >> 1) & 1, hl = f2 & 1;
                *reinterpret_cast<bf16x8*>(rec + REC_X + f2 * FRAG + ln * 16) =
                    col8_tr(smem, hl ? P_XTL : P_XTH, SN, 32 * s + lk, 16 * R, li);
            } else {  // P' [R][s], fp16, from the row-major hi/lo planes
                const int f2 = fr - 32, R = f2 >> 1, s = f2 & 1;
                const int o = ((16 * R + li) * SN + 32 * s + lk) * 2;
                const floatx8 x = bf8_to_f(ld8(smem, P_PH + o)) + bf8_to_f(ld8(smem, P_PL + o));
                *reinterpret_cast<halfx8*>(rec + REC_P + f2 * FRAG + ln * 16) = __builtin_convertvector(x, halfx8);
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(5);
    }
    KDA_PHASE_END;
}

// --------------------------------------------------------------------------
template <typename TOut, int NTL>
__global__ __launch_bounds__(NT) void scan_kernel(
    const bf16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ offsets,
    const unsigned char* __restrict__ records, const float* initial_state, TOut* __restrict__ out,
    float* final_state, int num_seqs, int num_heads) {
    using L_ = ScanLds<NTL>;
    __shared__ __align__(16) unsigned char smem[L_::BYTES];
    const int chain = blockIdx.x;
    if (chain >= num_seqs * num_heads) return;
    KDA_PHASE_BEGIN
    const int n = chain / num_heads, h = chain % num_heads;
    const int col0 = blockIdx.y * L_::COLS;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane0 = static_cast<int>(threadIdx.x) & 63;
    // Waves 0-3 form D (row block R = wave & 3), waves 4-7 the outputs of the
    // same row blocks; each SIMD (waves w and w+4) holds one of each.
    const int R = wave & 3;
    const bool forms_d = wave < 4;
    const bool wide = R >= 2;       // row blocks 2, 3 reach past the first 32 columns of X' and P'
    const int c_begin = offsets[n], c_end = offsets[n + 1];
    const int64_t t_first = cu_seqlens[n], t_last = cu_seqlens[n + 1];
    const int row_stride = num_heads * D;

    // This wave's rows 16 wave .. +15 of the state, NTL tiles of 16 columns.
    const size_t head_state = (static_cast<size_t>(n) * num_heads + h) * D * D;
    floatx4 S[NTL];
    {
        const int l16 = lane0 & 15, l4 = lane0 >> 4;
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[t][j] = initial_state
                              ? initial_state[head_state + (16 * wave + 4 * l4 + j) * D + col0 + DVT * t + l16]
                              : 0.f;
    }

    // Operands of one chunk held in registers.
    //   waves 0-3: a Psi'_R (fp16), b X'_R diag(rk beta) (bf16 hi/lo), vv values of V
    //   waves 4-7: a Qg'_R (fp16), b P'_R (fp16)
    //   all waves:  kt Ke^T rows 16 wave .. +15 (fp16); wave 0 also the chunk's vectors (gv)
    struct Frag {
        uint4 a[4];   // [s]
        uint4 b[4];   // [s*2 + hi/lo] (waves 4-7: hi slot only); s = 1 only for wide row blocks
        uint4 kt[2];  // [s]
        uint4 gv;     // wave 0: 16 bytes of the vector block (lane l: floats 4l .. 4l+3)
        uint32_t vv[NTL][4];  // bf16 bits, zero-extended (packed only at use)
    };
    // The loads come in three parts, issued at three points of the previous
    // chunk's step, so the memory pipeline never holds a whole chunk's requests
    // in front of the step's own instructions.
    auto load = [&](Frag& F, int cg, int lane, int part) {
        const unsigned char* rec = records + (static_cast<size_t>(cg) * num_heads + h) * REC_BYTES;
        const int l16 = lane & 15, l4 = lane >> 4;
        if (part == 0) {
            {
                // V rows of this wave's row block (waves 4-7 load them too, so
                // every wave runs the same loads); rows past the chunk's end
                // read as zero
                const int64_t tok0 = t_first + static_cast<int64_t>(C) * (cg - c_begin);
                const int L = static_cast<int>(min64(C, t_last - tok0));
                const auto vr = buffer_rsrc(v + (static_cast<size_t>(tok0) * num_heads + h) * D + col0,
                                            L * row_stride * 2);
#pragma unroll
                for (int t = 0; t < NTL; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        F.vv[t][j] = __builtin_amdgcn_raw_buffer_load_b16(
                            vr, ((16 * R + 4 * l4 + j) * row_stride + DVT * t + l16) * 2, 0, 0);
            }
            const int abase = forms_d ? REC_PSI : REC_QG;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                F.a[s] = *reinterpret_cast<const uint4*>(rec + abase + (R * 4 + s) * FRAG + lane * 16);
        } else if (part == 1) {
            // waves 0-3: X' (bf16 hi/lo) in b[2s + hl]; waves 4-7: P' (fp16) in b[2s]
            const unsigned char* xb = rec + REC_X + (R * 2 * 2) * FRAG + lane * 16;
            const unsigned char* pb = rec + REC_P + (R * 2) * FRAG + lane * 16;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s == 1 && !wide) break;
                F.b[2 * s] = *reinterpret_cast<const uint4*>(forms_d ? xb + (2 * s) * FRAG : pb + s * FRAG);
                if (forms_d) F.b[2 * s + 1] = *reinterpret_cast<const uint4*>(xb + (2 * s + 1) * FRAG);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                F.kt[s] = *reinterpret_cast<const uint4*>(rec + REC_KE + (wave * 2 + s) * FRAG + lane * 16);
            if (wave == 0) F.gv = *reinterpret_cast<const uint4*>(rec + REC_VEC + lane * 16);
        }
    };
    // One chunk.  An inactive step (the pad after an odd chunk count) leaves
    // S unchanged and stores nothing.  Fn / cg_next: the buffer and chunk
    // whose loads are issued during this step.
    auto step = [&](const Frag& F, int cg, int lane, bool active, Frag& Fn, int cg_next) {
        const int l16 = lane & 15, l4 = lane >> 4;
        const int64_t tok0 = t_first + static_cast<int64_t>(C) * (cg - c_begin);
        const int L = active ? static_cast<int>(min64(C, t_last - tok0)) : 0;
        const int slot = L_::VEC + (cg & 1) * 1024;
        load(Fn, cg_next, lane, 0);
        // (a) S^T (fp16 hi/lo), V^T (bf16), the chunk's vectors
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            halfx4 hi, lo;
            split4h(S[t], hi, lo);
            const int o = ((DVT * t + l16) * SW + 16 * wave + 4 * l4) * 2;
            *reinterpret_cast<halfx4*>(smem + L_::STH + o) = hi;
            *reinterpret_cast<halfx4*>(smem + L_::STL + o) = lo;
            if (forms_d) {
                const uint2 vp = {F.vv[t][0] | (F.vv[t][1] << 16), F.vv[t][2] | (F.vv[t][3] << 16)};
                *reinterpret_cast<uint2*>(smem + L_::V + ((DVT * t + l16) * SN + 16 * R + 4 * l4) * 2) = vp;
            }
        }
        if (wave == 0) *reinterpret_cast<uint4*>(smem + slot + lane * 16) = F.gv;
        lds_barrier();
        KDA_PHASE_MARK(8);
        load(Fn, cg_next, lane, 1);
        // (b) waves 0-3: D_R = X'_R diag(rk beta) V - Psi'_R S; waves 4-7: Qg'_R S
        floatx4 acc[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            // two accumulation chains, summed at the end
            floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s += 2) {
                const int ko = ((DVT * t + l16) * SW + 32 * s + 8 * l4) * 2;
                const halfx8 x0 = as_halfx8(F.a[s]), x1 = as_halfx8(F.a[s + 1]);
                a0 = mmah(x0, ldh8(smem, L_::STH + ko), a0);
                a0 = mmah(x0, ldh8(smem, L_::STL + ko), a0);
                a1 = mmah(x1, ldh8(smem, L_::STH + ko + 64), a1);
                a1 = mmah(x1, ldh8(smem, L_::STL + ko + 64), a1);
            }
            acc[t] = a0 + a1;
            if (forms_d) {
                floatx4 d0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s == 1 && !wide) break;
                    const bf16x8 vb = ld8(smem, L_::V + ((DVT * t + l16) * SN + 32 * s + 8 * l4) * 2);
                    d0 = mma(as_bf16x8(F.b[2 * s]), vb, d0);
                    d0 = mma(as_bf16x8(F.b[2 * s + 1]), vb, d0);
                }
                halfx4 hi, lo;
                split4h(d0 - acc[t], hi, lo);
                const int o = ((DVT * t + l16) * SN + 16 * R + 4 * l4) * 2;
                *reinterpret_cast<halfx4*>(smem + L_::DH + o) = hi;
                *reinterpret_cast<halfx4*>(smem + L_::DL + o) = lo;
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(9);
        load(Fn, cg_next, lane, 2);
        // (c) U = Ke^T D and the state update; waves 4-7: O_R = Qg'_R S + P'_R D
        {
            const floatx4 gl = *reinterpret_cast<const floatx4*>(smem + slot + (VEC_GL + 16 * wave + 4 * l4) * 4);
            const halfx8 k0 = as_halfx8(F.kt[0]), k1 = as_halfx8(F.kt[1]);
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                floatx4 u = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
                const int ko = ((DVT * t + l16) * SN + 8 * l4) * 2;
                u = mmah(k0, ldh8(smem, L_::DH + ko), u);
                u1 = mmah(k1, ldh8(smem, L_::DH + ko + 64), u1);
                u = mmah(k0, ldh8(smem, L_::DL + ko), u);
                u1 = mmah(k1, ldh8(smem, L_::DL + ko + 64), u1);
                const floatx4 s_new = gl * S[t] + (u + u1);
                S[t] = active ? s_new : S[t];
            }
        }
        if (!forms_d) {
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s == 1 && !wide) break;
                    const int ko = ((DVT * t + l16) * SN + 32 * s + 8 * l4) * 2;
                    const halfx8 pb = as_halfx8(F.b[2 * s]);
                    acc[t] = mmah(pb, ldh8(smem, L_::DH + ko), acc[t]);
                    acc[t] = mmah(pb, ldh8(smem, L_::DL + ko), acc[t]);
                }
            }
        }
        // Exactly 4 NTL stores per lane on every wave, so the wait counts in
        // the chunk loop are fixed: waves 0-3 (no output) and rows past the
        // chunk's end go through an empty or shorter range and are dropped.
        const int out_bytes = forms_d ? 0 : L * row_stride * static_cast<int>(sizeof(TOut));
        const auto orr = buffer_rsrc(out + (static_cast<size_t>(tok0) * num_heads + h) * D + col0, out_bytes);
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int off = ((16 * R + 4 * l4 + j) * row_stride + DVT * t + l16) * static_cast<int>(sizeof(TOut));
                if constexpr (sizeof(TOut) == 4)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[t][j]), orr, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[t][j]).bits, orr, off, 0, 0);
            }
        KDA_PHASE_MARK(10);
    };

    // Two register buffers: the loads for chunk c+1 are issued during chunk
    // c.  Loads past the last chunk re-read it, and the pad step is inactive,
    // so no memory operation depends on data, and the wait after each step
    // names exactly what may still be in flight: that step's stores.
    // (Left to itself the compiler loses count across the loop's back edge and
    // drains every load, prefetch included, before each chunk.)
    if (c_begin < c_end) {
        Frag F0, F1;
        load(F0, c_begin, lane0, 0);
        load(F0, c_begin, lane0, 1);
        load(F0, c_begin, lane0, 2);
        wait_vmcnt<0>();
        for (int cg = c_begin; cg < c_end; cg += 2) {
            const int lane = opaque(lane0);
            step(F0, cg, lane, true, F1, min(cg + 1, c_end - 1));
            wait_vmcnt<4 * NTL>();
            KDA_PHASE_MARK(11);
            step(F1, cg + 1, lane, cg + 1 < c_end, F0, min(cg + 2, c_end - 1));
            wait_vmcnt<4 * NTL>();
            KDA_PHASE_MARK(11);
        }
    }

    if (final_state) {
        const int l16 = lane0 & 15, l4 = lane0 >> 4;
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                final_state[head_state + (16 * wave + 4 * l4 + j) * D + col0 + DVT * t + l16] = S[t][j];
    }
    KDA_PHASE_END;
}

// --------------------------------------------------------------------------
#ifndef SCAN_NTL
#define SCAN_NTL 1  // 16-column tiles per scan workgroup
#endif

bool split_prefill_applies(const PrefillArgs& a) { return a.qkv_bf16 && a.head_dim == D; }

size_t split_workspace_bytes(int64_t total_tokens, int num_seqs, int num_heads) {
    const size_t off_bytes = (static_cast<size_t>(num_seqs + 1) * 4 + 255) & ~size_t(255);
    const size_t max_chunks = static_cast<size_t>((total_tokens + C - 1) / C) + static_cast<size_t>(num_seqs);
    return off_bytes + max_chunks * static_cast<size_t>(num_heads) * REC_BYTES;
}

static int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

template <typename TOut>
static hipError_t launch_split_t(const PrefillArgs& a, void* workspace, hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws);
    unsigned char* records = ws + ((static_cast<size_t>(a.num_seqs + 1) * 4 + 255) & ~size_t(255));
    const size_t max_chunks = static_cast<size_t>((a.total_tokens + C - 1) / C) + static_cast<size_t>(a.num_seqs);
    chunk_map_kernel<<<1, 1024, 0, stream>>>(a.cu_seqlens, a.num_seqs, a.total_tokens, static_cast<int>(max_chunks),
                                             offsets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t max_items = max_chunks * static_cast<size_t>(a.num_heads);
    const unsigned prep_grid = static_cast<unsigned>(max_items < static_cast<size_t>(device_cu_count()) ? max_items : static_cast<size_t>(device_cu_count()));
    if (prep_grid > 0) {
        prep_kernel<<<prep_grid, NT, 0, stream>>>(static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                                                  a.g, a.beta, a.cu_seqlens, offsets, records, a.num_seqs,
                                                  a.num_heads, a.scale, a.l2norm);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned chains = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
    // tiles of one chain (linear ids chain + k * grid.x) share an XCD when grid.x % 8 == 0
    const dim3 grid((chains + 7u) & ~7u, D / (DVT * SCAN_NTL));
    scan_kernel<TOut, SCAN_NTL><<<grid, NT, 0, stream>>>(static_cast<const bf16_t*>(a.v), a.cu_seqlens, offsets,
                                                         records, a.initial_state, static_cast<TOut*>(a.out),
                                                         a.final_state, a.num_seqs, a.num_heads);
    return hipGetLastError();
}

hipError_t launch_prefill_split(const PrefillArgs& a, void* workspace, hipStream_t stream) {
    return a.out_bf16 ? launch_split_t<bf16_t>(a, workspace, stream) : launch_split_t<float>(a, workspace, stream);
}

}  // namespace kda
