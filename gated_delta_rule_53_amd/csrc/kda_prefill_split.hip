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
//                     cu_seqlens (device side, no host synchronisation) and
//                     the order in which the scan takes the sequences.
//   prep_kernel       persistent, fully parallel over (chunk, head): builds
//                     Kg/Qg/Ki, A and P on MFMA, the four 16x16 diagonal
//                     inverses, W_RJ = -X_RR A'_RJ, and solves for Psi' and X'
//                     by block forward substitution.  Writes -Psi', Qg', Ke^T,
//                     X', P' and e^{G_last} to a per-(chunk, head) record, in
//                     the lane order the scan's MFMA operands use.
//   scan_kernel       one workgroup per (sequence, head, one or two 16-column
//                     value tiles) carries the chunk chain above.  One wave
//                     per tile holds the state tile in MFMA accumulators and
//                     feeds it back as the B operand without moving it (see
//                     "accumulator order"); three more waves copy the record
//                     into LDS ahead of them, form Delta0 ahead of them and
//                     form the output behind them, for all its tiles.
// Inside prep, operands are bf16 hi/lo pairs (hi*hi + hi*lo + lo*hi), except
// k.k in A (inverted afterwards; pairs too in the blocks that chunks too steep
// for the reference token form on MFMA); the 16x16 diagonal inverses are fp32.
#include <type_traits>

#include "kda_bf16_mfma.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;       // chunk length
constexpr int D = 128;      // head size
constexpr int DVT = 16;     // value columns of one MFMA tile in the scan
constexpr int PNT = 1024;   // threads per prep workgroup (16 waves)
constexpr int SW = D + 8;   // bf16 row stride of 128-wide LDS planes
constexpr int SN = C + 8;   // bf16 row stride of 64-wide LDS planes

// ---- per-(chunk, head) record written by prep_kernel ----
// A fragment is one wave-wide MFMA A operand: 64 lanes x 16 bytes, lane l
// holding row row0 + l%16 at the eight K indices of lane group g = l/16.
// Accumulator order: within each 32-wide K block, group g holds K indices
// 4g .. 4g+3 and 16+4g .. 16+4g+3.  Those are exactly the rows a pair of
// 16x16 accumulator tiles (K rows 0-15 and 16-31 of the block) leaves in the
// lanes of group g, so an accumulator pair converts into a B operand in
// place.  Every fragment below is in accumulator order.
constexpr int FRAG = 1024;
// The operands the state meets (Psi', Qg', Ke^T, P') are single fp16; the
// state side (S, D) is an fp16 hi/lo pair.  fp16 keeps 11 significant bits,
// and every one of these operands is bounded: Qg' by |q_hat|, P' by
// |q_hat||k_hat|, Ke = k e^{G_last - G} by |k|, Psi' by the scaled inverse.
// X' diag(rk beta) is single fp16 too; the scan multiplies it by V taken to
// fp16 (exact for bf16 values in fp16's normal range).
// X' and P' are lower triangular: only the six (R, s) blocks with
// 32 s <= 16 R + 15 are stored (tri_block).
constexpr int REC_NPSI = 0;                   // -Psi' : [R 4][s 4] fragments, fp16
constexpr int REC_QG = 16 * FRAG;             // Qg'   : [R 4][s 4], fp16
constexpr int REC_KE = 32 * FRAG;             // Ke^T  : [channel block 8][s 2], fp16
constexpr int REC_X = 48 * FRAG;              // X' diag(rk beta) : [tri 6], fp16
constexpr int REC_P = 54 * FRAG;              // P'    : [tri 6], fp16
constexpr int REC_VEC = 60 * FRAG;            // fp32 e^{G_last}[128]
constexpr int REC_BYTES = REC_VEC + D * 4;    // 61952

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
// X_RR and X_RR diag(rk^2 beta) are stored transposed, block R at R * BLK:
// row c holds column c of the block (written by one lane as two 16-byte stores).
constexpr int P_XDH = P_LDT + 4 * 16 * LDS_STR * 4;             // X_RR^T [4][16][24] bf16
constexpr int P_XDL = P_XDH + 4 * BLK;
constexpr int P_XFH = P_XDL + 4 * BLK;                          // (X_RR diag(rk^2 beta))^T
constexpr int P_XFL = P_XFH + 4 * BLK;
constexpr int P_RK = P_XFL + 4 * BLK;                           // fp32 [64]
constexpr int P_RQ = P_RK + C * 4;
constexpr int P_BETA = P_RQ + C * 4;
constexpr int P_EM = P_BETA + C * 4;                            // fp32 [128] e^{G_31}
constexpr int P_EL = P_EM + D * 4;                              // e^{G_last - G_31}
constexpr int P_GL = P_EL + D * 4;                              // e^{G_last}
constexpr int P_G31 = P_GL + D * 4;                             // fp32 [128] G_31 (natural log)
constexpr int P_GLL = P_G31 + D * 4;                            // fp32 [128] G_last (natural log)
constexpr int P_FLAG = P_GLL + D * 4;                           // int: the item takes the exact path
constexpr int P_CW = P_FLAG + 16;                               // conv taps of the item's head: k, q [4][128] bf16
constexpr int P_LDS = P_CW + 2 * 4 * D * 2;
static_assert(P_LDS <= 160 * 1024, "prep LDS budget");
constexpr int P_WT = P_XDH;                                     // 16 wave totals [16][128] fp32 (phase 1 only)
static_assert(16 * D * 4 <= 4 * 4 * BLK, "wave totals alias X_RR and X_RR diag(rk^2 beta)");
// Exact path (a chunk whose decay is too strong for the reference token):
// raw k and q of every row, bf16 [64][128] (the values are bf16 already), and
// e^g and G (the cumulative log-decay from the chunk's start), fp32 [64][128],
// in regions 1-3 before the planes are formed there.
constexpr int P_GK = 0, P_GQ = C * D * 2, P_GE = 2 * C * D * 2, P_GG = P_GE + C * D * 4;
static_assert(P_GG + C * D * 4 <= P_R3_END && P_R3_END <= P_PH, "exact-path arrays fit below P'");
// Fused convolution: the raw k and q rows -4 .. 63 of the chunk (row -4 + i
// at i * 256 bytes), in region 1 from the top of an item until its planes.
constexpr int P_CVK = 0, P_CVQ = (C + 4) * D * 2;
static_assert(P_CVQ + (C + 4) * D * 2 <= P_R2, "raw rows fit in region 1");
// Largest |G_r - G_31| (natural log) the reference-token factors may span:
// e^{60} and e^{-60} are well inside the float32 and bf16 normal range.
constexpr float kRefSpan = 60.f;

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }

// Stored (R, s) blocks of the triangular operands: R = 0, 1 have s = 0 only.
__host__ __device__ constexpr int tri_block(int R, int s) { return R < 2 ? R : 2 * R - 2 + s; }
__host__ __device__ constexpr int tri_R(int b) { return b < 2 ? b : 2 + ((b - 2) >> 1); }
__host__ __device__ constexpr int tri_s(int b) { return b < 2 ? 0 : (b - 2) & 1; }

// (R, I) block of A and P computed by waves 1-10 of prep_kernel (one each).
// The table only feeds constant evaluation: the kernel reads it as two packed
// immediates, so selecting a wave's block costs scalar shifts and no memory
// load (a load here would also wait on the next item's prefetch in flight).
constexpr int8_t kPrepUnit[16][2] = {
    {-1, -1}, {1, 0}, {3, 3}, {2, 0}, {2, 2}, {2, 1}, {1, 1}, {3, 0},
    {0, 0}, {3, 1}, {3, 2}, {-1, -1}, {-1, -1}, {-1, -1}, {-1, -1}, {-1, -1},
};
constexpr uint32_t pack_prep_unit(int col) {
    uint32_t r = 0;
    for (int w = 0; w < 16; ++w) r |= static_cast<uint32_t>(kPrepUnit[w][col] & 3) << (2 * w);
    return r;
}
constexpr uint32_t kPrepUnitR = pack_prep_unit(0), kPrepUnitI = pack_prep_unit(1);
constexpr bool prep_unit_packing_ok() {
    for (int w = 0; w < 16; ++w) {
        const bool has = w >= 1 && w <= 10;
        if (has != (kPrepUnit[w][0] >= 0)) return false;
        if (has && (static_cast<int>((kPrepUnitR >> (2 * w)) & 3) != kPrepUnit[w][0] ||
                    static_cast<int>((kPrepUnitI >> (2 * w)) & 3) != kPrepUnit[w][1]))
            return false;
    }
    return true;
}
static_assert(prep_unit_packing_ok(), "waves 1-10 own one block each");

__device__ __forceinline__ const unsigned char* frag_ptr(const unsigned char* rec, int base, int unit, int ns,
                                                         int s, int hl, int lane) {
    return rec + base + ((unit * ns + s) * 2 + hl) * FRAG + lane * 16;
}

// A' and P' of a chunk whose decay is too steep for one reference token,
// exactly (every factor at most 1, so none overflows; the ones that underflow
// are zero).  The chunk's 64 rows form eight 8-row groups.
// - Inside each group, elementwise: wave pw takes columns i = 4 pw .. 4 pw + 3
//   (one per lane group; lane l16 holds 8 channels) and carries
//   z = k_i e^{G_r - G_i} down the group's rows r >= i as a running product of
//   e^{g_r} <= 1, forming k_r . z and q_r . z per row.
// - Everything else below the diagonal, on MFMA, with both operands referred
//   to the last token e of the column block (columns k_i e^{G_e - G_i}, rows
//   k_r e^{G_r - G_e}, q_r for P'), bf16 hi/lo pairs built in registers: the
//   six 16x16 blocks R > I (e = 16 I + 15), and in each diagonal block the
//   rows 8 .. 15 against the columns 0 .. 7 (e = 16 R + 7), two diagonal blocks
//   to one product (its two cross quarters mix references and are dropped;
//   their factors are at most 1 too).  The waves whose groups have the fewest
//   rows take these eight products, two per SIMD.
// With the factored path's scalings, A'[r][i] = beta_r rk_r^2 (k_r . z) for
// i < r and P'[r][i] = rq_r (q_r . z) for i <= r (z = k_i e^{G_r - G_i}), and
// written where that path puts its own: A' blocks below the diagonal and P' as
// bf16 hi/lo planes, the diagonal blocks of L' in fp32.  Entries above the
// diagonal are not written: the inverses do not read them, and the P' planes
// are cleared beforehand.
__device__ __forceinline__ void exact_ap(unsigned char* smem, int wave, int l16, int l4) {
    const float* ge = reinterpret_cast<const float*>(smem + P_GE);
    const float* gg = reinterpret_cast<const float*>(smem + P_GG);
    const float* srk = reinterpret_cast<const float*>(smem + P_RK);
    const float* srq = reinterpret_cast<const float*>(smem + P_RQ);
    const float* sbeta = reinterpret_cast<const float*>(smem + P_BETA);
    auto f32row8 = [&](const float* base, int r, int c0) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(base + r * D + c0);
        const floatx4 b = *reinterpret_cast<const floatx4*>(base + r * D + c0 + 4);
        return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };
    auto bfrow8 = [&](int plane, int r, int c0) { return bf8_to_f(ld8(smem, plane + (r * D + c0) * 2)); };
    // ---- inside the 8-row groups ----
    // Column group pw starts at row 4 pw and runs to its 8-row group's end (8
    // rows for even pw, 4 for odd).  The four waves sharing a SIMD (wave mod 4)
    // get two of each.
    const int pw = ((wave >> 2) & 1) ? (wave ^ 3) : wave;
    const int r0 = 4 * pw, i = r0 + l4, co = 8 * l16;
    const int rend = (r0 | 7) + 1;
    const floatx8 ki = bfrow8(P_GK, i, co);
    floatx8 z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float av = 0.f, pv = 0.f;  // lane l16 keeps the sums of row 16 (r / 16) + l16
    // Row r of the sums: z is born at r == i (the first four rows of the
    // group), decayed by e^{g_r} afterwards; the group ends at r % 8 == 7.
    auto step = [&](int r, bool birth) {
        const floatx8 er = f32row8(ge, r, co);
        if (birth) {
#pragma unroll
            for (int c = 0; c < 8; ++c) z[c] = r == i ? ki[c] : z[c] * er[c];
        } else {
            z *= er;
        }
        const floatx8 kr = bfrow8(P_GK, r, co), qr = bfrow8(P_GQ, r, co);
        float a = 0.f, p = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            a += kr[c] * z[c];
            p += qr[c] * z[c];
        }
        a = row16_sum(a);
        p = row16_sum(p);
        av = l16 == (r & 15) ? a : av;
        pv = l16 == (r & 15) ? p : pv;
        if ((r & 7) != 7) return;
        const int rr = (r & ~15) + l16;
        if (rr < i || rr > r) return;  // lanes of the group's rows at or below the diagonal
        uint32_t h, l;
        split2(srq[rr] * pv, 0.f, h, l);
        *reinterpret_cast<uint16_t*>(smem + P_PH + (rr * SN + i) * 2) = static_cast<uint16_t>(h);
        *reinterpret_cast<uint16_t*>(smem + P_PL + (rr * SN + i) * 2) = static_cast<uint16_t>(l);
        if (rr == i) return;
        const float rk = srk[rr];
        const int R = rr >> 4;
        *reinterpret_cast<float*>(smem + P_LDT + ((R * 16 + (i & 15)) * LDS_STR + (rr & 15)) * 4) =
            sbeta[rr] * rk * rk * av;
    };
    for (int r = r0; r < r0 + 4; ++r) step(r, true);
    for (int r = r0 + 4; r < rend; ++r) step(r, false);

    // ---- the rest below the diagonal, on MFMA ----
    // jobs 0-5: block (R, I) = (1,0), (2,0), (2,1), (3,0), (3,1), (3,2); jobs 6,
    // 7: the lower-left quarters of diagonal blocks 0, 1 and 2, 3.  Lane l16 is
    // the row (A operand) and the column (B operand) of its 16.
    const int b = wave == 1 ? 0 : wave == 3 ? 1 : wave == 4 ? 2 : wave == 6 ? 3 : wave == 9 ? 4 : wave == 11 ? 5
                : wave == 12 ? 6 : wave == 14 ? 7 : -1;
    if (b < 0) return;
    int rrow, icol, e;
    if (b < 6) {
        const int R = b < 1 ? 1 : b < 3 ? 2 : 3;
        const int I = b < 1 ? 0 : b < 3 ? b - 1 : b - 3;
        rrow = 16 * R + l16;
        icol = 16 * I + l16;
        e = 16 * I + 15;
    } else {
        const int Rd = 2 * (b - 6) + (l16 >> 3);  // this lane's diagonal block
        rrow = 16 * Rd + 8 + (l16 & 7);
        icol = 16 * Rd + (l16 & 7);
        e = 16 * Rd + 7;
    }
    floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int s = 0; s < 4; ++s) {
        const int c0 = 32 * s + 8 * l4;
        // columns up to e: k_i e^{G_e - G_i}, G_e <= G_i
        const floatx8 gm = f32row8(gg, e, c0);
        bf16x8 bh, bl;
        {
            const floatx8 gc = f32row8(gg, icol, c0), kc = bfrow8(P_GK, icol, c0);
            floatx8 xb;
#pragma unroll
            for (int c = 0; c < 8; ++c) xb[c] = kc[c] * fast_exp2((gm[c] - gc[c]) * kLog2e);
            split8(xb, bh, bl);
        }
        // rows after e: e^{G_r - G_e}, G_r <= G_e, shared by A' (k_r) and P' (q_r)
        floatx8 fr;
        {
            const floatx8 gr = f32row8(gg, rrow, c0);
#pragma unroll
            for (int c = 0; c < 8; ++c) fr[c] = fast_exp2((gr[c] - gm[c]) * kLog2e);
        }
        {
            const floatx8 kr = bfrow8(P_GK, rrow, c0);
            bf16x8 ah, al;
            split8(kr * fr, ah, al);
            accA = mma3(ah, al, bh, bl, accA);
        }
        {
            const floatx8 qr = bfrow8(P_GQ, rrow, c0);
            bf16x8 ph, pl;
            split8(qr * fr, ph, pl);
            accP = mma3(ph, pl, bh, bl, accP);
        }
    }
    // accumulator j of lane (l4, l16): A operand row m = 4 l4 + j, B operand
    // column n = l16, stored as the factored path stores them
    if (b < 6) {
        const int R = b < 1 ? 1 : b < 3 ? 2 : 3;
        const int I = b < 1 ? 0 : b < 3 ? b - 1 : b - 3;
        floatx4 a, pq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * R + 4 * l4 + j;
            const float rk = srk[r];
            a[j] = sbeta[r] * rk * rk * accA[j];
            pq[j] = srq[r] * accP[j];
        }
        bf16x4 hi, lo;
        split4(a, hi, lo);
        const int o = ((pair_index(R, I) * 16 + l16) * WSTR + 4 * l4) * 2;
        *reinterpret_cast<bf16x4*>(smem + P_ATH + o) = hi;
        *reinterpret_cast<bf16x4*>(smem + P_ATL + o) = lo;
        split4(pq, hi, lo);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int o2 = ((16 * R + 4 * l4 + j) * SN + 16 * I + l16) * 2;
            *reinterpret_cast<__bf16*>(smem + P_PH + o2) = hi[j];
            *reinterpret_cast<__bf16*>(smem + P_PL + o2) = lo[j];
        }
    } else if ((l4 >> 1) == (l16 >> 3)) {  // rows and column of the same diagonal block
        const int Rd = 2 * (b - 6) + (l16 >> 3);
        const int cl = l16 & 7;  // column 16 Rd + cl
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rl = 8 + 4 * (l4 & 1) + j;  // row 16 Rd + rl
            const int r = 16 * Rd + rl;
            const float rk = srk[r];
            *reinterpret_cast<float*>(smem + P_LDT + ((Rd * 16 + cl) * LDS_STR + rl) * 4) =
                sbeta[r] * rk * rk * accA[j];
            uint32_t h, l;
            split2(srq[r] * accP[j], 0.f, h, l);
            *reinterpret_cast<uint16_t*>(smem + P_PH + (r * SN + 16 * Rd + cl) * 2) = static_cast<uint16_t>(h);
            *reinterpret_cast<uint16_t*>(smem + P_PL + (r * SN + 16 * Rd + cl) * 2) = static_cast<uint16_t>(l);
        }
    }
}

// ---- the short convolution fused into the q/k/v loads ----
// Its four taps (K < 4: leading taps of weight zero) meet the rows r - 3 ..
// r of the fused projection; the arithmetic is that of kda_short_conv term
// for term (the tap that meets row r first, then one fused multiply-add per
// step back), then y * sigmoid(y) with silu, rounded to bf16 as the
// standalone convolution's output is, so the core sees the same inputs.

// Lane l gets lane l - 1's words (lane 0 gets lane 63's): a DPP whole-wave rotate.
__device__ __forceinline__ uint4 ror1_u4(const uint4& v) {
    constexpr int kWaveRor1 = 0x13C;
    return uint4{static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v.x), kWaveRor1, 0xF, 0xF, false)),
                 static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v.y), kWaveRor1, 0xF, 0xF, false)),
                 static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v.z), kWaveRor1, 0xF, 0xF, false)),
                 static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v.w), kWaveRor1, 0xF, 0xF, false))};
}

// x0 .. x3: the eight channels' inputs 0 .. 3 steps back; t: their tap pairs.
// The convolution of kda_short_conv (conv8_bf16), then silu, rounded to bf16;
// zero for rows past the chunk's end.
// Channels 2e, 2e + 1 for the words e in [E0, E1) (the others are left zero).
template <int E0 = 0, int E1 = 4>
__device__ __forceinline__ floatx8 conv8(const uint4& x0, const uint4& x1, const uint4& x2, const uint4& x3,
                                        const ConvTaps8& t, int silu, bool live) {
    float a[8] = {};
    conv8_bf16<E0, E1>(x0, x1, x2, x3, t, a);
    if (silu) {
#pragma unroll
        for (int i = 2 * E0; i < 2 * E1; ++i) a[i] *= gate_sigmoid(a[i]);
    }
    // bf16 round to nearest even in hardware, as the standalone kernel rounds
    floatx8 y = {};
#pragma unroll
    for (int i = 2 * E0; i < 2 * E1; i += 2) {
        const uint32_t p = pack_bf16x2(a[i], a[i + 1]);
        y[i] = live ? __uint_as_float(p << 16) : 0.f;
        y[i + 1] = live ? __uint_as_float(p & 0xffff0000u) : 0.f;
    }
    return y;
}

// One lane's part of a record fragment, as fp16.  A record is written once
// and read once, by the chain pass.  NT: a non-temporal store (config 2: about
// 2 % faster); the chain pass with the fused convolution, whose helper waves
// touch fewer record lines ahead, reads them faster from the last-level cache
// after ordinary stores (201 against 207 us).
template <bool NT>
__device__ __forceinline__ void store_frag(unsigned char* p, const floatx8& x) {
    if constexpr (NT)
        __builtin_nontemporal_store(__builtin_convertvector(x, halfx8), reinterpret_cast<halfx8*>(p));
    else
        *reinterpret_cast<halfx8*>(p) = __builtin_convertvector(x, halfx8);
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
// order[r] is the sequence with the r-th most chunks (ties by index), so the
// scan dispatches the longest chains first and the short ones fill the tail
// (longest-processing-time-first list scheduling).  Beyond SORT_MAX sequences
// order is the identity.
constexpr int SORT_MAX = 1024;

__device__ inline int seq_chunks(const int32_t* __restrict__ cu, int i, int64_t total_tokens) {
    const int64_t a = cu[i], b = cu[i + 1];
    return (a >= 0 && b <= total_tokens && b >= a) ? static_cast<int>((b - a + C - 1) / C) : 0;
}

// Where prep_kernel and chain_kernel find each sequence's chunks: the chunk
// map's offsets and order in the workspace, or, with offsets null (at most
// kLaneMapSeqs sequences, every chain running at once so their order does not
// matter), offsets each wave computes from cu_seqlens at its start and the
// sequences in index order.  One kernel launch fewer per call.
struct ChunkMap {
    const int32_t* offsets;  // [N + 1], or null
    const int32_t* order;    // [N], or null
    int64_t total_tokens;
    int max_chunks;          // the workspace's record capacity in chunks
};
constexpr int kLaneMapSeqs = 63;

// The chunk map's offsets in a wave's lanes: lane n (n <= num_seqs) holds
// offsets[n], clamped to max_chunks as chunk_map_kernel clamps them.
__device__ __forceinline__ int lane_offsets(const int32_t* __restrict__ cu, int num_seqs, const ChunkMap& cm,
                                            int lane) {
    const int mine = lane < num_seqs ? seq_chunks(cu, lane, cm.total_tokens) : 0;
    int x = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        x += lane >= off ? y : 0;
    }
    return min(x - mine, cm.max_chunks);
}

// find_seq over lane-held offsets: the last n < num_seqs with offsets[n] <= cg.
__device__ __forceinline__ int find_seq_lanes(int lane_off, int lane, int num_seqs, int cg) {
    const unsigned long long m = __ballot(lane < num_seqs && lane_off <= cg);
    return m ? 63 - __clzll(static_cast<long long>(m)) : 0;
}

__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                         int64_t total_tokens, int max_chunks,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ order) {
    __shared__ int wsum[16];
    __shared__ __align__(16) int slen[SORT_MAX];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (num_seqs <= SORT_MAX) {
        const int i = tid;
        const int mine = i < num_seqs ? seq_chunks(cu, i, total_tokens) : 0;
        if (i < num_seqs) slen[i] = mine;
        __syncthreads();
        if (i < num_seqs) {
            int rank = 0;
            for (int m = 0; m < num_seqs; ++m) {
                const int other = slen[m];
                rank += (other > mine) | ((other == mine) & (m < i));
            }
            order[rank] = i;
        }
    } else {
        for (int i = tid; i < num_seqs; i += 1024) order[i] = i;
    }
    int carry = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int i = base + tid;
        const int nch = i < num_seqs ? seq_chunks(cu, i, total_tokens) : 0;
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
// With GATED, g and beta are the raw gate and raw beta (bf16), activated as
// each item is consumed; rows past a sequence's end get g = beta = 0.
// With CONV, q and k are column blocks of the fused projection (qk_row
// elements per token) before the short convolution, which is applied here:
// at the top of an item every thread puts its raw k and q row into LDS
// (region 1, free until the planes), beside the four rows before the chunk
// (from the previous chunk, or the request's conv state for a sequence's
// first chunk) and the head's taps, which waves 0-3 fetched with the item's
// other inputs; after the first barrier each row is convolved from rows
// r - 3 .. r.
template <bool GATED, bool GPH, bool CONV, bool LMAP>
__global__ __launch_bounds__(PNT) void prep_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const void* __restrict__ g_in,
    const void* __restrict__ beta_in, GateParams gp, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ offsets, unsigned char* __restrict__ records, int num_seqs, int num_heads,
    float scale, int l2norm, int qk_row, ConvParams cv, int64_t total_tokens, int max_chunks) {
    const ChunkMap cm{offsets, nullptr, total_tokens, max_chunks};
    const float* __restrict__ g = static_cast<const float*>(g_in);
    const float* __restrict__ beta = static_cast<const float*>(beta_in);
    const bf16_t* __restrict__ graw = static_cast<const bf16_t*>(g_in);
    const bf16_t* __restrict__ braw = static_cast<const bf16_t*>(beta_in);
    __shared__ __align__(16) unsigned char smem[P_LDS];
    float* sWT = reinterpret_cast<float*>(smem + P_WT);
    float* srk = reinterpret_cast<float*>(smem + P_RK);
    float* srq = reinterpret_cast<float*>(smem + P_RQ);
    float* sbeta = reinterpret_cast<float*>(smem + P_BETA);
    float* sEm = reinterpret_cast<float*>(smem + P_EM);
    float* sEL = reinterpret_cast<float*>(smem + P_EL);
    float* sGL = reinterpret_cast<float*>(smem + P_GL);
    float* sG31 = reinterpret_cast<float*>(smem + P_G31);
    float* sGLL = reinterpret_cast<float*>(smem + P_GLL);
    int* sFlag = reinterpret_cast<int*>(smem + P_FLAG);

    KDA_PHASE_BEGIN
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    // LMAP: the chunk offsets in the wave's lanes (cm.offsets is null)
    const int lane_off = LMAP ? lane_offsets(cu_seqlens, num_seqs, cm, static_cast<int>(threadIdx.x) & 63) : 0;
    // offsets[n] of sequence n (n uniform), from the map or from the lanes
    auto offset_of = [&](int n) {
        if constexpr (LMAP)
            return __builtin_amdgcn_readlane(lane_off, n);
        else
            return offsets[n];
    };
    const int n_chunks = offset_of(num_seqs);
    const int items = n_chunks * num_heads;

    // Prefetch registers: row tid/16, channels 8(tid%16) .. +7 of k, q, g; beta.
    // Gated: the raw gate row in pgr.  One decay per head (GPH): the row's one
    // value in pgs (raw bf16 bits in pgs_raw when gated).  pL: the item's valid
    // length.  Buffer loads over the chunk's valid rows: rows past its end read
    // as zero with no branch, and nothing here waits for a load in flight (the
    // gated values are activated, and masked, where they are consumed).
    uint4 pk, pq, pgr = {0u, 0u, 0u, 0u};
    uint4 pcv = {0u, 0u, 0u, 0u};  // CONV: waves 0, 1: k, q rows -4 .. -1; waves 2, 3: k, q taps
    floatx4 pg0 = {0.f, 0.f, 0.f, 0.f}, pg1 = {0.f, 0.f, 0.f, 0.f};
    float pb = 0.f, pgs = 0.f;
    uint32_t pgs_raw = 0, pb_raw = 0;
    int pL = 0;
    const int row_bytes = num_heads * D * 2;  // one token's g row of all heads, bf16 (twice that in fp32)
    const int qk_bytes = qk_row * 2;          // one token's q or k row
    auto fetch = [&](int item, int tid) {
        const int cg = item / num_heads, h = item - (item / num_heads) * num_heads;
        const int n = LMAP ? find_seq_lanes(lane_off, static_cast<int>(threadIdx.x) & 63, num_seqs, cg)
                           : find_seq(offsets, num_seqs, cg);
        const int first_chunk = offset_of(n);
        const int64_t start = cu_seqlens[n] + static_cast<int64_t>(C) * (cg - first_chunk);
        const int L = max(static_cast<int>(min64(C, cu_seqlens[n + 1] - start)), 0);
        const int r = tid >> 4, cc = tid & 15;
        const size_t head0 = static_cast<size_t>(start) * num_heads + h;  // (first row, head)
        const int voff = r * row_bytes + 16 * cc;
        const size_t qk0 = static_cast<size_t>(start) * qk_row + h * D;
        const int qoff = r * qk_bytes + 16 * cc;
        pk = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(k + qk0, L * qk_bytes), qoff, 0, 0));
        pq = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(q + qk0, L * qk_bytes), qoff, 0, 0));
        if constexpr (CONV) {
            // lane (l4, cc) of waves 0 and 1: the row -4 + l4 before the chunk
            // of k and of q: from the previous chunk, or for a sequence's first
            // chunk the conv state's row K - 5 + l4 (entries past its range, or
            // with no state, read as zero); of waves 2 and 3: tap l4 of the
            // head's k and q channels 8 cc .. 8 cc + 7 (taps padded at the front
            // to four); the other waves read nothing (an empty range)
            const int l4 = r & 3;
            const bool first = cg == first_chunk;
            const int srow_bytes = cv.channels * 2;
            const bool is_k = (wave & 1) == 0;
            const int blk = is_k ? num_heads * D : 0;  // channel block of k or q
            const int s_idx = cv.K - 5 + l4;
            const int s_range = cv.state ? (cv.K - 1) * srow_bytes : 0;
            const int tap = l4 - (4 - cv.K);
            const int w_range = (cv.K - 1) * srow_bytes + D * 2;
            const bf16_t* xs = is_k ? k : q;
            const bf16_t* base;
            int range, off;
            if (wave < 2) {
                base = first ? (cv.state ? cv.state + static_cast<size_t>(n) * (cv.K - 1) * cv.channels + blk + h * D : xs)
                             : xs + qk0 - 4 * static_cast<size_t>(qk_row);
                range = first ? s_range : 4 * qk_bytes;
                off = first ? (s_idx >= 0 ? s_idx * srow_bytes + 16 * cc : s_range) : l4 * qk_bytes + 16 * cc;
            } else {
                base = wave < 4 ? cv.weight + blk + h * D : xs;
                range = wave < 4 ? w_range : 0;
                off = wave < 4 && tap >= 0 ? tap * srow_bytes + 16 * cc : range;
            }
            pcv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(base, range), off, 0, 0));
        }
        if constexpr (GATED) {
            if constexpr (GPH)
                pgs_raw = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(graw + head0, L * num_heads * 2), r * num_heads * 2, 0, 0);
            else
                pgr = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(graw + head0 * D, L * row_bytes), voff, 0, 0));
        } else {
            if constexpr (GPH) {
                pgs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(g + head0, L * num_heads * 4), r * num_heads * 4, 0, 0));
            } else {
                const auto gr_ = buffer_rsrc(g + head0 * D, 2 * L * row_bytes);
                pg0 = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(gr_, 2 * voff, 0, 0));
                pg1 = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(gr_, 2 * voff + 16, 0, 0));
            }
        }
        if (tid < C) {
            if constexpr (GATED)
                pb_raw = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(braw + head0, L * num_heads * 2), tid * num_heads * 2, 0, 0);
            else
                pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(beta + head0, L * num_heads * 4), tid * num_heads * 4, 0, 0));
        }
        pL = L;
    };
    // Items run from the last chunk to the first: the records the state scan
    // reads first are the ones written last, still in the last-level cache.
    if (static_cast<int>(blockIdx.x) < items) fetch(items - 1 - static_cast<int>(blockIdx.x), threadIdx.x);

    // -Psi', X', P' fragments of an item out of LDS (K indices in accumulator
    // order).  Called at the top of the next item, once its prefetched inputs
    // are in registers: the stores are then issued after that prefetch, and
    // waiting for the prefetch never waits for them (loads and stores retire
    // in issue order).  The last item's fragments go out after the loop.
    auto frags_out = [&](unsigned char* rec, int tid) {
        for (int f = tid; f < 28 * 64; f += PNT) {
            const int fr = f >> 6, ln = f & 63;
            const int li = ln & 15, ka = 4 * (ln >> 4);
            if (fr < 16) {  // -Psi' [R][s], fp16: -Psi'[16R + li][32s + k] = -Psi'^T[32s + k][16R + li]
                const int R = fr >> 2, s = fr & 3, r0 = 32 * s + ka;
                const floatx8 x = bf8_to_f(col8_tr2(smem, P_PTH, SN, r0, r0 + 16, 16 * R, li)) +
                                  bf8_to_f(col8_tr2(smem, P_PTL, SN, r0, r0 + 16, 16 * R, li));
                store_frag<!CONV>(rec + REC_NPSI + fr * FRAG + ln * 16, -x);
            } else if (fr < 22) {  // X' diag(rk beta) [tri], fp16: X'^T[32s + k][16R + li]
                const int b = fr - 16;
                const int R = tri_R(b), r0 = 32 * tri_s(b) + ka;
                const floatx8 x = bf8_to_f(col8_tr2(smem, P_XTH, SN, r0, r0 + 16, 16 * R, li)) +
                                  bf8_to_f(col8_tr2(smem, P_XTL, SN, r0, r0 + 16, 16 * R, li));
                store_frag<!CONV>(rec + REC_X + b * FRAG + ln * 16, x);
            } else {  // P' [tri], fp16, from the row-major hi/lo planes
                const int b = fr - 22, R = tri_R(b);
                const int o = ((16 * R + li) * SN + 32 * tri_s(b) + ka) * 2;
                const bf16x4 h0 = ld4(smem, P_PH + o), h1 = ld4(smem, P_PH + o + 32);
                const bf16x4 q0 = ld4(smem, P_PL + o), q1 = ld4(smem, P_PL + o + 32);
                floatx8 x;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = static_cast<float>(h0[i]) + static_cast<float>(q0[i]);
                    x[4 + i] = static_cast<float>(h1[i]) + static_cast<float>(q1[i]);
                }
                store_frag<!CONV>(rec + REC_P + b * FRAG + ln * 16, x);
            }
        }
    };
    unsigned char* prev_rec = nullptr;  // the item whose fragments are still in LDS
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int item = items - 1 - it;
        const int lane = opaque(static_cast<int>(threadIdx.x) & 63);
        const int tid = wave * 64 + lane;
        const int l16 = lane & 15, l4 = lane >> 4;
        const int rp = tid >> 4, cc = tid & 15;  // phase 1: row rp, channels 8cc .. 8cc+7
        const int cg = item / num_heads, h = item - cg * num_heads;
        unsigned char* rec = records + (static_cast<size_t>(cg) * num_heads + h) * REC_BYTES;

        // ======== phase 1: norms, cumulative log-decay, operand planes ========
        // rows past the chunk's end were loaded as zeros; only activated gates need a mask
        if (tid == 0) *sFlag = 0;  // last read after the previous item's second barrier
        floatx8 kf, qf;
        if constexpr (CONV) {
            // raw rows into region 1 (convolved after the first barrier)
            *reinterpret_cast<uint4*>(smem + P_CVK + (4 + rp) * D * 2 + 16 * cc) = pk;
            *reinterpret_cast<uint4*>(smem + P_CVQ + (4 + rp) * D * 2 + 16 * cc) = pq;
            if (wave < 2)
                *reinterpret_cast<uint4*>(smem + (wave == 0 ? P_CVK : P_CVQ) + l4 * D * 2 + 16 * cc) = pcv;
            else if (wave < 4)
                *reinterpret_cast<uint4*>(smem + P_CW + (wave - 2) * 4 * D * 2 + l4 * D * 2 + 16 * cc) = pcv;
        } else {
            kf = unpack8(pk);
            qf = unpack8(pq);
        }
        // inclusive prefix of g over the wave's four rows (16-lane groups), then
        // the totals of the 16 waves through LDS
        floatx8 gr;
        if constexpr (GATED) {
            const bool live = rp < pL;
            const float a = gate_exp(gp.a_log[h]);
            if constexpr (GPH) {
                const float x0 = __uint_as_float(pgs_raw << 16);
                const float gv = live ? gate_g(x0, gp.dt_bias[h], a, gp.lower_bound, gp.has_lower_bound) : 0.f;
                gr = floatx8{gv, gv, gv, gv, gv, gv, gv, gv};
            } else {
                const floatx8 x = unpack8(pgr);
                const floatx4 b0 = *reinterpret_cast<const floatx4*>(gp.dt_bias + h * D + 8 * cc);
                const floatx4 b1 = *reinterpret_cast<const floatx4*>(gp.dt_bias + h * D + 8 * cc + 4);
                const float bias[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    gr[i] = live ? gate_g(x[i], bias[i], a, gp.lower_bound, gp.has_lower_bound) : 0.f;
            }
        } else {
            if constexpr (GPH)
                gr = floatx8{pgs, pgs, pgs, pgs, pgs, pgs, pgs, pgs};
            else
                gr = floatx8{pg0[0], pg0[1], pg0[2], pg0[3], pg1[0], pg1[1], pg1[2], pg1[3]};
        }
        floatx8 incl = gr;
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
        // the previous item's fragments; the barrier below also ends their LDS reads
        // (the wave totals live in the X_RR planes, which they do not read)
        if (prev_rec) frags_out(prev_rec, tid);
        lds_barrier();
        if constexpr (CONV) {
            // row rp from the raw rows rp - 3 .. rp and the head's taps
            auto conv_rows = [&](int base, int taps, const uint4& own) {
                uint4 w[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = *reinterpret_cast<const uint4*>(smem + taps + t * D * 2 + 16 * cc);
                const unsigned char* row = smem + base + (4 + rp) * D * 2 + 16 * cc;
                const uint4 x1 = *reinterpret_cast<const uint4*>(row - D * 2);
                const uint4 x2 = *reinterpret_cast<const uint4*>(row - 2 * D * 2);
                const uint4 x3 = *reinterpret_cast<const uint4*>(row - 3 * D * 2);
                return conv8(own, x1, x2, x3, conv_taps8(w), cv.silu, rp < pL);
            };
            kf = conv_rows(P_CVK, P_CW, pk);
            qf = conv_rows(P_CVQ, P_CW + 4 * D * 2, pq);
        }
        // Channel threads turn the wave totals of channel c into offsets in
        // place: with P_w the sum of the totals of waves 0 .. w-1, entry (w, c)
        // becomes P_w - P_8, the cumulative g before wave w's first row minus
        // G_31 (token 31 is the last row of wave 7); and e^{G_31}, e^{G_last -
        // G_31}, e^{G_last}.  Meanwhile every thread forms its row norms.
        if (tid < D) {
            float t[16];
#pragma unroll
            for (int w2 = 0; w2 < 16; ++w2) t[w2] = sWT[w2 * D + tid];
            float pre[17];
            pre[0] = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 16; ++w2) pre[w2 + 1] = pre[w2] + t[w2];
#pragma unroll
            for (int w2 = 0; w2 < 16; ++w2) sWT[w2 * D + tid] = pre[w2] - pre[8];
            sEm[tid] = fast_exp2(pre[8] * kLog2e);
            sEL[tid] = fast_exp2((pre[16] - pre[8]) * kLog2e);
            sGL[tid] = fast_exp2(pre[16] * kLog2e);
            sG31[tid] = pre[8];
            sGLL[tid] = pre[16];
            // With g <= 0, G_r - G_31 lies in [pre[16] - pre[8], -pre[8]]; past
            // kRefSpan the chunk takes the exact path (a NaN sum does too).
            if (!(-pre[8] <= kRefSpan && pre[8] - pre[16] <= kRefSpan)) *sFlag = 1;
        }
        {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sk += kf[i] * kf[i];
                sq += qf[i] * qf[i];
            }
            sk = row16_sum(sk);
            sq = row16_sum(sq);
            if (cc == 0) {
                srk[rp] = l2norm ? rsqrtf(sk + kNormEps) : 1.f;
                srq[rp] = (l2norm ? rsqrtf(sq + kNormEps) : 1.f) * scale;
            }
        }
        if (tid < C) {
            float bv;
            if constexpr (GATED)
                bv = gate_sigmoid(__uint_as_float(pb_raw << 16));
            else
                bv = pb;
            sbeta[tid] = tid < pL ? bv : 0.f;
        }
        lds_barrier();
        // Operand planes: Kg = k e^{d}, Qg = q e^{d}, Ki = k e^{dt} (bf16 hi/lo).
        auto planes = [&](const floatx8& d, const floatx8& dt) {
            const int o = (rp * SW + 8 * cc) * 2;
            floatx8 e, ei;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = fast_exp2(d[i]);
                ei[i] = fast_exp2(dt[i]);
            }
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
        };
        // G_r - G_31 for this row
        auto offsets8 = [&](const float* base) {
            const floatx4 a = *reinterpret_cast<const floatx4*>(base);
            const floatx4 b = *reinterpret_cast<const floatx4*>(base + 4);
            return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        };
        // Decay too strong for the reference token somewhere in the chunk:
        // A' and P' come from exact_ap, and the planes take the chunk's start
        // (Kg, Qg) and end (Ki) as references, every factor at most 1, with
        // e^{G_31} and e^{G_last - G_31} replaced by 1 downstream.
        // a plain LDS read (the barrier's memory clobber makes it a fresh one; a
        // volatile generic pointer would compile to a flat load, which the
        // compiler waits for together with every vector memory operation in flight)
        const bool exact = __builtin_amdgcn_readfirstlane(*sFlag) != 0;
        if (exact) {
            const int o = rp * D + 8 * cc;
            floatx8 eg;
#pragma unroll
            for (int i = 0; i < 8; ++i) eg[i] = fast_exp2(gr[i] * kLog2e);
            // G_r (from the chunk's start)
            const floatx8 dl = offsets8(sWT + wave * D + 8 * cc) + incl + offsets8(sG31 + 8 * cc);
            float* ge = reinterpret_cast<float*>(smem + P_GE);
            float* gg = reinterpret_cast<float*>(smem + P_GG);
            auto pack8 = [](const floatx8& x) {  // exact: the values are bf16 already
                return uint4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                             pack_bf16x2(x[6], x[7])};
            };
            *reinterpret_cast<uint4*>(smem + P_GK + o * 2) = pack8(kf);
            *reinterpret_cast<uint4*>(smem + P_GQ + o * 2) = pack8(qf);
            *reinterpret_cast<floatx4*>(ge + o) = floatx4{eg[0], eg[1], eg[2], eg[3]};
            *reinterpret_cast<floatx4*>(ge + o + 4) = floatx4{eg[4], eg[5], eg[6], eg[7]};
            *reinterpret_cast<floatx4*>(gg + o) = floatx4{dl[0], dl[1], dl[2], dl[3]};
            *reinterpret_cast<floatx4*>(gg + o + 4) = floatx4{dl[4], dl[5], dl[6], dl[7]};
            // P' planes (hi and lo, adjacent) cleared: exact_ap writes i <= r only
            static_assert(P_PL == P_PH + PN && 2 * PN % 16 == 0, "P' planes adjacent");
            for (int u = tid; u < 2 * PN / 16; u += PNT)
                *reinterpret_cast<uint4*>(smem + P_PH + 16 * u) = uint4{0u, 0u, 0u, 0u};
            if (tid < D) {
                sEm[tid] = 1.f;
                sEL[tid] = 1.f;
            }
            lds_barrier();
            exact_ap(smem, wave, l16, l4);
            // k, q and G of this row back from LDS (nothing is kept live across
            // exact_ap), before the barrier after which the planes overwrite them
            kf = bf8_to_f(ld8(smem, P_GK + o * 2));
            qf = bf8_to_f(ld8(smem, P_GQ + o * 2));
            const floatx8 dg = offsets8(gg + o);
            lds_barrier();
            // d = G_r (from the chunk's start), dt = G_last - G_r
            planes(dg * kLog2e, (offsets8(sGLL + 8 * cc) - dg) * kLog2e);
        } else {
            const floatx8 d = (offsets8(sWT + wave * D + 8 * cc) + incl) * kLog2e;
            planes(d, -d);
        }
        // the next item's loads fly from here on
        if (it + static_cast<int>(gridDim.x) < items) fetch(items - 1 - (it + static_cast<int>(gridDim.x)), tid);
        lds_barrier();
        KDA_PHASE_MARK(0);

        // ======== phase 2: A' and P' blocks (K = 128 channels), one per wave 1-10 ========
        const bool has_unit = wave >= 1 && wave <= 10;
        const int uR = has_unit ? static_cast<int>((kPrepUnitR >> (2 * wave)) & 3) : -1;
        const int uI = has_unit ? static_cast<int>((kPrepUnitI >> (2 * wave)) & 3) : -1;
        floatx4 pacc = {0.f, 0.f, 0.f, 0.f};
        if (uR >= 0 && !exact) {
            const int ar = (16 * uR + l16) * SW, br = (16 * uI + l16) * SW;
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ko = 32 * s + 8 * l4;
                const bf16x8 bh = ld8(smem, P_KIH + (br + ko) * 2);
                const bf16x8 bl = ld8(smem, P_KIL + (br + ko) * 2);
                accA = mma(ld8(smem, P_KGH + (ar + ko) * 2), bh, accA);
                accP = mma3(ld8(smem, P_QGH + (ar + ko) * 2), ld8(smem, P_QGL + (ar + ko) * 2), bh, bl, accP);
            }
            floatx4 a;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * uR + 4 * l4 + j;
                const float rk = srk[r];
                a[j] = sbeta[r] * rk * rk * accA[j];
                pacc[j] = srq[r] * accP[j];
            }
            if (uI < uR) {
                bf16x4 hi, lo;
                split4(a, hi, lo);
                const int o = ((pair_index(uR, uI) * 16 + l16) * WSTR + 4 * l4) * 2;
                *reinterpret_cast<bf16x4*>(smem + P_ATH + o) = hi;
                *reinterpret_cast<bf16x4*>(smem + P_ATL + o) = lo;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int lr = 4 * l4 + j;
                    a[j] = l16 < lr ? a[j] : (l16 == lr ? 1.f : 0.f);
                    pacc[j] = l16 <= lr ? pacc[j] : 0.f;
                }
                *reinterpret_cast<floatx4*>(smem + P_LDT + ((uR * 16 + l16) * LDS_STR + 4 * l4) * 4) = a;
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(1);

        // ======== phase 3: diagonal inverses (wave 0); P' (waves 1-10), Ke^T, Qg', vectors ========
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
            // column l16 of block l4 is row l16 of the transposed block: 16
            // consecutive bf16 per plane, hi = RNE(x) and lo = RNE(x - hi)
            uint32_t xh[8], xl[8], fh[8], fl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a = x[2 * i], b = x[2 * i + 1];
                const uint32_t h = pack_bf16x2(a, b);
                xh[i] = h;
                xl[i] = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
                const float fa = a * sphi, fb = b * sphi;
                const uint32_t hf = pack_bf16x2(fa, fb);
                fh[i] = hf;
                fl[i] = pack_bf16x2(fa - __uint_as_float(hf << 16), fb - __uint_as_float(hf & 0xffff0000u));
            }
            const int o = (l4 * 16 + l16) * WSTR * 2;
            *reinterpret_cast<uint4*>(smem + P_XDH + o) = uint4{xh[0], xh[1], xh[2], xh[3]};
            *reinterpret_cast<uint4*>(smem + P_XDH + o + 16) = uint4{xh[4], xh[5], xh[6], xh[7]};
            *reinterpret_cast<uint4*>(smem + P_XDL + o) = uint4{xl[0], xl[1], xl[2], xl[3]};
            *reinterpret_cast<uint4*>(smem + P_XDL + o + 16) = uint4{xl[4], xl[5], xl[6], xl[7]};
            *reinterpret_cast<uint4*>(smem + P_XFH + o) = uint4{fh[0], fh[1], fh[2], fh[3]};
            *reinterpret_cast<uint4*>(smem + P_XFH + o + 16) = uint4{fh[4], fh[5], fh[6], fh[7]};
            *reinterpret_cast<uint4*>(smem + P_XFL + o) = uint4{fl[0], fl[1], fl[2], fl[3]};
            *reinterpret_cast<uint4*>(smem + P_XFL + o + 16) = uint4{fl[4], fl[5], fl[6], fl[7]};
        } else {
            if (uR >= 0) {
                // P' from this wave's accumulator of phase 2 (exact path: in place already)
                if (!exact) {
                    bf16x4 hi, lo;
                    split4(pacc, hi, lo);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int o = ((16 * uR + 4 * l4 + j) * SN + 16 * uI + l16) * 2;
                        *reinterpret_cast<__bf16*>(smem + P_PH + o) = hi[j];
                        *reinterpret_cast<__bf16*>(smem + P_PL + o) = lo[j];
                    }
                }
            } else if (wave == 15) {
                // blocks (0,1) and (2,3) lie in the K range of 32-wide steps and read as zero
                const int blk = lane >> 5, row = (lane >> 1) & 15, part = lane & 1;
                const int r = (blk ? 32 : 0) + row, c0 = (blk ? 48 : 16) + 8 * part;
                const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
                *reinterpret_cast<bf16x8*>(smem + P_PH + (r * SN + c0) * 2) = z;
                *reinterpret_cast<bf16x8*>(smem + P_PL + (r * SN + c0) * 2) = z;
            }
            const int t1 = tid - 64;  // 0..959: 32 fragments over waves 1-15
            for (int f = t1; f < 32 * 64; f += PNT - 64) {
                const int fr = f >> 6, ln = f & 63;
                const int li = ln & 15, ka = 4 * (ln >> 4);  // K indices ka .. ka+3, ka+16 .. ka+19
                if (fr < 16) {
                    // Ke^T [w][s]: Ki[32s + k][16w + li] e^{G_last - G_31}[16w + li]
                    //   = k e^{G_last - G} (the decay to the chunk's end) at tokens 32s + k
                    const int w = fr >> 1, s = fr & 1;
                    const int r0 = 32 * s + ka;
                    floatx8 x = bf8_to_f(col8_tr2(smem, P_KIH, SW, r0, r0 + 16, 16 * w, li)) +
                                bf8_to_f(col8_tr2(smem, P_KIL, SW, r0, r0 + 16, 16 * w, li));
                    x *= sEL[16 * w + li];
                    store_frag<!CONV>(rec + REC_KE + fr * FRAG + ln * 16, x);
                } else {
                    // Qg' [R][s]: rq_r Qg[r][c] e^{G_31}[c] at channels c = 32s + k
                    const int f2 = fr - 16, R = f2 >> 2, s = f2 & 3;
                    const int r = 16 * R + li, c0 = 32 * s + ka;
                    const int o = (r * SW + c0) * 2;
                    const bf16x4 h0 = ld4(smem, P_QGH + o), h1 = ld4(smem, P_QGH + o + 32);
                    const bf16x4 q0 = ld4(smem, P_QGL + o), q1 = ld4(smem, P_QGL + o + 32);
                    const floatx4 e0 = *reinterpret_cast<const floatx4*>(sEm + c0);
                    const floatx4 e1 = *reinterpret_cast<const floatx4*>(sEm + c0 + 16);
                    const float rq = srq[r];
                    floatx8 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = (static_cast<float>(h0[i]) + static_cast<float>(q0[i])) * (rq * e0[i]);
                        x[4 + i] = (static_cast<float>(h1[i]) + static_cast<float>(q1[i])) * (rq * e1[i]);
                    }
                    store_frag<!CONV>(rec + REC_QG + f2 * FRAG + ln * 16, x);
                }
            }
            float* vec = reinterpret_cast<float*>(rec + REC_VEC);
            if (t1 < D) vec[t1] = sGL[t1];
        }
        lds_barrier();
        KDA_PHASE_MARK(2);

        // ======== phase 4: W_RJ = -X_RR A'_RJ (six blocks, K = 16) ========
        if (wave < 6) {
            const int R = wave < 1 ? 1 : wave < 3 ? 2 : 3;
            const bool ok = l4 < 2;
            // X_RR[l16][8 l4 .. +7] = column l16 of the transposed block (K past 16 reads as zero)
            const int xr = ok ? 8 * l4 : 0;
            const bf16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
            const bf16x8 xh8 = col8_tr(smem, P_XDH + R * BLK, WSTR, xr, 0, l16);
            const bf16x8 xl8 = col8_tr(smem, P_XDL + R * BLK, WSTR, xr, 0, l16);
            const int bo = ((wave * 16 + l16) * WSTR + 8 * l4) * 2;
            floatx4 w = {0.f, 0.f, 0.f, 0.f};
            w = mma3(ok ? xh8 : z8, ok ? xl8 : z8, ld8_if(smem, P_ATH + bo, ok), ld8_if(smem, P_ATL + bo, ok), w);
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
        // Waves 0-7: column tile t = wave of Psi'; waves 8-11: column tile
        // t = wave - 8 of X'.  Step R: out_R = rhs_R + sum_{J<R} W_RJ out_J,
        // with out kept transposed in LDS (each wave reads only its own rows).
        // Every term has K = 16, so two of them share one 32-wide product:
        // lanes of groups 0-1 supply block J and groups 2-3 block J+1 (W_RJ and
        // W_R,J+1 are adjacent, and so are the rows of out_J and out_J+1).
        // A lone term masks the upper half of K.
        if (wave < 12) {
            const bool ok = l4 < 2;
            const int xr = ok ? 8 * l4 : 0;
            const bf16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
            const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
            const bool psi = wave < 8;
            const int t = psi ? wave : wave - 8;
            // out^T planes and the first step this wave solves
            const int oh = psi ? P_PTH : P_XTH, ol = psi ? P_PTL : P_XTL;
            const int orow = 16 * t + l16;  // the wave's own row of out^T
            const int j0 = psi ? 0 : t;
            floatx4 rhs[4];
            if (psi) {
                // rhs_R = (X_RR diag(rk^2 beta)) Kg_R[:, tile] e^{G_31}[col], independent of the substitution
                const float em = sEm[16 * t + l16];
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    // rows past 16R + 15 (lanes with l4 >= 2) read other LDS data and are zeroed
                    const bf16x8 xfh8 = col8_tr(smem, P_XFH + R * BLK, WSTR, xr, 0, l16);
                    const bf16x8 xfl8 = col8_tr(smem, P_XFL + R * BLK, WSTR, xr, 0, l16);
                    const bf16x8 kgh8 = col8_tr(smem, P_KGH, SW, 16 * R + 8 * l4, 16 * t, l16);
                    const bf16x8 kgl8 = col8_tr(smem, P_KGL, SW, 16 * R + 8 * l4, 16 * t, l16);
                    rhs[R] = mma3(ok ? xfh8 : z8, ok ? xfl8 : z8, ok ? kgh8 : z8, ok ? kgl8 : z8, zero4) * em;
                }
            } else {
                // X'_tt = X_tt, columns scaled by rk beta (the scan multiplies this X' by V directly):
                // X_tt[4 l4 + j][l16] is row l16 of the transposed block
                const float cs = srk[16 * t + l16] * sbeta[16 * t + l16];
                const int o = ((t * 16 + l16) * WSTR + 4 * l4) * 2;
                const bf16x4 xh4 = ld4(smem, P_XDH + o), xl4 = ld4(smem, P_XDL + o);
#pragma unroll
                for (int R = 0; R < 4; ++R) rhs[R] = zero4;
                floatx4 d;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) d[jj] = (static_cast<float>(xh4[jj]) + static_cast<float>(xl4[jj])) * cs;
#pragma unroll
                for (int R = 0; R < 4; ++R)
                    if (R == t) rhs[R] = d;
            }
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                // X' waves: blocks R < t of the tile are the upper triangle and are stored as zeros
                floatx4 acc = rhs[R];
                int J = j0;
                for (; J + 1 < R; J += 2) {
                    const int wo = ((pair_index(R, J + (l4 >> 1)) * 16 + l16) * WSTR + 8 * (l4 & 1)) * 2;
                    const int po = (orow * SN + 16 * J + 8 * l4) * 2;
                    acc = mma3(ld8(smem, P_WH + wo), ld8(smem, P_WL + wo), ld8(smem, oh + po), ld8(smem, ol + po), acc);
                }
                if (J < R) {
                    const int wo = ((pair_index(R, J) * 16 + l16) * WSTR + 8 * l4) * 2;
                    const int po = (orow * SN + 16 * J + 8 * l4) * 2;
                    acc = mma3(ld8_if(smem, P_WH + wo, ok), ld8_if(smem, P_WL + wo, ok), ld8_if(smem, oh + po, ok),
                               ld8_if(smem, ol + po, ok), acc);
                }
                bf16x4 hi, lo;
                split4(acc, hi, lo);
                const int oo = (orow * SN + 16 * R + 4 * l4) * 2;
                *reinterpret_cast<bf16x4*>(smem + oh + oo) = hi;
                *reinterpret_cast<bf16x4*>(smem + ol + oo) = lo;
                asm volatile("" ::: "memory");
            }
        }
        lds_barrier();
        KDA_PHASE_MARK(4);
        prev_rec = rec;
    }
    if (prev_rec) frags_out(prev_rec, static_cast<int>(threadIdx.x));
    KDA_PHASE_END;
}

// --------------------------------------------------------------------------
// ---- scan_kernel: NT + 3 waves per (sequence, head, NT 16-column value tiles) ----
// Waves 0 .. NT-1 (the state waves) each carry the chunk recurrence of one
// tile alone: D from S, then S'.  Wave NT+2 copies their operands (-Psi',
// Ke^T), which do not depend on the value columns and so serve every tile,
// into LDS three chunks ahead; wave NT forms Delta0 = X' diag(rk beta) V of
// the tiles two chunks ahead; wave NT+1 (the output wave) forms O = Qg' S +
// P' D of the tiles one chunk behind, from S and D handed over through LDS
// already in B-operand form.  One barrier per chunk.  The copy wave never
// reads its own copies, so nothing makes it wait for them before the barrier
// two chunks later.  With NT = 2 a workgroup reads each record once for two
// tiles: half the L2 traffic per tile, for when there are more tiles than
// compute units; with NT = 1 a chain's chunk takes the least time.
constexpr int SB_NP = 0;                       // -Psi' [m 4][s 4]
constexpr int SB_KE = 16 * FRAG;               // Ke^T [w 8][s 2]
// LDS regions, each its own array: the compiler then sees that the direct
// loads into one region do not write the others, and waits only where needed.
constexpr int SB_BYTES = 32 * FRAG;            // one of three state buffers (chunk mod 3)
constexpr int XV_X = 0, XV_V = 6 * FRAG;       // X' buffers: X' [tri 6] fp16, V rows [64][16 NT] bf16,
                                               // then e^{G_last} [128] fp32 (the copy fills 1 KiB)
constexpr int DG_D = 0;                        // two slots: Delta0 of tile t (accumulator layout) at 4t fragments,
                                               // then e^{G_last} [128] fp32
// The output is not fed back, so it takes S and D as single fp16 (their high
// parts); the state side keeps the hi/lo pairs.
constexpr int XCH_S = 0;                       // exchange, two slots, per tile: S as B operand [s 4], fp16
constexpr int XCH_D = 4 * FRAG;                // D as B operand [s 2]
constexpr int XCH_TILE = 6 * FRAG;

template <int NT>
struct ScanShape {
    // X' buffers: with one tile three, so the Delta0 wave forms Delta0 from a
    // copy requested two chunks earlier; with two tiles two (one chunk earlier).
    static constexpr int XVB = NT == 1 ? 3 : 2;
    static constexpr int XV_GL = XV_V + C * NT * DVT * 2;
    static constexpr int XV_BYTES = XV_GL + FRAG;
    static constexpr int DG_GL = NT * 4 * FRAG;
    static constexpr int DG_SLOT = DG_GL + D * 4;
    static constexpr int XCH_SLOT = NT * XCH_TILE;
    static constexpr int LDS = 3 * SB_BYTES + XVB * XV_BYTES + 2 * DG_SLOT + 2 * XCH_SLOT + 256;
    static constexpr int THREADS = 64 * (NT + 3);
    static constexpr int UNITS = D / (NT * DVT);  // workgroups per chain
    static_assert(LDS <= 160 * 1024, "scan LDS budget");
    static_assert(UNITS * NT * DVT == D && (UNITS == 8 || UNITS == 4), "eight or four workgroups per chain");
};

template <typename TOut, int NT>
__global__ __launch_bounds__(ScanShape<NT>::THREADS) void scan_kernel(
    const bf16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ order, const unsigned char* __restrict__ records, const float* initial_state, TOut* __restrict__ out,
    float* final_state, const int32_t* __restrict__ slots, int num_slots, int num_seqs, int num_heads,
    int state_trans) {
    __shared__ __align__(16) unsigned char lds_sb[3 * SB_BYTES];
    using SS = ScanShape<NT>;
    constexpr int DG_GL = SS::DG_GL, DG_SLOT = SS::DG_SLOT, XCH_SLOT = SS::XCH_SLOT;
    // the X' buffers are separate arrays, so the compiler sees that a copy
    // into one does not write what is being read from the other
    __shared__ __align__(16) unsigned char lds_xv0[SS::XV_BYTES];
    __shared__ __align__(16) unsigned char lds_xv1[SS::XV_BYTES];
    __shared__ __align__(16) unsigned char lds_xv2[SS::XVB == 3 ? SS::XV_BYTES : 16];
    __shared__ __align__(16) unsigned char lds_dg[2 * DG_SLOT];
    __shared__ __align__(16) unsigned char lds_xch[2 * XCH_SLOT];
    __shared__ __align__(16) unsigned char lds_touch[256];  // sink of the L2 touches, never read
    // Workgroup id -> (chain rank, unit of NT tiles): each run of 8 UNITS ids
    // holds the units of 8 consecutive chains, and id mod 8 (the XCD the
    // workgroup lands on) is the chain's, so the units of a chain run
    // together on one XCD and read its records through one L2.
    const int id = static_cast<int>(blockIdx.x);
    const int crank = (id / (8 * SS::UNITS)) * 8 + (id & 7);
    const int unit = (id >> 3) % SS::UNITS;
    if (crank >= num_seqs * num_heads) return;
    KDA_PHASE_BEGIN
    const int n = order[crank / num_heads], h = crank % num_heads;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane0 = static_cast<int>(threadIdx.x) & 63;
    const int colp = unit * NT * DVT;  // first value column of the unit
    const int c_begin = offsets[n], c_end = offsets[n + 1];
    const int nc = c_end - c_begin;
    const int64_t t_first = cu_seqlens[n], t_last = cu_seqlens[n + 1];
    const int row_stride = num_heads * D;
    size_t head_state = 0;
    const bool has_state = state_block(slots, num_slots, n, h, num_heads, D, head_state);
    const float* init = has_state ? initial_state : nullptr;
    float* fin = has_state ? final_state : nullptr;
    auto rec_of = [&](int j) { return records + (static_cast<size_t>(c_begin + j) * num_heads + h) * REC_BYTES; };
    auto tok_of = [&](int j) { return t_first + static_cast<int64_t>(C) * j; };
    auto len_of = [&](int j) { return static_cast<int>(min64(C, t_last - tok_of(j))); };

    if (wave < NT) {
        // ================= state waves (tile t = wave) =================
        // S[w][j] = S[16w + 4(l/16) + j][col0 + l%16]: the accumulator layout of U = Ke^T D.
        const int col0 = colp + DVT * wave;
        const int dg_t = DG_D + 4 * FRAG * wave, xch_t = XCH_TILE * wave;
        floatx4 S[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) S[w] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (init) {
            const int l16 = lane0 & 15, g = lane0 >> 4;
#pragma unroll
            for (int w = 0; w < 8; ++w)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    S[w][j] = init[head_state + state_elem(16 * w + 4 * g + j, col0 + l16, D, state_trans)];
        }
        // Step j from state buffer sb (chunk j mod 3) and slots of parity p.
        // D = Delta0 - Psi' S runs K block by K block (32 rows of S each): the
        // -Psi' fragments of the next block are read, the next block of S is
        // split and handed over, Ke^T is read and the block of S just used is
        // decayed by e^{G_last} while the current block's eight MFMAs run.  U
        // then accumulates in S itself (S' = diag(e^{G_last}) S + Ke^T D),
        // rows 0-31 of D first, so the second half of D is split while the
        // first sixteen products run.
        auto step = [&](int sbuf, int p, int lane) {
            const unsigned char* sb = lds_sb + sbuf * SB_BYTES;
            const unsigned char* dg = lds_dg + p * DG_SLOT;
            unsigned char* xch = lds_xch + p * XCH_SLOT + xch_t;
            const int g = lane >> 4, lo16 = lane * 16;
            floatx4 Dm[4];
            halfx8 fa[4], fb[4], fk[16];
            halfx8 sh, sl, shn, sln;
#pragma unroll
            for (int m = 0; m < 4; ++m) Dm[m] = *reinterpret_cast<const floatx4*>(dg + dg_t + m * FRAG + lo16);
#pragma unroll
            for (int m = 0; m < 4; ++m) fa[m] = ldh8(sb, SB_NP + 4 * m * FRAG + lo16);
            split8h(S[0], S[1], sh, sl);
            *reinterpret_cast<halfx8*>(xch + XCH_S + lo16) = sh;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) {
#pragma unroll
                    for (int m = 0; m < 4; ++m) fb[m] = ldh8(sb, SB_NP + (4 * m + s + 1) * FRAG + lo16);
                    split8h(S[2 * s + 2], S[2 * s + 3], shn, sln);
                    *reinterpret_cast<halfx8*>(xch + XCH_S + (s + 1) * FRAG + lo16) = shn;
                }
#pragma unroll
                for (int q = 4 * s; q < 4 * s + 4; ++q) fk[q] = ldh8(sb, SB_KE + q * FRAG + lo16);
#pragma unroll
                for (int w = 2 * s; w < 2 * s + 2; ++w)
                    S[w] *= *reinterpret_cast<const floatx4*>(dg + DG_GL + (16 * w + 4 * g) * 4);
                if (s < 3) {
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                        for (int m = 0; m < 4; ++m) Dm[m] = mmah(fa[m], hl ? sl : sh, Dm[m]);
                } else {
                    // rows 0-31 of D complete first
#pragma unroll
                    for (int half = 0; half < 2; ++half)
#pragma unroll
                        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                            for (int m = 2 * half; m < 2 * half + 2; ++m) Dm[m] = mmah(fa[m], hl ? sl : sh, Dm[m]);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) fa[m] = fb[m];
                sh = shn;
                sl = sln;
                // A wave hides only about two of its own VALU instructions
                // under each MFMA: spread the split and the decay over the
                // block's eight products, reads first.
                __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            KDA_PHASE_MARK(8);
            // U: D as the B operand, in two halves, each handed over
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                halfx8 dh, dl;
                split8h(Dm[2 * s], Dm[2 * s + 1], dh, dl);
                *reinterpret_cast<halfx8*>(xch + XCH_D + s * FRAG + lo16) = dh;
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                    for (int w = 0; w < 8; ++w) S[w] = mmah(fk[2 * w + s], hl ? dl : dh, S[w]);
            }
            KDA_PHASE_MARK(9);
            lds_barrier();
            KDA_PHASE_MARK(10);
        };

        lds_barrier();  // the first chunks' operands are in place
        int sbuf = 0;
        for (int j = 0; j < nc; j += 2) {
            const int lane = opaque(lane0);
            step(sbuf, 0, lane);
            sbuf = sbuf == 2 ? 0 : sbuf + 1;
            // the pad step after an odd chunk count only keeps the barrier count
            if (j + 1 < nc)
                step(sbuf, 1, lane);
            else
                lds_barrier();
            sbuf = sbuf == 2 ? 0 : sbuf + 1;
        }
        if (fin) {
            const int l16 = lane0 & 15, g = lane0 >> 4;
#pragma unroll
            for (int w = 0; w < 8; ++w)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    fin[head_state + state_elem(16 * w + 4 * g + j, col0 + l16, D, state_trans)] = S[w][j];
        }
    } else if (wave == NT + 2) {
        // ================= state-copy wave =================
        // -Psi' and Ke^T of chunk j into state buffer sbuf (32 copies).
        // The eight 4 KiB groups (four of -Psi', then four of Ke^T) are taken
        // in an order rotated by the unit, so the units of a chain do not ask
        // for the same lines at the same moment.
        const int rot = (NT * unit) & 7;
        auto fetch_state = [&](int sbuf, int j, int lane) {
            lds_u8* dst = (lds_u8*)lds_sb + sbuf * SB_BYTES;
            const unsigned char* rec = rec_of(j) + lane * 16;
            static_assert(SB_NP == 0 && SB_KE == 16 * FRAG && REC_NPSI == 0, "group g at 4g fragments of the buffer");
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int g = (i + rot) & 7;
                const unsigned char* src = rec + (g < 4 ? REC_NPSI + 4 * g * FRAG : REC_KE + 4 * (g - 4) * FRAG);
                lds_u8* d = dst + 4 * g * FRAG;
                copy16_to_lds<0>(src, d);
                copy16_to_lds<1024>(src, d);
                copy16_to_lds<2048>(src, d);
                copy16_to_lds<3072>(src, d);
            }
        };
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < nc) fetch_state(j, j, lane0);
        wait_vmcnt<0>();
        lds_barrier();
        // Step j (while the state wave runs chunk j+1): chunk j+3 into buffer
        // j mod 3, last read by the state wave in step j.  Before each barrier
        // only the copies of the step just ended may still be in flight, so a
        // chunk's copies land by the barrier two steps after they are issued.
        // The first unit of a chain also touches every 128-byte line of the
        // record four chunks ahead (one 4-byte load per line, into a scratch
        // LDS row), so the record is in L2 when the waves of all its units
        // read it and none of them waits on HBM latency.  Lanes past the
        // record's end fall outside the buffer range and access nothing.
        constexpr int TOUCHES = (REC_BYTES + 64 * 128 - 1) / (64 * 128);
        const bool toucher = unit == 0;
        auto touch = [&](int j, int lane) {
            const auto r = buffer_rsrc(rec_of(j), REC_BYTES);
#pragma unroll
            for (int i = 0; i < TOUCHES; ++i) copy4_to_lds_buf(r, (64 * i + lane) * 128, (lds_u8*)lds_touch);
        };
        auto step = [&](int sbuf, int lane, int j) {
            if (j + 3 < nc) {
                // Its copies are needed two chunks later: let the Delta0 and
                // output waves, whose loads are needed sooner, reach the CU's
                // memory queue first (a wave blocked on a full queue stalls
                // its MFMAs too).  512 cycles measured best of 0 / 512 / 1024.
                __builtin_amdgcn_s_sleep(8);
                fetch_state(sbuf, j + 3, lane);
                if (toucher && j + 4 < nc) {
                    touch(j + 4, lane);
                    wait_vmcnt<32 + TOUCHES>();
                } else {
                    wait_vmcnt<32>();
                }
            } else {
                wait_vmcnt<0>();
            }
        };
        int sbuf = 0;
        for (int j = 0; j < nc; j += 2) {
            const int lane = opaque(lane0);
            lds_barrier();
            step(sbuf, lane, j);
            sbuf = sbuf == 2 ? 0 : sbuf + 1;
            lds_barrier();
            step(sbuf, lane, j + 1);
            sbuf = sbuf == 2 ? 0 : sbuf + 1;
        }
        wait_vmcnt<0>();
    } else if (wave == NT) {
        // ================= Delta0 wave =================
        // X', V rows and e^{G_last} of chunk j into X' buffer xb.
        const int xrot = unit % 6;
        auto fetch_xv = [&](int xb, int j, int lane) {
            lds_u8* xv = (lds_u8*)(xb == 0 ? lds_xv0 : xb == 1 ? lds_xv1 : lds_xv2);
            const unsigned char* rec = rec_of(j) + lane * 16;
            // six 1 KiB fragments, in an order rotated by the unit
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int f = (i + xrot) % 6;
                copy16_to_lds<0>(rec + REC_X + f * FRAG, xv + XV_X + f * FRAG);
            }
            // V rows of the unit's 16 NT columns, 2 NT lanes per row (8 columns
            // each), 32 / NT rows per copy; rows past the chunk's end read as zero
            const auto vr = buffer_rsrc(v + (static_cast<size_t>(tok_of(j)) * num_heads + h) * D + colp,
                                        len_of(j) * row_stride * 2);
            constexpr int LPR = 2 * NT;
#pragma unroll
            for (int k = 0; k < 2 * NT; ++k)
                copy16_to_lds_buf(vr, ((lane / LPR + (64 / LPR) * k) * row_stride + 8 * (lane % LPR)) * 2,
                                  xv + XV_V + k * FRAG);
            // 512 bytes; lanes 32-63 read past the record's end as zero
            copy16_to_lds_buf(buffer_rsrc(rec_of(j), REC_BYTES), REC_VEC + lane * 16, xv + SS::XV_GL);
        };
        // Delta0 = X' diag(rk beta) V of every tile from X' buffer xb into slot
        // p, and e^{G_last} along with it.
        auto delta0 = [&](int xb, int p, int lane) {
            const unsigned char* xv = xb == 0 ? lds_xv0 : xb == 1 ? lds_xv1 : lds_xv2;
            const int l16 = lane & 15, g = lane >> 4, lo16 = lane * 16;
            unsigned char* dg = lds_dg + p * DG_SLOT;
            *reinterpret_cast<floatx2*>(dg + DG_GL + lane * 8) =
                *reinterpret_cast<const floatx2*>(xv + SS::XV_GL + lane * 8);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                halfx8 vb[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int r0 = 32 * s + 4 * g;
                    vb[s] = __builtin_convertvector(bf8_to_f(col8_tr2(xv, XV_V, NT * DVT, r0, r0 + 16, DVT * t, l16)),
                                                    halfx8);
                }
                floatx4 Dm[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) Dm[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (s < (m < 2 ? 1 : 2))
                            Dm[m] = mmah(ldh8(xv, XV_X + tri_block(m, s) * FRAG + lo16), vb[s], Dm[m]);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    *reinterpret_cast<floatx4*>(dg + DG_D + (4 * t + m) * FRAG + lo16) = Dm[m];
            }
        };
        // Chunks 0 and 1 before the first barrier; then in step j (while the
        // state wave runs chunk j+1) chunk j+2 into slot j mod 2, last read by
        // the state wave in step j.  Chunk c's X', V rows and e^{G_last} are in
        // X' buffer c mod XVB.  With three buffers chunk j+2 was requested in
        // step j-2 and chunk j+4 is requested once chunk j+2's Delta0 is
        // formed, into the buffer chunk j+1 has left; with two, chunk j+2 was
        // requested in step j-1 and chunk j+3 follows.  Past the end the last
        // chunk is requested again into a buffer that is not read any more (no
        // branch, so no join merges the copies' wait state).  Requesting before
        // forming Delta0 was measured slower: the copies then meet the output
        // wave's loads in the memory queue.
        constexpr int XVB = SS::XVB;
        constexpr int XV_COPIES = 6 + 2 * NT + 1;  // copy instructions per fetch_xv
#pragma unroll
        for (int j = 0; j < XVB; ++j)
            if (j < nc) fetch_xv(j, j, lane0);
        wait_vmcnt<0>();
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (j < nc) delta0(j, j, lane0);
        // the reads of buffer 0 are done before the copy into it is issued
        __builtin_amdgcn_s_waitcnt(0xC07F);
        if (XVB < nc) fetch_xv(0, XVB, lane0);
        lds_barrier();
        // step j with its buffers as constants: Delta0 of chunk j+2 from buffer
        // (j+2) mod XVB, then chunk j+XVB+1 requested into buffer (j+1) mod XVB
        auto step = [&](int p, int lane, int j, int rb, int wb) {
            if (j + 2 < nc) {
                if constexpr (XVB == 3)
                    wait_vmcnt<XV_COPIES>();
                else
                    wait_vmcnt<0>();
                delta0(rb, p, lane);
                fetch_xv(wb, min(j + XVB + 1, nc - 1), lane);
            }
        };
        constexpr int U = 2 * XVB;  // steps per loop pass: slot parity and buffer index both repeat
        const int nce = (nc + 1) & ~1;  // barriers the other waves run after the first
        for (int j = 0; j < nce; j += U) {
            const int lane = opaque(lane0);
#pragma unroll
            for (int k = 0; k < U; ++k) {
                if (j + k < nce) {
                    lds_barrier();
                    step(k & 1, lane, j + k, (k + 2) % XVB, (k + 1) % XVB);
                }
            }
        }
        wait_vmcnt<0>();
    } else {
        // ================= output wave =================
        struct Ops {
            uint4 q[16];  // Qg' [m][s]
            uint4 p[6];   // P' [tri]
        };
        auto load = [&](Ops& o, int j, int lane) {
            const unsigned char* rec = rec_of(j) + lane * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) o.q[i] = *reinterpret_cast<const uint4*>(rec + REC_QG + i * FRAG);
#pragma unroll
            for (int i = 0; i < 6; ++i) o.p[i] = *reinterpret_cast<const uint4*>(rec + REC_P + i * FRAG);
        };
        // Output rows of chunk j.  O is formed transposed (O^T = S^T Qg'^T +
        // D^T P'^T: the S and D fragments in B-operand form are the A operands
        // of S^T and D^T, and the Qg', P' fragments the B operands of their
        // transposes), so lane l holds columns 4(l/16) .. +3 of row 16m + l%16
        // in O[m]: one 8-byte (bf16) or 16-byte (fp32) store per row block.
        // Rows past the chunk's end, and everything when L = 0, fall outside
        // the range and are dropped.
        auto store_o = [&](const floatx4 (&O)[NT][4], int j, int L, int lane) {
            const int l16 = lane & 15, g = lane >> 4;
            const int out_bytes = L * row_stride * static_cast<int>(sizeof(TOut));
            const auto orr = buffer_rsrc(out + (static_cast<size_t>(tok_of(j)) * num_heads + h) * D + colp, out_bytes);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int off = ((16 * m + l16) * row_stride + DVT * t + 4 * g) * static_cast<int>(sizeof(TOut));
                if constexpr (sizeof(TOut) == 4) {
                    typedef int intx4 __attribute__((ext_vector_type(4)));
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(intx4, O[t][m]), orr, off, 0, 0);
                } else {
                    typedef int intx2 __attribute__((ext_vector_type(2)));
                    const intx2 pk = {static_cast<int>(pack_bf16x2(O[t][m][0], O[t][m][1])),
                                      static_cast<int>(pack_bf16x2(O[t][m][2], O[t][m][3]))};
                    __builtin_amdgcn_raw_buffer_store_b64(pk, orr, off, 0, 0);
                }
            }
        };
        // Step j (between the state wave's barriers j and j+1): store chunk
        // j-1's outputs, request chunk j+1's operands and form chunk j's
        // outputs.  Everything has landed before the barrier.
        auto step = [&](Ops& cur, Ops& nxt, int b, int lane, int j, floatx4 (&O)[NT][4], int& o_len) {
            const int lo16 = lane * 16;
            store_o(O, j - 1, o_len, lane);
            o_len = j < nc ? len_of(j) : 0;
            load(nxt, min(j + 1, nc - 1), lane);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const unsigned char* xch = lds_xch + b * XCH_SLOT + XCH_TILE * t;
                halfx8 sh[4], dh[2];
#pragma unroll
                for (int s = 0; s < 4; ++s) sh[s] = ldh8(xch, XCH_S + s * FRAG + lo16);
#pragma unroll
                for (int s = 0; s < 2; ++s) dh[s] = ldh8(xch, XCH_D + s * FRAG + lo16);
#pragma unroll
                for (int m = 0; m < 4; ++m) O[t][m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m) O[t][m] = mmah(sh[s], as_halfx8(cur.q[4 * m + s]), O[t][m]);
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (s < (m < 2 ? 1 : 2)) O[t][m] = mmah(dh[s], as_halfx8(cur.p[tri_block(m, s)]), O[t][m]);
            }
            wait_vmcnt<0>();
        };

        Ops B0, B1;
        floatx4 O[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) O[t][m] = floatx4{0.f, 0.f, 0.f, 0.f};
        int o_len = 0;
        if (nc > 0) {
            load(B0, 0, lane0);
            wait_vmcnt<0>();
        }
        lds_barrier();
        for (int j = 0; j < nc; j += 2) {
            const int lane = opaque(lane0);
            lds_barrier();
            step(B0, B1, 0, lane, j, O, o_len);
            lds_barrier();
            step(B1, B0, 1, lane, j + 1, O, o_len);
        }
        store_o(O, (nc + 1) / 2 * 2 - 1, o_len, lane0);
    }
    KDA_PHASE_END;
}

// --------------------------------------------------------------------------
// ---- chain_kernel: four waves per (sequence, head, 16-column value tile) ----
// Wave m (0..3) owns the state rows 32m .. 32m+31 of the tile (two 16x16
// accumulator tiles) and the 16 token rows 16m .. 16m+15 of D and of the
// output.  Per chunk, with every operand in registers (loaded straight from
// the record one chunk ahead, no LDS staging):
//   1. the wave's S rows go to LDS as fp16 hi/lo B operands (K block m);
//      barrier;
//   2. all of S is read back; D_m = Delta0_m - Psi'[m,:] S (Delta0_m =
//      X'[m,:] diag(rk beta) V, V from LDS) and O^T_m = S^T Qg'[m,:]^T;
//   3. D_m goes to LDS as hi/lo (half of a 32-token K block); barrier;
//   4. all of D is read back; S <- diag(e^{G_last}) S + Ke^T D for the
//      wave's rows, O^T_m += D^T P'[m,:]^T, and the output rows are stored.
// Two barriers per chunk; each wave issues at most 24 MFMAs per chunk.
// A fifth wave pulls the record and the V rows of the chunk TOUCH_AHEAD steps
// ahead into L2 (one 4-byte load per 128-byte line, into an LDS sink; the
// eight units of a chain take every eighth line each), so the four waves'
// loads, requested one chunk ahead, find their lines in L2 instead of HBM.
// It also copies each chunk's V rows into LDS, two chunks ahead.  The four
// waves issue only their register loads and output stores: a direct-to-LDS
// copy among them would make the compiler wait for it before LDS reads, and
// any branch around a memory operation makes it count conservatively.
// Measured (config 2, per chunk, clock64 in wave 0): about 2.4k cycles,
// against 2.5k for scan_kernel with one tile per workgroup.
constexpr int CH_SX_BYTES = 8 * FRAG;    // S: K block s, hi/lo -> (2 s + hl) fragments
constexpr int CH_DX_BYTES = 4 * FRAG;    // D: K block s, hi/lo -> (2 s + hl) fragments
constexpr int CH_VBYTES = C * DVT * 2;   // V rows of a chunk, [64][16] bf16 (three buffers)
constexpr int CH_SINK = 1024;            // sink of the touch waves' loads
// two workgroups with 64 KiB of padding each exceed 160 KiB
constexpr int CH_LDS = CH_SX_BYTES + CH_DX_BYTES + 3 * CH_VBYTES + CH_SINK;
static_assert(2 * (CH_LDS + 64 * 1024) > 160 * 1024, "padding keeps one workgroup per CU");

constexpr int CH_THREADS = 320;           // four state waves and the touch wave
constexpr int CH_THREADS_CONV = 512;      // with the convolution fused: four helper waves
constexpr int TOUCH_AHEAD = 6;

// With CONV, v is the value block of the fused projection (v_row elements
// per token) before the short convolution, and the touch wave convolves the
// chunk's V rows instead of copying them (see below).
template <typename TOut, bool CONV>
__global__ __launch_bounds__(CONV ? CH_THREADS_CONV : CH_THREADS) void chain_kernel(
    const bf16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens, ChunkMap cm,
    const unsigned char* __restrict__ records, const float* initial_state,
    TOut* __restrict__ out, float* final_state, const int32_t* __restrict__ slots, int num_slots, int num_seqs,
    int num_heads, int state_trans, int v_row, ConvParams cv, bf16_t* conv_state_out) {
    __shared__ __align__(16) unsigned char lds_sx[CH_SX_BYTES];
    __shared__ __align__(16) unsigned char lds_dx[CH_DX_BYTES];
    __shared__ __align__(16) unsigned char lds_vb[3 * CH_VBYTES];  // chunk j's V rows in buffer j mod 3
    __shared__ __align__(16) unsigned char lds_sink[CH_SINK];  // never read
    extern __shared__ __align__(16) unsigned char lds_pad[];  // sized at launch to keep one workgroup per CU
    (void)lds_pad;
    // Workgroup id -> (chain rank, unit): the eight units of a chain share
    // id mod 8, so they run on one XCD and read the chain's records through
    // one L2 (as in scan_kernel).
    const int id = static_cast<int>(blockIdx.x);
    const int crank = (id / 64) * 8 + (id & 7);
    const int unit = (id >> 3) & 7;
    if (crank >= num_seqs * num_heads) return;
    const int n = cm.order ? cm.order[crank / num_heads] : crank / num_heads, h = crank % num_heads;
    const int m = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane0 = static_cast<int>(threadIdx.x) & 63;
    const int col0 = unit * DVT;
    int c_begin, c_end;
    if (cm.offsets) {
        c_begin = cm.offsets[n];
        c_end = cm.offsets[n + 1];
    } else {
        const int lane_off = lane_offsets(cu_seqlens, num_seqs, cm, lane0);
        c_begin = __builtin_amdgcn_readlane(lane_off, n);
        c_end = __builtin_amdgcn_readlane(lane_off, n + 1);
    }
    const int nc = c_end - c_begin;
    const int64_t t_first = cu_seqlens[n], t_last = cu_seqlens[n + 1];
    const int row_stride = num_heads * D;
    size_t head_state = 0;
    const bool has_state = state_block(slots, num_slots, n, h, num_heads, D, head_state);
    const float* init = has_state ? initial_state : nullptr;
    float* fin = has_state ? final_state : nullptr;
    auto rec_of = [&](int j) { return records + (static_cast<size_t>(c_begin + j) * num_heads + h) * REC_BYTES; };
    auto tok_of = [&](int j) { return t_first + static_cast<int64_t>(C) * j; };
    auto len_of = [&](int j) { return static_cast<int>(min64(C, t_last - tok_of(j))); };
    const int ns = m < 2 ? 1 : 2;  // 32-token K blocks of the triangular X' and P' rows of block m

    // output rows 16 r .. 16 r + 15 of chunk j (the tile of wave r), L of the
    // chunk's rows valid: lane (g, l16) holds token 16 r + l16, columns 4g .. 4g+3
    auto store_o = [&](const floatx4& O, int r, int j, int L, int lane) {
        const int l16 = lane & 15, g = lane >> 4;
        const int out_bytes = L * row_stride * static_cast<int>(sizeof(TOut));
        const auto orr = buffer_rsrc(out + (static_cast<size_t>(tok_of(j)) * num_heads + h) * D + col0, out_bytes);
        const int off = ((16 * r + l16) * row_stride + 4 * g) * static_cast<int>(sizeof(TOut));
        if constexpr (sizeof(TOut) == 4) {
            typedef int intx4 __attribute__((ext_vector_type(4)));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(intx4, O), orr, off, 0, 0);
        } else {
            typedef int intx2 __attribute__((ext_vector_type(2)));
            const intx2 pk = {static_cast<int>(pack_bf16x2(O[0], O[1])), static_cast<int>(pack_bf16x2(O[2], O[3]))};
            __builtin_amdgcn_raw_buffer_store_b64(pk, orr, off, 0, 0);
        }
    };

    // V rows of chunk j (64 rows of the unit's 16 columns) into V buffer j & 1:
    // copy k, lane l: row 32 k + l / 2, columns 8 (l & 1) .. +7; rows past the
    // chunk's end read as zero.
    auto v_rows = [&](int j) {  // the chunk's V rows of this head, v_row elements apart
        return buffer_rsrc(v + static_cast<size_t>(tok_of(j)) * v_row + h * D + col0, len_of(j) * v_row * 2);
    };
    auto copy_v = [&](int j, unsigned char* vbuf, int lane) {
        const auto vr = v_rows(j);
#pragma unroll
        for (int k = 0; k < 2; ++k)
            copy16_to_lds_buf(vr, ((32 * k + (lane >> 1)) * v_row + 8 * (lane & 1)) * 2,
                              (lds_u8*)vbuf + k * 32 * DVT * 2);
    };
    if (m >= 4) {
        // ---- touch wave: chunk j + TOUCH_AHEAD into L2 during step j ----
        lds_u8* sink = (lds_u8*)lds_sink;
        constexpr int REC_LINES = (REC_BYTES + 127) / 128;  // 484
        auto touch = [&](int j, int lane) {
            const int i = unit + 8 * lane;  // this unit's lines: unit, unit + 8, ...
            // record lines (lanes past its end fall outside the range and access nothing)
            copy4_to_lds_buf(buffer_rsrc(rec_of(j), REC_BYTES), i < REC_LINES ? 128 * i : REC_BYTES, sink);
            // V: the chunk's rows of this head, 256 bytes = 2 lines each
            const auto vr = buffer_rsrc(v + static_cast<size_t>(tok_of(j)) * v_row + h * D, len_of(j) * v_row * 2);
            copy4_to_lds_buf(vr, ((i >> 1) * v_row + 64 * (i & 1)) * 2, sink);
        };
        // Chunks past the last are clamped to it, so every step issues the
        // same operations (the clamped ones hit lines already in L2).
        const int lane = lane0;
        if constexpr (CONV) {
            // Four helper waves, hi = m - 4, one per SIMD beside a state wave:
            // lane l convolves row l of a chunk in columns 4 hi .. 4 hi + 3
            // (words we0 = 2 (hi & 1), we0 + 1 of the 16-byte half hf = hi / 2)
            // from the raw rows l - 3 .. l (of this chunk in the lanes below,
            // of the previous chunk, or before a sequence's first chunk its
            // conv state, in lanes 61 .. 63 of p).  Chunk j + 2 is convolved
            // into its V buffer during step j (the buffer was last read in
            // step j - 1): word we0 between the two barriers, we0 + 1 after the
            // second, while the state waves work; its raw rows were loaded
            // during step j - 1.  The three raw-row registers rotate by
            // unrolling, so none waits on a load by being copied.  Helper 1
            // touches the V lines, the others the record lines.
            const int hi = m - 4, hf = hi >> 1;
            uint4 prev, ra, rb, rc, r0;
            ConvTaps8 taps;
            {
                const int wrow = cv.channels * 2, range = (cv.K - 1) * wrow + 32;
                const auto wr = buffer_rsrc(cv.weight + 2 * num_heads * D + h * D + col0, range);
                uint4 w[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int jt = t - (4 - cv.K);
                    w[t] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, jt >= 0 ? jt * wrow + 16 * hf : range, 0, 0));
                }
                taps = conv_taps8(w);
                const int srow = cv.channels * 2, s_range = cv.state ? (cv.K - 1) * srow : 0;
                const auto sr = buffer_rsrc(cv.state ? cv.state + static_cast<size_t>(n) * (cv.K - 1) * cv.channels +
                                                           2 * num_heads * D + h * D + col0
                                                     : v,
                                            s_range);
                const int s_idx = cv.K - 65 + lane;  // lanes 61 .. 63: 3 .. 1 steps before the sequence
                prev = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(sr, s_idx >= 0 ? s_idx * srow + 16 * hf : s_range, 0, 0));
            }
            auto raw = [&](int j) {
                return __builtin_bit_cast(uint4,
                                          __builtin_amdgcn_raw_buffer_load_b128(v_rows(j), lane * v_row * 2 + 16 * hf, 0, 0));
            };
            // word e (channels 2e, 2e + 1 of the half) of chunk j's V rows from
            // its raw rows x and the previous chunk's p
            auto conv_word = [&](int j, const uint4& x, const uint4& p, auto ew) {
                constexpr int E = decltype(ew)::value;
                const bool live = lane < len_of(j);
                // rows l - 1, l - 2, l - 3 by rotating the wave (lanes 61 .. 63
                // hand over the previous chunk's rows where the wrap needs them)
                const uint4 x1 = ror1_u4(lane == 63 ? p : x);
                const uint4 x2 = ror1_u4(ror1_u4(lane >= 62 ? p : x));
                const uint4 x3 = ror1_u4(ror1_u4(ror1_u4(lane >= 61 ? p : x)));
                const floatx8 y = conv8<E, E + 1>(x, x1, x2, x3, taps, cv.silu, live);
                *reinterpret_cast<uint32_t*>(lds_vb + (j % 3) * CH_VBYTES + lane * DVT * 2 + 16 * hf + 4 * E) =
                    pack_bf16x2(y[2 * E], y[2 * E + 1]);
            };
            using IA = std::integral_constant<int, 0>;
            using IB = std::integral_constant<int, 1>;
            using IC = std::integral_constant<int, 2>;
            using ID = std::integral_constant<int, 3>;
            // the helper's two words (we0 = 0 or 2, chosen at run time: one
            // call per case keeps E a constant)
            auto conv_first = [&](int j, const uint4& x, const uint4& p) {
                if (hi & 1) conv_word(j, x, p, IC{});
                else conv_word(j, x, p, IA{});
            };
            auto conv_second = [&](int j, const uint4& x, const uint4& p) {
                if (hi & 1) conv_word(j, x, p, ID{});
                else conv_word(j, x, p, IB{});
            };
            // helper 1 touches V rows of this head (from its first column, 2
            // lines each), the others record lines: one load, its address
            // chosen by arithmetic (a branch around it would make the compiler
            // count loads in flight conservatively)
            const uint64_t pick = hi == 1 ? 0 : ~uint64_t(0);
            auto touch_reg = [&](int j) {
                const int i = unit + 8 * lane;
                const uint64_t a = reinterpret_cast<uint64_t>(rec_of(j));
                const uint64_t b = reinterpret_cast<uint64_t>(v + static_cast<size_t>(tok_of(j)) * v_row + h * D);
                const unsigned char* base = reinterpret_cast<const unsigned char*>((a & pick) | (b & ~pick));
                const int range = hi != 1 ? REC_BYTES : len_of(j) * v_row * 2;
                const int off = hi != 1 ? (i < REC_LINES ? 128 * i : REC_BYTES) : ((i >> 1) * v_row + 64 * (i & 1)) * 2;
                return __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(base, range), off, 0, 0);
            };
            uint32_t sum = 0, tka = 0, tkb = 0, tkc = 0;
            if (nc > 0) {
                // chunks 0 and 1 before the loop; ra, rb: the raw rows of chunks 1, 2
                r0 = raw(0);
                ra = raw(min(1, nc - 1));
                rb = raw(min(2, nc - 1));
#pragma unroll
                for (int j = 3; j < TOUCH_AHEAD; ++j) touch(min(j, nc - 1), lane);
                wait_vmcnt<0>();  // once: the direct-to-LDS touches are done before the loop's LDS writes
                conv_first(0, r0, prev);
                conv_second(0, r0, prev);
                if (nc > 1) {
                    conv_first(1, ra, r0);
                    conv_second(1, ra, r0);
                }
            }
            // step j with x1, x2 the raw rows of chunks j + 1, j + 2; x3
            // receives chunk j + 3's.  Per step: one raw load after the first
            // barrier, one touch at the end, so chunk j + 2's rows are older
            // than the last 2 operations once x3 is issued.  A touch's value is
            // folded in three steps later (the line comes from HBM).  The
            // scheduling barriers keep each part of the work between its two
            // barriers.
            KDA_PHASE_BEGIN
            auto step_t = [&](int j, const uint4& x1, const uint4& x2, uint4& x3, uint32_t& tk) {
                KDA_PHASE_MARK(24);
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
                KDA_PHASE_MARK(25);
                x3 = raw(min(j + 3, nc - 1));
                wait_vmcnt<2>();
                if (j + 2 < nc) conv_first(j + 2, x2, x1);
                KDA_PHASE_MARK(26);
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
                KDA_PHASE_MARK(27);
                if (j + 2 < nc) conv_second(j + 2, x2, x1);
                KDA_PHASE_MARK(28);
                sum += tk;
                tk = touch_reg(min(j + TOUCH_AHEAD, nc - 1));
                KDA_PHASE_MARK(29);
            };
            int j = 0;
            for (; j + 3 <= nc; j += 3) {
                step_t(j, ra, rb, rc, tka);
                step_t(j + 1, rb, rc, ra, tkb);
                step_t(j + 2, rc, ra, rb, tkc);
            }
            if (j < nc) step_t(j, ra, rb, rc, tka);
            if (j + 1 < nc) step_t(j + 1, rb, rc, ra, tkb);
            KDA_PHASE_END;
            wait_vmcnt<0>();
            sum += tka + tkb + tkc;
            reinterpret_cast<uint32_t*>(lds_sink)[hi * 64 + lane] = sum;
            // The request's new conv state, this unit's 16 channels of its
            // head's q, k and v blocks: row r is entry len + r of the window
            // (the input row when that lies past the old state, else the old
            // state's row, else zero).  Lane: block p = lane / 6, row r = (lane
            // / 2) % 3, half lane & 1.  Each slice of the old state is read by
            // this workgroup alone (its v columns above, q and k by the prep
            // pass before), and every lane's load precedes the stores, so the
            // new state may overwrite the old.
            if (hi == 0 && conv_state_out && cv.K > 1) {
                const int S = cv.K - 1;
                const int p = lane / 6, r = (lane >> 1) % 3;
                const int64_t start = t_first, end = t_last;
                const int64_t len = start < 0 || end > cm.total_tokens || end < start ? 0 : end - start;
                const size_t Cc = static_cast<size_t>(cv.channels);
                const size_t c = static_cast<size_t>(p) * num_heads * D + h * D + col0 + 8 * (lane & 1);
                const bf16_t* x0 = v - 2 * static_cast<size_t>(num_heads) * D;  // the fused projection
                const bool live = lane < 18 && r < S;
                const int64_t i = len + r;
                const bf16_t* src = i >= S ? x0 + static_cast<size_t>(start + i - S) * Cc + c
                                           : (cv.state ? cv.state + (static_cast<size_t>(n) * S + i) * Cc + c : nullptr);
                uint4 val = {0u, 0u, 0u, 0u};
                if (live && src) val = *reinterpret_cast<const uint4*>(src);
                if (live) *reinterpret_cast<uint4*>(conv_state_out + (static_cast<size_t>(n) * S + r) * Cc + c) = val;
            }
            return;
        }
        if (nc > 0) {
            copy_v(0, lds_vb, lane);
            copy_v(min(1, nc - 1), lds_vb + CH_VBYTES, lane);
#pragma unroll
            for (int j = 2; j < TOUCH_AHEAD; ++j) touch(min(j, nc - 1), lane);
            static_assert(2 + 2 * (TOUCH_AHEAD - 2) == 10, "ops after chunk 0's copies");
            wait_vmcnt<2 + 2 * (TOUCH_AHEAD - 2)>();
        }
        // Only the V copy goes between the two barriers (so this wave reaches
        // the second one on time); the touches and the stores of chunk j - 1's
        // output rows follow it, while the other waves update the state.
        // Chunk j + 2's V rows are copied during step j into the buffer chunk
        // j - 1 left; per step this wave issues 2 copies and 2 touches, so
        // before step j's first barrier chunk j's copies are the ops older
        // than the last 6 (step 1: the last 10; step 0: the last 10).
        auto vbuf = [&](int j) { return lds_vb + (j % 3) * CH_VBYTES; };
        KDA_PHASE_BEGIN
        for (int j = 0; j < nc; ++j) {
            if (j == 1)
                wait_vmcnt<10>();
            else if (j > 1)
                wait_vmcnt<6>();
            KDA_PHASE_MARK(24);
            lds_barrier();
            KDA_PHASE_MARK(25);
            const int jv = min(j + 2, nc - 1);
            copy_v(jv, vbuf(jv), lane);
            KDA_PHASE_MARK(26);
            lds_barrier();
            KDA_PHASE_MARK(27);
            touch(min(j + TOUCH_AHEAD, nc - 1), lane);
            KDA_PHASE_MARK(28);
        }
        KDA_PHASE_END;

        wait_vmcnt<0>();
        return;
    }


    KDA_PHASE_BEGIN
    // state rows 32m + 4g + j (tile 0) and 32m + 16 + 4g + j (tile 1), column col0 + l16
    floatx4 S[2];
    {
        const int l16 = lane0 & 15, g = lane0 >> 4;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[a][j] = init ? init[head_state + state_elem(32 * m + 16 * a + 4 * g + j, col0 + l16, D, state_trans)]
                               : 0.f;
    }

    // The operands of chunk j, wave m: -Psi'[m][s], Qg'[m][s] (s = 0..3), Ke^T
    // of channel blocks 2m, 2m+1 (K blocks 0, 1), X' and P' blocks (m, s <
    // ns; a second, unused copy of block (m, 0) when ns = 1, so every wave
    // issues the same loads), e^{G_last} of the wave's state rows.
    struct Ops {
        uint4 np[4], qg[4], ke[4], x[2], p[2];
        floatx4 gl[2];
    };
    // The loads come in three groups, each issued between the MFMAs of one
    // part of the step (a wave issues in order and would otherwise stall on
    // the memory queue before its products), in the order the next chunk
    // uses them: X', -Psi' (D); Qg' (output); Ke^T, e^{G_last}, P' (update).
    // X' and P' block (m, 1) exists for m >= 2 only: for m < 2 it is read
    // at an offset past the record's range, which returns zeros (no branch,
    // no mask written over a register with a load in flight).
    const int blk1_off = ns > 1 ? 0 : REC_BYTES;
    auto tri_load = [&](const __amdgpu_buffer_rsrc_t& rr, int base, int s_, int lane) {
        const int off = s_ == 0 ? base + tri_block(m, 0) * FRAG + lane * 16
                                : base + tri_block(m, 1) * FRAG + lane * 16 + blk1_off;
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0));
    };
    auto load_a = [&](Ops& o, const unsigned char* rec, const __amdgpu_buffer_rsrc_t& rr, int i, int lane) {
        if (i < 2) {
            o.x[i] = tri_load(rr, REC_X, i, lane);
        } else {
            o.np[i - 2] = *reinterpret_cast<const uint4*>(rec + REC_NPSI + (4 * m + i - 2) * FRAG);
        }
    };
    auto load_b = [&](Ops& o, const unsigned char* rec, int i) {  // i = 0 .. 3
        o.qg[i] = *reinterpret_cast<const uint4*>(rec + REC_QG + (4 * m + i) * FRAG);
    };
    auto load_c = [&](Ops& o, const unsigned char* rec, const unsigned char* vec, const __amdgpu_buffer_rsrc_t& rr,
                      int i, int lane) {  // i = 0 .. 7
        if (i < 4) {
            o.ke[i] = *reinterpret_cast<const uint4*>(rec + REC_KE + ((2 * m + (i >> 1)) * 2 + (i & 1)) * FRAG);
        } else if (i < 6) {
            o.gl[i - 4] = *reinterpret_cast<const floatx4*>(vec + 16 * (i - 4) * 4);
        } else {
            o.p[i - 6] = tri_load(rr, REC_P, i - 6, lane);
        }
    };
    auto load = [&](Ops& o, int j, int lane) {
        const unsigned char* rec = rec_of(j) + lane * 16;
        const unsigned char* vec = rec_of(j) + REC_VEC + (32 * m + 4 * (lane >> 4)) * 4;
        const auto rr = buffer_rsrc(rec_of(j), REC_BYTES);
#pragma unroll
        for (int i = 0; i < 6; ++i) load_a(o, rec, rr, i, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_b(o, rec, i);
#pragma unroll
        for (int i = 0; i < 8; ++i) load_c(o, rec, vec, rr, i, lane);
    };
    // One chunk with its operands in cur; the next chunk's go into nxt, in
    // three groups between this chunk's products (18 loads; the compiler
    // waits for each where it is used).
    auto step = [&](Ops& cur, Ops& nxt, int j, floatx4& O, int& L, int lane) {
        const unsigned char* vb_cur = lds_vb + (j % 3) * CH_VBYTES;
        const int lo16 = lane * 16, l16 = lane & 15, g = lane >> 4;
        const int jn = min(j + 1, nc - 1);
        const unsigned char* nrec = rec_of(jn) + lane * 16;
        const unsigned char* nvec = rec_of(jn) + REC_VEC + (32 * m + 4 * g) * 4;
        const auto nrr = buffer_rsrc(rec_of(jn), REC_BYTES);
        // (1) this wave's rows of S into LDS as the B operand of K block m
        {
            halfx8 sh, sl;
            split8h(S[0], S[1], sh, sl);
            *reinterpret_cast<halfx8*>(lds_sx + (2 * m) * FRAG + lo16) = sh;
            *reinterpret_cast<halfx8*>(lds_sx + (2 * m + 1) * FRAG + lo16) = sl;
        }
        KDA_PHASE_MARK(16);
        KDA_PHASE_MARK(17);
        lds_barrier();
        KDA_PHASE_MARK(18);
        // (2) S (all 128 rows) back as B operands; V rows of this chunk as B operands
        halfx8 shs[4], sls[4], vb[2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            shs[s] = ldh8(lds_sx, (2 * s) * FRAG + lo16);
            sls[s] = ldh8(lds_sx, (2 * s + 1) * FRAG + lo16);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int r0 = 32 * s + 4 * g;
            vb[s] = __builtin_convertvector(
                bf8_to_f(col8_tr2(vb_cur, 0, DVT, r0, r0 + 16, 0, l16)), halfx8);
        }
        // the products of D in two independent accumulators (K blocks 0, 1 and
        // 2, 3 of S), each product followed by one load of the next chunk
        // (pinned order)
        const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
        floatx4 Da = mmah(as_halfx8(cur.x[0]), vb[0], z4);
        __builtin_amdgcn_sched_barrier(0);
        load_a(nxt, nrec, nrr, 0, lane);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 Db = mmah(as_halfx8(cur.x[1]), vb[1], z4);
        __builtin_amdgcn_sched_barrier(0);
        load_a(nxt, nrec, nrr, 1, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            Da = mmah(as_halfx8(cur.np[s]), shs[s], Da);
            Db = mmah(as_halfx8(cur.np[2 + s]), shs[2 + s], Db);
            __builtin_amdgcn_sched_barrier(0);
            load_a(nxt, nrec, nrr, 2 + 2 * s, lane);
            __builtin_amdgcn_sched_barrier(0);
            Da = mmah(as_halfx8(cur.np[s]), sls[s], Da);
            Db = mmah(as_halfx8(cur.np[2 + s]), sls[2 + s], Db);
            __builtin_amdgcn_sched_barrier(0);
            load_a(nxt, nrec, nrr, 3 + 2 * s, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
        const floatx4 Dm = Da + Db;
        // (3) D_m into LDS: rows 16m .. 16m+15 are half (m & 1) of K block m >> 1
        {
            halfx4 dh, dl;
            split4h(Dm, dh, dl);
            const int o = (2 * (m >> 1)) * FRAG + lo16 + 8 * (m & 1);
            *reinterpret_cast<halfx4*>(lds_dx + o) = dh;
            *reinterpret_cast<halfx4*>(lds_dx + o + FRAG) = dl;
        }
        floatx4 Oa = z4, Ob = z4;
#pragma unroll
        for (int s = 0; s < 4; s += 2) {
            Oa = mmah(shs[s], as_halfx8(cur.qg[s]), Oa);
            __builtin_amdgcn_sched_barrier(0);
            load_b(nxt, nrec, s);
            __builtin_amdgcn_sched_barrier(0);
            Ob = mmah(shs[s + 1], as_halfx8(cur.qg[s + 1]), Ob);
            __builtin_amdgcn_sched_barrier(0);
            load_b(nxt, nrec, s + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        O = Oa + Ob;
        L = len_of(j);
        KDA_PHASE_MARK(19);
        lds_barrier();
        KDA_PHASE_MARK(20);
        // (4) D back; state update of the wave's rows; output
        halfx8 dh[2], dl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            dh[s] = ldh8(lds_dx, (2 * s) * FRAG + lo16);
            dl[s] = ldh8(lds_dx, (2 * s + 1) * FRAG + lo16);
        }
        S[0] *= cur.gl[0];
        S[1] *= cur.gl[1];
        // the update's products and the output's, each followed by one load of the next chunk
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                S[a] = mmah(as_halfx8(cur.ke[2 * a + s]), dh[s], S[a]);
                __builtin_amdgcn_sched_barrier(0);
                load_c(nxt, nrec, nvec, nrr, 2 * s + a, lane);
                __builtin_amdgcn_sched_barrier(0);
                S[a] = mmah(as_halfx8(cur.ke[2 * a + s]), dl[s], S[a]);
                __builtin_amdgcn_sched_barrier(0);
                load_c(nxt, nrec, nvec, nrr, 4 + 2 * s + a, lane);
                __builtin_amdgcn_sched_barrier(0);
            }
        O = mmah(dh[0], as_halfx8(cur.p[0]), O);
        O = mmah(dh[1], as_halfx8(cur.p[1]), O);
        store_o(O, m, j, L, lane);
        KDA_PHASE_MARK(21);
        (void)l16;
    };

    if (nc > 0) {
        Ops B0, B1;
        floatx4 O = {0.f, 0.f, 0.f, 0.f};
        int L = 0;
        load(B0, 0, lane0);
        // Needed by the first step anyway; waiting here also keeps the
        // compiler's count at the loop head to what the loop itself issues
        // (it merges the entry path into every iteration).
        wait_vmcnt<0>();
        int j = 0;
        for (; j + 1 < nc; j += 2) {
            const int lane = opaque(lane0);
            step(B0, B1, j, O, L, lane);
            step(B1, B0, j + 1, O, L, lane);
        }
        if (j < nc) step(B0, B1, j, O, L, opaque(lane0));
        wait_vmcnt<0>();
    }
    if (fin) {
        const int l16 = lane0 & 15, g = lane0 >> 4;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fin[head_state + state_elem(32 * m + 16 * a + 4 * g + j, col0 + l16, D, state_trans)] = S[a][j];
    }
    KDA_PHASE_END;
}

// --------------------------------------------------------------------------

bool split_prefill_applies(const PrefillArgs& a) { return a.qkv_bf16 && a.head_dim == D; }

// Workspace: chunk offsets [N + 1] and the dispatch order [N] (int32), padded
// to 256 bytes, then the records.
static size_t map_bytes(int num_seqs) { return (static_cast<size_t>(2 * num_seqs + 1) * 4 + 255) & ~size_t(255); }

size_t split_workspace_bytes(int64_t total_tokens, int num_seqs, int num_heads) {
    const size_t off_bytes = map_bytes(num_seqs);
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
    int32_t* order = offsets + a.num_seqs + 1;
    unsigned char* records = ws + map_bytes(a.num_seqs);
    const size_t max_chunks = static_cast<size_t>((a.total_tokens + C - 1) / C) + static_cast<size_t>(a.num_seqs);
    const unsigned chains = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
    const unsigned groups = (chains + 7u) & ~7u;
    // While every 16-column tile has a compute unit of its own, the chunk
    // chain's latency is the limit: chain_kernel (four waves share a tile's
    // chain; 64 KiB of LDS padding keeps one workgroup per CU).  When tiles
    // outnumber CUs, throughput is: scan_kernel with two tiles per workgroup
    // reads each record once for both.
    // With the convolution fused, chain_kernel (whose touch wave convolves
    // V) runs in both cases, without the padding when tiles outnumber CUs.
    const bool pairs = static_cast<size_t>(chains) * (D / DVT) > static_cast<size_t>(device_cu_count());
    // Every chain running at once and few sequences: the kernels find the
    // chunks themselves, with no chunk-map launch.
    const bool lane_map = !pairs && a.num_seqs <= kLaneMapSeqs;
    const ChunkMap cm{lane_map ? nullptr : offsets, lane_map ? nullptr : order, a.total_tokens,
                      static_cast<int>(max_chunks)};
    hipError_t e = hipSuccess;
    if (!lane_map) {
        chunk_map_kernel<<<1, 1024, 0, stream>>>(a.cu_seqlens, a.num_seqs, a.total_tokens,
                                                 static_cast<int>(max_chunks), offsets, order);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t max_items = max_chunks * static_cast<size_t>(a.num_heads);
    const unsigned prep_grid = static_cast<unsigned>(max_items < static_cast<size_t>(device_cu_count()) ? max_items : static_cast<size_t>(device_cu_count()));
    if (prep_grid > 0) {
        const bf16_t* q = static_cast<const bf16_t*>(a.q);
        const bf16_t* k = static_cast<const bf16_t*>(a.k);
        auto pick = [&](auto conv, auto lmap) {
            constexpr bool CV = decltype(conv)::value, LM = decltype(lmap)::value;
            return a.gate.a_log ? (a.gate_per_head ? prep_kernel<true, true, CV, LM> : prep_kernel<true, false, CV, LM>)
                                : (a.gate_per_head ? prep_kernel<false, true, CV, LM> : prep_kernel<false, false, CV, LM>);
        };
        auto pick_map = [&](auto lmap) { return a.conv.weight ? pick(std::true_type{}, lmap) : pick(std::false_type{}, lmap); };
        auto* kern = lane_map ? pick_map(std::true_type{}) : pick_map(std::false_type{});
        kern<<<prep_grid, PNT, 0, stream>>>(q, k, a.g, a.beta, a.gate, a.cu_seqlens, cm.offsets, records,
                                            a.num_seqs, a.num_heads, a.scale, a.l2norm, static_cast<int>(a.qkv_row),
                                            a.conv, a.total_tokens, static_cast<int>(max_chunks));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.conv.weight) {
        chain_kernel<TOut, true><<<groups * 8, CH_THREADS_CONV, pairs ? 0 : 64 * 1024, stream>>>(
            static_cast<const bf16_t*>(a.v), a.cu_seqlens, cm, records, a.initial_state,
            static_cast<TOut*>(a.out), a.final_state, a.slots, a.num_slots, a.num_seqs, a.num_heads,
            a.state_trans, static_cast<int>(a.qkv_row), a.conv, static_cast<bf16_t*>(a.conv_state_out));
        return hipGetLastError();
    }
    if (!pairs) {
        chain_kernel<TOut, false><<<groups * 8, CH_THREADS, 64 * 1024, stream>>>(
            static_cast<const bf16_t*>(a.v), a.cu_seqlens, cm, records, a.initial_state,
            static_cast<TOut*>(a.out), a.final_state, a.slots, a.num_slots, a.num_seqs, a.num_heads,
            a.state_trans, static_cast<int>(a.qkv_row), a.conv, nullptr);
        return hipGetLastError();
    }
    scan_kernel<TOut, 2><<<groups * ScanShape<2>::UNITS, ScanShape<2>::THREADS, 0, stream>>>(
        static_cast<const bf16_t*>(a.v), a.cu_seqlens, offsets, order, records, a.initial_state,
        static_cast<TOut*>(a.out), a.final_state, a.slots, a.num_slots, a.num_seqs, a.num_heads,
        a.state_trans);
    return hipGetLastError();
}

hipError_t launch_prefill_split(const PrefillArgs& a, void* workspace, hipStream_t stream) {
    return a.out_bf16 ? launch_split_t<bf16_t>(a, workspace, stream) : launch_split_t<float>(a, workspace, stream);
}

}  // namespace kda
