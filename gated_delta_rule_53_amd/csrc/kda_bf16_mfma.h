// Private helpers for the bf16 MFMA kernels (gfx950, wave64).
//
// Operands are carried as bf16 hi/lo pairs (x = hi + lo to about 2^-17
// relative); products use hi*hi + hi*lo + lo*hi on the 16x16x32 bf16 MFMA with
// fp32 accumulation.  Lane layout of v_mfma_f32_16x16x32_bf16: lane l supplies
// A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16]; the accumulator holds
// D[4*(l/16)+j][l%16] in element j.
#pragma once

#include "kda_common.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ floatx4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, floatx4 c) {
    c = mma(ah, bh, c);
    c = mma(ah, bl, c);
    return mma(al, bh, c);
}

// fp16 operands (v_mfma_f32_16x16x32_f16 has the same lane layout as the
// bf16 instruction).
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mmah(halfx8 a, halfx8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ halfx8 ldh8(const unsigned char* smem, int off_bytes) {
    return *reinterpret_cast<const halfx8*>(smem + off_bytes);
}

__device__ __forceinline__ halfx8 as_halfx8(const uint4& u) { return __builtin_bit_cast(halfx8, u); }

// fp16 hi/lo pair of four floats (x = hi + lo to about 2^-22 relative while
// |x| stays in the fp16 normal range).
__device__ __forceinline__ void split4h(const floatx4& x, halfx4& hi, halfx4& lo) {
    hi = __builtin_convertvector(x, halfx4);
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, floatx4), halfx4);
}

// fp16 hi/lo pair of eight floats (a then b) in MFMA operand order.  hi is
// the rounded conversion; lo = round(x - hi) comes from one mixed-precision
// FMA per value (x - hi is exact in fp32, so the single rounding gives the
// same lo as converting hi back and subtracting).
__device__ __forceinline__ void split8h(const floatx4& a, const floatx4& b, halfx8& hi, halfx8& lo) {
    const halfx4 ha = __builtin_convertvector(a, halfx4), hb = __builtin_convertvector(b, halfx4);
    hi = halfx8{ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
    const uint4 h = __builtin_bit_cast(uint4, hi);
    uint4 l = {0u, 0u, 0u, 0u};
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    uint32_t lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "+v"(lw[k]) : "v"(x[2 * k]), "v"(hw[k]));
        asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
            : "+v"(lw[k])
            : "v"(x[2 * k + 1]), "v"(hw[k]));
    }
    lo = __builtin_bit_cast(halfx8, uint4{lw[0], lw[1], lw[2], lw[3]});
}

__device__ __forceinline__ bf16x8 ld8(const unsigned char* smem, int off_bytes) {
    return *reinterpret_cast<const bf16x8*>(smem + off_bytes);
}

// Operand fragment or zeros (K ranges past the valid rows).
__device__ __forceinline__ bf16x8 ld8_if(const unsigned char* smem, int off_bytes, bool valid) {
    const bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    return valid ? ld8(smem, off_bytes) : z;
}

// Eight bf16 at base[0], base[stride], ..., base[7*stride] (a column gather).
__device__ __forceinline__ bf16x8 gather8(const __bf16* base, int stride) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = base[i * stride];
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// Column read through the transposing LDS load ds_read_b64_tr_b16.  Within
// each group of 16 lanes, lane L reads 8 bytes at its own address and lane i
// receives element i%4 of the reads of lanes i/4, i/4+4, i/4+8, i/4+12.  So
// if lane L reads row r0 + L/4, columns c0 + 4(L%4) .. +3 of a row-major
// 16-bit array, lane i gets column c0 + i of rows r0 .. r0+3.  col8_tr does
// that twice: lane i of the group gets rows r0 .. r0+7 of column c0 + i (the
// same result as gather8, in two LDS instructions instead of eight).
// base: byte offset of the array in LDS, stride: row stride in elements,
// r0, c0: per 16-lane group; l16: the lane's index in its group.
// col8_tr2 takes the two groups of four rows from independent starts r0, r1.
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 col8_tr2(const unsigned char* smem, int base, int stride, int r0, int r1, int c0,
                                           int l16) {
    const int col = c0 + 4 * (l16 & 3);
    typedef __attribute__((address_space(3))) shortx4* lds_v4;
    const shortx4 a =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(smem + base + ((r0 + (l16 >> 2)) * stride + col) * 2));
    const shortx4 b =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(smem + base + ((r1 + (l16 >> 2)) * stride + col) * 2));
    const short t[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = __builtin_bit_cast(__bf16, t[i]);
    return r;
}

__device__ __forceinline__ bf16x8 col8_tr(const unsigned char* smem, int base, int stride, int r0, int c0, int l16) {
    return col8_tr2(smem, base, stride, r0, r0 + 4, c0, l16);
}

// Four bf16 at smem[off_bytes] (8-byte aligned).
__device__ __forceinline__ bf16x4 ld4(const unsigned char* smem, int off_bytes) {
    return *reinterpret_cast<const bf16x4*>(smem + off_bytes);
}

// Direct copy global -> LDS: each lane's 16 bytes at src + off land at
// lds + off + 16 * lane (lds is wave-uniform; it goes to M0; the constant
// off is the instruction offset, which applies to both addresses).  Counted
// by vmcnt like any other load; the data is in LDS once the count says so.
typedef __attribute__((address_space(3))) unsigned char lds_u8;
template <int OFF>
__device__ __forceinline__ void copy16_to_lds(const void* src, lds_u8* lds) {
    typedef __attribute__((address_space(1))) void gvoid;
    typedef __attribute__((address_space(3))) void lvoid;
    __builtin_amdgcn_global_load_lds((const gvoid*)src, (lvoid*)lds, 16, OFF, 0);
}

// Buffer form: lane l's 16 bytes at byte voff of the resource land at
// lds + 16 l; bytes past the resource's end read as zero.
__device__ __forceinline__ void copy16_to_lds_buf(__amdgpu_buffer_rsrc_t r, int voff, lds_u8* lds) {
    typedef __attribute__((address_space(3))) void lvoid;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lvoid*)lds, 16, voff, 0, 0, 0);
}

// Four bytes per lane at byte voff of the resource into lds + 4 l.  Used to
// pull lines into L2 ahead of their readers (the LDS copy is the load's only
// visible effect, so the compiler keeps it).
__device__ __forceinline__ void copy4_to_lds_buf(__amdgpu_buffer_rsrc_t r, int voff, lds_u8* lds) {
    typedef __attribute__((address_space(3))) void lvoid;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lvoid*)lds, 4, voff, 0, 0, 0);
}

// The same with off = 1024 q, q = 0 .. 3 chosen at run time (a constant after unrolling).
__device__ __forceinline__ void copy16_to_lds_q(const void* src, lds_u8* lds, int q) {
    switch (q) {
        case 0: copy16_to_lds<0>(src, lds); break;
        case 1: copy16_to_lds<1024>(src, lds); break;
        case 2: copy16_to_lds<2048>(src, lds); break;
        default: copy16_to_lds<3072>(src, lds); break;
    }
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load, which would expose the latency of a
// prefetch issued before it; here only this wave's LDS operations are
// drained.  The memory clobber keeps the compiler from moving loads or
// stores across it.
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

__device__ __forceinline__ floatx8 bf8_to_f(const bf16x8& b) { return unpack8(__builtin_bit_cast(uint4, b)); }

// Split two floats into packed bf16 hi and lo words.  The high halves are
// recovered from the packed word with integer ops so the rounding
// conversion runs once per pair.
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

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero and stores past the end are dropped by the hardware, so ragged tails
// need no branches and every wave issues the same number of memory operations.
// Word 3 selects 32-bit data format with no swizzle (gfx9 family).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).  Emitted
// through the builtin, so the compiler's own wait insertion knows about it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Opaque copy of a lane-dependent value: re-materialised where it is used so
// the compiler cannot hoist lane-dependent constants out of long loops (kept
// live across them they would be spilled).
__device__ __forceinline__ int opaque(int x) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

}  // namespace kda
