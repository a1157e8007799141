// Output epilogue of the KDA layer: gated RMSNorm over the value channels.
//
// The Ascend model file's attention output path (`_project_out` with its
// `KimiRMSNorm` o_norm) takes each (token, head) row of the core output, of
// length dv, divides it by its root mean square (eps added to the mean of
// squares inside the root), scales it by the norm weight (one value per
// channel) and by the sigmoid of the output-gate projection:
//
//   y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate)
//
// HBM-bound: per row, o and gate are read once and y written once.  Launch:
// 256 threads per workgroup, dv / 8 lanes per row, eight values per lane (one
// 16-byte load of bf16, two of fp32), fully coalesced; the mean of squares is
// a sum over the row's lanes.  A lane reads all of its values of a row before
// it writes any of them, so out may be o itself.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

template <typename T>
__device__ __forceinline__ void load8(float (&x)[8], const T* p) {
    T v[8];
    load_vec<8>(v, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(v[i]);
}

// bf16 rounded by pairs in hardware
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(T) == 2) {
        __builtin_nontemporal_store(u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                                          pack_bf16x2(x[6], x[7])},
                                    reinterpret_cast<u32x4*>(p));
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(x)[i], reinterpret_cast<u32x4*>(p) + i);
    }
}

}  // namespace

// Each lane group takes RPG rows, RPB apart, with all their loads issued
// before any arithmetic; y is stored non-temporally (nothing reads it back
// here).  One row per lane group measured best (T=4096, H=32, dv=128, bf16:
// 17.3 us against 17.5 / 18.0 / 18.7 us for 2 / 4 / 8): more workgroups keep
// more loads in flight than more rows per lane.
constexpr int RPG = 1;

template <int DV, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const TIn* __restrict__ o, const TIn* __restrict__ gate,
                                                            const float* __restrict__ weight, float eps,
                                                            TOut* out, int64_t rows) {
    constexpr int LPR = DV / 8;      // lanes per row
    constexpr int RPB = 256 / LPR;   // rows per workgroup and pass
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * RPB * RPG + threadIdx.x / LPR;
    const int c0 = (threadIdx.x % LPR) * 8;
    float x[RPG][8], g[RPG][8], w[8];
    *reinterpret_cast<floatx4*>(w) = *reinterpret_cast<const floatx4*>(weight + c0);
    *reinterpret_cast<floatx4*>(w + 4) = *reinterpret_cast<const floatx4*>(weight + c0 + 4);
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
        const int64_t row = row0 + static_cast<int64_t>(k) * RPB;
        // a row past the end reads row 0 (in bounds) and is not stored
        const size_t off = static_cast<size_t>(row < rows ? row : 0) * DV + c0;
        load8(x[k], o + off);
        load8(g[k], gate + off);
    }
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
        const int64_t row = row0 + static_cast<int64_t>(k) * RPB;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += x[k][i] * x[k][i];
        // the sum stays within the row's LPR lanes
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float r = rsqrtf(ss * (1.f / DV) + eps);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[k][i] = x[k][i] * r * w[i] * gate_sigmoid(g[k][i]);
        if (row < rows) store8(out + static_cast<size_t>(row) * DV + c0, x[k]);
    }
}

template <int DV, typename TIn, typename TOut>
static hipError_t launch_epi_t(const EpilogueArgs& a, hipStream_t stream) {
    constexpr int RPB = 256 / (DV / 8) * RPG;
    const int64_t blocks = (a.rows + RPB - 1) / RPB;
    gated_rmsnorm_kernel<DV, TIn, TOut><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
        static_cast<const TIn*>(a.o), static_cast<const TIn*>(a.gate), a.weight, a.eps, static_cast<TOut*>(a.out),
        a.rows);
    return hipGetLastError();
}

template <int DV>
static hipError_t launch_epi_d(const EpilogueArgs& a, hipStream_t stream) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_epi_t<DV, bf16_t, bf16_t>(a, stream) : launch_epi_t<DV, bf16_t, float>(a, stream);
    return a.out_bf16 ? launch_epi_t<DV, float, bf16_t>(a, stream) : launch_epi_t<DV, float, float>(a, stream);
}

hipError_t launch_gated_rmsnorm(const EpilogueArgs& a, hipStream_t stream) {
    return a.head_v == 128 ? launch_epi_d<128>(a, stream) : launch_epi_d<64>(a, stream);
}

}  // namespace kda
