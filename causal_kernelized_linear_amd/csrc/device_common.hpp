// Device-side helpers shared by the gfx950 kernels: element traits, the
// feature map, and the 16x16 MFMA step used by every chunk contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kThreads = 256;      // four waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

// phi(x) = elu(x) + 1: x + 1 above zero, exp(x) at or below it.  exp(x) is
// 2^(x * log2 e) on the hardware exp2 unit; for large positive x it overflows to
// +inf, which the select discards (NaN inputs stay NaN).
__device__ __forceinline__ float phi(float x) {
    const float e = __builtin_amdgcn_exp2f(x * kLog2e);
    return x > 0.0f ? x + 1.0f : e;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the 64 lanes of a wave, every lane active: DPP row shifts by
// 1, 2, 4 and 8 scan each 16-lane row (a source outside the row reads 0), then
// row_bcast:15 adds the last lane of row r - 1 to rows 1 and 3 and row_bcast:31 adds
// lane 31 (the total of rows 0 and 1) to rows 2 and 3.  Six VALU steps, no LDS.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add_from(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, true));
}
// Sum over each aligned group of G consecutive lanes (G = 8 or 16), every lane getting
// its group's sum: quad swaps, then the half-row mirror, then (G = 16) the row mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int G>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
    x += dpp_mov<0xB1>(x);      // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);      // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x141>(x);     // row_half_mirror
    if constexpr (G == 16) x += dpp_mov<0x140>(x);   // row_mirror
    return x;
}

__device__ __forceinline__ float wave_incl_scan(float x) {
    x = dpp_add_from<0x111, 0xF>(x);   // row_shr:1
    x = dpp_add_from<0x112, 0xF>(x);   // row_shr:2
    x = dpp_add_from<0x114, 0xF>(x);   // row_shr:4
    x = dpp_add_from<0x118, 0xF>(x);   // row_shr:8
    x = dpp_add_from<0x142, 0xA>(x);   // row_bcast:15
    x = dpp_add_from<0x143, 0xC>(x);   // row_bcast:31
    return x;
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Element traits.  bf16 travels as its 16-bit pattern (uint16_t); widening is a
// shift, narrowing is the hardware round-to-nearest-even conversion.
template <typename E> struct Elem;

template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
    static __device__ __forceinline__ uint16_t from_f32(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
};

template <> struct Elem<float> {
    static __device__ __forceinline__ float to_f32(float x) { return x; }
    static __device__ __forceinline__ float from_f32(float f) { return f; }
};

// Eight consecutive elements: one MFMA operand fragment of one lane.
template <typename E> struct alignas(16) F8 { E x[8]; };
// Four consecutive elements (half a fragment, or one accumulator row quad).
template <typename E> struct alignas(8) F4 { E x[4]; };

// One 16x16 output tile step over 32 values of the contraction index:
//   C[m][n] += sum_k A[m][k] B[k][n]
// Lane l supplies row m = l % 16 of A and column n = l % 16 of B, each with the
// eight contraction slots of lane group l / 16; A and B must fill the same slot
// with the same contraction index.  The accumulator holds C[4*(l/16) + r][l % 16].
// bf16 uses one v_mfma_f32_16x16x32_bf16; float uses eight v_mfma_f32_16x16x4_f32,
// slot s of every lane feeding step s, so no value is ever rounded below fp32.
__device__ __forceinline__ f32x4_t mma(const F8<uint16_t>& a, const F8<uint16_t>& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma(const F8<float>& a, const F8<float>& b, f32x4_t c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[s], b.x[s], c, 0, 0, 0);
    return c;
}

template <typename E>
__device__ __forceinline__ F8<E> zero8() {
    F8<E> r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.x[i] = E(0);
    return r;
}

template <typename E>
__device__ __forceinline__ F8<E> lds_f8(const E* p) { return *reinterpret_cast<const F8<E>*>(p); }

// One fragment from global memory, plain or non-temporal (NT: the data is not expected to
// be read again while it could still be in the caches).
template <bool NT, typename E>
__device__ __forceinline__ F8<E> global_f8(const E* p) {
    if constexpr (!NT) {
        return *reinterpret_cast<const F8<E>*>(p);
    } else {
        constexpr int NV = int(sizeof(F8<E>)) / 16;
        f32x4_t v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + i);
        return __builtin_bit_cast(F8<E>, v);
    }
}

template <typename E>
__device__ __forceinline__ F4<E> lds_f4(const E* p) { return *reinterpret_cast<const F4<E>*>(p); }

template <typename E>
__device__ __forceinline__ F8<E> join(const F4<E>& lo, const F4<E>& hi) {
    F8<E> r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r.x[i] = lo.x[i]; r.x[4 + i] = hi.x[i]; }
    return r;
}

}  // namespace linattn
