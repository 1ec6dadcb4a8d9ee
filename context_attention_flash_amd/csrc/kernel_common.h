// Device helpers shared by the HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D = A * B + C on a 32x32x16 bf16 tile.  Lane l holds, for A (32 x 16):
// row l%32, k = 8*(l/32) .. +7; for B (16 x 32): column l%32, the same k; for
// C/D: column l%32, rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap(x, x) returns
// two registers: the first holds x[l] on lanes 0-31 and x[l-32] on lanes
// 32-63, the second x[l+32] on lanes 0-31 and x[l] on lanes 32-63; combining
// the two gives the pair reduction on every lane.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                              __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                              __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Plan arrays (tile lists, orders) are never written while a kernel runs; reading
// them through the constant address space lets uniform indices use scalar
// loads, which do not wait behind outstanding vector memory operations.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ cint_ptr as_const(const int32_t* p) { return (cint_ptr)(p); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Blocks of a launch are dealt to the 8 XCDs round-robin; this remaps the
// block index so that each XCD receives one contiguous range of work items
// (neighbouring items share K/V and therefore that XCD's L2).  grid % 8 == 0.
__device__ __forceinline__ int xcd_work_index(int bid, int grid) {
    return (bid & 7) * (grid >> 3) + (bid >> 3);
}

}  // namespace ra
