// bi_common.hpp -- helpers shared by the HIP kernels of libbi.so (gfx950 only).
//
// Numerics policy for every kernel in the library (it is what makes "the same
// source expression gives the same bits" hold across kernels):
//   * built with -ffp-contract=off and without fast-math: every + and * is an
//     IEEE operation rounded on its own; fused multiply-adds appear only where
//     written explicitly with __fmaf_rn;
//   * fp32 -> bf16 is round-to-nearest-even by the gfx950 instruction
//     v_cvt_pk_bf16_f32 (two values per instruction); compared on the device
//     against round-to-nearest-even done on the bit pattern for all 2^32 fp32
//     inputs: identical, NaNs included (a NaN keeps its sign and top payload
//     bits and comes out quiet);
//   * exp2 is the hardware v_exp_f32 (one instruction, deterministic);
//   * no atomics anywhere: every reduction has one fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bi.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h16)
{
    return __uint_as_float(h16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ u32x4 zero_u32x4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One 16x16x32 bf16 MFMA: D = A*B + C.  Lane l supplies A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16], j = 0..7, and holds D[4(l/16)+r][l%16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- host side
static inline bool bi_aligned(const void* p, uintptr_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }

static inline int bi_launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

#define BI_TRY_BEGIN try {
#define BI_TRY_END } catch (...) { return BI_ERR_LAUNCH; }
