// Device-side helpers shared by the prefill and decode kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

constexpr int kDqk = 192;  // q/k head size
constexpr int kDv = 128;   // v head size
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Reductions across lane pairs (lane, lane ^ 32) and (lane, lane ^ 16) with the gfx950
// lane-swap instructions: after v_permlane32_swap(x, x) one result holds x of the lower
// half and the other x of the upper half in every lane, so combining the two results
// combines each lane with its partner.
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Pack two floats to two bf16 (round to nearest even, v_cvt_pk_bf16_f32): lo = a, hi = b.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Byte-select of two dwords (v_perm_b32): result byte i = sel byte i over {hi:lo} bytes
// numbered lo.b0..b3 = 0..3, hi.b0..b3 = 4..7.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
// {lo16(a), lo16(b)} and {hi16(a), hi16(b)}
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// Transpose an 8x8 block of 16-bit values held as r[e] = row e (8 values, 4 dwords):
// returns w[d] = column d = { r[0][d], r[1][d], ..., r[7][d] }.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 r[8], u32x4 w[8]) {
#pragma unroll
    for (int dp = 0; dp < 4; ++dp) {  // dword dp of each row holds columns 2dp, 2dp+1
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // output dword k holds rows 2k, 2k+1
            w[2 * dp][k] = lo_halves(r[2 * k][dp], r[2 * k + 1][dp]);
            w[2 * dp + 1][k] = hi_halves(r[2 * k][dp], r[2 * k + 1][dp]);
        }
    }
}

}  // namespace sinkattn
