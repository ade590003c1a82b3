// Partial rotary position embedding of a 192-wide q or k row ("MiMo-V2-Flash 模型架构深度拆解",
// CH 10.3: the first 64 dimensions rotate, the other 128 do not; "MiMo-V2-Flash 架构 QA", Q2.7:
// pair i turns by pos * theta^(-2i/64)).  Pair i is dimensions i and i + 32.  Shared by the
// prologue kernels and the fused decode step, so that both round identically.
#pragma once

#include "common.h"

namespace sinkattn {

constexpr int kRopeDims = 64;  // rotated leading dimensions of the 192
constexpr int kRopePairs = kRopeDims / 2;
constexpr double kTwoPi = 6.283185307179586;

// cos and sin of pos * theta^(-2i/64) for the 32 pairs, into LDS (threads 0..31).  The angle
// is formed and reduced to [-pi, pi] in double precision (a position near 262144 times a
// frequency near 1 would lose about 0.02 rad in float), then its sine and cosine are taken
// in float.
__device__ __forceinline__ void rope_angles(const double *inv_freq, int pos, float *cs, float *sn) {
    const int i = threadIdx.x;
    if (i < kRopePairs) {
        double ang = (double)pos * inv_freq[i];
        ang -= kTwoPi * __builtin_rint(ang / kTwoPi);
        sincosf((float)ang, &sn[i], &cs[i]);
    }
}

// Pairs i0 .. i0 + 7: lo holds dimensions i0 .. i0 + 7 and hi dimensions 32 + i0 .. 32 + i0 + 7
// (bf16); the rotated values x cos - y sin and y cos + x sin (float32, one rounded product and
// one fused multiply-add each), rounded to bf16 (nearest even), in the same places.
__device__ __forceinline__ void rope_rotate8(u32x4 lo, u32x4 hi, int i0, const float *cs, const float *sn,
                                             u32x4 &lo_out, u32x4 &hi_out) {
    uint32_t rl[4], rh[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float ro[2], rp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = i0 + 2 * w + h;
            const float a = __builtin_bit_cast(float, h ? (lo[w] & 0xffff0000u) : (lo[w] << 16));
            const float b = __builtin_bit_cast(float, h ? (hi[w] & 0xffff0000u) : (hi[w] << 16));
            // explicit fused multiply-adds: every kernel that rotates rounds the same way
            // (left to contraction, the compiler may fuse either product)
            ro[h] = __builtin_fmaf(a, cs[i], -(b * sn[i]));
            rp[h] = __builtin_fmaf(b, cs[i], a * sn[i]);
        }
        rl[w] = pack_bf16x2(ro[0], ro[1]);
        rh[w] = pack_bf16x2(rp[0], rp[1]);
    }
    lo_out = u32x4{rl[0], rl[1], rl[2], rl[3]};
    hi_out = u32x4{rh[0], rh[1], rh[2], rh[3]};
}

}  // namespace sinkattn
