// The steps on the near side of the attention ("MiMo-V2-Flash 模型架构深度拆解", CH 10.3
// forward steps 3-6): partial rotary position embedding of q and k, and writing the new
// tokens' keys and values into the KV cache (ring slots or pages, bf16 or E4M3).
//
// Both are elementwise and memory-bound: each element is read and written once with 16-byte
// (append) or coalesced 2-byte (rotation) accesses.
#include "common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kRopeDims = 64;            // rotated leading dimensions of the 192
constexpr int kRopePairs = kRopeDims / 2;
constexpr int kRopeRowsPerBlock = 8;     // 8 rows x 32 pairs = 256 threads
constexpr double kTwoPi = 6.283185307179586;

// One thread per (sequence, row, pair i); it turns dimensions i and i + 32 of that row in
// every head by pos * theta^(-2i/64).  The angle is formed and reduced to [-pi, pi] in double
// precision (a position near 262144 times a frequency near 1 would lose about 0.02 rad in
// float), then its sine and cosine are taken in float.
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
    const int i = threadIdx.x & (kRopePairs - 1);
    const int r = blockIdx.x * kRopeRowsPerBlock + (threadIdx.x >> 5);
    const int b = blockIdx.y;
    if (r >= p.rows) return;
    const int pos = (p.seq_lens ? p.seq_lens[b] - p.rows : p.pos0) + r;
    double ang = (double)pos * p.inv_freq[i];
    ang -= kTwoPi * __builtin_rint(ang / kTwoPi);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    uint16_t *x = p.x + (((size_t)b * p.heads) * p.rows + r) * kDqk;
    const size_t head_stride = (size_t)p.rows * kDqk;
    for (int h = 0; h < p.heads; ++h, x += head_stride) {
        const float a = __builtin_bit_cast(float, (uint32_t)x[i] << 16);
        const float c = __builtin_bit_cast(float, (uint32_t)x[i + kRopePairs] << 16);
        const uint32_t pk = pack_bf16x2(a * cs - c * sn, c * cs + a * sn);
        x[i] = (uint16_t)(pk & 0xffffu);
        x[i + kRopePairs] = (uint16_t)(pk >> 16);
    }
}

// 16 bytes of bf16 -> 8 E4M3 codes of value / scale (round to nearest even, clamped to the
// largest finite code 448).
__device__ __forceinline__ u32x2 bf16x8_to_e4m3(u32x4 v, float scale) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
        f[2 * e] = __builtin_bit_cast(float, w << 16);
        f[2 * e + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = fminf(fmaxf(f[e] / scale, -448.f), 448.f);  // IEEE division
    uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], (int)lo, true);
    uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], (int)hi, true);
    return u32x2{lo, hi};
}

// One workgroup per (sequence, new token): its K rows (hkv x 192) and V rows (hkv x 128)
// move in 16-byte pieces (8 elements) to the cache row of the token's position.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
    const int t = blockIdx.x, b = blockIdx.y;
    const int n = p.seq_lens[b];
    const int pos = n - p.n_new + t;
    if (pos < 0) return;
    size_t row;  // cache row (in units of one key) of this position for KV head 0
    if (!p.paged) {
        if (pos < n - p.window) return;  // overwritten by a later token of this call
        row = ((size_t)b * p.hkv) * p.window + pos % p.window;
    } else {
        if (pos / p.page_size >= p.max_pages) return;
        const int page = p.block_table[(size_t)b * p.max_pages + pos / p.page_size];
        if (page < 0 || page >= p.num_pages) return;
        row = ((size_t)page * p.hkv) * p.page_size + pos % p.page_size;
    }
    const size_t head_rows = p.paged ? (size_t)p.page_size : (size_t)p.window;
    constexpr int kK16 = kDqk / 8, kV16 = kDv / 8;  // 16-byte pieces per row
    const int total = p.hkv * (kK16 + kV16);
    for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
        const bool isk = idx < p.hkv * kK16;
        const int j = isk ? idx : idx - p.hkv * kK16;
        const int per = isk ? kK16 : kV16, width = isk ? kDqk : kDv;
        const int h = j / per, c = j % per;
        const uint16_t *src = (isk ? p.k_new : p.v_new) + (((size_t)b * p.hkv + h) * p.n_new + t) * width + 8 * c;
        const u32x4 v = ldg16(src);
        const size_t dst_elem = (row + h * head_rows) * width + 8 * c;
        if (p.fp8) {
            uint8_t *dst = (isk ? p.k_cache8 : p.v_cache8) + dst_elem;
            *reinterpret_cast<u32x2 *>(dst) = bf16x8_to_e4m3(v, isk ? p.k_scale : p.v_scale);
        } else {
            uint16_t *dst = (isk ? p.k_cache : p.v_cache) + dst_elem;
            *reinterpret_cast<u32x4 *>(dst) = v;
        }
    }
}

}  // namespace

int launch_rope(const RopeParams &prm, hipStream_t stream) {
    RopeParams p = prm;
    void *args[] = {&p};
    const dim3 grid((p.rows + kRopeRowsPerBlock - 1) / kRopeRowsPerBlock, p.batch);
    return hipLaunchKernel(reinterpret_cast<const void *>(&rope_kernel), grid, dim3(256), args, 0, stream) ==
                   hipSuccess
               ? 0
               : -1;
}

int launch_kv_append(const AppendParams &prm, hipStream_t stream) {
    AppendParams p = prm;
    void *args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(&kv_append_kernel), dim3(p.n_new, p.batch), dim3(256), args,
                           0, stream) == hipSuccess
               ? 0
               : -1;
}

}  // namespace sinkattn
