// The steps on the near side of the attention ("MiMo-V2-Flash 模型架构深度拆解", CH 10.3
// forward steps 3-6): partial rotary position embedding of q and k, and writing the new
// tokens' keys and values into the KV cache (ring slots or pages, bf16 or E4M3).
//
// Both are elementwise and memory-bound: each element is read and written once, in 16-byte
// pieces.
#include "common.h"
#include "launch.h"
#include "rope.h"

namespace sinkattn {

namespace {

// Rotation task c (0..3) of one 192-wide row: dimensions 8c .. 8c+7 turn with 32 + 8c ..
// 32 + 8c + 7 (pairs i = 8c + e), two 16-byte loads and two 16-byte stores; results rounded
// to bf16 (nearest even).  src and dst may be the same row.
__device__ __forceinline__ void rope_task(const uint16_t *src, uint16_t *dst, int c, const float *cs, const float *sn,
                                          u32x4 &lo_out, u32x4 &hi_out) {
    const u32x4 lo = ldg16(src + 8 * c), hi = ldg16(src + kRopePairs + 8 * c);
    rope_rotate8(lo, hi, 8 * c, cs, sn, lo_out, hi_out);
    if (dst) {
        *reinterpret_cast<u32x4 *>(dst + 8 * c) = lo_out;
        *reinterpret_cast<u32x4 *>(dst + kRopePairs + 8 * c) = hi_out;
    }
}

// One workgroup per (sequence, row): the row's 32 angles once, then one thread per (head,
// rotation task): 16-byte loads and stores.  The 128 trailing dimensions are not touched.
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
    __shared__ float cs[kRopePairs], sn[kRopePairs];
    const int r = blockIdx.x, b = blockIdx.y;
    const int pos = (p.seq_lens ? p.seq_lens[b] - p.rows : p.pos0) + r;
    rope_angles(p.inv_freq, pos, cs, sn);
    __syncthreads();
    for (int task = threadIdx.x; task < p.heads * 4; task += blockDim.x) {
        const int h = task >> 2, c = task & 3;
        uint16_t *x = p.x + (((size_t)b * p.heads + h) * p.rows + r) * kDqk;
        u32x4 lo, hi;
        rope_task(x, x, c, cs, sn, lo, hi);
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

// Cache row (in units of one key, for KV head 0) of position pos of sequence b with n tokens,
// or -1 when the position is not written: before the sequence, overwritten in a ring by a
// later token of the same call, or a page id outside the pool.
__device__ __forceinline__ int64_t cache_row(const AppendParams &p, int b, int n, int pos) {
    if (pos < 0) return -1;
    if (!p.paged) {
        if (pos < n - p.window) return -1;
        return ((int64_t)b * p.hkv) * p.window + pos % p.window;
    }
    if (pos / p.page_size >= p.max_pages) return -1;
    const int page = p.block_table[(size_t)b * p.max_pages + pos / p.page_size];
    if (page < 0 || page >= p.num_pages) return -1;
    return ((int64_t)page * p.hkv) * p.page_size + pos % p.page_size;
}

// 16 bytes of bf16 (8 elements) into the cache at element offset `elem`, as bf16 or as E4M3
// codes of value / scale.
__device__ __forceinline__ void cache_store(const AppendParams &p, bool isk, size_t elem, u32x4 v) {
    if (p.fp8) {
        uint8_t *dst = (isk ? p.k_cache8 : p.v_cache8) + elem;
        *reinterpret_cast<u32x2 *>(dst) = bf16x8_to_e4m3(v, isk ? p.k_scale : p.v_scale);
    } else {
        *reinterpret_cast<u32x4 *>((isk ? p.k_cache : p.v_cache) + elem) = v;
    }
}

// The decode prologue in one pass ("MiMo-V2-Flash 模型架构深度拆解", CH 10.3 forward steps 3-6):
// one workgroup per (sequence, new token, KV head) computes the token's 32 rotary angles,
// then rotates the rows of the KV head's query heads into q_out, rotates the new key row and
// writes it with the value row into the cache (bf16 or E4M3), all in 16-byte pieces: at one
// new token and 8 query heads per KV head that is one piece per thread.  The rotated keys are
// rounded to bf16 before an 8-bit cache encodes them, as a separate rotation and append would.
__global__ __launch_bounds__(256) void decode_prologue_kernel(PrologueParams pp) {
    __shared__ float cs[kRopePairs], sn[kRopePairs];
    const AppendParams &p = pp.a;
    const int t = blockIdx.x, b = blockIdx.y, g = blockIdx.z;
    const int G = pp.hq / p.hkv;
    const int n = p.seq_lens[b];
    const int pos = n - p.n_new + t;
    rope_angles(pp.inv_freq, pos, cs, sn);
    const int64_t row = cache_row(p, b, n, pos);
    const size_t head_rows = p.paged ? (size_t)p.page_size : (size_t)p.window;
    __syncthreads();
    constexpr int kCopy = (kDqk - kRopeDims) / 8;  // 16 plain 16-byte pieces of a q or k row
    const bool q_copy = pp.q_out != pp.q_in;
    const int nq = G * (4 + (q_copy ? kCopy : 0));  // tasks: this KV head's query rows
    const int nk = 4 + kCopy;                       // its rotated key row
    const int nv = kDv / 8;                         // its value row
    const int total = nq + (row >= 0 ? nk + nv : 0);
    for (int task = threadIdx.x; task < total; task += blockDim.x) {
        if (task < nq) {
            const int per = 4 + (q_copy ? kCopy : 0);
            const int h = g * G + task / per, c = task % per;
            const size_t off = (((size_t)b * pp.hq + h) * p.n_new + t) * kDqk;
            if (c < 4) {
                u32x4 lo, hi;
                rope_task(pp.q_in + off, pp.q_out + off, c, cs, sn, lo, hi);
            } else {
                const int e = kRopeDims + 8 * (c - 4);
                *reinterpret_cast<u32x4 *>(pp.q_out + off + e) = ldg16(pp.q_in + off + e);
            }
        } else if (task < nq + nk) {
            const int h = g, c = task - nq;
            const uint16_t *src = p.k_new + (((size_t)b * p.hkv + h) * p.n_new + t) * kDqk;
            const size_t dst = ((size_t)row + h * head_rows) * kDqk;
            if (c < 4) {
                u32x4 lo, hi;
                rope_task(src, nullptr, c, cs, sn, lo, hi);
                cache_store(p, true, dst + 8 * c, lo);
                cache_store(p, true, dst + kRopePairs + 8 * c, hi);
            } else {
                const int e = kRopeDims + 8 * (c - 4);
                cache_store(p, true, dst + e, ldg16(src + e));
            }
        } else {
            const int h = g, c = task - nq - nk;
            const uint16_t *src = p.v_new + (((size_t)b * p.hkv + h) * p.n_new + t) * kDv;
            cache_store(p, false, ((size_t)row + h * head_rows) * kDv + 8 * c, ldg16(src + 8 * c));
        }
    }
}

}  // namespace

int launch_decode_prologue(const PrologueParams &prm, hipStream_t stream) {
    PrologueParams p = prm;
    void *args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(&decode_prologue_kernel),
                           dim3(p.a.n_new, p.a.batch, p.a.hkv), dim3(256), args, 0, stream) == hipSuccess
               ? 0
               : -1;
}

int launch_rope(const RopeParams &prm, hipStream_t stream) {
    RopeParams p = prm;
    void *args[] = {&p};
    const dim3 grid(p.rows, p.batch);
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
