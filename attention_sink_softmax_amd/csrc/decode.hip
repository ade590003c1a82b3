// Decode kernels: one new query token per sequence against a sliding-window ring cache or a
// paged cache, with a per-head sink term in the softmax denominator, for gfx950.
//
// Decode is bound by reading the KV cache (paper-notes page "MiMo-V2-Flash Technical
// Report", §1.1: at long context the decode step is limited by KV-read bandwidth).  The key
// range of each (sequence, KV head) is split across workgroups so that even 8 sequences
// fill 256 CUs; every split produces unnormalised partial results (running max m, sum l,
// and o = sum of exp(a - m) v) and a second kernel merges them.  The sink term
// exp(sink - M) enters exactly once, in that merge (or in the single-split epilogue), as
// the sink softmax of "MiMo-V2-Flash 架构 QA" Q3.8 requires.
//
// Work of one workgroup (4 waves): keys are taken 128 at a time, 32 per wave.  The G query
// heads that share the KV head (up to 16) form the N dimension of
// v_mfma_f32_16x16x32_bf16, so every key byte read from HBM serves all of them:
//   S^T[16 keys][16 heads] = K Q^T    K straight from global memory into the A operand,
//                                     Q^T held in registers;
//   O^T[16 dv][16 heads]  += V^T P^T  P^T is the score tile itself (same lane layout),
//                                     V^T is V transposed in registers (8x8 bf16 blocks)
//                                     and staged through a per-wave LDS tile.
// Row statistics need two lane exchanges (xor 16, xor 32).  At the end the 4 waves'
// states are merged through LDS.
#include "common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerWave = 32;
constexpr int kBlock = kWaves * kKeysPerWave;  // keys per workgroup iteration
constexpr int kPart = kDv + 4;                  // partial record: o[128], m, l, 2 pad (16-byte rows)

// Per-wave V^T tile [128 dv][32 keys]: 4 chunks of 8 keys per row, chunk c stored at
// c ^ ((r >> 2) & 3) so the 16 rows of one MFMA operand read hit distinct banks.
__device__ __forceinline__ int vt_off(int row, int chunk) { return row * 32 + ((chunk ^ (row >> 2)) & 3) * 8; }

// Key (0..31 within the wave's slice) supplied as element e by k-group q of the PV product:
// the 16x16 MFMA output gives lane group q the rows 4q..4q+3 of each 16-key score tile, and
// the two tiles' registers are concatenated into one 32-key k-step.
__device__ __forceinline__ int vkey(int q, int e) { return (e < 4) ? (4 * q + e) : (16 + 4 * q + (e - 4)); }

struct KeyAddr {
    const uint16_t *k;  // row of d_qk values, or nullptr when the key is not readable
    const uint16_t *v;
    bool bad;           // page id outside the pool
};

// Address of visible key number j (0-based within [kbeg, kend)) of sequence b.
__device__ __forceinline__ KeyAddr key_addr(const DecodeParams &p, int b, int kvh, int j) {
    KeyAddr a{nullptr, nullptr, false};
    if (!p.paged) {
        // ring: the visible keys are slots 0..min(n, W)-1 (position p lives in slot p mod W,
        // and the W most recent positions occupy distinct slots)
        const size_t row = ((size_t)b * p.Hkv + kvh) * p.window + j;
        a.k = p.k + row * kDqk;
        a.v = p.v + row * kDv;
        return a;
    }
    const int page = p.block_table[(size_t)b * p.max_pages + j / p.page_size];
    if (page < 0 || page >= p.num_pages) {
        a.bad = true;
        return a;
    }
    const size_t row = ((size_t)page * p.Hkv + kvh) * p.page_size + (j % p.page_size);
    a.k = p.k + row * kDqk;
    a.v = p.v + row * kDv;
    return a;
}

__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kWaves][kDv * kKeysPerWave];
    __shared__ float red_m[kWaves][16], red_l[kWaves][16];

    const int split = blockIdx.x;
    const int kvh = blockIdx.y % p.Hkv, hc = blockIdx.y / p.Hkv;
    const int b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hl = lane & 15, q = lane >> 4;  // head column, k-group
    const int hidx = hc * 16 + hl;            // head within the KV group
    const bool head_ok = hidx < p.G;
    const int h = kvh * p.G + hidx;

    const int n = p.seq_lens[b];
    // visible keys: positions [max(0, n-W), n) (sliding) or [0, n) (global); the ring
    // enumerates them as slots [0, min(n, W))
    int kbeg, kend;
    if (!p.paged) {
        kbeg = 0;
        kend = min(n, p.window);
    } else {
        kbeg = p.swa ? max(0, n - p.window) : 0;
        kend = n;
    }
    const bool seq_ok = n >= 1 && n <= p.max_seq_len && (!p.paged || n <= p.max_pages * p.page_size);
    const int s_lo = kbeg + split * p.chunk;
    const int s_hi = seq_ok ? min(kend, s_lo + p.chunk) : s_lo;  // empty when the length is invalid

    // Q^T fragments: lane supplies q[h][32kk + 8q .. +8]
    bf16x8 qf[6];
    {
        const uint16_t *qrow = p.q + ((size_t)b * p.Hq + (head_ok ? h : 0)) * kDqk + 8 * q;
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) qf[kk] = as_bf16x8(head_ok ? ldg16(qrow + 32 * kk) : u32x4{0, 0, 0, 0});
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = false;
    uint16_t *vt = Vt[wave];

    for (int blk = s_lo; blk < s_hi; blk += kBlock) {
        const int w0 = blk + kKeysPerWave * wave;  // first key of this wave's slice
        // ---- K operand: two 16-key tiles, lane key = w0 + 16*sb + hl, d chunk 8q + 32kk
        bf16x8 kf[2][6];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int j = w0 + 16 * sb + hl;
            const bool in = j < s_hi;
            const KeyAddr a = in ? key_addr(p, b, kvh, j) : KeyAddr{nullptr, nullptr, false};
            bad |= a.bad;
            const bool rd = in && !a.bad;
#pragma unroll
            for (int kk = 0; kk < 6; ++kk)
                kf[sb][kk] = as_bf16x8(rd ? ldg16(a.k + 32 * kk + 8 * q) : u32x4{0, 0, 0, 0});
        }
        // ---- V: lane owns k-group kq (8 keys) x dv chunk c (8 values); transpose into LDS
        {
            const int kq = lane & 3, c = lane >> 2;
            u32x4 r[8], w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = w0 + vkey(kq, e);
                const bool in = j < s_hi;
                const KeyAddr a = in ? key_addr(p, b, kvh, j) : KeyAddr{nullptr, nullptr, false};
                r[e] = (in && !a.bad) ? ldg16(a.v + 8 * c) : u32x4{0, 0, 0, 0};
            }
            transpose8x8_b16(r, w);
#pragma unroll
            for (int d = 0; d < 8; ++d) *reinterpret_cast<u32x4 *>(&vt[vt_off(8 * c + d, kq)]) = w[d];
        }
        // ---- scores
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 6; ++kk)
                s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[sb][kk], qf[kk], s[sb], 0, 0, 0);
        }
        // lane holds keys w0 + 16sb + 4q + i for head hl
        float x[8];
        float mx = m_run;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = w0 + 16 * sb + 4 * q + i;
                const float v = j < s_hi ? s[sb][i] * p.scale_log2 : -INFINITY;
                x[4 * sb + i] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = fmaxf(mx, xor16(mx));
        mx = fmaxf(mx, xor32(mx));
        const float mu = (mx == -INFINITY) ? 0.f : mx;
        const float alpha = exp2f_fast(m_run - mu);
        m_run = mx;
        float ps = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p0 = exp2f_fast(x[2 * i] - mu), p1 = exp2f_fast(x[2 * i + 1] - mu);
            ps += p0 + p1;
            pk[i] = pack_bf16x2(p0, p1);
        }
        l_run = l_run * alpha + ps;
        const bf16x8 pf = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&vt[vt_off(16 * db + hl, q)]);
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[db] * alpha, 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- merge the 4 waves' states through LDS (reusing the V tiles as float storage)
    float lsum = l_run + xor16(l_run);
    lsum += xor32(lsum);
    const bool any_bad = __syncthreads_or(bad) != 0;
    float *ob = reinterpret_cast<float *>(&Vt[0][0]);  // [4 waves][16 heads][128 dv] floats = 32 KB
    if (q == 0) {
        red_m[wave][hl] = m_run;
        red_l[wave][hl] = lsum;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[(wave * 16 + hl) * kDv + 16 * db + 4 * q + i] = acc[db][i];
    __syncthreads();

    // thread -> (head hh, 8 dv values)
    const int hh = tid >> 4, d0 = (tid & 15) * 8;
    const int hidx2 = hc * 16 + hh;
    if (hidx2 >= p.G) return;
    const int h2 = kvh * p.G + hidx2;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float sc = exp2f_fast(red_m[w][hh] - Mu);
        L += sc * red_l[w][hh];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] += sc * ob[(w * 16 + hh) * kDv + d0 + i];
    }

    if (p.nsplit == 1) {
        // final output: add the sink term once, normalise, round to bf16
        uint16_t *orow = p.out + ((size_t)b * p.Hq + h2) * kDv + d0;
        float res[8];
        if (n <= 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) res[i] = 0.f;
        } else if (!seq_ok || any_bad) {
#pragma unroll
            for (int i = 0; i < 8; ++i) res[i] = __builtin_nanf("");
        } else {
            const float sk = p.sink ? p.sink[h2] : -INFINITY;
            if (sk == INFINITY) {
#pragma unroll
                for (int i = 0; i < 8; ++i) res[i] = 0.f;
            } else {
                const float sl = sk * kLog2e;
                const float M2 = fmaxf(M, sl);
                const float sc = exp2f_fast(M - M2);
                const float Lt = L * sc + (sk == -INFINITY ? 0.f : exp2f_fast(sl - M2));
                const float inv = 1.f / Lt;
#pragma unroll
                for (int i = 0; i < 8; ++i) res[i] = o[i] * sc * inv;
            }
        }
        *reinterpret_cast<u32x4 *>(orow) = u32x4{pack_bf16x2(res[0], res[1]), pack_bf16x2(res[2], res[3]),
                                                 pack_bf16x2(res[4], res[5]), pack_bf16x2(res[6], res[7])};
    } else {
        float *rec = p.ws + (((size_t)b * p.Hq + h2) * p.nsplit + split) * kPart;
#pragma unroll
        for (int i = 0; i < 8; i += 4) *reinterpret_cast<f32x4 *>(rec + d0 + i) = f32x4{o[i], o[i + 1], o[i + 2], o[i + 3]};
        if ((tid & 15) == 0) {
            rec[kDv] = M;
            rec[kDv + 1] = any_bad ? __builtin_nanf("") : L;
        }
    }
}

// One wave per (sequence, query head): merge the splits' partials and add the sink once.
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
    const int bh = blockIdx.x;
    const int b = bh / p.Hq, h = bh % p.Hq;
    const int lane = threadIdx.x;
    const int n = p.seq_lens[b];
    uint16_t *orow = p.out + (size_t)bh * kDv + 2 * lane;
    const bool seq_ok = n >= 1 && n <= p.max_seq_len && (!p.paged || n <= p.max_pages * p.page_size);
    if (n <= 0 || !seq_ok) {
        const float z = n <= 0 ? 0.f : __builtin_nanf("");
        *reinterpret_cast<uint32_t *>(orow) = pack_bf16x2(z, z);
        return;
    }
    const int kbeg = p.paged ? (p.swa ? max(0, n - p.window) : 0) : 0;
    const int kend = p.paged ? n : min(n, p.window);
    const int used = (kend - kbeg + p.chunk - 1) / p.chunk;  // splits that saw keys
    const float *base = p.ws + (size_t)bh * p.nsplit * kPart;

    const float sk = p.sink ? p.sink[h] : -INFINITY;
    const bool sink_inf = sk == INFINITY;
    const float sl = (sink_inf ? -INFINITY : sk) * kLog2e;  // an infinite sink is applied at the end
    float M = sl;
    for (int s = lane; s < used; s += 64) M = fmaxf(M, base[(size_t)s * kPart + kDv]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = (sl == -INFINITY) ? 0.f : exp2f_fast(sl - Mu);
    float o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < used; ++s) {
        const float *rec = base + (size_t)s * kPart;
        const float sc = exp2f_fast(rec[kDv] - Mu);
        L += sc * rec[kDv + 1];  // a NaN sum marks an unreadable page and poisons L
        o0 += sc * rec[2 * lane];
        o1 += sc * rec[2 * lane + 1];
    }
    float r0 = o0 / L, r1 = o1 / L;
    if (sink_inf && !__builtin_isnan(L)) r0 = r1 = 0.f;
    *reinterpret_cast<uint32_t *>(orow) = pack_bf16x2(r0, r1);
}

}  // namespace

int launch_decode(const DecodeParams &prm, hipStream_t stream) {
    DecodeParams p = prm;
    void *args[] = {&p};
    const dim3 grid(p.nsplit, p.Hkv * p.hchunks, p.B);
    if (hipLaunchKernel(reinterpret_cast<const void *>(&decode_split_kernel), grid, dim3(256), args, 0, stream) !=
        hipSuccess)
        return -1;
    if (p.nsplit > 1) {
        if (hipLaunchKernel(reinterpret_cast<const void *>(&decode_merge_kernel), dim3(p.B * p.Hq), dim3(64), args, 0,
                            stream) != hipSuccess)
            return -1;
    }
    return 0;
}

}  // namespace sinkattn
