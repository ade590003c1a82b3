// Backward of prefill attention with a per-head sink, for gfx950.
//
// With the forward weights recomputed from the saved log-sum-exp, P_ij = exp(a_ij - LSE_i), the
// sink's weight exp(sink - LSE_i), and dO the gradient of the output:
//   D_i = dO_i . O_i   dS_ij = P_ij (dO_i . v_j - D_i)   dq = scale dS k   dk = scale dS^T q
//   dv = P^T dO        dsink_h = -sum_i exp(sink_h - LSE_i) D_i
// (the sink enters the outputs only through the shared softmax denominator and has no value
// vector: "MiMo-V2-Flash 架构 QA", Q3.8; it is a learnable per-head scalar: "MiMo-V2-Flash 模型
// 架构深度拆解", CH 10.1).
//
// Four kernels on one stream:
//   bwd_pre     D_i and the per-block partial sums of the sink gradient;
//   bwd_dkdv    one workgroup per 128 keys of a (sequence, KV head): each wave keeps its 32 keys'
//               K and V operands and its dK, dV accumulators in registers and walks every query
//               head of the group and every 32-row query tile that sees its keys:
//                 S = Q K^T, dP = dO V^T (query rows x keys), dS = P (dP - D),
//                 dV += P^T dO, dK += dS^T Q       (P and dS feed the A operand as they are;
//                                                    dO and Q arrive through transposing reads);
//   bwd_dq      one workgroup per 32 query rows of four query heads of one KV head: each wave
//               keeps its head's Q and dO operands and dQ^T in registers and walks the key tiles:
//                 S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T;
//   bwd_dsink   sums the sink gradient partials in a fixed order (deterministic).
// All products are v_mfma_f32_32x32x16_bf16 with float32 accumulation; P and dS enter them as
// bf16.  Tiles pass through double-buffered LDS (one barrier per tile) with their 16-byte
// chunks XOR-swizzled by row so that both the row reads and the transposing reads spread over
// the banks.  Masking is branch-free and only runs on tiles that cross the causal diagonal, the
// window's edge or the sequence end.
#include "common.h"
#include "launch.h"

namespace sinkattn {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Tiles travel HBM -> LDS with 16-byte (4-byte for row statistics) buffer loads that write
// LDS directly: lane l of one instruction fills bytes 16 l .. 16 l + 15 of a 1 KB block, so
// each lane fetches the global chunk that the swizzled layout puts there.  A buffer region
// covers one (sequence, head) matrix; offsets past its end read zeros, which pads the last
// tile of a sequence.
constexpr int kRawDword3 = 0x00020000;  // untyped 32-bit data, no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region(const void *base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRawDword3);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

constexpr int kQT = 32;                    // query rows per tile
constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWg = 4 * kKeysPerWave;  // bwd_dkdv
constexpr int kKT = 64;                    // keys per tile in bwd_dq
constexpr int kPreRows = 16;               // rows per bwd_pre workgroup

// Byte offset of 16-byte chunk c of row r: rows of 192 (384 B) and of 128 (256 B) elements.
// The chunk index is XORed with swz(r), which takes the 8 values 0..7 over any 8 aligned rows
// and 4 values with distinct bits 1-2 over any 4 aligned rows: no two lanes of a 128-byte
// phase of a row read, or of a 16-lane transposing read, share a bank if the banks serve
// 128 bytes per cycle.  The hardware serves 256 bytes per cycle (16 lanes of a row read), and
// its counters show conflicts in 12-15% of cycles here.  A swizzle built for that wider phase
// removed them but made the dQ kernel slower (its addresses took more registers), so this
// one stays.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int off192(int r, int c) { return r * 384 + ((c ^ swz(r)) << 4); }
__device__ __forceinline__ int off128(int r, int c) { return r * 256 + ((c ^ swz(r)) << 4); }

template <int W>
__device__ __forceinline__ int tile_off(int r, int c) {
    if constexpr (W == 192) return off192(r, c);
    else return off128(r, c);
}
// Source offset (bytes, from the tile's first row) of the chunk that lands in 16-byte slot
// `slot` of a swizzled tile of W-element rows.
template <int W>
__device__ __forceinline__ int src_of_slot(int slot) {
    constexpr int kChunks = W / 8;
    const int r = slot / kChunks, c = (slot % kChunks) ^ swz(r);
    return r * (W * 2) + c * 16;
}

// Row m of a 32x32 MFMA result held in register e by lane group g.
__device__ __forceinline__ int mrow(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// 8 elements of column `col0 + (lane & 31)` of a swizzled row-major tile, from rows
// rbase + {4g .. 4g+3} and rbase + 8 + {4g .. 4g+3} (g = lane >> 5): the operand, in the k
// order of a score tile's registers, of a product that contracts over those rows.
template <int W>
__device__ __forceinline__ bf16x8 col_operand(const char *tile, int rbase, int col0, int lane) {
    const int g = lane >> 5, gl = (lane >> 4) & 1, i = lane & 15;
    const int r = i >> 2, c4 = i & 3;
    const int col = col0 + 16 * gl + 4 * c4;
    const int chunk = col >> 3, half = (col >> 2) & 1;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(tile + tile_off<W>(rbase + 4 * g + r, chunk) + 8 * half));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(tile + tile_off<W>(rbase + 8 + 4 * g + r, chunk) + 8 * half));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 8 elements of row rbase + (lane & 31), chunk 2kk + g, of a swizzled row-major tile.
template <int W>
__device__ __forceinline__ bf16x8 row_operand(const char *tile, int rbase, int kk, int lane) {
    return *reinterpret_cast<const bf16x8 *>(tile + tile_off<W>(rbase + (lane & 31), 2 * kk + (lane >> 5)));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// Pack registers e0 .. e0+7 of a score tile to the bf16 operand of one 16-wide k-step.
__device__ __forceinline__ bf16x8 pack8(const f32x16 &x, int e0) {
    return as_bf16x8(u32x4{pack_bf16x2(x[e0], x[e0 + 1]), pack_bf16x2(x[e0 + 2], x[e0 + 3]),
                           pack_bf16x2(x[e0 + 4], x[e0 + 5]), pack_bf16x2(x[e0 + 6], x[e0 + 7])});
}

__device__ __forceinline__ bool visible(const BwdParams &p, int qpos, int key) {
    return qpos < p.L && key <= qpos && (!p.swa || key > qpos - p.window);
}

// True when every (query, key) pair of queries q0 .. q0+31 and keys k0 .. k0+31 is visible.
__device__ __forceinline__ bool all_visible(const BwdParams &p, int q0, int k0) {
    return k0 + 31 <= q0 && q0 + 31 < p.L && (!p.swa || k0 > q0 + 31 - p.window);
}

// ---- D_i = dO_i . O_i and the sink gradient's partial sums
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
    __shared__ float part[256 / 16];
    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
    const int i = blockIdx.x * kPreRows + r;
    float dsum = 0.f;
    if (i < p.L) {
        const size_t row = ((size_t)b * p.Hq + h) * p.L + i;
        const u32x4 o = ldg16(p.out + row * kDv + 8 * c), d = ldg16(p.dout + row * kDv + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dsum += bf16_to_f32(o[e] & 0xffffu) * bf16_to_f32(d[e] & 0xffffu);
            dsum += bf16_to_f32(o[e] >> 16) * bf16_to_f32(d[e] >> 16);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m, 16);
    float contrib = 0.f;
    if (i < p.L && c == 0) {
        const size_t row = ((size_t)b * p.Hq + h) * p.L + i;
        p.delta[row] = dsum;
        if (p.sink) {
            const float sk = p.sink[h];
            // the sink's weight exp(sink - LSE); with a sink of +inf every output is 0 (D = 0)
            if (sk != INFINITY && sk != -INFINITY) contrib = -exp2f_fast((sk - p.lse[row]) * kLog2e) * dsum;
        }
    }
    if (c == 0) part[r] = contrib;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int k = 0; k < 256 / 16; ++k) s += part[k];
        p.dsink_part[((size_t)b * p.Hq + h) * gridDim.x + blockIdx.x] = s;
    }
}

// One workgroup per head: thread t sums the partials t, t + 256, ... of every sequence in a
// fixed order, then a fixed tree adds the 256 sums (the result does not depend on timing).
__global__ __launch_bounds__(256) void bwd_dsink_kernel(BwdParams p, int nblk) {
    __shared__ float part[256];
    const int h = blockIdx.x, tid = threadIdx.x;
    float s = 0.f;
    for (int b = 0; b < p.B; ++b)
        for (int k = tid; k < nblk; k += 256) s += p.dsink_part[((size_t)b * p.Hq + h) * nblk + k];
    part[tid] = s;
    __syncthreads();
#pragma unroll
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) part[tid] += part[tid + w];
        __syncthreads();
    }
    if (tid == 0) p.dsink[h] = part[0];
}

// ---- dK and dV
// LDS tile of one query tile: Q [32][192] (12 KB = 12 blocks of 1 KB), dO [32][128] (8 blocks),
// and the LSE and D of its rows (64 floats each: the 32 rows of the tile and 32 unused).
constexpr int kDkQBytes = kQT * kDqk * 2, kDkOBytes = kQT * kDv * 2;

struct DkTile {
    char *q, *o;
    float *lse, *d;
};

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char qa[kDkQBytes], qb[kDkQBytes], qc[kDkQBytes];
    __shared__ __attribute__((aligned(1024))) char oa[kDkOBytes], ob[kDkOBytes], oc[kDkOBytes];
    __shared__ __attribute__((aligned(256))) float la[64], lb[64], lc[64], da[64], db_[64], dc[64];

    // workgroup -> (key block, sequence, KV head): KV heads vary fastest, so that the
    // workgroups that the hardware places on one XCD (ids equal mod 8) share a KV head, and
    // the key blocks with the most query tiles come first
    int bid = blockIdx.x;
    const int kvh = bid % p.Hkv;
    bid /= p.Hkv;
    const int b = bid % p.B;
    const int kb0 = (bid / p.B) * kKeysPerWg;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int kw0 = kb0 + kKeysPerWave * wave;  // this wave's first key
    const int key = kw0 + n;                    // this lane's key (B-operand column)

    // this wave's K and V rows as the B operands of S = Q K^T and dP = dO V^T
    bf16x8 kB[12], vB[8];
    {
        const bool ok = key < p.L;
        const size_t kr = ((size_t)b * p.Hkv + kvh) * p.L + (ok ? key : 0);
#pragma unroll
        for (int kk = 0; kk < 12; ++kk)
            kB[kk] = as_bf16x8(ok ? ldg16(p.k + kr * kDqk + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            vB[kk] = as_bf16x8(ok ? ldg16(p.v + kr * kDv + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
        // parked in AGPRs (the matrix unit reads them there), leaving the VGPRs to the
        // operands streamed from LDS
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) asm volatile("" : "+a"(kB[kk]));
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+a"(vB[kk]));
    }
    f32x16 dK[6], dV[4];
#pragma unroll
    for (int i = 0; i < 6; ++i) dK[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < 4; ++i) dV[i] = f32x16{};

    // query tiles that can see keys kb0 .. kb0 + 127
    const int qt_lo = kb0 / kQT;
    const int q_last = p.swa ? min(p.L - 1, kb0 + kKeysPerWg - 1 + p.window - 1) : p.L - 1;
    const int qt_hi = kb0 < p.L ? q_last / kQT : qt_lo - 1;
    const int ntile = qt_hi - qt_lo + 1;
    const int total = ntile > 0 ? ntile * p.G : 0;

    // Item it = (query tile qt_hi - it / G, head it % G): every workgroup walks the query
    // tiles from the last one down, so the workgroups of one KV head that run together read
    // the same tiles at about the same time (shared in L2).  Wave w loads blocks w, w + 4,
    // w + 8 of Q and w, w + 4 of dO; waves 0 and 1 also load the LSE and D rows.
    const int qsrc0 = src_of_slot<192>(64 * wave + lane), qsrc1 = src_of_slot<192>(64 * (wave + 4) + lane),
              qsrc2 = src_of_slot<192>(64 * (wave + 8) + lane);
    const int osrc0 = src_of_slot<128>(64 * wave + lane), osrc1 = src_of_slot<128>(64 * (wave + 4) + lane);
    auto issue = [&](int it, const DkTile &t) {
        const int hq = kvh * p.G + it % p.G, q0 = (qt_hi - it / p.G) * kQT;
        const size_t rbase = ((size_t)b * p.Hq + hq) * p.L;
        const auto rq = region(p.q + rbase * kDqk, (size_t)p.L * kDqk * 2);
        const auto ro = region(p.dout + rbase * kDv, (size_t)p.L * kDv * 2);
        dma16(rq, t.q + 1024 * wave, qsrc0, q0 * (kDqk * 2));
        dma16(rq, t.q + 1024 * (wave + 4), qsrc1, q0 * (kDqk * 2));
        dma16(rq, t.q + 1024 * (wave + 8), qsrc2, q0 * (kDqk * 2));
        dma16(ro, t.o + 1024 * wave, osrc0, q0 * (kDv * 2));
        dma16(ro, t.o + 1024 * (wave + 4), osrc1, q0 * (kDv * 2));
        if (wave == 0) dma4(region(p.lse + rbase, (size_t)p.L * 4), t.lse, 4 * lane, 4 * q0);
        if (wave == 1) dma4(region(p.delta + rbase, (size_t)p.L * 4), t.d, 4 * lane, 4 * q0);
    };
    auto compute = [&](const DkTile &t, int it) {
        const int q0 = (qt_hi - it / p.G) * kQT;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 12; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<192>(t.q, 0, kk, lane), kB[kk], s, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<128>(t.o, 0, kk, lane), vB[kk], dp, 0, 0, 0);
        // lane: key column n, query rows mrow(e, g) = 8 (e / 4) + 4 g + e % 4
        if (!all_visible(p, q0, kw0)) {  // wave-uniform
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (!visible(p, q0 + mrow(e, g), key)) s[e] = -INFINITY;
        }
        f32x16 pr, ds;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 l4 = *reinterpret_cast<const f32x4 *>(t.lse + 8 * j + 4 * g);
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(t.d + 8 * j + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * j + i;
                const float pv = exp2f_fast(__builtin_fmaf(s[e], p.scale_log2, -l4[i] * kLog2e));
                pr[e] = pv;
                ds[e] = pv * (dp[e] - d4[i]);
            }
        }
        const bf16x8 pa0 = pack8(pr, 0), pa1 = pack8(pr, 8), da0 = pack8(ds, 0), da1 = pack8(ds, 8);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            dV[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0, col_operand<128>(t.o, 0, 32 * nb, lane), dV[nb], 0, 0, 0);
            dV[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1, col_operand<128>(t.o, 16, 32 * nb, lane), dV[nb], 0, 0, 0);
        }
#pragma unroll
        for (int nb = 0; nb < 6; ++nb) {
            dK[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da0, col_operand<192>(t.q, 0, 32 * nb, lane), dK[nb], 0, 0, 0);
            dK[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da1, col_operand<192>(t.q, 16, 32 * nb, lane), dK[nb], 0, 0, 0);
        }
    };
    // Item it uses buffer it % 3 and its loads are issued two items ahead: after the barrier
    // of item it - 2, when every wave has finished item it - 3, the last reader of that
    // buffer.  Before the barrier of item it each wave waits for all but its newest loads
    // (those of item it + 1: six instructions on waves 0 and 1, five on the others); past
    // the last item the loads repeat the last item, so that the count never changes.
    const DkTile ta{qa, oa, la, da}, tb{qb, ob, lb, db_}, tc{qc, oc, lc, dc};
    auto step = [&](int it, const DkTile &cur, const DkTile &fut) {
        if (wave < 2) __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
        else __builtin_amdgcn_s_waitcnt(0x0F75);           // vmcnt(5)
        __syncthreads();
        issue(min(it + 2, total - 1), fut);
        compute(cur, it);
    };
    if (total > 0) {
        issue(0, ta);
        issue(min(1, total - 1), tb);
    }
    int it = 0;
    for (; it + 2 < total; it += 3) {
        step(it, ta, tc);
        step(it + 1, tb, ta);
        step(it + 2, tc, tb);
    }
    if (it < total) step(it, ta, tc);
    if (it + 1 < total) step(it + 1, tb, ta);
    wait_dma();  // no load into LDS outlives the workgroup

    // rows: this wave's keys mrow(e, g); columns: dims 32 nb + n
    const float scale = p.scale;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int kr = kw0 + mrow(e, g);
        if (kr >= p.L) continue;
        const size_t row = ((size_t)b * p.Hkv + kvh) * p.L + kr;
#pragma unroll
        for (int nb = 0; nb < 6; ++nb) p.dk[row * kDqk + 32 * nb + n] = dK[nb][e] * scale;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) p.dv[row * kDv + 32 * nb + n] = dV[nb][e];
    }
}

// ---- dQ
// LDS tile of 64 keys: K [64][192] (24 blocks of 1 KB) and V [64][128] (16 blocks), triple
// buffered (120 KB).  Each wave runs a software pipeline over 32-key sub-blocks so that the
// softmax arithmetic of one sub-block overlaps the products of the next:
//   phase A: S^T, dP^T of (t, 1)       with  dS^T of (t, 0)
//   phase B: dQ^T += K(t, 0)^T dS^T(t, 0)
//   barrier: tile t + 1 has landed, the buffer of tile t - 1 is free; tile t + 2 starts
//   phase C: S^T, dP^T of (t + 1, 0)   with  dS^T of (t, 1)
//   phase D: dQ^T += K(t, 1)^T dS^T(t, 1)
// Sub-blocks past the last row or before the window are computed and masked to zero, and
// past the last tile the loads and scores repeat the last tile unused, so that no branch
// splits a phase.
constexpr int kDqKBytes = kKT * kDqk * 2, kDqVBytes = kKT * kDv * 2;

__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char K0[kDqKBytes], K1[kDqKBytes], K2[kDqKBytes];
    __shared__ __attribute__((aligned(1024))) char V0[kDqVBytes], V1[kDqVBytes], V2[kDqVBytes];

    // workgroup -> (query tile, sequence, group of four heads): head groups vary fastest and
    // the query tiles with the most key tiles come first
    int bid = blockIdx.x;
    const int hgroup = bid % (p.Hq / 4);
    bid /= p.Hq / 4;
    const int b = bid % p.B;
    const int q0 = ((p.L + kQT - 1) / kQT - 1 - bid / p.B) * kQT;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int hq = hgroup * 4 + wave, kvh = (hgroup * 4) / p.G;
    const int qpos = q0 + n;  // this lane's query (B-operand column)
    const size_t qrow = ((size_t)b * p.Hq + hq) * p.L + (qpos < p.L ? qpos : 0);
    const bool qok = qpos < p.L;
    if (q0 >= p.L) return;  // uniform over the workgroup

    bf16x8 qB[12], oB[8];
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) qB[kk] = as_bf16x8(qok ? ldg16(p.q + qrow * kDqk + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) oB[kk] = as_bf16x8(qok ? ldg16(p.dout + qrow * kDv + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
    // a row past the sequence end has every pair masked; its LSE only has to be finite
    const float nlse2 = qok ? -p.lse[qrow] * kLog2e : 0.f, d_q = qok ? p.delta[qrow] : 0.f;
    f32x16 dQ[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) dQ[i] = f32x16{};

    // key tiles that rows q0 .. q0 + 31 see
    const int q_hi = min(p.L, q0 + kQT) - 1;
    const int k_lo = p.swa ? max(0, q0 - p.window + 1) : 0;
    const int t0 = k_lo / kKT, t1 = q_hi / kKT;
    const size_t kvbase = ((size_t)b * p.Hkv + kvh) * p.L;
    const auto rk = region(p.k + kvbase * kDqk, (size_t)p.L * kDqk * 2);
    const auto rv = region(p.v + kvbase * kDv, (size_t)p.L * kDv * 2);

    // wave w loads blocks w + 4 i of K (24 blocks) and of V (16 blocks)
    int ksrc[6], vsrc[4];
#pragma unroll
    for (int i = 0; i < 6; ++i) ksrc[i] = src_of_slot<192>(64 * (wave + 4 * i) + lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) vsrc[i] = src_of_slot<128>(64 * (wave + 4 * i) + lane);
    auto issue = [&](int t, char *kt, char *vt) {
        const int kbase = t * kKT;
#pragma unroll
        for (int i = 0; i < 6; ++i) dma16(rk, kt + 1024 * (wave + 4 * i), ksrc[i], kbase * (kDqk * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(rv, vt + 1024 * (wave + 4 * i), vsrc[i], kbase * (kDv * 2));
    };
    // S^T = K Q^T and dP^T = V dO^T of sub-block sb of a tile
    auto scores = [&](const char *kt, const char *vt, int sb, f32x16 &s, f32x16 &dp) {
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 12; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<192>(kt, 32 * sb, kk, lane), qB[kk], s, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<128>(vt, 32 * sb, kk, lane), oB[kk], dp, 0, 0, 0);
    };
    // dS^T = P^T (dP^T - D) of the sub-block whose first key is kbase, as two bf16 k-steps;
    // lane: query column n, key rows mrow(e, g)
    auto dscores = [&](f32x16 s, const f32x16 &dp, int kbase, bf16x8 &d0, bf16x8 &d1) {
        if (!all_visible(p, q0, kbase)) {  // uniform
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (!visible(p, qpos, kbase + mrow(e, g))) s[e] = -INFINITY;
        }
        f32x16 ds;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float pv = exp2f_fast(__builtin_fmaf(s[e], p.scale_log2, nlse2));
            ds[e] = pv * (dp[e] - d_q);
        }
        d0 = pack8(ds, 0);
        d1 = pack8(ds, 8);
    };
    auto dq_acc = [&](const char *kt, int sb, const bf16x8 &d0, const bf16x8 &d1) {
#pragma unroll
        for (int db = 0; db < 6; ++db) {
            dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_operand<192>(kt, 32 * sb, 32 * db, lane), d0, dQ[db], 0, 0, 0);
            dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_operand<192>(kt, 32 * sb + 16, 32 * db, lane), d1, dQ[db], 0, 0, 0);
        }
    };

    f32x16 s0, dp0, s1, dp1;
    bf16x8 da, db;
    auto step = [&](int t, const char *Kc, const char *Vc, const char *Kn, const char *Vn, char *Kf, char *Vf) {
        const int kb = t * kKT;
        scores(Kc, Vc, 1, s1, dp1);        // phase A
        dscores(s0, dp0, kb, da, db);
        dq_acc(Kc, 0, da, db);             // phase B
        wait_dma();
        __syncthreads();
        issue(min(t + 2, t1), Kf, Vf);
        scores(Kn, Vn, 0, s0, dp0);        // phase C (unused after the last tile)
        dscores(s1, dp1, kb + 32, da, db);
        dq_acc(Kc, 1, da, db);             // phase D
    };
    issue(t0, K0, V0);
    issue(min(t0 + 1, t1), K1, V1);
    wait_dma();
    __syncthreads();
    scores(K0, V0, 0, s0, dp0);
    for (int t = t0; t <= t1; t += 3) {
        step(t, K0, V0, K1, V1, K2, V2);
        if (t + 1 <= t1) step(t + 1, K1, V1, K2, V2, K0, V0);
        if (t + 2 <= t1) step(t + 2, K2, V2, K0, V0, K1, V1);
    }
    wait_dma();  // no load into LDS outlives the workgroup
    if (!qok) return;
    // dQ^T: lane holds query qpos, dims 32 db + mrow(e, g): four consecutive dims per group of 4
    float *dst = p.dq + qrow * kDqk;
#pragma unroll
    for (int i = 0; i < 6; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4 *>(dst + 32 * i + 8 * j + 4 * g) =
                f32x4{dQ[i][4 * j] * p.scale, dQ[i][4 * j + 1] * p.scale, dQ[i][4 * j + 2] * p.scale,
                      dQ[i][4 * j + 3] * p.scale};
}

}  // namespace

size_t backward_workspace_bytes(int B, int Hq, int L) {
    const size_t nblk = ((size_t)L + kPreRows - 1) / kPreRows;
    return ((size_t)B * Hq * L + (size_t)B * Hq * nblk) * sizeof(float);
}

int launch_backward(const BwdParams &prm, hipStream_t stream) {
    BwdParams p = prm;
    const int nblk = (p.L + kPreRows - 1) / kPreRows;
    void *args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_pre_kernel), dim3(nblk, p.Hq, p.B), dim3(256), args, 0,
                        stream) != hipSuccess)
        return -1;
    if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_dkdv_kernel),
                        dim3(((p.L + kKeysPerWg - 1) / kKeysPerWg) * p.Hkv * p.B), dim3(256), args, 0, stream) != hipSuccess)
        return -1;
    if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_dq_kernel), dim3(((p.L + kQT - 1) / kQT) * (p.Hq / 4) * p.B),
                        dim3(256), args, 0, stream) != hipSuccess)
        return -1;
    if (p.sink) {
        void *args2[] = {&p, (void *)&nblk};
        if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_dsink_kernel), dim3(p.Hq), dim3(256), args2,
                            0, stream) != hipSuccess)
            return -1;
    }
    return 0;
}

}  // namespace sinkattn
