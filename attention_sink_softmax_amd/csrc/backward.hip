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
//   bwd_dkdv    one workgroup per 128 keys of a (sequence, KV head): the two waves of each 32-key
//               group keep its K and dV, or V and dK, in registers and walk every query head of
//               the group and every 32-row query tile that sees its keys:
//                 S = Q K^T, dP = dO V^T (query rows x keys), dS = P (dP - D),
//                 dV += P^T dO, dK += dS^T Q       (P and dS feed the A operand as they are;
//                                                    dO and Q arrive through transposing reads);
//   bwd_dq      one workgroup per 64 query rows of four query heads of one KV head: each wave
//               keeps its head's Q and dO operands and dQ^T for 32 rows in registers and walks
//               the key tiles:
//                 S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T;
//   bwd_dsink   sums the sink gradient partials in a fixed order (deterministic).
// All products are v_mfma_f32_32x32x16_bf16 with float32 accumulation; P and dS enter them as
// bf16.  Tiles pass through LDS (four buffers in bwd_dkdv, three in bwd_dq, loaded two steps
// ahead, one barrier per step) with their 16-byte chunks XOR-swizzled by row so that both the
// row reads and the transposing reads spread over the banks.  Masking is branch-free and only runs on tiles that cross the causal diagonal, the
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
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// The loads are written as inline asm.  The compiler does not see them,
// so it adds no wait for them before reads of other LDS buffers (its own tracking of loads
// into LDS loses the buffer across the loop and waits for the next tile's loads as well).
// The kernels wait for these loads themselves (vmcnt) before each barrier.  m0 carries the
// LDS address (one wait state before the load) and is restored for the compiler's use; the
// asm has no register output, so no load in flight can land in a register.
__device__ __forceinline__ void dma16_async(__amdgpu_buffer_rsrc_t r, char *lds, int voff, int soff) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)lds;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(base), "v"(voff), "s"(r), "s"(soff)
        : "memory");
}
__device__ __forceinline__ void dma4_async(__amdgpu_buffer_rsrc_t r, void *lds, int voff, int soff) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)lds;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(base), "v"(voff), "s"(r), "s"(soff)
        : "memory");
}

// Workgroup barrier over LDS: this wave's LDS writes are complete, then every wave meets.
// The caller first waits for the loads into LDS that the next step reads (vmcnt); the
// barrier itself does not wait for the others, which stay in flight across it.  (A
// __syncthreads() fence would wait for every outstanding load.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int kQT = 32;                    // query rows per tile
constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWg = 4 * kKeysPerWave;  // bwd_dkdv
constexpr int kKT = 64;                    // keys per tile in bwd_dq
constexpr int kPreRows = 16;               // rows per bwd_pre workgroup

// Byte offset of 16-byte chunk c of row r in an LDS tile of W-element rows.  Rows are 448
// bytes apart for W = 192 and 320 for W = 128 (64 bytes unused at the end of each), and chunk c
// sits at c ^ ((r >> 2) & 3).  With banks serving 256 bytes per cycle (16 lanes of a 16-byte
// read, 32 lanes of an 8-byte transposing read):
//   * a transposing read (4 rows of a 4-aligned group x 4 chunks of a 4-aligned group) puts
//     each row's 4 chunks in a run of 4 slots that the XOR only permutes, and the row stride
//     (28 or 20 slots, 4 mod 8) sets the 4 runs 4 slots apart;
//   * a row read (rows r .. r + 15 of a 16-aligned group, one chunk) gets 4 bank positions
//     from the stride (r mod 4) and the other 4 from the XOR ((r >> 2) & 3).
// The XOR touches only the low two bits of the chunk index, which are lane bits in the
// transposing reads and half lane bits in the row reads, so each read's address is a lane
// register plus a constant offset (two registers per operand kind).
template <int W>
constexpr int kTileRow = W == 192 ? 448 : 320;
template <int W>
__device__ __forceinline__ int tile_off(int r, int c) {
    return r * kTileRow<W> + ((c ^ ((r >> 2) & 3)) << 4);
}
// Source offset (bytes, from the tile's first row) of the chunk that lands in 16-byte slot
// `slot` of a tile of W-element rows.  The unused slots at a row's end take a copy of one of
// the row's chunks (nobody reads them), so that every lane of a load instruction loads.
template <int W>
__device__ __forceinline__ int src_of_slot(int slot) {
    constexpr int kSlots = kTileRow<W> / 16, kChunks = W / 8;
    const int r = slot / kSlots, pc = slot % kSlots;
    return r * (W * 2) + ((pc % kChunks) ^ ((r >> 2) & 3)) * 16;
}

// Row m of a 32x32 MFMA result held in register e by lane group g.
__device__ __forceinline__ int mrow(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// The lane-dependent parts of the operand reads of a tile of W-element rows.  Every read
// starts at a row rbase that is a multiple of 16, so (row >> 2) & 3 depends on the lane only,
// and the XOR stays in the low two bits of the chunk index: each address is one of these
// registers plus a compile-time offset.
//   row[p]: row rbase + (lane & 31), chunk 2 kk + g with kk & 1 = p (g = lane >> 5);
//   col[h]: row rbase + 8h + 4g + (i >> 2), chunk 4 nb + 2 gl + (c4 >> 1), half c4 & 1
//           (i = lane & 15, gl = (lane >> 4) & 1, c4 = i & 3).
template <int W>
struct LaneOff {
    int row[2], col[2];
    __device__ __forceinline__ explicit LaneOff(int lane) {
        constexpr int S = kTileRow<W>;
        const int g = lane >> 5, gl = (lane >> 4) & 1, i = lane & 15, c4 = i & 3, r = lane & 31;
#pragma unroll
        for (int p = 0; p < 2; ++p) row[p] = r * S + (((2 * p + g) ^ ((r >> 2) & 3)) << 4);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            col[h] = (4 * g + (i >> 2)) * S + (((2 * gl + (c4 >> 1)) ^ ((2 * h + g) & 3)) << 4) + 8 * (c4 & 1);
    }
};

// 8 elements of column `col0 + (lane & 31)` of a tile, from rows rbase + {4g .. 4g+3} and
// rbase + 8 + {4g .. 4g+3} (g = lane >> 5): the operand, in the k order of a score tile's
// registers, of a product that contracts over those rows.  col0 is a multiple of 32.
template <int W>
__device__ __forceinline__ bf16x8 col_operand(const char *tile, int rbase, int col0, const LaneOff<W> &lo) {
    const char *base = tile + rbase * kTileRow<W> + 2 * col0;  // chunk 4 nb = col0 / 8
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + lo.col[0]));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + 8 * kTileRow<W> + lo.col[1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 8 elements of row rbase + (lane & 31), chunk 2kk + g, of a tile.
template <int W>
__device__ __forceinline__ bf16x8 row_operand(const char *tile, int rbase, int kk, const LaneOff<W> &lo) {
    return *reinterpret_cast<const bf16x8 *>(tile + rbase * kTileRow<W> + (kk >> 1) * 64 + lo.row[kk & 1]);
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

// ---- D_i = dO_i . O_i, -LSE_i log2(e), and the sink gradient's partial sums
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
        p.nlse2[row] = -p.lse[row] * kLog2e;
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
// One workgroup per 128 keys of a (sequence, KV head), eight waves.  Key group kg = wave % 4
// owns keys kb0 + 32 kg .. +31, and its two waves split the products of every item (query
// tile, head) between them:
//   wave kg     (role P):  S = Q K^T, P = exp(scale S - LSE), dV += P^T dO;  P goes to LDS
//   wave kg + 4 (role dS): dP = dO V^T, dS = P (dP - D),    dK += dS^T Q   (one item later)
// Each role keeps half of the per-key state in registers (K and dV, or V and dK), so two
// waves share a SIMD and one's products run while the other waits or does its softmax
// arithmetic.  The P tile passes in float32, so the results are those of computing both
// halves in one wave.
// LDS tile of one query tile: Q [32][192] (14 blocks of 1 KB) and dO [32][128] (10 blocks),
// and -LSE log2(e) and D of its rows (64 floats each: the 32 rows of the tile and 32 unused;
// the pre-pass writes -LSE log2(e), so P is one fused multiply-add and an exp2 per element).
constexpr int kDkQBytes = kQT * kTileRow<192>, kDkOBytes = kQT * kTileRow<128>;  // 14 and 10 KB

struct DkTile {
    char *q, *o;
    float *nl2, *d;  // -lse log2(e) and D of the tile's rows
};

__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char q0b[kDkQBytes], q1b[kDkQBytes], q2b[kDkQBytes], q3b[kDkQBytes];
    __shared__ __attribute__((aligned(1024))) char o0b[kDkOBytes], o1b[kDkOBytes], o2b[kDkOBytes], o3b[kDkOBytes];
    __shared__ __attribute__((aligned(256))) float l0[64], l1[64], l2[64], l3[64], d0[64], d1[64], d2[64], d3[64];
    // P of one item per key group, float32, [key group][register quad j][lane] of 16 bytes;
    // two slots: role P writes slot it % 2 during step it, role dS reads it during step it + 1
    __shared__ __attribute__((aligned(1024))) f32x4 pslot[2][4][4][64];

    // workgroup -> (key block, sequence, KV head): KV heads vary fastest, so that the
    // workgroups that the hardware places on one XCD (ids equal mod 8) share a KV head, and
    // the key blocks with the most query tiles come first
    int bid = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const int kvh = bid % p.Hkv;
    bid /= p.Hkv;
    const int b = bid % p.B;
    const int kb0 = (bid / p.B) * kKeysPerWg;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3;
    const bool role_p = wave < 4;
    const LaneOff<192> lq(lane);  // Q tiles
    const LaneOff<128> lo(lane);  // dO tiles
    const int n = lane & 31, g = lane >> 5;
    const int kw0 = kb0 + kKeysPerWave * kg;  // this key group's first key
    const int key = kw0 + n;                  // this lane's key (B-operand column)
    const bool key_ok = key < p.L;
    const size_t krow = ((size_t)b * p.Hkv + kvh) * p.L + (key_ok ? key : 0);

    // query tiles that can see keys kb0 .. kb0 + 127
    const int qt_lo = kb0 / kQT;
    const int q_last = p.swa ? min(p.L - 1, kb0 + kKeysPerWg - 1 + p.window - 1) : p.L - 1;
    const int qt_hi = kb0 < p.L ? q_last / kQT : qt_lo - 1;
    const int ntile = qt_hi - qt_lo + 1;
    const int total = ntile > 0 ? ntile * p.G : 0;

    // Item it = (query tile qt_hi - it / G, head it % G): every workgroup walks the query
    // tiles from the last one down, so the workgroups of one KV head that run together read
    // the same tiles at about the same time (shared in L2).  Wave w loads blocks w of Q and
    // dO, waves 0-5 also block w + 8 of Q, waves 0-1 block w + 8 of dO, wave 6 the -LSE log2(e)
    // rows and wave 7 the D rows: four load instructions per item on waves 0-1, three on the
    // others.
    const int qsrc0 = src_of_slot<192>(64 * wave + lane), qsrc1 = src_of_slot<192>(64 * (wave + 8) + lane);
    const int osrc0 = src_of_slot<128>(64 * wave + lane), osrc1 = src_of_slot<128>(64 * (wave + 8) + lane);
    auto issue = [&](int it, const DkTile &t) {
        const int hq = kvh * p.G + it % p.G, q0 = (qt_hi - it / p.G) * kQT;
        const size_t rbase = ((size_t)b * p.Hq + hq) * p.L;
        const auto rq = region(p.q + rbase * kDqk, (size_t)p.L * kDqk * 2);
        const auto ro = region(p.dout + rbase * kDv, (size_t)p.L * kDv * 2);
        dma16_async(rq, t.q + 1024 * wave, qsrc0, q0 * (kDqk * 2));
        if (wave < 6) dma16_async(rq, t.q + 1024 * (wave + 8), qsrc1, q0 * (kDqk * 2));
        dma16_async(ro, t.o + 1024 * wave, osrc0, q0 * (kDv * 2));
        if (wave < 2) dma16_async(ro, t.o + 1024 * (wave + 8), osrc1, q0 * (kDv * 2));
        if (wave == 6) dma4_async(region(p.nlse2 + rbase, (size_t)p.L * 4), t.nl2, 4 * lane, 4 * q0);
        if (wave == 7) dma4_async(region(p.delta + rbase, (size_t)p.L * 4), t.d, 4 * lane, 4 * q0);
    };
    // Item it uses buffer it % 4; its loads are issued two items ahead, after the barrier of
    // step it - 2, by when the previous item in that buffer, it - 4, is done (role P ran it
    // in step it - 4, role dS in step it - 3).  Step s runs item s on role P and
    // item s - 1 on role dS; there are total + 1 steps.  Before the barrier of each step
    // every wave waits for all but its newest loads (those of the item after the next);
    // past the last item the loads repeat it, so that the count never changes.
    const DkTile t0{q0b, o0b, l0, d0}, t1{q1b, o1b, l1, d1}, t2{q2b, o2b, l2, d2}, t3{q3b, o3b, l3, d3};
    const int nsteps = total > 0 ? total + 1 : 0;
    auto sync_issue = [&](int s, const DkTile &fut) {
        if (wave < 2) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
        else __builtin_amdgcn_s_waitcnt(0x0F73);           // vmcnt(3)
        lds_barrier();
        issue(min(s + 2, total - 1), fut);
    };
    if (total > 0) {
        issue(0, t0);
        issue(min(1, total - 1), t1);
    }
    const float scale = p.scale;

    if (role_p) {
        // this key group's K rows as the B operand of S = Q K^T (in AGPRs, which the matrix
        // unit reads directly)
        bf16x8 kB[12];
#pragma unroll
        for (int kk = 0; kk < 12; ++kk)
            kB[kk] = as_bf16x8(key_ok ? ldg16(p.k + krow * kDqk + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) asm volatile("" : "+a"(kB[kk]));
        f32x16 dV[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dV[i] = f32x16{};
        auto compute = [&](const DkTile &t, int it) __attribute__((always_inline)) {
            const int q0 = (qt_hi - it / p.G) * kQT;
            f32x16 s = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 12; ++kk)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<192>(t.q, 0, kk, lq), kB[kk], s, 0, 0, 0);
            // lane: key column n, query rows mrow(e, g) = 8 (e / 4) + 4 g + e % 4
            if (!all_visible(p, q0, kw0)) {  // wave-uniform
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (!visible(p, q0 + mrow(e, g), key)) s[e] = -INFINITY;
            }
            f32x16 pr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(t.nl2 + 8 * j + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) pr[4 * j + i] = exp2f_fast(__builtin_fmaf(s[4 * j + i], p.scale_log2, l4[i]));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pslot[it & 1][kg][j][lane] = f32x4{pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]};
            const bf16x8 pa0 = pack8(pr, 0), pa1 = pack8(pr, 8);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                dV[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0, col_operand<128>(t.o, 0, 32 * nb, lo), dV[nb], 0, 0, 0);
                dV[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1, col_operand<128>(t.o, 16, 32 * nb, lo), dV[nb], 0, 0, 0);
            }
        };
        auto step = [&](int s, const DkTile &cur, const DkTile &fut) __attribute__((always_inline)) {
            sync_issue(s, fut);
            if (s < total) compute(cur, s);
        };
        int s = 0;
        for (; s + 3 < nsteps; s += 4) {
            step(s, t0, t2);
            step(s + 1, t1, t3);
            step(s + 2, t2, t0);
            step(s + 3, t3, t1);
        }
        if (s < nsteps) step(s, t0, t2);
        if (s + 1 < nsteps) step(s + 1, t1, t3);
        if (s + 2 < nsteps) step(s + 2, t2, t0);
        wait_dma();  // no load into LDS outlives the workgroup
        // rows: this group's keys mrow(e, g); columns: dims 32 nb + n
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int kr = kw0 + mrow(e, g);
            if (kr >= p.L) continue;
            const size_t row = ((size_t)b * p.Hkv + kvh) * p.L + kr;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) p.dv[row * kDv + 32 * nb + n] = dV[nb][e];
        }
    } else {
        // this key group's V rows as the B operand of dP = dO V^T
        bf16x8 vB[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            vB[kk] = as_bf16x8(key_ok ? ldg16(p.v + krow * kDv + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+a"(vB[kk]));
        f32x16 dK[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) dK[i] = f32x16{};
        auto compute = [&](const DkTile &t, int it) __attribute__((always_inline)) {
            f32x16 dp = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<128>(t.o, 0, kk, lo), vB[kk], dp, 0, 0, 0);
            f32x16 ds;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 d4 = *reinterpret_cast<const f32x4 *>(t.d + 8 * j + 4 * g);
                const f32x4 p4 = pslot[it & 1][kg][j][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) ds[4 * j + i] = p4[i] * (dp[4 * j + i] - d4[i]);
            }
            const bf16x8 da0 = pack8(ds, 0), da1 = pack8(ds, 8);
#pragma unroll
            for (int nb = 0; nb < 6; ++nb) {
                dK[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da0, col_operand<192>(t.q, 0, 32 * nb, lq), dK[nb], 0, 0, 0);
                dK[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da1, col_operand<192>(t.q, 16, 32 * nb, lq), dK[nb], 0, 0, 0);
            }
        };
        // step s: item s - 1, in buffer (s - 1) % 4
        auto step = [&](int s, const DkTile &prev, const DkTile &fut) __attribute__((always_inline)) {
            sync_issue(s, fut);
            if (s >= 1) compute(prev, s - 1);
        };
        int s = 0;
        for (; s + 3 < nsteps; s += 4) {
            step(s, t3, t2);
            step(s + 1, t0, t3);
            step(s + 2, t1, t0);
            step(s + 3, t2, t1);
        }
        if (s < nsteps) step(s, t3, t2);
        if (s + 1 < nsteps) step(s + 1, t0, t3);
        if (s + 2 < nsteps) step(s + 2, t1, t0);
        wait_dma();
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int kr = kw0 + mrow(e, g);
            if (kr >= p.L) continue;
            const size_t row = ((size_t)b * p.Hkv + kvh) * p.L + kr;
#pragma unroll
            for (int nb = 0; nb < 6; ++nb) p.dk[row * kDqk + 32 * nb + n] = dK[nb][e] * scale;
        }
    }
}

// ---- dQ
// One workgroup per 64 query rows of four query heads of one KV head, eight waves: wave w
// takes head 4 hgroup + w % 4 and rows q0 + 32 (w / 4) .. +31, keeps that head's Q and dO
// operands and dQ^T in registers, and walks the key tiles.  LDS tile of 64 keys: K [64][192]
// (28 blocks of 1 KB) and V [64][128] (20 blocks), triple buffered (144 KB), shared by the
// eight waves; two waves per SIMD, so one's products run while the other does its softmax
// arithmetic.  Per 32-key sub-block:
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// A sub-block that none of the wave's rows sees is skipped (wave-uniform); one that crosses
// the diagonal, the window's edge or the sequence end is masked.
constexpr int kDqKBytes = kKT * kTileRow<192>, kDqVBytes = kKT * kTileRow<128>;  // 28 and 20 KB
constexpr int kDqRows = 2 * kQT;  // query rows per workgroup

__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char K0[kDqKBytes], K1[kDqKBytes], K2[kDqKBytes];
    __shared__ __attribute__((aligned(1024))) char V0[kDqVBytes], V1[kDqVBytes], V2[kDqVBytes];

    // workgroup -> (query block, sequence, group of four heads): head groups vary fastest and
    // the query blocks with the most key tiles come first
    int bid = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const int hgroup = bid % (p.Hq / 4);
    bid /= p.Hq / 4;
    const int b = bid % p.B;
    const int qb0 = ((p.L + kDqRows - 1) / kDqRows - 1 - bid / p.B) * kDqRows;
    if (qb0 >= p.L) return;  // uniform over the workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int hq = hgroup * 4 + (wave & 3), kvh = (hgroup * 4) / p.G;
    const LaneOff<192> lk(lane);  // K tiles
    const LaneOff<128> lv(lane);  // V tiles
    const int q0 = qb0 + kQT * (wave >> 2);  // this wave's first row
    const int qpos = q0 + n;                 // this lane's query (B-operand column)
    const size_t qrow = ((size_t)b * p.Hq + hq) * p.L + (qpos < p.L ? qpos : 0);
    const bool qok = qpos < p.L;

    bf16x8 qB[12], oB[8];
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) qB[kk] = as_bf16x8(qok ? ldg16(p.q + qrow * kDqk + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) oB[kk] = as_bf16x8(qok ? ldg16(p.dout + qrow * kDv + 16 * kk + 8 * g) : u32x4{0, 0, 0, 0});
    // a row past the sequence end has every pair masked; its LSE only has to be finite
    const float nlse2 = qok ? p.nlse2[qrow] : 0.f, d_q = qok ? p.delta[qrow] : 0.f;
    // these loads land before the loop: the compiler does not count the tile loads, so a wait
    // for them inside the loop would wait for every tile load in flight
    wait_dma();
    f32x16 dQ[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) dQ[i] = f32x16{};

    // key tiles that rows qb0 .. qb0 + 63 see, and the keys this wave's rows see
    const int q_hi = min(p.L, qb0 + kDqRows) - 1;
    const int k_lo = p.swa ? max(0, qb0 - p.window + 1) : 0;
    const int t0 = k_lo / kKT, t1 = q_hi / kKT;
    const int wk_hi = min(p.L, q0 + kQT) - 1;                       // last key of any row
    const int wk_lo = p.swa ? q0 - p.window + 1 : INT32_MIN / 2;  // first key of the last row
    const size_t kvbase = ((size_t)b * p.Hkv + kvh) * p.L;
    const auto rk = region(p.k + kvbase * kDqk, (size_t)p.L * kDqk * 2);
    const auto rv = region(p.v + kvbase * kDv, (size_t)p.L * kDv * 2);

    // wave w loads blocks w, w + 8, w + 16 of K and w, w + 8 of V, and waves 0-3 also block
    // w + 24 of K and w + 16 of V: seven load instructions per tile on waves 0-3, five on 4-7
    int ksrc[4], vsrc[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) ksrc[i] = src_of_slot<192>(64 * (wave + 8 * i) + lane);
#pragma unroll
    for (int i = 0; i < 3; ++i) vsrc[i] = src_of_slot<128>(64 * (wave + 8 * i) + lane);
    auto issue = [&](int t, char *kt, char *vt) {
        const int kbase = t * kKT;
#pragma unroll
        for (int i = 0; i < 3; ++i) dma16_async(rk, kt + 1024 * (wave + 8 * i), ksrc[i], kbase * (kDqk * 2));
        if (wave < 4) dma16_async(rk, kt + 1024 * (wave + 24), ksrc[3], kbase * (kDqk * 2));
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_async(rv, vt + 1024 * (wave + 8 * i), vsrc[i], kbase * (kDv * 2));
        if (wave < 4) dma16_async(rv, vt + 1024 * (wave + 16), vsrc[2], kbase * (kDv * 2));
    };
    // one 32-key sub-block: lane holds query column n, key rows kbase + mrow(e, g)
    auto sub = [&](const char *kt, const char *vt, int sb, int kbase) __attribute__((always_inline)) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 12; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<192>(kt, 32 * sb, kk, lk), qB[kk], s, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<128>(vt, 32 * sb, kk, lv), oB[kk], dp, 0, 0, 0);
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
        const bf16x8 d0 = pack8(ds, 0), d1 = pack8(ds, 8);
#pragma unroll
        for (int db = 0; db < 6; ++db) {
            dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_operand<192>(kt, 32 * sb, 32 * db, lk), d0, dQ[db], 0, 0, 0);
            dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_operand<192>(kt, 32 * sb + 16, 32 * db, lk), d1, dQ[db], 0, 0, 0);
        }
    };
    // Tile t uses buffer (t - t0) % 3; its loads are issued two tiles ahead, after the barrier
    // of tile t - 2, when every wave has finished tile t - 3, the last reader of that buffer.
    // Before each barrier a wave waits for all but its newest loads (those of the next tile);
    // past the last tile the loads repeat it, so that the count never changes.
    auto step = [&](int t, const char *Kc, const char *Vc, char *Kf, char *Vf) __attribute__((always_inline)) {
        if (wave < 4) __builtin_amdgcn_s_waitcnt(0x0F77);  // vmcnt(7)
        else __builtin_amdgcn_s_waitcnt(0x0F75);           // vmcnt(5)
        lds_barrier();
        issue(min(t + 2, t1), Kf, Vf);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int kbase = t * kKT + 32 * sb;
            const bool dead = q0 >= p.L || kbase > wk_hi || kbase + 31 < wk_lo;  // uniform
            if (!dead) sub(Kc, Vc, sb, kbase);
        }
    };
    issue(t0, K0, V0);
    issue(min(t0 + 1, t1), K1, V1);
    for (int t = t0; t <= t1; t += 3) {
        step(t, K0, V0, K2, V2);
        if (t + 1 <= t1) step(t + 1, K1, V1, K0, V0);
        if (t + 2 <= t1) step(t + 2, K2, V2, K1, V1);
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
    return (2 * (size_t)B * Hq * L + (size_t)B * Hq * nblk) * sizeof(float);
}

int launch_backward(const BwdParams &prm, hipStream_t stream) {
    BwdParams p = prm;
    p.reverse = grid_reversed();
    const int nblk = (p.L + kPreRows - 1) / kPreRows;
    void *args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_pre_kernel), dim3(nblk, p.Hq, p.B), dim3(256), args, 0,
                        stream) != hipSuccess)
        return -1;
    if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_dkdv_kernel),
                        dim3(((p.L + kKeysPerWg - 1) / kKeysPerWg) * p.Hkv * p.B), dim3(512), args, 0, stream) != hipSuccess)
        return -1;
    if (hipLaunchKernel(reinterpret_cast<const void *>(&bwd_dq_kernel),
                        dim3(((p.L + kDqRows - 1) / kDqRows) * (p.Hq / 4) * p.B), dim3(512), args, 0, stream) != hipSuccess)
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
