// Prefill kernel: causal / sliding-window GQA attention with a per-head sink term in the
// softmax denominator, bf16 in, fp32 accumulate, bf16 out, for gfx950.
//
// Method: the sink softmax of "MiMo-V2-Flash 架构 QA" (Q3.7 max including the sink, Q3.8
// formula), computed as an online softmax over key tiles.  The sink enters by starting
// each row's running max at the sink logit and its running denominator at exp(0) = 1, so
// it is counted exactly once, never receives a value, and keeps every later rescale
// consistent.  Sliding-window rows only visit the key tiles that intersect their band
// (the chunk = window observation of Q3.6: a query needs at most its own and the previous
// chunk), causal rows only the tiles at or below the diagonal.
//
// Layout of the work (gfx950, wave64):
//   * Causal attention over a group of 8 or 16 query heads per KV head (the global layers):
//     a workgroup of 8 waves, one query head each, all at the same 32 query positions, so
//     one K / V^T tile staged in LDS feeds all eight; two waves share each SIMD and hide
//     each other's LDS waits.
//   * Sliding window (W <= 128, group a multiple of 8, whole sequence): the ring kernel below,
//     8 waves walking a run of consecutive query blocks with the band's keys kept in LDS.
//   * Everything else (other sliding-window shapes, chunked sliding-window prefill, other
//     group sizes): a workgroup of 4 waves, each owning HPW query heads (2 when the group
//     size is even and the mode causal) and 32 positions; with two heads per wave every K
//     and V fragment read from LDS feeds two MFMAs.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K comes
//     from LDS as the A operand, Q^T stays in registers as the B operand for the whole
//     kernel.  In the output layout a lane holds one query column and 16 key rows, so the
//     row statistics need only one exchange with the partner lane (lane ^ 32), and the
//     probabilities P^T are already in the B-operand layout of the second product
//     O^T = V^T P^T.
//   * A first, HBM-bound kernel writes V^T into the caller's workspace, tile by tile
//     (contiguous 16 KB blocks), with the keys of every 16-key group in MFMA k-order, so
//     the A operand of V^T P^T is one 16-byte LDS read per lane.  K and V^T tiles then
//     travel HBM -> LDS with 16-byte direct-to-LDS loads (no registers, no transposing in
//     the hot loop) into blocks of 16 rows x 4 chunks stored chunk-major: every 16-lane
//     group of an MFMA operand read is one contiguous 256-byte run (no bank conflicts) and
//     a lane's operand addresses differ only by compile-time offsets.  Tiles are double
//     (general kernel) or triple (causal kernel) buffered in distinct LDS objects, so the
//     loads of the next tiles overlap the math of the current one.
//   * Softmax: the logit scale is folded into one FMA per score (exp2 domain), and the
//     reference max moves, with a rescale of the output accumulator, only when a row's max
//     grows by more than 2^8 (the result is exact for any reference max; this only bounds
//     the size of the unnormalised terms).  The causal and ring kernels detect the growth
//     on the weights themselves (a lane whose 16 weights sum past 2^8) and form the row max
//     only inside the rare rescale; the general kernel takes the max of every sub-block.
//   * Sub-blocks fully inside every row's visible range take a branch-free path; diagonal
//     and band-edge sub-blocks take a masked path.
//   * Workgroup ids are remapped so that the workgroups sharing one KV head and position
//     block land on the same XCD (each XCD has its own L2), heaviest causal rows first.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kBQ = 32;    // query positions per wave
constexpr int kBN = 64;    // keys per LDS tile
constexpr int kKTileBytes = kBN * kDqk * 2;  // 24 KB
constexpr int kVTileBytes = kDv * kBN * 2;   // 16 KB
constexpr float kLazyRescale = 8.f;          // log2 growth of a row max that forces a rescale

typedef __attribute__((address_space(3))) void lds_void;

// ---- K tile layout: 24 blocks of 1 KB; block (rg, cg) holds rows 16rg..16rg+15 (keys) and
// 16-byte chunks 4cg..4cg+3 (8 consecutive d each); chunk c of row r sits in slot 16c + r.
// A 16-lane group of an MFMA operand read (16 consecutive rows, one chunk) is one
// contiguous 256-byte run, and for a fixed lane the offsets of all (sub-block, k-step)
// reads differ only by compile-time constants.
[[maybe_unused]] __device__ __forceinline__ int k_off(int row, int chunk) {
    return ((row >> 4) * 6 + (chunk >> 2)) * 1024 + ((chunk & 3) * 16 + (row & 15)) * 16;
}
// ---- V^T tile [128 dv][64 keys] of bf16: 16 blocks of 1 KB; block (rg, kg) holds dv rows
// 16rg..16rg+15 and key chunks 4kg..4kg+3 (8 keys each, in MFMA k-order); chunk c of row r
// sits in slot 16c + r.  Byte offsets.
[[maybe_unused]] __device__ __forceinline__ int vt_off(int row, int chunk) {
    return ((row >> 4) * 2 + (chunk >> 2)) * 1024 + ((chunk & 3) * 16 + (row & 15)) * 16;
}
// Key (within a 64-key tile) supplied as element e by lane group g for the 16-key group gam.
// In the 32x32 MFMA output a lane of group g holds, for register r, the key row
// 8*(r/4) + 4*g + r%4 of a 32-key block; the PV product consumes registers 0..7 and 8..15
// as two 16-key k-steps, so k-step gam, group g, element e is this key.  The transposed V
// copy stores chunk 2*gam + g of every 64-key tile in this order.
__device__ __forceinline__ int vkey(int gam, int g, int e) {
    return 16 * gam + ((e < 4) ? (4 * g + e) : (8 + 4 * g + (e - 4)));
}

struct WaveCtx {
    int L, swa, window;
    float c;  // logit scale * log2(e)
    int qpos0, qi, g, lq, lane;
    int klane, vlane;  // lane parts of the K and V^T operand offsets
};

// K tile rows kb..kb+63 -> LDS: block blk (0..23) = (rg, cg) is one wave instruction; lane l
// fetches row 16rg + (l & 15), chunk 4cg + (l >> 4) (four lanes read 64 contiguous bytes of
// each of 16 rows).  Rows past the sequence end are clamped to the last row (their scores
// are masked).
// The loads go through buffer resources (one per K or V^T region of a (batch, KV head)):
// a buffer load into LDS counts only towards vmcnt, so the LDS operand reads that overlap
// it can wait for each other one at a time (lgkmcnt(n)); a global load into LDS would make
// every such wait a wait for all of them.  An offset past the region reads zeros.
struct TileSrc {
    __amdgpu_buffer_rsrc_t k, vt;
};
__device__ __forceinline__ TileSrc tile_src(const PrefillParams &p, int b, int kvh) {
    constexpr int kRawDword3 = 0x00020000;  // untyped 32-bit data, no swizzle
    TileSrc t;
    t.k = __builtin_amdgcn_make_buffer_rsrc((void *)(p.k + ((size_t)b * p.Hkv + kvh) * p.L * kDqk), 0,
                                            p.L * (kDqk * 2), kRawDword3);
    t.vt = __builtin_amdgcn_make_buffer_rsrc((void *)(p.vt + ((size_t)b * p.Hkv + kvh) * kDv * p.lpad), 0,
                                             p.lpad * (kDv * 2), kRawDword3);
    return t;
}
__device__ __forceinline__ void dma_k_block(char *Kt, const TileSrc &src, int kb, int L, int blk, int lane) {
    const int rg = blk / 6, cg = blk % 6;
    const int row = min(kb + 16 * rg + (lane & 15), L - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, (lds_void *)(Kt + blk * 1024), 16,
                                             row * (kDqk * 2) + (4 * cg + (lane >> 4)) * 16, 0, 0, 0);
}
// V^T tile (keys kb..kb+63) -> LDS.  The transposed copy is stored tile by tile, each tile a
// contiguous 16 KB block [128 dv][64 keys], so a tile load touches one small address range.
// Block blk (0..15) = (rg, kg); lane l fetches dv row 16rg + (l & 15), key chunk
// 4kg + (l >> 4).
__device__ __forceinline__ void dma_vt_block(char *Vt, const TileSrc &src, int kb, int blk, int lane) {
    const int rg = blk >> 1, kg = blk & 1;
    const int row = 16 * rg + (lane & 15);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.vt, (lds_void *)(Vt + blk * 1024), 16,
                                             kb * (kDv * 2) + row * (kBN * 2) + (4 * kg + (lane >> 4)) * 16, 0, 0, 0);
}
// The same 16-byte loads into LDS, written as instructions the compiler does not interpret.
// In the causal kernel's loop the compiler cannot tell that the LDS reads after such a load
// read other buffers. With the builtin it waits for the load before them, which makes the
// load synchronous. Here it inserts no wait; the kernel waits itself (vmcnt(0)) before each
// barrier, and the data is read only after the barrier.
__device__ __forceinline__ void dma16_opaque(__amdgpu_buffer_rsrc_t r, char *lds, int voff) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)lds;
    uint32_t saved;
    // m0 carries the LDS address; one wait state between writing it and the load; m0 is
    // restored for the compiler's own use
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(base), "v"(voff), "s"(r)
        : "memory");
}
// Wave w issues blocks w, w+4, ... of the 24 K and 16 V^T blocks of a tile (10 per wave).
__device__ __forceinline__ void issue_tile(char *Kt, char *Vt, const TileSrc &src, int kb, int L, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 6; ++i) dma_k_block(Kt, src, kb, L, wave + 4 * i, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_vt_block(Vt, src, kb, wave + 4 * i, lane);
}

// ---- the four steps of a 32-key sub-block (keys kb + 32sb .. +31) for one wave

// S^T = K Q^T for each of the wave's heads.
template <int HPW>
__device__ __forceinline__ void qk_scores(const char *Kt, int sb, const bf16x8 (&qf)[HPW][12], f32x16 (&s)[HPW],
                                          const WaveCtx &w) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) s[h] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
        // = Kt + k_off(32 sb + lq, 2 kk + g): lane part plus a compile-time offset
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Kt + w.klane + (sb * 12288 + (kk >> 1) * 1024 + (kk & 1) * 512));
#pragma unroll
        for (int h = 0; h < HPW; ++h) s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[h][kk], s[h], 0, 0, 0);
    }
}

// Scores of keys outside row qi's visible range (or past the sequence end) become -inf.
// Lane register r holds key row 8*(r/4) + 4g + r%4 of the sub-block.
template <int HPW>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[HPW], int kb, int sb, const WaveCtx &w) {
    // visible keys of row qi: [lo, hi]; register r holds key base + c_r, c_r known at compile
    // time, so each test is two compares against lane constants (no branches)
    const int base = kb + 32 * sb + 4 * w.g;
    const int hi = min(w.qi, w.L - 1) - base;
    const int lo = (w.swa ? w.qi - w.window + 1 : INT32_MIN / 2) - base;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        const bool ok = (c >= lo) & (c <= hi);
#pragma unroll
        for (int h = 0; h < HPW; ++h) s[h][r] = ok ? s[h][r] : -INFINITY;
    }
}

// New running max from raw scores (the scale is positive); true when some row's max grew
// by more than 2^kLazyRescale (branch-free).
template <int HPW>
__device__ __forceinline__ bool row_max(const f32x16 (&s)[HPW], const float (&m_run)[HPW], float (&mnew)[HPW],
                                        const WaveCtx &w) {
    bool grow = false;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        // one v_max then seven v_max3
        float mx = __builtin_fmaxf(s[h][0], s[h][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[h][r]), s[h][r + 1]);
        mx = max_xor32(mx) * w.c;
        mnew[h] = fmaxf(m_run[h], mx);
        grow |= mnew[h] > m_run[h] + kLazyRescale;
    }
    return grow;
}

// The exponent offset of probs: -m, or 0 while a row has no reference yet (m = -inf).  Kept
// beside m and recomputed only when m moves.
template <int HPW>
__device__ __forceinline__ void neg_ref(const float (&m_run)[HPW], float (&neg)[HPW]) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) neg[h] = (m_run[h] == -INFINITY) ? 0.f : -m_run[h];
}

// Lazy rescale: when some row of the wave grew past the threshold, every row moves its
// reference to its new max and rescales its accumulator and denominator.
template <int HPW>
__device__ __forceinline__ void rescale(bool grow, const float (&mnew)[HPW], f32x16 (&acc)[HPW][4],
                                        float (&m_run)[HPW], float (&l_run)[HPW], float (&neg)[HPW]) {
    if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            // unchanged max (including a row with no visible key yet, -inf) keeps alpha = 1;
            // a first finite max after -inf gives 0
            const float alpha = (mnew[h] == m_run[h]) ? 1.f : exp2f_fast(m_run[h] - mnew[h]);
            l_run[h] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) acc[h][db] *= alpha;
            m_run[h] = mnew[h];
        }
        neg_ref<HPW>(m_run, neg);
    }
}

// Running max and lazy rescale together (general kernel).
template <int HPW>
__device__ __forceinline__ void row_update(const f32x16 (&s)[HPW], f32x16 (&acc)[HPW][4], float (&m_run)[HPW],
                                           float (&l_run)[HPW], float (&neg)[HPW], const WaveCtx &w) {
    float mnew[HPW];
    const bool grow = row_max<HPW>(s, m_run, mnew, w);
    rescale<HPW>(grow, mnew, acc, m_run, l_run, neg);
}

// P = 2^(c*s - m) rounded to bf16 in the B-operand layout of the PV product; l += sum(P).
// neg is neg_ref of the running max.
template <int HPW>
__device__ __forceinline__ void probs(const f32x16 (&s)[HPW], const float (&neg)[HPW], float (&l_run)[HPW],
                                      bf16x8 (&pf)[HPW][2], const WaveCtx &w) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        float ps;
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float p0 = exp2f_fast(__builtin_fmaf(s[h][2 * r], w.c, neg[h]));
            const float p1 = exp2f_fast(__builtin_fmaf(s[h][2 * r + 1], w.c, neg[h]));
            ps = r == 0 ? p0 + p1 : ps + (p0 + p1);
            pk[r] = pack_bf16x2(p0, p1);
        }
        l_run[h] += ps;
        pf[h][0] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
        pf[h][1] = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
        // computed here, not sunk past a following branch towards their use
        asm volatile("" : "+v"(pf[h][0]), "+v"(pf[h][1]), "+v"(l_run[h]));
    }
}

// O^T += V^T P^T.
template <int HPW>
__device__ __forceinline__ void pv_accum(const char *Vt, int sb, const bf16x8 (&pf)[HPW][2], f32x16 (&acc)[HPW][4],
                                         const WaveCtx &w) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            // = Vt + vt_off(32 db + lq, 4 sb + 2 k2 + g)
            const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(Vt + w.vlane + (db * 4096 + sb * 1024 + k2 * 512));
#pragma unroll
            for (int h = 0; h < HPW; ++h)
                acc[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[h][k2], acc[h][db], 0, 0, 0);
        }
    }
}

// One 64-key tile for one wave, sub-block by sub-block.  Sub-blocks wholly outside this
// wave's rows are skipped; sub-blocks wholly inside are not masked.
template <int HPW>
__device__ __forceinline__ void compute_tile(const char *Kt, const char *Vt, int kb, const bf16x8 (&qf)[HPW][12],
                                             f32x16 (&acc)[HPW][4], float (&m_run)[HPW], float (&l_run)[HPW],
                                             float (&neg)[HPW], const WaveCtx &w) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const int k0 = kb + 32 * sb;
        const bool dead = k0 > w.qpos0 + kBQ - 1 || k0 >= w.L || (w.swa && k0 + 31 < w.qpos0 - w.window + 1);
        if (dead) continue;
        const bool full = k0 + 31 <= w.qpos0 && k0 + 32 <= w.L && (!w.swa || k0 >= w.qpos0 + kBQ - w.window);
        f32x16 s[HPW];
        qk_scores<HPW>(Kt, sb, qf, s, w);
        if (!full) mask_scores<HPW>(s, kb, sb, w);
        row_update<HPW>(s, acc, m_run, l_run, neg, w);
        bf16x8 pf[HPW][2];
        probs<HPW>(s, neg, l_run, pf, w);
        pv_accum<HPW>(Vt, sb, pf, acc, w);
    }
}

// ---- per-wave setup shared by the kernels

struct WaveSetup {
    int b, kvh, h0, qpos0, wg_q0, wg_q1;
    bool valid;
};

// Workgroup -> (position group, batch, kv head, head group).  The mapping is XCD-aware: the
// hgroups workgroups that share one KV head and position group get ids that the hardware
// dispatches to the same XCD one after another; position groups run heaviest first.
template <int HPW>
__device__ __forceinline__ WaveSetup wave_setup(const PrefillParams &p, int wave) {
    WaveSetup ws;
    const int C = p.hgroups;
    const int bid = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int lam = (((slot / C) * 8 + xcd) * C) + slot % C;
    ws.valid = lam < p.n_items;
    int t = lam;
    const int hg = t % C;
    t /= C;
    ws.kvh = t % p.Hkv;
    t /= p.Hkv;
    ws.b = t % p.B;
    t /= p.B;
    const int pbw = p.n_pbw - 1 - t;
    const int wh = p.hw / HPW;  // waves along heads
    ws.h0 = ws.kvh * p.G + hg * p.hw + (wave % wh) * HPW;
    ws.qpos0 = p.q0 + (pbw * p.pw + wave / wh) * kBQ;
    ws.wg_q0 = p.q0 + pbw * p.pw * kBQ;
    ws.wg_q1 = min(p.L, ws.wg_q0 + p.pw * kBQ);
    return ws;
}

// Q^T fragments (B operand): lane supplies row qi - q0 of q[h], elements 16kk + 8g .. +8.
// A lane past the sequence end (or, in the ring kernel's first block of a chunk, before the
// chunk's first position) reads row 0 instead: its scores are finite, it never shares
// statistics with a valid row, and its output is never stored.  The loads are unconditional
// and their values used as they are, so the compiler waits for them only at their first use.
template <int HPW>
__device__ __forceinline__ void load_q(const PrefillParams &p, const WaveSetup &ws, const WaveCtx &w,
                                       bf16x8 (&qf)[HPW][12]) {
    const bool ok = w.qi >= p.q0 && w.qi < p.L;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        const uint16_t *qrow = p.q + ((((size_t)ws.b * p.Hq + ws.h0 + h) * p.Lq) + (ok ? w.qi - p.q0 : 0)) * kDqk + 8 * w.g;
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) qf[h][kk] = as_bf16x8(ldg16(qrow + 16 * kk));
    }
}

// The sink starts each row's running max and denominator: m = sink, l = exp(0) = 1 (counted
// on one lane of the pair that shares the row).  No sink: m = -inf, l = 0.
template <int HPW>
__device__ __forceinline__ void init_state_from(const float (&sink)[HPW], const WaveCtx &w, f32x16 (&acc)[HPW][4],
                                                float (&m_run)[HPW], float (&l_run)[HPW], bool (&sink_inf)[HPW],
                                                float (&neg)[HPW]) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        const float sk = sink[h];
        const bool has_sink = sk != -INFINITY;
        sink_inf[h] = sk == INFINITY;
        m_run[h] = has_sink ? sk * kLog2e : -INFINITY;
        l_run[h] = (has_sink && w.g == 0) ? 1.f : 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[h][db] = f32x16{};
    }
    neg_ref<HPW>(m_run, neg);
}
template <int HPW>
__device__ __forceinline__ void load_sink(const PrefillParams &p, const WaveSetup &ws, float (&sink)[HPW]) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) sink[h] = p.sink ? p.sink[ws.h0 + h] : -INFINITY;
}
template <int HPW>
__device__ __forceinline__ void init_state(const PrefillParams &p, const WaveSetup &ws, const WaveCtx &w,
                                           f32x16 (&acc)[HPW][4], float (&m_run)[HPW], float (&l_run)[HPW],
                                           bool (&sink_inf)[HPW], float (&neg)[HPW]) {
    float sink[HPW];
    load_sink<HPW>(p, ws, sink);
    init_state_from<HPW>(sink, w, acc, m_run, l_run, sink_inf, neg);
}

// O = out_scale * acc / l rounded to bf16; lane holds dv 32db + 8i + 4g + j of query qi (row
// qi - q0).  On request the row's log-sum-exp in natural log, (m + log2 l) ln 2: m is the
// reference the sums are kept against (log2 units of the scaled logits, the sink included).
template <int HPW>
__device__ __forceinline__ void store_out(const PrefillParams &p, const WaveSetup &ws, const WaveCtx &w, bool live,
                                          const f32x16 (&acc)[HPW][4], const float (&m_run)[HPW],
                                          const float (&l_run)[HPW], const bool (&sink_inf)[HPW]) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        const float lt = sum_xor32(l_run[h]);
        if (!live || w.qi >= p.L) continue;
        const float inv = p.out_scale / lt;
        const size_t row = (((size_t)ws.b * p.Hq + ws.h0 + h) * p.Lq) + (w.qi - p.q0);
        if (p.lse && w.g == 0) p.lse[row] = (m_run[h] + __builtin_amdgcn_logf(lt)) * kLn2;
        uint16_t *orow = p.out + row * kDv + 4 * w.g;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o0 = acc[h][db][4 * i] * inv, o1 = acc[h][db][4 * i + 1] * inv;
                float o2 = acc[h][db][4 * i + 2] * inv, o3 = acc[h][db][4 * i + 3] * inv;
                if (sink_inf[h]) o0 = o1 = o2 = o3 = 0.f;
                *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * i) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
            }
        }
    }
}

// store_out with the same stores on every path, for a loop that prefetches across it.  A
// branch around the stores makes the compiler's wait analysis assume the path without them,
// so a later wait for a prefetch issued before the stores would wait for the stores as well.
// Here every lane always issues its 16 output stores and one log-sum-exp store through a
// buffer resource spanning the rows of its (sequence, head); a row past the sequence end, a
// lane that does not own the log-sum-exp, or a missing log-sum-exp buffer (an empty range)
// gets an offset past the range, and the hardware drops such stores.
template <int HPW>
__device__ __forceinline__ void store_out_fixed(const PrefillParams &p, const WaveSetup &ws, const WaveCtx &w,
                                                const f32x16 (&acc)[HPW][4], const float (&m_run)[HPW],
                                                const float (&l_run)[HPW], const bool (&sink_inf)[HPW]) {
    constexpr int kRawDword3 = 0x00020000;  // untyped 32-bit data, no swizzle
    constexpr int kDropped = 0x40000000;    // past any range below
    const bool row_ok = w.qi >= p.q0 && w.qi < p.L;  // a row of this call's output
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        const float lt = sum_xor32(l_run[h]);
        const float inv = p.out_scale / lt;
        const size_t row0 = ((size_t)ws.b * p.Hq + ws.h0 + h) * p.Lq;
        const __amdgpu_buffer_rsrc_t orr =
            __builtin_amdgcn_make_buffer_rsrc(p.out + row0 * kDv, 0, p.Lq * (kDv * 2), kRawDword3);
        const __amdgpu_buffer_rsrc_t lrr =
            __builtin_amdgcn_make_buffer_rsrc(p.lse ? p.lse + row0 : nullptr, 0, p.lse ? p.Lq * 4 : 0, kRawDword3);
        const int ooff = row_ok ? (w.qi - p.q0) * (kDv * 2) + 8 * w.g : kDropped;
        const int loff = row_ok && w.g == 0 ? (w.qi - p.q0) * 4 : kDropped;
        const float lse = (m_run[h] + __builtin_amdgcn_logf(lt)) * kLn2;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lrr, loff, 0, 0);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o0 = acc[h][db][4 * i] * inv, o1 = acc[h][db][4 * i + 1] * inv;
                float o2 = acc[h][db][4 * i + 2] * inv, o3 = acc[h][db][4 * i + 3] * inv;
                if (sink_inf[h]) o0 = o1 = o2 = o3 = 0.f;
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)}, orr,
                                                      ooff + (32 * db + 8 * i) * 2, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ WaveCtx make_ctx(const PrefillParams &p, const WaveSetup &ws, int lane) {
    WaveCtx w;
    w.L = p.L;
    w.swa = p.swa;
    w.window = p.window;
    w.c = p.scale_log2;
    w.qpos0 = ws.qpos0;
    w.lane = lane;
    w.g = lane >> 5;
    w.lq = lane & 31;
    w.qi = ws.qpos0 + w.lq;
    // k_off and vt_off of the lane's operand reads split into a lane part (here) and a part
    // known at compile time, which the LDS read instructions take as an immediate offset
    w.klane = (w.lq >> 4) * 6144 + w.g * 256 + (w.lq & 15) * 16;
    w.vlane = (w.lq >> 4) * 2048 + w.g * 256 + (w.lq & 15) * 16;
    return w;
}

// ---- general kernel (sliding window, odd group sizes): double-buffered tiles, each
// sub-block computed start to finish.
template <int HPW>
__global__ __launch_bounds__(256, 3 - HPW) void prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(1024))) char KA[kKTileBytes];
    __shared__ __attribute__((aligned(1024))) char KB[kKTileBytes];
    __shared__ __attribute__((aligned(1024))) char VA[kVTileBytes];
    __shared__ __attribute__((aligned(1024))) char VB[kVTileBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const WaveSetup ws = wave_setup<HPW>(p, wave);
    if (!ws.valid) return;  // padding workgroup (uniform: before any barrier)
    const WaveCtx w = make_ctx(p, ws, lane);
    const bool wave_live = ws.qpos0 < p.L;

    bf16x8 qf[HPW][12];
    load_q<HPW>(p, ws, w, qf);
    float m_run[HPW], l_run[HPW], neg[HPW];
    bool sink_inf[HPW];
    f32x16 acc[HPW][4];
    init_state<HPW>(p, ws, w, acc, m_run, l_run, sink_inf, neg);

    const TileSrc src = tile_src(p, ws.b, ws.kvh);
    const int k_lo = p.swa ? max(0, ws.wg_q0 - p.window + 1) : 0;
    const int t0 = k_lo / kBN, t1 = (ws.wg_q1 - 1) / kBN;

    issue_tile(KA, VA, src, t0 * kBN, p.L, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // Tile kt from (Kc, Vc) while tile kt+1 streams into (Kn, Vn).
    auto step = [&](int kt, const char *Kc, const char *Vc, char *Kn, char *Vn) {
        const bool more = kt < t1;
        if (more) issue_tile(Kn, Vn, src, (kt + 1) * kBN, p.L, wave, lane);
        if (wave_live) compute_tile<HPW>(Kc, Vc, kt * kBN, qf, acc, m_run, l_run, neg, w);
        if (more) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile kt+1 has landed
        __syncthreads();
    };
    for (int kt = t0; kt <= t1; kt += 2) {
        step(kt, KA, VA, KB, VB);
        if (kt + 1 <= t1) step(kt + 1, KB, VB, KA, VA);
    }
    store_out<HPW>(p, ws, w, wave_live, acc, m_run, l_run, sink_inf);
}

// ---- causal kernel: eight waves, one head each, all at the same 32 positions (the eight
// heads of one KV head's group share every K and V^T tile), two waves per SIMD so that one
// wave's LDS waits and dependency stalls are filled by the other.  Each wave runs a
// software pipeline over 32-key sub-blocks so that the softmax arithmetic of one sub-block
// overlaps the matrix products of another:
//
//   phase A: S(t,1) = K(t)Q^T              with  P(t,0) = exp(S(t,0)), its test, the rare rescale
//   phase B: O += V(t)^T P(t,0)
//   barrier; tiles t+2 start streaming in
//   phase C: S(t+1,0) = K(t+1)Q^T          with  P(t,1) = exp(S(t,1)), its test, the rare rescale
//   phase D: O += V(t)^T P(t,1)
//
// K runs one tile ahead of V, so both are triple buffered (120 KB of LDS); loads issued
// after the barrier of tile t land by the barrier of tile t+1.  The loop is unrolled by 3
// so that every buffer is a distinct LDS object and the compiler can tell the loads in
// flight from the reads.  Every rescale happens after the PV product that used the old
// reference max, so the accumulator and the denominator always share one reference.
constexpr int kCausalWaves = 8;

// The tile of keys kb .. kb + 63 of one (sequence, KV head) as buffer resources that start at
// row kb, so that the lane part of every load is the same for all tiles.  K rows past the
// sequence end fall outside the K range and read zeros (their scores are masked); the V^T
// copy is padded to whole tiles.
__device__ __forceinline__ TileSrc tile_src_at(const PrefillParams &p, int b, int kvh, int kb) {
    constexpr int kRawDword3 = 0x00020000;  // untyped 32-bit data, no swizzle
    const size_t bh = (size_t)b * p.Hkv + kvh;
    TileSrc t;
    t.k = __builtin_amdgcn_make_buffer_rsrc((void *)(p.k + (bh * p.L + kb) * kDqk), 0, (p.L - kb) * (kDqk * 2),
                                            kRawDword3);
    t.vt = __builtin_amdgcn_make_buffer_rsrc((void *)(p.vt + bh * kDv * p.lpad + (size_t)kb * kDv), 0,
                                             (p.lpad - kb) * (kDv * 2), kRawDword3);
    return t;
}

// An LDS address in a register the compiler cannot see into.  Reads at constant distances from
// it take the distance as the instruction's 16-bit offset; from a known buffer address the
// compiler would add every offset above 64 KB with an instruction of its own.
__device__ __forceinline__ uint32_t lds_reg(const char *p) {
    uint32_t a = (uint32_t)(uintptr_t)(lds_void *)p;
    asm("" : "+v"(a));
    return a;
}
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
__device__ __forceinline__ bf16x8 lds_read16(uint32_t a, int off) { return *(lds_bf16x8 *)(a + off); }

// The weights P = 2^(c s - m) of one head's sub-block as probs() forms them, without adding
// them to the denominator; returns the lane's sum of its 16 weights.
__device__ __forceinline__ float weights(const f32x16 &s, float neg, bf16x8 (&pf)[1][2], const WaveCtx &w) {
    float ps;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float p0 = exp2f_fast(__builtin_fmaf(s[2 * r], w.c, neg));
        const float p1 = exp2f_fast(__builtin_fmaf(s[2 * r + 1], w.c, neg));
        ps = r == 0 ? p0 + p1 : ps + (p0 + p1);
        pk[r] = pack_bf16x2(p0, p1);
    }
    pf[0][0] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
    pf[0][1] = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
    return ps;
}
// The limit on a lane's weight sum that keeps the reference: 2^kLazyRescale, or -1 while the
// row has no reference yet (m = -inf), so that its first visible sub-block takes the rescale.
__device__ __forceinline__ float sum_limit(float m) { return m == -INFINITY ? -1.f : 256.f; }
static_assert(kLazyRescale == 8.f, "sum_limit holds 2^kLazyRescale");
// probs() with the lazy-rescale test on the weights themselves: while a lane's 16 weights sum
// to at most 2^kLazyRescale none of them exceeds it, and the reference stands.  Otherwise
// (some score grew past the reference by more than 4, or the row has no reference yet) the
// rare path forms the row max over both lanes of the pair, rescales the accumulator and the
// denominator (which does not hold this sub-block's weights yet), and forms the weights again.
__device__ __forceinline__ void probs_lazy(const f32x16 &s, f32x16 (&acc)[1][4], float (&m_run)[1],
                                           float (&l_run)[1], float (&neg)[1], float &limit, bf16x8 (&pf)[1][2],
                                           const WaveCtx &w) {
    float ps = weights(s, neg[0], pf, w);
    if (__builtin_expect(__any(!(ps <= limit)), 0)) {
        float mx = __builtin_fmaxf(s[0], s[1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[r]), s[r + 1]);
        float mnew[1] = {fmaxf(m_run[0], max_xor32(mx) * w.c)};
        rescale<1>(true, mnew, acc, m_run, l_run, neg);
        limit = sum_limit(m_run[0]);
        ps = weights(s, neg[0], pf, w);
    }
    l_run[0] += ps;
    // computed here, not sunk past a following branch towards their use
    asm volatile("" : "+v"(pf[0][0]), "+v"(pf[0][1]), "+v"(l_run[0]));
}

// qk_scores and pv_accum of one head reading through such registers: kr = K tile + klane,
// vr = V^T tile + vlane.
__device__ __forceinline__ void qk_scores_r(uint32_t kr, int sb, const bf16x8 (&qf)[1][12], f32x16 (&s)[1]) {
    s[0] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 12; ++kk)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read16(kr, sb * 12288 + (kk >> 1) * 1024 + (kk & 1) * 512),
                                                       qf[0][kk], s[0], 0, 0, 0);
}
__device__ __forceinline__ void pv_accum_r(uint32_t vr, int sb, const bf16x8 (&pf)[1][2], f32x16 (&acc)[1][4]) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read16(vr, db * 4096 + sb * 1024 + k2 * 512),
                                                                 pf[0][k2], acc[0][db], 0, 0, 0);
}

// Wave w of the causal kernel issues blocks w, w+8, ... of the 24 K and 16 V^T blocks.
__device__ __forceinline__ void dma_k_part(char *Kt, const TileSrc &src, int kb, int L, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 3; ++i) dma_k_block(Kt, src, kb, L, wave + kCausalWaves * i, lane);
}
__device__ __forceinline__ void dma_vt_part(char *Vt, const TileSrc &src, int kb, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma_vt_block(Vt, src, kb, wave + kCausalWaves * i, lane);
}

__global__ __launch_bounds__(64 * kCausalWaves, 1) void prefill_causal_kernel(PrefillParams p) {
    constexpr int HPW = 1;
    __shared__ __attribute__((aligned(1024))) char K0[kKTileBytes];
    __shared__ __attribute__((aligned(1024))) char K1[kKTileBytes];
    __shared__ __attribute__((aligned(1024))) char K2[kKTileBytes];
    __shared__ __attribute__((aligned(1024))) char V0[kVTileBytes];
    __shared__ __attribute__((aligned(1024))) char V1[kVTileBytes];
    __shared__ __attribute__((aligned(1024))) char V2[kVTileBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const WaveSetup ws = wave_setup<HPW>(p, wave);
    if (!ws.valid) return;  // padding workgroup (uniform: before any barrier)
    const WaveCtx w = make_ctx(p, ws, lane);

    bf16x8 qf[HPW][12];
    load_q<HPW>(p, ws, w, qf);
    float m_run[HPW], l_run[HPW], neg[HPW];
    bool sink_inf[HPW];
    f32x16 acc[HPW][4];
    init_state<HPW>(p, ws, w, acc, m_run, l_run, sink_inf, neg);

    const TileSrc src = tile_src(p, ws.b, ws.kvh);
    const int t1 = (ws.wg_q1 - 1) / kBN;  // tiles 0..t1

    // a sub-block needs masking when its last key lies past the first query row
    auto masked = [&](int t, int sb) { return t * kBN + 32 * sb + 31 > w.qpos0; };
    // lane parts of this wave's tile loads (K blocks wave + 8i, V^T blocks wave + 8j) against
    // resources that start at the tile's first row
    int kl[3], vl[2];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int blk = wave + kCausalWaves * i, rg = blk / 6, cg = blk % 6;
        kl[i] = (16 * rg + (lane & 15)) * (kDqk * 2) + (4 * cg + (lane >> 4)) * 16;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int blk = wave + kCausalWaves * j, rg = blk >> 1, kg = blk & 1;
        vl[j] = (16 * rg + (lane & 15)) * (kBN * 2) + (4 * kg + (lane >> 4)) * 16;
    }
    const uint32_t kr0 = lds_reg(K0 + w.klane), kr1 = lds_reg(K1 + w.klane), kr2 = lds_reg(K2 + w.klane);
    const uint32_t vr0 = lds_reg(V0 + w.vlane), vr1 = lds_reg(V1 + w.vlane), vr2 = lds_reg(V2 + w.vlane);

    dma_k_part(K0, src, 0, p.L, wave, lane);
    dma_vt_part(V0, src, 0, wave, lane);
    if (t1 >= 1) {
        dma_k_part(K1, src, kBN, p.L, wave, lane);
        dma_vt_part(V1, src, kBN, wave, lane);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    f32x16 s0[HPW], s1[HPW];
    bf16x8 pf[HPW][2];
    qk_scores<HPW>(K0, 0, qf, s0, w);
    if (masked(0, 0)) mask_scores<HPW>(s0, 0, 0, w);
    row_update<HPW>(s0, acc, m_run, l_run, neg, w);
    float limit = sum_limit(m_run[0]);

    // Tile t: K(t) in Kc, K(t+1) in Kn, V(t) in Vc; tiles t+2 go to (Kf, Vf).  The loads of
    // tile t+2 are issued unconditionally (past the last tile they re-read tile t1 into a
    // buffer nobody reads any more), so that no branch splits phases C and D.
    auto step = [&](int t, uint32_t Kc, uint32_t Kn, uint32_t Vc, char *Kf, char *Vf) {
        const int kb = t * kBN;
        const TileSrc nsrc = tile_src_at(p, ws.b, ws.kvh, min(t + 2, t1) * kBN);
        // phase A: S(t,1) with P(t,0) and its lazy-rescale test (after PV of P(t-1,1))
        qk_scores_r(Kc, 1, qf, s1);
        probs_lazy(s0[0], acc, m_run, l_run, neg, limit, pf, w);
        if (masked(t, 1)) mask_scores<HPW>(s1, kb, 1, w);
        // phase B: O += V(t)^T P(t,0)
        pv_accum_r(Vc, 0, pf, acc);
        // tiles t+1 have landed everywhere; the buffers of tiles t-1 (V) and t (K) are free
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        // phase C: S(t+1,0) with P(t,1) and its test, and the K loads of tile t+2 (the scores
        // of tile t+1 are unused after the last tile)
        qk_scores_r(Kn, 0, qf, s0);
        probs_lazy(s1[0], acc, m_run, l_run, neg, limit, pf, w);
#pragma unroll
        for (int i = 0; i < 3; ++i) dma16_opaque(nsrc.k, Kf + (wave + kCausalWaves * i) * 1024, kl[i]);
        if (t < t1 && masked(t + 1, 0)) mask_scores<HPW>(s0, kb + kBN, 0, w);
        // phase D: O += V(t)^T P(t,1) and the V^T loads of tile t+2
        pv_accum_r(Vc, 1, pf, acc);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_opaque(nsrc.vt, Vf + (wave + kCausalWaves * i) * 1024, vl[i]);
    };
    for (int t = 0; t <= t1; t += 3) {
        step(t, kr0, kr1, vr0, K2, V2);
        if (t + 1 <= t1) step(t + 1, kr1, kr2, vr1, K0, V0);
        if (t + 2 <= t1) step(t + 2, kr2, kr0, vr2, K1, V1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the workgroup
    store_out<HPW>(p, ws, w, true, acc, m_run, l_run, sink_inf);
}

// ---- sliding-window ring kernel (window <= 128, group size a multiple of 8, whole-sequence
// prefill).  A workgroup of 8 waves, one query head each, owns a run of consecutive 32-position
// blocks of one (sequence, KV head, 8 heads).  The keys a block sees, [32j - W + 1, 32j + 31],
// lie in the five 32-key sub-blocks j - 4 .. j, so K and V^T stay in LDS as a ring of six
// sub-blocks: each step computes block j from five of them while sub-block j + 1 and the next
// block's queries load, and every K/V row is read from HBM once per run.  The queries and
// outputs, which are most of the traffic, stream with a step of latency to hide behind.
// Two waves per SIMD overlap each other's softmax with their products.
constexpr int kSwaWaves = 8;
constexpr int kRingSlots = 6;
constexpr int kSubKBytes = 32 * kDqk * 2;  // 12 KB: rows of a K tile's first 32 keys
constexpr int kSubVBytes = 32 * kDv * 2;   // 8 KB: V [32 keys][128 dv]
constexpr int kSlotBytes = kSubKBytes + kSubVBytes;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// V rows of a sub-block in LDS, row-major [32 keys][128 dv] with 16-byte chunk c of key row r
// at chunk c ^ vswz(r).  The banks serve 256 bytes per cycle and every 256-byte row starts on
// the same bank, so vswz takes 16 distinct values over any 16 aligned rows (a 16-lane row
// write) and 4 distinct values of bits 2-3 over any 4 aligned rows (the 4 rows x 4 adjacent
// chunks of a 32-lane transposing read).
__device__ __forceinline__ int vswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int v_off(int r, int c) { return r * (kDv * 2) + ((c ^ vswz(r)) << 4); }

// One 32-key sub-block, global -> registers: K chunk idx lands at byte 16 idx of the K part in
// the K tile layout (rows 0..31); thread t also moves chunk t & 15 of V row t >> 4, stored at
// v_off.  Thread t moves K chunks t and 512 + t (t < 256); every thread issues the same three
// loads (the second K load of threads 256 .. 511 is not stored), so the number in flight is
// the same on every path.  Rows past the sequence end read the last row (their weights are 0).
struct SubStage {
    u32x4 k0, k1, v;
};
// Row `row` (0 .. L-1) of K or V: from k / v, or (kPrefix: a ring-cache prefix read in place)
// rows below q0 from the ring and the rest from the chunk's rows.
template <bool kPrefix>
__device__ __forceinline__ const uint16_t *kv_src(const PrefillParams &p, const uint16_t *chunk,
                                                  const uint16_t *prefix, int width, size_t bkv, int row) {
    if constexpr (!kPrefix) return chunk + (bkv * p.L + row) * width;
    if (row < p.q0) return prefix + (bkv * p.prefix_w + (p.prefix_base + row) % p.prefix_w) * width;
    return chunk + (bkv * p.Lq + (row - p.q0)) * width;
}
template <bool kPrefix>
__device__ __forceinline__ void sub_load(SubStage &st, const PrefillParams &p, int b, int kvh, int sub, int tid) {
    const size_t bkv = (size_t)b * p.Hkv + kvh;
    auto kchunk = [&](int idx) {
        const int blk = idx >> 6, l = idx & 63;
        const int row = min(32 * sub + 16 * (blk / 6) + (l & 15), p.L - 1);
        return ldg16(kv_src<kPrefix>(p, p.k, p.prefix_k, kDqk, bkv, row) + (4 * (blk % 6) + (l >> 4)) * 8);
    };
    st.k0 = kchunk(tid);
    st.k1 = kchunk(512 + (tid & 255));
    const int vrow = min(32 * sub + (tid >> 4), p.L - 1);
    st.v = ldg16(kv_src<kPrefix>(p, p.v, p.prefix_v, kDv, bkv, vrow) + (tid & 15) * 8);
}
__device__ __forceinline__ void sub_store(const SubStage &st, char *slot, int tid) {
    *reinterpret_cast<u32x4 *>(slot + 16 * tid) = st.k0;
    if (tid < 256) *reinterpret_cast<u32x4 *>(slot + 16 * (512 + tid)) = st.k1;
    *reinterpret_cast<u32x4 *>(slot + kSubKBytes + v_off(tid >> 4, tid & 15)) = st.v;
}

// O^T += V^T P^T from the V rows of a sub-block (layout of sub_store).  The A operand of
// k-step k2 is, for lane (g, dv row 32 db + lq), V at the keys that P^T's registers hold:
// 16 k2 + {4g .. 4g + 3} and 16 k2 + 8 + {4g .. 4g + 3}.  Two transposing reads give them:
// in a 16-lane group, lane 4r + c4 addresses key row r and dv columns 4 c4 .. +3 of its
// 16-column block, and lane i receives dv column i of the 4 rows.
__device__ __forceinline__ void pv_sub(const char *Vs, const bf16x8 (&pf)[1][2], f32x16 (&acc)[1][4], const WaveCtx &w) {
    const int gl = (w.lane >> 4) & 1, i = w.lane & 15, r = i >> 2, c4 = i & 3;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int col = 32 * db + 16 * gl + 4 * c4;
        const int chunk = col >> 3, half = (col >> 2) & 1;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int r0 = 16 * k2 + 4 * w.g + r;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(Vs + v_off(r0, chunk) + 8 * half));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(Vs + v_off(r0 + 8, chunk) + 8 * half));
            const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[0][k2], acc[0][db], 0, 0, 0);
        }
    }
}

template <bool kPrefix>
__global__ __launch_bounds__(64 * kSwaWaves, 1) void prefill_swa_kernel(PrefillParams p) {
    constexpr int HPW = 1;
    __shared__ __attribute__((aligned(1024))) char ring[kRingSlots * kSlotBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroup -> (chunk of blocks, batch, KV head, group of 8 heads).  Query blocks are
    // 32 positions of the sequence, from the block holding the first query row q0 (rows
    // before q0 in that block are computed but not stored) to the last.
    const int nqb = (p.L + kBQ - 1) / kBQ, jb0 = p.q0 / kBQ;
    const int nchunk = (nqb - jb0 + p.chunk - 1) / p.chunk;
    int u = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const int hg = u % p.hgroups;
    u /= p.hgroups;
    const int kvh = u % p.Hkv;
    u /= p.Hkv;
    const int b = u % p.B;
    const int c = u / p.B;
    if (c >= nchunk) return;  // uniform: before any barrier
    const int j_lo = jb0 + c * p.chunk, j_hi = min(nqb, j_lo + p.chunk);

    WaveSetup ws;
    ws.b = b;
    ws.kvh = kvh;
    ws.h0 = kvh * p.G + hg * kSwaWaves + wave;
    ws.valid = true;
    auto setup_block = [&](int j) {
        ws.qpos0 = kBQ * j;
        ws.wg_q0 = ws.qpos0;
        ws.wg_q1 = min(p.L, ws.qpos0 + kBQ);
        return make_ctx(p, ws, lane);
    };

    // the sub-blocks of the first block's band
    {
        SubStage st[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int sub = j_lo - 4 + i;
            if (sub >= 0) sub_load<kPrefix>(st[i], p, b, kvh, sub, tid);
        }
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int sub = j_lo - 4 + i;
            if (sub >= 0) sub_store(st[i], ring + (sub % kRingSlots) * kSlotBytes, tid);
        }
    }
    bf16x8 qa[HPW][12], qb[HPW][12];
    float sink[HPW];  // loaded once: a load inside the loop would wait for the prefetches
    load_sink<HPW>(p, ws, sink);
    {
        const WaveCtx w0 = setup_block(j_lo);
        load_q<HPW>(p, ws, w0, qa);
    }
    // Nothing may stay in flight into the loop: the compiler's wait analysis merges the
    // conditional prologue loads into every later use and would wait for all loads (the
    // prefetches included) in each step.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // The loads for the next step are unconditional (the last step of a run reloads its own
    // block and the last sub-block of the sequence into places nobody reads again), so the
    // compiler can count them exactly and wait for nothing but what each use needs.
    auto step = [&](int j, const bf16x8 (&qc)[HPW][12], bf16x8 (&qn)[HPW][12]) {
        SubStage st;
        sub_load<kPrefix>(st, p, b, kvh, min(j + 1, nqb - 1), tid);
        {
            const WaveCtx wn = setup_block(min(j + 1, j_hi - 1));
            load_q<HPW>(p, ws, wn, qn);
        }
        const WaveCtx w = setup_block(j);
        float m_run[HPW], l_run[HPW], neg[HPW];
        bool sink_inf[HPW];
        f32x16 acc[HPW][4];
        init_state_from<HPW>(sink, w, acc, m_run, l_run, sink_inf, neg);
        float limit = sum_limit(m_run[0]);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int sub = j - 4 + i, k0 = kBQ * sub;
            const bool dead = sub < 0 || k0 >= p.L || k0 + 31 < w.qpos0 - p.window + 1;
            if (dead) continue;
            const bool full = k0 + 31 <= w.qpos0 && k0 + 32 <= p.L && k0 >= w.qpos0 + kBQ - p.window;
            const char *slot = ring + (sub % kRingSlots) * kSlotBytes;
            f32x16 sc[HPW];
            qk_scores<HPW>(slot, 0, qc, sc, w);
            if (!full) mask_scores<HPW>(sc, k0, 0, w);
            bf16x8 pf[HPW][2];
            probs_lazy(sc[0], acc, m_run, l_run, neg, limit, pf, w);
            pv_sub(slot + kSubKBytes, pf, acc, w);
        }
        // slot (j + 1) % 6 held sub-block j - 5, outside this block's band
        sub_store(st, ring + ((j + 1) % kRingSlots) * kSlotBytes, tid);
        store_out_fixed<HPW>(p, ws, w, acc, m_run, l_run, sink_inf);
        __syncthreads();
    };
    for (int j = j_lo; j < j_hi; j += 2) {
        step(j, qa, qb);
        if (j + 1 < j_hi) step(j + 1, qb, qa);
    }
}

// V -> V^T tile by tile: tile t of (batch, kv head) is a contiguous [128 dv][64 keys] block
// with the keys of every 16-key group in MFMA k-order (chunk 2*gam + g holds the keys
// vkey(gam, g, 0..7)); keys past L are zero.  One workgroup per (batch x kv head, tile).
__global__ __launch_bounds__(256) void transpose_v_kernel(const uint16_t *v, uint16_t *vt, int L, int lpad) {
    __shared__ uint16_t tile[kBN][kDv + 8];
    const int kb = blockIdx.x * kBN;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const uint16_t *src = v + bh * (size_t)L * kDv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;
        const int key = idx >> 4, c = idx & 15;
        const u32x4 val = kb + key < L ? ldg16(src + (size_t)(kb + key) * kDv + 8 * c) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x2 *>(&tile[key][8 * c]) = u32x2{val.x, val.y};
        *reinterpret_cast<u32x2 *>(&tile[key][8 * c + 4]) = u32x2{val.z, val.w};
    }
    __syncthreads();
    uint16_t *dst = vt + (bh * (size_t)lpad + kb) * kDv;  // this tile's block
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;
        const int row = idx >> 3, kc = idx & 7;
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = tile[vkey(kc >> 1, kc & 1, 2 * i)][row];
            const uint32_t hi = tile[vkey(kc >> 1, kc & 1, 2 * i + 1)][row];
            wv[i] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4 *>(dst + row * kBN + 8 * kc) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
}

// Keys and values of positions base + r, r < Lc, into contiguous rows: 16 rows of one
// (sequence, KV head) per workgroup, 16-byte chunks, consecutive threads on consecutive chunks
// of a row.  A prefix position whose page id lies outside the pool gets a zero key and NaN
// values, so every output row that sees it is NaN.
__global__ __launch_bounds__(256) void gather_prefix_kernel(GatherParams g) {
    constexpr int kKC = kDqk / 8, kVC = kDv / 8;  // 16-byte chunks per row
    const int r0 = blockIdx.x * 16;
    const int bh = blockIdx.y, b = bh / g.Hkv, kvh = bh % g.Hkv;
    for (int idx = threadIdx.x; idx < 16 * (kKC + kVC); idx += 256) {
        const bool is_k = idx < 16 * kKC;
        const int w = is_k ? kKC : kVC;
        const int rel = is_k ? idx : idx - 16 * kKC;
        const int r = r0 + rel / w, c = rel % w;
        if (r >= g.Lc) continue;
        const int pos = g.base + r;
        const int width = is_k ? kDqk : kDv;
        const uint16_t *src;
        bool bad = false;
        if (pos >= g.q0) {
            src = (is_k ? g.k_chunk : g.v_chunk) + ((size_t)bh * g.Lq + (pos - g.q0)) * width;
        } else if (!g.paged) {
            src = (is_k ? g.k_cache : g.v_cache) + ((size_t)bh * g.window + pos % g.window) * width;
        } else {
            const int page = g.block_table[(size_t)b * g.max_pages + pos / g.page_size];
            bad = page < 0 || page >= g.num_pages;
            src = (is_k ? g.k_cache : g.v_cache) +
                  (((size_t)(bad ? 0 : page) * g.Hkv + kvh) * g.page_size + pos % g.page_size) * width;
        }
        u32x4 val = bad ? u32x4{0, 0, 0, 0} : ldg16(src + 8 * c);
        if (bad && !is_k) val = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};  // bf16 NaN
        *reinterpret_cast<u32x4 *>((is_k ? g.k_out : g.v_out) + ((size_t)bh * g.Lc + r) * width + 8 * c) = val;
    }
}

}  // namespace

int launch_gather_prefix(const GatherParams &g, hipStream_t stream) {
    if (g.Lc <= 0 || g.B * g.Hkv <= 0) return 0;
    GatherParams gp = g;
    void *args[] = {&gp};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gather_prefix_kernel), dim3((g.Lc + 15) / 16, g.B * g.Hkv),
                           dim3(256), args, 0, stream) == hipSuccess ? 0 : -1;
}

namespace {
bool causal_layout(const PrefillParams &p) { return !p.swa && p.hpw == 1 && p.hw == kCausalWaves; }
// Compute units of the current device (256 on a whole MI355X, fewer on a partition); only the
// length of the ring kernel's runs depends on it.
int compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}
}  // namespace

// Causal mode with a group size divisible by 8: the eight-wave kernel, one head per wave.
// Otherwise the general kernel, with as many waves along heads as divide the group (at most
// 4) and the rest along positions: one head per wave in sliding-window mode (two workgroups
// share a CU, so one's loads overlap the other's math on this short, memory-bound work), two
// heads per wave for causal attention over an even group (half the LDS reads per MFMA).
int64_t plan_prefill(PrefillParams &p) {
    p.ring = 0;
    p.chunk = 0;
    if (p.swa && p.window <= 128 && p.G % kSwaWaves == 0) {
        // ring kernel: runs of consecutive blocks, about one workgroup per compute unit
        p.ring = 1;
        p.hpw = 1;
        p.hw = kSwaWaves;
        p.pw = 1;
        p.hgroups = p.G / kSwaWaves;
        const int64_t units = (int64_t)p.B * p.Hkv * p.hgroups;
        const int64_t nqb = (p.L + 31) / 32 - p.q0 / 32;  // query blocks from the one holding q0
        const int64_t cus = compute_units();
        const int64_t split = std::max<int64_t>(1, std::min<int64_t>(nqb, (cus + units - 1) / units));
        p.chunk = (int)((nqb + split - 1) / split);
        p.n_pbw = (int)((nqb + p.chunk - 1) / p.chunk);
        const int64_t items = units * p.n_pbw;
        p.n_items = items > INT32_MAX ? INT32_MAX : (int)items;
        return items;
    }
    if (!p.swa && p.G % kCausalWaves == 0) {
        p.hpw = 1;
        p.hw = kCausalWaves;
        p.pw = 1;
    } else {
        p.hpw = (!p.swa && p.G % 2 == 0) ? 2 : 1;
        p.hw = p.hpw;
        while (p.hw * 2 <= 4 * p.hpw && p.G % (p.hw * 2) == 0) p.hw *= 2;
        p.pw = 4 * p.hpw / p.hw;
    }
    const int64_t npb = (p.Lq + 31) / 32;
    p.n_pbw = (int)((npb + p.pw - 1) / p.pw);
    p.hgroups = p.G / p.hw;
    const int64_t items = (int64_t)p.n_pbw * p.B * p.Hkv * p.hgroups;
    p.n_items = items > INT32_MAX ? INT32_MAX : (int)items;
    return ((items + 8 * p.hgroups - 1) / (8 * p.hgroups)) * 8 * p.hgroups;
}

size_t prefill_workspace_bytes(int B, int Hkv, int L) {
    const size_t lpad = ((size_t)L + kBN - 1) / kBN * kBN;
    return (size_t)B * Hkv * kDv * lpad * 2;
}

int grid_reversed() {
    const char *e = getenv("SINKATTN_GRID_ORDER");
    return e && strcmp(e, "reversed") == 0;
}

int launch_prefill(const PrefillParams &prm, hipStream_t stream) {
    PrefillParams p = prm;
    p.reverse = grid_reversed();
    if (!p.ring) {  // the ring kernel reads V rows directly
        void *targs[] = {(void *)&p.v, (void *)&p.vt, (void *)&p.L, (void *)&p.lpad};
        if (hipLaunchKernel(reinterpret_cast<const void *>(&transpose_v_kernel), dim3(p.lpad / kBN, p.B * p.Hkv),
                            dim3(256), targs, 0, stream) != hipSuccess)
            return -1;
    }
    void *args[] = {&p};
    if (p.ring)
        return hipLaunchKernel(p.prefix_k ? reinterpret_cast<const void *>(&prefill_swa_kernel<true>)
                                          : reinterpret_cast<const void *>(&prefill_swa_kernel<false>),
                               dim3(p.n_items),
                               dim3(64 * kSwaWaves), args, 0, stream) == hipSuccess ? 0 : -1;
    const int grid = ((p.n_items + 8 * p.hgroups - 1) / (8 * p.hgroups)) * 8 * p.hgroups;
    if (causal_layout(p)) {
        return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_causal_kernel), dim3(grid),
                               dim3(64 * kCausalWaves), args, 0, stream) == hipSuccess ? 0 : -1;
    }
    const void *fn = p.hpw == 2 ? reinterpret_cast<const void *>(&prefill_kernel<2>)
                                : reinterpret_cast<const void *>(&prefill_kernel<1>);
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, stream) == hipSuccess ? 0 : -1;
}

}  // namespace sinkattn
