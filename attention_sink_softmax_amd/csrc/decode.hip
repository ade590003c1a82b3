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
// Work of one workgroup (4 waves, one per SIMD, the whole 160 KB of LDS): each wave walks
// its own 32-key slices of the split.  A slice's K (12 KB) and V (8 KB) go from HBM
// straight into a per-wave LDS buffer with 16-byte direct-to-LDS loads (no registers
// spent on staging), double buffered so the next slice is in flight while this one is
// computed.  The G query heads that share the KV head (up to 16) form the N dimension of
// v_mfma_f32_16x16x32_bf16, so every key byte read from HBM serves all of them:
//   S^T[16 keys][16 heads] = K Q^T    K from LDS (one contiguous 1 KB read per operand),
//                                     Q^T held in registers;
//   O^T[16 dv][16 heads]  += V^T P^T  P^T is the score tile itself (same lane layout),
//                                     V^T comes from the row-major V slice through the
//                                     transposing LDS read ds_read_b64_tr_b16.
// Row statistics need two lane exchanges (lane ^ 16, lane ^ 32).  At the end the 4 waves'
// states are merged through LDS.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "rope.h"
#include "sinkattn.h"

namespace sinkattn {

namespace {

constexpr int kWaves = 4;
constexpr int kSlice = 32;                           // keys per wave step
constexpr float kLazyRescale = 8.f;                  // log2 growth of a max that forces a rescale
constexpr int kKBytes = kSlice * kDqk * 2;           // 12 KB: 12 blocks of 1 KB
constexpr int kVBytes = kSlice * kDv * 2;            // 8 KB: 8 blocks of 1 KB
constexpr int kBufBytes = kKBytes + kVBytes;         // one slice
constexpr int kObRow = kDv + 4;                      // floats per column record in the wave merge
constexpr int kPart = kDv + 4;                       // partial record: o[128], m, l, 2 pad
constexpr int kDmaPerSlice = (kKBytes + kVBytes) / 1024;  // 20 wave-wide 1 KB loads
// 8-bit (E4M3) cache: the same slice in half the bytes
constexpr int kKBytes8 = kSlice * kDqk;                  // 6 KB
constexpr int kVBytes8 = kSlice * kDv;                   // 4 KB
constexpr int kBufBytes8 = kKBytes8 + kVBytes8;
constexpr int kDmaPerSlice8 = kBufBytes8 / 1024;         // 10

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Non-temporal loads, for data read once per call.  Over 4 GiB read in whole cache lines per
// instruction, MI355X streamed 7.1 TB/s with them against 6.3 TB/s with the default policy,
// for 16-byte loads into registers and into LDS alike.  Where an instruction reads only part
// of each line and later instructions read the rest, they lose the reuse of the line: the
// sliding-window prefill took 38% longer with its query and K/V loads non-temporal (and 3.4x
// with its output stores so), so only the decode cache loads here use them.
constexpr int kLoadNT = 2;  // cache-policy argument of the load-to-LDS builtins: nt
__device__ __forceinline__ u32x4 ldg16_nt(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Chunk swizzle of the bf16 K layout (below): key k of a 16-key block.
__device__ __forceinline__ int kswz(int k) { return (k >> 1) & 7; }

// E4M3 K of a 16-key block: 16 rows of 192 bytes, 3 KB, loaded by three instructions of 64
// lanes x 16 bytes.  Two keys 2p, 2p+1 span three whole 128-byte lines (A: key 2p chunks 0-7,
// B: key 2p chunks 8-11 and key 2p+1 chunks 0-3, C: key 2p+1 chunks 4-11); instruction i
// loads line A, B or C of all eight pairs, so every instruction reads whole lines.  Within an
// instruction, chunk c of key k has residue r = (k + c) mod 16 and goes to slot r + 16 t,
// t its rank among the four chunks of that residue there.  For a fixed chunk the 16 keys
// have 16 residues, so an operand read of 16 keys (8 bytes each for two lane groups) meets
// no bank twice in a 256-byte phase.
// Instruction i, lane l -> the key k and 16-byte chunk c it loads.
__device__ __forceinline__ void k8_lane_chunk(int i, int l, int &k, int &c) {
    const int r = l & 15, t = l >> 4;
    if (i == 0) c = 2 * t + (r & 1);
    else if (i == 1) c = t < 2 ? 8 + 2 * t + (r & 1) : 2 * (t - 2) + ((r + 1) & 1);
    else c = 4 + 2 * t + ((r + 1) & 1);
    k = (r - c) & 15;
}
// Byte offset of key k, chunk c within the 3 KB block (the inverse of k8_lane_chunk).
__device__ __forceinline__ int k8_off(int k, int c) {
    const int r = (k + c) & 15;
    int i, t;
    if ((k & 1) == 0) {
        i = c < 8 ? 0 : 1;
        t = c < 8 ? c >> 1 : (c - 8) >> 1;
    } else {
        i = c < 4 ? 1 : 2;
        t = c < 4 ? 2 + (c >> 1) : (c - 4) >> 1;
    }
    return i * 1024 + (r + 16 * t) * 16;
}

// 16 bytes per lane from global memory into LDS at dst + 16 * lane (dst wave-uniform), with
// cache policy AUX.  The cache is read once per step and every kernel here loads it
// non-temporal.  Measured on two boxes against the default policy: 1.3-2.7% faster for the
// paged bf16 cache at 8 x 256K, 0.6-1.8% for the E4M3 cache, 20% per call for the 128-slot
// rings at B = 128; the q_len = 4 verify was 0-3% slower while its K loads read half cache
// lines, and 3.9% faster once they read whole lines.
template <int AUX>
__device__ __forceinline__ void dma16(const void *src, char *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 16, 0, AUX);
}

// LDS layout of one slice (per wave, per buffer):
//   K: block 6 sb + 3 kh + c (1 KB) holds keys 16 sb + 8 kh .. +7 and bytes 128 c .. +127 of
//      their rows, one whole cache line per key, so each load instruction reads whole lines.
//      Key k (0..15 within the 16-key block) keeps its 16-byte chunk m of the line at slot
//      8 (k & 7) + (m ^ kswz(k)): the 16 lanes of an A-operand read (keys 0..15, one chunk)
//      hit 16 distinct 16-byte slots of a 256-byte bank phase.
//   V: block m = keys 4m .. 4m+3, 256 bytes each; row r keeps its 16-byte chunk c in slot
//      c ^ 2r ^ 8 (m & 1).  A transposing read takes 4 rows x 32 bytes of one block per
//      16-lane group, and the two groups that the banks serve together read blocks of
//      opposite parity, so the 32 lanes hit 32 distinct 8-byte bank slots of a 256-byte
//      phase (without the 8 (m & 1) term they met in pairs).

// 8-bit cache layout of one slice (per wave, per buffer):
//   K: for each 16-key half sb (3 KB), 16-byte chunk c (d = 16c .. 16c+15) of key k sits in
//      slot 16c + k, so an operand read (8 bytes: d = 32kk + 8q .. +8) of 16 keys x 2 halves
//      of one chunk covers 256 contiguous bytes.
//   V: key k (0..31) keeps 128 bytes, its 16-byte chunk c in slot c ^ vswz(k); the
//      transposing byte read gathers 8 keys x 16 dv per 16-lane group, and vswz spreads the
//      keys a group (and a pair of groups) reads over distinct banks.
__device__ __forceinline__ int vswz(int k) { return ((k >> 1) & 3) | ((k >> 2) & 4); }

// Eight E4M3 codes (two dwords, code i in byte i % 4 of dword i / 4) -> eight bf16, exactly
// (every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(v2i32 c) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c[0], 1.f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c[0], 1.f, true);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c[1], 1.f, false);
    const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c[1], 1.f, true);
    return bf16x8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
}

// Row of key j (general path): ring slot j, or page block_table[b][j / page_size].  With
// the new tokens' keys beside the cache (p.k_new), j is a position: positions from n - q_len
// on are rows of `side`, earlier ones ring slot j mod window or the page lookup.
__device__ __forceinline__ const uint16_t *kv_row(const DecodeParams &p, int b, int kvh, int j, const uint16_t *base,
                                                  const uint16_t *side, int width, int n, bool &bad) {
    if (p.k_new && j >= n - p.q_len)
        return side + (((size_t)b * p.Hkv + kvh) * p.q_len + (j - (n - p.q_len))) * width;
    if (!p.paged) return base + (((size_t)b * p.Hkv + kvh) * p.window + (p.k_new ? j % p.window : j)) * width;
    const int page = p.block_table[(size_t)b * p.max_pages + j / p.page_size];
    if (page < 0 || page >= p.num_pages) {
        bad = true;
        return base;
    }
    return base + (((size_t)page * p.Hkv + kvh) * p.page_size + (j % p.page_size)) * width;
}

// Keys that sequence b's queries can see, as the range the splits walk: [kbeg, kend).  The
// new queries sit at positions n - q_len .. n - 1; a ring enumerates its slots [0, min(n, W))
// (one query, every valid slot visible), except with the new tokens beside it, when keys are
// walked by position as in a paged cache.
__device__ __forceinline__ void key_range(const DecodeParams &p, int n, int &kbeg, int &kend) {
    if (!p.paged && !p.k_new) {
        kbeg = 0;
        kend = min(n, p.window);
    } else {
        kbeg = p.swa ? max(0, n - p.q_len - p.window + 1) : 0;
        kend = n;
    }
}

__device__ __forceinline__ bool seq_valid(const DecodeParams &p, int n) {
    const int cached = p.k_new ? n - p.q_len : n;  // positions the page table must cover
    return n >= 1 && n <= p.max_seq_len && (!p.paged || cached <= p.max_pages * p.page_size);
}

// Columns: the G * q_len (query head, new token) pairs of one KV head, column c = head-in-
// group * q_len + token; a workgroup takes NCB blocks of 16 columns, and every K and V
// fragment it reads from LDS feeds all NCB blocks (one pass over the cache per KV head).
//
// kSingle: every wave holds at most one slice (a split of at most 4 x 32 keys, e.g. a
// 128-slot ring).  Its K goes straight into registers (the direct-to-LDS layout below is
// lane-private: lane l writes exactly the 16 bytes it later reads as its MFMA operand) and
// only V passes through LDS, 34 KB per workgroup, so four workgroups share a CU and a whole
// batch of rings is in flight at once.
//
// kFp8: K and V are E4M3 codes (8-bit cache, fast paged layout only); they are converted to
// bf16 after the LDS read, the K scale is part of the logit scale and the V scale multiplies
// the unnormalised output.
//
// kStep (with kSingle): the decode step fused ("MiMo-V2-Flash 模型架构深度拆解", CH 10.3 forward
// steps 3-6 and the attention): the queries are rotated in registers (a lane holds both
// halves of its rotation pairs), and the wave whose slice holds the new token's slot loads
// the new key and value rows in place of that slot's old rows, rotates the key in
// registers, and writes both to the ring.  Bit-identical to the prologue kernel followed by
// the attention.
template <bool kFast, bool kSingle, int NCB, bool kFp8 = false, bool kStep = false>
__global__ __launch_bounds__(256, kSingle ? (kFast ? 4 : 2) : 1) void decode_split_kernel(DecodeParams p) {
    static_assert(!kFp8 || (kFast && !kSingle), "8-bit caches use the double-buffered fast path");
    static_assert(!kStep || (kFast && kSingle && NCB == 1 && !kFp8), "the fused step is a single-slice ring path");
    constexpr int kSliceBytes = kFp8 ? kBufBytes8 : kBufBytes;
    constexpr int kDma = kFp8 ? kDmaPerSlice8 : kDmaPerSlice;
    // slice buffers: even slices in bufA, odd ones in a second object (declared below, only
    // when a wave has more than one slice) so that the compiler can tell the loads in flight
    // into one from the reads of the other.  The single-slice buffer holds V only, plus room
    // for the merge's row statistics.
    constexpr int kBufA = kSingle ? kVBytes + 512 : kSliceBytes;
    __shared__ __attribute__((aligned(1024))) char bufA[kWaves][kBufA];
    static_assert((kWaves * 16 * kObRow + 2 * kWaves * 16 + kWaves) * 4 <= kWaves * kBufA,
                  "the wave merge's records fit in the slice buffers");

    const int split = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const int by = p.reverse ? gridDim.y - 1 - blockIdx.y : blockIdx.y;
    const int kvh = by % p.Hkv, hc = by / p.Hkv;
    const int b = p.reverse ? gridDim.z - 1 - blockIdx.z : blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hl = lane & 15, q = lane >> 4;  // column within a block, k-group
    // E4M3 cache: lane part of the K operand address of k-step kk (key hl, chunk 2 kk + q / 2,
    // byte half q & 1 of it), layout of k8_lane_chunk
    int k8lane[6];
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) k8lane[kk] = k8_off(hl, 2 * kk + (q >> 1)) + (q & 1) * 8;
    // lane part of the K operand address (layout of the K loads) for even and odd k-steps:
    // key hl of the 16-key block, chunk 4 (kk & 1) + q of line kk / 2
    const int klane[2] = {3072 * (hl >> 3) + (8 * (hl & 7) + (q ^ kswz(hl))) * 16,
                          3072 * (hl >> 3) + (8 * (hl & 7) + ((4 + q) ^ kswz(hl))) * 16};
    const int rows = p.G * p.q_len;

    const int n = p.seq_lens[b];
    int kbeg, kend;
    key_range(p, n, kbeg, kend);
    const bool seq_ok = seq_valid(p, n);
    // slices are aligned to 32 keys
    const int kb0 = kbeg & ~(kSlice - 1);
    const int s_lo = kb0 + split * p.chunk;
    const int s_hi = seq_ok ? min(kend, s_lo + p.chunk) : s_lo;  // empty when the length is invalid
    const int nslices = s_hi > s_lo ? (s_hi - s_lo + kSlice - 1) / kSlice : 0;
    const int nmine = nslices > wave ? (nslices - wave + kWaves - 1) / kWaves : 0;

    // this lane's columns: Q^T fragments (lane supplies q[32kk + 8q .. +8]) and the keys each
    // one sees, [lo_c, hi_c] within this split
    bf16x8 qf[NCB][6];
    int lo_c[NCB], hi_c[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int c = (hc * NCB + cb) * 16 + hl;
        const bool ok = c < rows;
        const int hq = kvh * p.G + (ok ? c / p.q_len : 0), tok = ok ? c % p.q_len : 0;
        const int pos = n - p.q_len + tok;
        const bool by_pos = p.paged || p.k_new;  // keys walked by position
        lo_c[cb] = max(kbeg, (by_pos && p.swa) ? pos - p.window + 1 : 0);
        hi_c[cb] = min(s_hi, by_pos ? pos + 1 : kend) - 1;
        const uint16_t *qrow = p.q + (((size_t)b * p.Hq + hq) * p.q_len + tok) * kDqk + 8 * q;
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) qf[cb][kk] = as_bf16x8(ok ? ldg16(qrow + 32 * kk) : u32x4{0, 0, 0, 0});
    }

    // fused step: the rotary angles of position n - 1 (the queries are rotated once the slice
    // has landed, next to the new key)
    __shared__ float rope_cs[kRopePairs], rope_sn[kRopePairs];
    if constexpr (kStep) {
        rope_angles(p.inv_freq, n - 1, rope_cs, rope_sn);
        __syncthreads();
    }
    // fused step: the new token's ring slot, and its key offset in this wave's slice
    const int slot_new = n >= 1 ? (n - 1) % max(p.window, 1) : -1;
    const int t_new = slot_new - (s_lo + kSlice * wave);
    const bool step_owner = kStep && n >= 1 && t_new >= 0 && t_new < kSlice;  // wave-uniform

    bool bad = false;

    // Page of each of this wave's slices (register r, lane i: slice 64 r + i), loaded before
    // the loop so that no table read sits between the direct-to-LDS loads (fast paged path).
    constexpr int kPageRegs = (kDecodeMaxChunk / (kSlice * kWaves) + 63) / 64;
    int page_reg[kPageRegs];
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r) {
        page_reg[r] = 0;
        if (kFast && p.paged && 64 * r + lane < nmine) {
            const int j0 = s_lo + kSlice * (wave + kWaves * (64 * r + lane));
            page_reg[r] = p.block_table[(size_t)b * p.max_pages + j0 / p.page_size];
        }
    }

    bf16x8 kreg[2][6];  // single-slice path: this wave's K operands
    // Issue the 20 loads of slice i (of this wave): K and V direct to LDS at `dst` (single-
    // slice path: K into kreg, V to `dst`).
    auto issue = [&](int i, char *dst) __attribute__((always_inline)) {
        const int j0 = s_lo + kSlice * (wave + kWaves * i);
        char *kb = dst;
        char *vb = kSingle ? dst : kb + kKBytes;
        const int r = lane >> 4, s = lane & 15;
        if (kFast) {
            // ring, or pages holding a multiple of 32 keys (one page per slice): rows
            // j0..j0+31 are contiguous; keys outside [kbeg, kend) read a clamped valid row
            // (their scores are masked)
            size_t row0;  // cache row of key offset 0 of this slice's page (or ring)
            int off0;
            if (p.paged) {
                int preg = page_reg[0];
#pragma unroll
                for (int r = 1; r < kPageRegs; ++r) preg = (i >> 6) == r ? page_reg[r] : preg;  // i is uniform
                const int page = __builtin_amdgcn_readlane(preg, i & 63);
                const bool ok = page >= 0 && page < p.num_pages;
                bad |= !ok;
                row0 = ((size_t)(ok ? page : 0) * p.Hkv + kvh) * p.page_size;
                off0 = j0 % p.page_size;
            } else {
                row0 = ((size_t)b * p.Hkv + kvh) * p.window;
                off0 = j0;
            }
            const uint16_t *kbase = p.k + row0 * kDqk, *vbase = p.v + row0 * kDv;
            const int lo = max(kbeg, j0) - j0, hi = min(kend, j0 + kSlice) - 1 - j0;  // valid key offsets
            if constexpr (kFp8) {
                // one byte per element: rows of kDqk and kDv bytes
                const uint8_t *kbase8 = reinterpret_cast<const uint8_t *>(p.k) + row0 * kDqk;
                const uint8_t *vbase8 = reinterpret_cast<const uint8_t *>(p.v) + row0 * kDv;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int i2 = 0; i2 < 3; ++i2) {
                        int kk8, c8;
                        k8_lane_chunk(i2, lane, kk8, c8);
                        const int t = min(max(16 * sb + kk8, lo), hi);
                        dma16<kLoadNT>(kbase8 + (size_t)(off0 + t) * kDqk + c8 * 16, kb + sb * 3072 + i2 * 1024);
                    }
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int key = 8 * m + (lane >> 3);
                    const int t = min(max(key, lo), hi);
                    dma16<kLoadNT>(vbase8 + (size_t)(off0 + t) * kDv + ((lane & 7) ^ vswz(key)) * 16,
                                             kb + kKBytes8 + m * 1024);
                }
                return;
            }
            if constexpr (kSingle) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const int t = min(max(16 * sb + s, lo), hi);
                    const uint16_t *kr = kbase + (size_t)(off0 + t) * kDqk + 8 * r;
                    // fused step: the new token's key (before rotation) in place of its slot's
                    // old row
                    if (kStep && step_owner && i == 0 && 16 * sb + s == t_new)
                        kr = p.k_step + ((size_t)b * p.Hkv + kvh) * kDqk + 8 * r;
#pragma unroll
                    for (int kk = 0; kk < 6; ++kk)
                        kreg[sb][kk] = as_bf16x8(ldg16_nt(kr + 32 * kk));
                }
            } else {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {
                        const int k16 = 8 * kh + (lane >> 3);
                        const int t = min(max(16 * sb + k16, lo), hi);
                        const uint16_t *kr = kbase + (size_t)(off0 + t) * kDqk + 8 * ((lane & 7) ^ kswz(k16));
#pragma unroll
                        for (int c = 0; c < 3; ++c)
                            dma16<kLoadNT>(kr + 64 * c, kb + (6 * sb + 3 * kh + c) * 1024);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int t = min(max(4 * m + r, lo), hi);
                const uint16_t *vr = vbase + (size_t)(off0 + t) * kDv;
                if (kStep && step_owner && i == 0 && 4 * m + r == t_new) vr = p.v_step + ((size_t)b * p.Hkv + kvh) * kDv;  // new value
                dma16<kLoadNT>(vr + 8 * (s ^ (2 * r) ^ (8 * (m & 1))), vb + m * 1024);
            }
        } else {
            const int lo = max(kbeg, j0), hi = min(kend, j0 + kSlice) - 1;
            if constexpr (kSingle) {
                // K rows looked up one by one, straight into the operand registers (lane (r, s):
                // key 16 sb + s, dimensions 32 kk + 8 r)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const int j = min(max(j0 + 16 * sb + s, lo), hi);
                    const uint16_t *kr = kv_row(p, b, kvh, j, p.k, p.k_new, kDqk, n, bad) + 8 * r;
#pragma unroll
                    for (int kk = 0; kk < 6; ++kk) kreg[sb][kk] = as_bf16x8(ldg16_nt(kr + 32 * kk));
                }
            } else {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {
                        const int k16 = 8 * kh + (lane >> 3);
                        const int j = min(max(j0 + 16 * sb + k16, lo), hi);
                        const uint16_t *kr =
                            kv_row(p, b, kvh, j, p.k, p.k_new, kDqk, n, bad) + 8 * ((lane & 7) ^ kswz(k16));
#pragma unroll
                        for (int c = 0; c < 3; ++c) dma16<kLoadNT>(kr + 64 * c, kb + (6 * sb + 3 * kh + c) * 1024);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int j = min(max(j0 + 4 * m + r, lo), hi);
                dma16<kLoadNT>(kv_row(p, b, kvh, j, p.v, p.v_new, kDv, n, bad) + 8 * (s ^ (2 * r) ^ (8 * (m & 1))),
                               vb + m * 1024);
            }
        }
    };

    // m: the reference the sums are kept against (log2 units of the scaled logits); thr =
    // (m + kLazyRescale) / scale, the growth threshold in raw-score units (the scale is
    // positive), moves only with m.
    float m_run[NCB], l_run[NCB], thr[NCB];
    f32x4 acc[NCB][8];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
        thr[cb] = -INFINITY;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Slice i: put slice i+1 in flight into `nxt`, wait for slice i, compute it from `cur`.
    auto step = [&](int i, const char *cur, char *nxt) __attribute__((always_inline)) {
        if (!kSingle && i + 1 < nmine) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of `nxt` are done
            issue(i + 1, nxt);
            // vmcnt(kDma): the loads just issued may stay in flight; slice i has landed
            __builtin_amdgcn_s_waitcnt(0x0F70 | (kDma & 15) | ((kDma >> 4) << 14));
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
        const char *kb = cur;
        const char *vb = kSingle ? cur : kb + (kFp8 ? kKBytes8 : kKBytes);
        const int j0 = s_lo + kSlice * (wave + kWaves * i);
        if constexpr (kStep) {
            // the queries: lane (hl, q) holds dimensions 8q .. 8q+7 in k-step 0 and their
            // rotation partners 32 + 8q .. in k-step 1
            {
                u32x4 lo, hi;
                rope_rotate8(__builtin_bit_cast(u32x4, qf[0][0]), __builtin_bit_cast(u32x4, qf[0][1]), 8 * q, rope_cs,
                             rope_sn, lo, hi);
                qf[0][0] = as_bf16x8(lo);
                qf[0][1] = as_bf16x8(hi);
            }
            if (step_owner && i == 0) {
                // the lanes that hold the new key (lane (r, s): key 16 sb + s, dimensions
                // 32 kk + 8 r) rotate it and write it to the ring; lane c < 16 moves chunk c
                // of the new value row from the V tile to the ring
                const int r = lane >> 4, s = lane & 15;
                const size_t ring_row = ((size_t)b * p.Hkv + kvh) * p.window + slot_new;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    if (16 * sb + s == t_new) {
                        u32x4 lo, hi;
                        rope_rotate8(__builtin_bit_cast(u32x4, kreg[sb][0]), __builtin_bit_cast(u32x4, kreg[sb][1]),
                                     8 * r, rope_cs, rope_sn, lo, hi);
                        kreg[sb][0] = as_bf16x8(lo);
                        kreg[sb][1] = as_bf16x8(hi);
                        uint16_t *kdst = const_cast<uint16_t *>(p.k) + ring_row * kDqk + 8 * r;
#pragma unroll
                        for (int kk = 0; kk < 6; ++kk)
                            *reinterpret_cast<u32x4 *>(kdst + 32 * kk) = __builtin_bit_cast(u32x4, kreg[sb][kk]);
                    }
                }
                if (lane < 16) {
                    const int m = t_new >> 2, rr = t_new & 3;
                    const u32x4 vv =
                        *reinterpret_cast<const u32x4 *>(vb + m * 1024 + rr * 256 + ((lane ^ (2 * rr) ^ (8 * (m & 1))) << 4));
                    *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(p.v) + ring_row * kDv + 8 * lane) = vv;
                }
            }
        }
        // ---- scores: S^T tiles of 16 keys x 16 columns
        f32x4 s[NCB][2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) s[cb][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 6; ++kk) {
                bf16x8 kf;
                if constexpr (kFp8)
                    kf = e4m3x8_to_bf16(*reinterpret_cast<const v2i32 *>(kb + sb * 3072 + k8lane[kk]));
                else
                    kf = kSingle ? kreg[sb][kk]
                                 : *reinterpret_cast<const bf16x8 *>(kb + (6 * sb + (kk >> 1)) * 1024 + klane[kk & 1]);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    s[cb][sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[cb][kk], s[cb][sb], 0, 0, 0);
            }
        }
        // lane holds keys j0 + 16sb + 4q + e for column hl of each block.  Keys outside a
        // column's range become -inf, on slices that cross some column's range only (a
        // wave-uniform test).
        bool inside = true;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) inside &= (j0 >= lo_c[cb]) & (j0 + kSlice - 1 <= hi_c[cb]);
        if (!__all(inside)) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = j0 + 16 * sb + 4 * q + e;
                        if (!((j >= lo_c[cb]) & (j <= hi_c[cb]))) s[cb][sb][e] = -INFINITY;
                    }
        }
        // The reference that the sums are kept against moves only when some column's max
        // grows by more than 2^kLazyRescale: the weights then stay below 2^kLazyRescale.  The
        // test compares each lane's largest raw score with the threshold; only the rare
        // rescale (a wave-uniform branch) forms the columns' maxima and keeps the
        // accumulators, the denominators and the reference consistent.
        float mxl[NCB];
        bool grow = false;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            float mx = fmaxf(s[cb][0][0], s[cb][0][1]);
#pragma unroll
            for (int e = 2; e < 8; e += 2) mx = fmaxf(fmaxf(mx, s[cb][e >> 2][e & 3]), s[cb][e >> 2][(e & 3) + 1]);
            mxl[cb] = mx;
            grow |= mx > thr[cb];
        }
        if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const float mnew = fmaxf(m_run[cb], max_xor32(max_xor16(mxl[cb])) * p.scale_log2);
                // an unchanged reference (including -inf, nothing visible yet) keeps alpha = 1
                const float alpha = (mnew == m_run[cb]) ? 1.f : exp2f_fast(m_run[cb] - mnew);
                l_run[cb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db) acc[cb][db] *= alpha;
                m_run[cb] = mnew;
                thr[cb] = (mnew + kLazyRescale) / p.scale_log2;
            }
        }
        bf16x8 pf[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const float neg = (m_run[cb] == -INFINITY) ? 0.f : -m_run[cb];
            float ps = 0.f;
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = exp2f_fast(__builtin_fmaf(s[cb][e >> 1][2 * (e & 1)], p.scale_log2, neg));
                const float p1 = exp2f_fast(__builtin_fmaf(s[cb][e >> 1][2 * (e & 1) + 1], p.scale_log2, neg));
                ps += p0 + p1;
                pk[e] = pack_bf16x2(p0, p1);
            }
            l_run[cb] += ps;
            pf[cb] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
        }

        // ---- O^T += V^T P^T; V^T through the transposing read: 16-lane group q, lane
        // 4r + c4 addresses row r (keys 4q + r, then 16 + 4q + r) at dv 16db + 4c4, and lane i
        // of the group receives dv 16db + i of the 4 rows
        const int r = hl >> 2, c4 = lane & 3;
        // 8-bit V: lane 2r8 + c2 of group q addresses key kr8 (rows r8 < 4: keys 4q + r8, then
        // 16 + 4q + r8 - 4) at dv 16db + 8c2, and lane i receives dv 16db + i of the 8 keys
        const int r8 = hl >> 1, c2 = hl & 1;
        const int kr8 = (r8 < 4) ? 4 * q + r8 : 12 + 4 * q + r8;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            bf16x8 vf;
            if constexpr (kFp8) {
                const v2i32 codes = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_v2i32 *)(vb + kr8 * 128 + (db ^ vswz(kr8)) * 16 + c2 * 8));
                vf = e4m3x8_to_bf16(codes);
            } else {
                const int c = 2 * db + (c4 >> 1);
                const int off = r * 256 + ((c ^ (2 * r) ^ (8 * (q & 1))) * 16) + (c4 & 1) * 8;  // blocks q, 4 + q
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + q * 1024 + off));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + (4 + q) * 1024 + off));
                vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                acc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[cb], acc[cb][db], 0, 0, 0);
        }
    };

    if (nmine > 0) issue(0, bufA[wave]);
    if constexpr (kSingle && kFast) {
        if (nmine > 0) step(0, bufA[wave], bufA[wave]);
    } else if constexpr (kSingle) {
        // one buffer: a wave's next slice (drafts beside a ring: at most two per wave) loads
        // after it has read the current one
        for (int i = 0; i < nmine; ++i) {
            if (i > 0) {
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of its V tile are done
                issue(i, bufA[wave]);
            }
            step(i, bufA[wave], bufA[wave]);
        }
    } else {
        __shared__ __attribute__((aligned(1024))) char bufB[kWaves][kSliceBytes];
        for (int i = 0; i < nmine; i += 2) {
            step(i, bufA[wave], bufB[wave]);
            if (i + 1 < nmine) step(i + 1, bufB[wave], bufA[wave]);
        }
    }

    // ---- merge the 4 waves' states through LDS (reusing the slice buffers), one block of
    // 16 columns at a time.  A column's record is padded to kObRow floats, so that the 16
    // lanes of a 16-byte write (16 columns, the same 4 dv) hit 16 distinct bank slots.
    const bool wave_bad = __any(bad);
    float *ob = reinterpret_cast<float *>(&bufA[0][0]);  // [4 waves][16 columns][kObRow]
    float *red_m = ob + kWaves * 16 * kObRow, *red_l = red_m + kWaves * 16, *red_bad = red_l + kWaves * 16;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const float lsum = sum_xor32(sum_xor16(l_run[cb]));
        __syncthreads();  // the slice buffers (or the previous block's records) are free
        if (q == 0) {
            red_m[wave * 16 + hl] = m_run[cb];
            red_l[wave * 16 + hl] = lsum;
        }
        if (lane == 0) red_bad[wave] = wave_bad ? 1.f : 0.f;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[(wave * 16 + hl) * kObRow + 16 * db + 4 * q + e] = acc[cb][db][e];
        __syncthreads();

        const bool any_bad = (red_bad[0] + red_bad[1] + red_bad[2] + red_bad[3]) != 0.f;
        // thread -> (column hh, 8 dv values)
        const int hh = tid >> 4, d0 = (tid & 15) * 8;
        const int c = (hc * NCB + cb) * 16 + hh;
        if (c < rows) {
            const int h2 = kvh * p.G + c / p.q_len, tok = c % p.q_len;
            const size_t row = ((size_t)b * p.Hq + h2) * p.q_len + tok;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * 16 + hh]);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = exp2f_fast(red_m[w * 16 + hh] - Mu);
                L += sc * red_l[w * 16 + hh];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += sc * ob[(w * 16 + hh) * kObRow + d0 + e];
            }
            if (p.nsplit == 1) {
                // final output: add the sink term once, normalise, scale, round to bf16; the
                // row's log-sum-exp (natural log) on request
                uint16_t *orow = p.out + row * kDv + d0;
                float res[8];
                const float sk = p.sink ? p.sink[h2] : -INFINITY;
                float lse;
                if (n - p.q_len + tok < 0) {  // no visible key: the sink alone
#pragma unroll
                    for (int e = 0; e < 8; ++e) res[e] = 0.f;
                    lse = sk;
                } else if (!seq_ok || any_bad) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) res[e] = __builtin_nanf("");
                    lse = __builtin_nanf("");
                } else if (sk == INFINITY) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) res[e] = 0.f;
                    lse = INFINITY;
                } else {
                    const float sl = sk * kLog2e;
                    const float M2 = fmaxf(M, sl);
                    const float sc = exp2f_fast(M - M2);
                    const float Lt = L * sc + (sk == -INFINITY ? 0.f : exp2f_fast(sl - M2));
                    const float inv = p.out_scale / Lt;
#pragma unroll
                    for (int e = 0; e < 8; ++e) res[e] = o[e] * sc * inv;
                    lse = (M2 + __builtin_amdgcn_logf(Lt)) * kLn2;
                }
                if (p.lse && (tid & 15) == 0) p.lse[row] = lse;
                *reinterpret_cast<u32x4 *>(orow) = u32x4{pack_bf16x2(res[0], res[1]), pack_bf16x2(res[2], res[3]),
                                                         pack_bf16x2(res[4], res[5]), pack_bf16x2(res[6], res[7])};
            } else {
                float *rec = p.ws + (row * p.nsplit + split) * kPart;
                *reinterpret_cast<f32x4 *>(rec + d0) = f32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<f32x4 *>(rec + d0 + 4) = f32x4{o[4], o[5], o[6], o[7]};
                if ((tid & 15) == 0) {
                    rec[kDv] = M;
                    rec[kDv + 1] = any_bad ? __builtin_nanf("") : L;
                }
            }
        }
    }
}

// One workgroup of 128 threads per (sequence, query head, new token): thread t owns output
// dim t.  Merges the splits' partials and adds the sink term once.
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
    __shared__ float red[128];
    const size_t row = p.reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x;  // (b * Hq + h) * q_len + token
    const int tok = (int)(row % p.q_len);
    const int h = (int)((row / p.q_len) % p.Hq), b = (int)(row / ((size_t)p.q_len * p.Hq));
    const int t = threadIdx.x;
    const int n = p.seq_lens[b];
    uint16_t *out = p.out + row * kDv + t;
    const bool seq_ok = seq_valid(p, n);
    const float sk = p.sink ? p.sink[h] : -INFINITY;
    if (n - p.q_len + tok < 0 || !seq_ok) {
        const bool before = n - p.q_len + tok < 0;  // no visible key: the sink alone
        *out = __builtin_bit_cast(uint16_t, (__bf16)(before ? 0.f : __builtin_nanf("")));
        if (p.lse && t == 0) p.lse[row] = before ? sk : __builtin_nanf("");
        return;
    }
    int kbeg, kend;
    key_range(p, n, kbeg, kend);
    const int kb0 = kbeg & ~(kSlice - 1);
    const int used = (kend - kb0 + p.chunk - 1) / p.chunk;  // splits that saw keys
    const float *base = p.ws + row * p.nsplit * kPart;


    const bool sink_inf = sk == INFINITY;
    const float sl = (sink_inf ? -INFINITY : sk) * kLog2e;  // an infinite sink is applied at the end
    float M = sl;
    for (int s = t; s < used; s += 128) M = fmaxf(M, base[(size_t)s * kPart + kDv]);
    red[t] = M;
    __syncthreads();
    for (int w = 64; w >= 1; w >>= 1) {
        if (t < w) red[t] = fmaxf(red[t], red[t + w]);
        __syncthreads();
    }
    M = red[0];
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = (sl == -INFINITY) ? 0.f : exp2f_fast(sl - Mu);
    float o = 0.f;
    int s = 0;
    for (; s + 4 <= used; s += 4) {
        float sc[4], lv[4], ov[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float *rec = base + (size_t)(s + u) * kPart;
            sc[u] = rec[kDv];
            lv[u] = rec[kDv + 1];
            ov[u] = rec[t];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float e = exp2f_fast(sc[u] - Mu);
            L += e * lv[u];  // a NaN sum marks an unreadable page and poisons L
            o += e * ov[u];
        }
    }
    for (; s < used; ++s) {
        const float *rec = base + (size_t)s * kPart;
        const float e = exp2f_fast(rec[kDv] - Mu);
        L += e * rec[kDv + 1];
        o += e * rec[t];
    }
    float r = o * (p.out_scale / L);
    if (sink_inf && !__builtin_isnan(L)) r = 0.f;
    *out = __builtin_bit_cast(uint16_t, (__bf16)r);
    if (p.lse && t == 0) p.lse[row] = sink_inf && !__builtin_isnan(L) ? INFINITY : (Mu + __builtin_amdgcn_logf(L)) * kLn2;
}

}  // namespace

// ---- scratch for the decode entry point that allocates nothing
//
// The split partials of that entry point live in this file-scope device array instead of a
// caller's workspace.  Each GPU the library runs on holds its own copy at its own address
// until the process ends; on the host the name only stands in for it, so the device address
// is looked up once per device (hipGetSymbolAddress, with that device current) and only that
// address reaches the kernels.  Calls on one GPU share the array: calls that overlap on a
// GPU race.  No part of it needs clearing: every split writes its whole record before the
// merge reads it.
constexpr size_t kScratchBytes = (size_t)SINKATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
float *scratch_ptr[kMaxDevices];  // device address of each device's copy, once looked up
}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

float *decode_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_ptr[dev] = static_cast<float *>(ptr);
    }
    return scratch_ptr[dev];
}

int launch_decode(const DecodeParams &prm, hipStream_t stream) {
    DecodeParams p = prm;
    p.reverse = grid_reversed();
    void *args[] = {&p};
    const dim3 grid(p.nsplit, p.Hkv * p.hchunks, p.B);
    // keys beside the cache take the general path (rows looked up one by one)
    const bool fast = !p.k_new && (!p.paged || (p.page_size % kSlice == 0));
    // a ring of at most 128 visible slots in one split: one slice per wave
    const bool single =
        !p.k_new && !p.paged && p.nsplit == 1 && p.ncb == 1 && min(p.window, p.max_seq_len) <= kWaves * kSlice;
    // drafts beside a ring, whose keys (window + q_len - 1, from a 32-aligned start) take at
    // most two slices per wave: K in registers, one slice buffer, two or more workgroups per CU
    const bool single_side = p.k_new && !p.paged && !p.fp8 && p.nsplit == 1 && p.ncb <= 2 &&
                             p.window + p.q_len - 1 + kSlice - 1 <= 2 * kWaves * kSlice;
    const void *fn;
    if (p.k_step) {
        // the fused decode step: a ring of at most 128 visible slots, one 16-column block
        if (!single || p.fp8 || p.q_len != 1) return -1;
        fn = reinterpret_cast<const void *>(&decode_split_kernel<true, true, 1, false, true>);
    } else if (p.fp8) {
        if (!p.paged || !fast) return -1;
        fn = p.ncb == 4   ? reinterpret_cast<const void *>(&decode_split_kernel<true, false, 4, true>)
             : p.ncb == 2 ? reinterpret_cast<const void *>(&decode_split_kernel<true, false, 2, true>)
                          : reinterpret_cast<const void *>(&decode_split_kernel<true, false, 1, true>);
    } else if (single) {
        fn = reinterpret_cast<const void *>(&decode_split_kernel<true, true, 1>);
    } else if (single_side) {
        fn = p.ncb == 2 ? reinterpret_cast<const void *>(&decode_split_kernel<false, true, 2>)
                        : reinterpret_cast<const void *>(&decode_split_kernel<false, true, 1>);
    } else if (fast) {
        fn = p.ncb == 4   ? reinterpret_cast<const void *>(&decode_split_kernel<true, false, 4>)
             : p.ncb == 2 ? reinterpret_cast<const void *>(&decode_split_kernel<true, false, 2>)
                          : reinterpret_cast<const void *>(&decode_split_kernel<true, false, 1>);
    } else {
        fn = p.ncb == 4   ? reinterpret_cast<const void *>(&decode_split_kernel<false, false, 4>)
             : p.ncb == 2 ? reinterpret_cast<const void *>(&decode_split_kernel<false, false, 2>)
                          : reinterpret_cast<const void *>(&decode_split_kernel<false, false, 1>);
    }
    if (hipLaunchKernel(fn, grid, dim3(256), args, 0, stream) != hipSuccess) return -1;
    if (p.nsplit > 1) {
        if (hipLaunchKernel(reinterpret_cast<const void *>(&decode_merge_kernel), dim3(p.B * p.Hq * p.q_len), dim3(128),
                            args, 0, stream) != hipSuccess)
            return -1;
    }
    return 0;
}

}  // namespace sinkattn
