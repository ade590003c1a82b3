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
//   * A workgroup is 4 waves.  Each wave owns one query head and 32 consecutive query
//     positions.  The 4 waves share one KV head (grouped-query attention), so one key/value
//     tile staged in LDS feeds all of them.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K comes
//     from LDS as the A operand, Q^T stays in registers as the B operand for the whole
//     kernel.  In the output layout a lane holds one query column and 16 key rows, so the
//     row statistics need only one exchange with the partner lane (lane ^ 32), and the
//     probabilities P^T are already in the B-operand layout of the second product
//     O^T = V^T P^T (no shuffle of P through LDS).
//   * V is transposed in registers (8x8 blocks of bf16) on its way into LDS, so the
//     A operand of O^T = V^T P^T is one 16-byte LDS read per lane.
//   * LDS tiles are XOR-swizzled so the MFMA operand reads are bank-conflict free.
//   * Workgroup ids are remapped so that the workgroups sharing one KV head and position
//     block land on the same XCD (each XCD has its own L2), heaviest causal rows first.
#include "common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kBQ = 32;    // query positions per wave
constexpr int kBN = 64;    // keys per LDS tile

// K tile [64 keys][192]: row r holds 24 chunks of 8 bf16; chunk c is stored at
// (c & ~7) | ((c ^ (r >> 1)) & 7) so 16 consecutive rows read at one column hit distinct banks.
__device__ __forceinline__ int ks_off(int row, int chunk) {
    return row * kDqk + ((chunk & ~7) | ((chunk ^ (row >> 1)) & 7)) * 8;
}
// V^T tile [128 dv][64 keys]: row r holds 8 chunks of 8 keys in MFMA k-order; chunk c is
// stored at (c ^ r ^ (r >> 3)) & 7.
__device__ __forceinline__ int vt_off(int row, int chunk) {
    return row * kBN + ((chunk ^ row ^ (row >> 3)) & 7) * 8;
}

// Key (within a 64-key tile) supplied as element e by lane group g for the 16-key group gam.
// In the 32x32 MFMA output a lane of group g holds, for register r, the key row
// 8*(r/4) + 4*g + r%4 of a 32-key block; the PV product consumes registers 0..7 and 8..15
// as two 16-key k-steps, so k-step gam, group g, element e is this key:
__device__ __forceinline__ int vkey(int gam, int g, int e) {
    return 16 * gam + ((e < 4) ? (4 * g + e) : (8 + 4 * g + (e - 4)));
}

__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * kDqk];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kDv * kBN];

    // ---- workgroup -> (position group, batch, kv head, head group), XCD-aware
    const int C = p.hgroups;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int lam = (((slot / C) * 8 + xcd) * C) + slot % C;
    if (lam >= p.n_items) return;  // padding workgroup (uniform: before any barrier)
    int t = lam;
    const int hg = t % C;
    t /= C;
    const int kvh = t % p.Hkv;
    t /= p.Hkv;
    const int b = t % p.B;
    t /= p.B;
    const int pbw = p.n_pbw - 1 - t;  // heaviest (latest) positions first

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 5, lq = lane & 31;
    const int h = kvh * p.G + hg * p.hw + (wave % p.hw);
    const int qpos0 = (pbw * p.pw + wave / p.hw) * kBQ;
    const int wg_q0 = pbw * p.pw * kBQ;
    const int wg_q1 = min(p.L, wg_q0 + p.pw * kBQ);
    const int qi = qpos0 + lq;
    const bool wave_live = qpos0 < p.L;

    // ---- Q^T fragments (B operand): lane supplies q[qi][16kk + 8g .. +8]
    bf16x8 qf[12];
    {
        const bool ok = qi < p.L;
        const uint16_t *qrow = p.q + ((((size_t)b * p.Hq + h) * p.L) + (ok ? qi : 0)) * kDqk + 8 * g;
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) {
            u32x4 v = ok ? ldg16(qrow + 16 * kk) : u32x4{0, 0, 0, 0};
            qf[kk] = as_bf16x8(v);
        }
    }

    // ---- running state: the sink starts the max and the denominator
    const float sk = p.sink ? p.sink[h] : -INFINITY;
    const bool has_sink = sk != -INFINITY;
    const bool sink_inf = sk == INFINITY;
    float m_run = has_sink ? sk * kLog2e : -INFINITY;
    float l_run = (has_sink && g == 0) ? 1.f : 0.f;  // exp2(sink - m) = 1, counted on one lane of the pair
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

    const size_t kvbase = ((size_t)b * p.Hkv + kvh) * p.L;
    const uint16_t *kg_base = p.k + kvbase * kDqk;
    const uint16_t *vg_base = p.v + kvbase * kDv;

    const int k_lo = p.swa ? max(0, wg_q0 - p.window + 1) : 0;
    const int t0 = k_lo / kBN, t1 = (wg_q1 - 1) / kBN;

    for (int kt = t0; kt <= t1; ++kt) {
        const int kb = kt * kBN;
        __syncthreads();  // the previous tile is no longer read
        if (tid >= 128) {
            // K tile: 64 rows x 24 chunks of 16 bytes over 128 threads, row-contiguous
            const int t2 = tid - 128;
#pragma unroll
            for (int e = 0; e < 12; ++e) {
                const int chunk = t2 + 128 * e;
                const int row = chunk / 24, col = chunk % 24;
                const int key = kb + row;
                u32x4 val = key < p.L ? ldg16(kg_base + (size_t)key * kDqk + col * 8) : u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4 *>(&Ks[ks_off(row, col)]) = val;
            }
        } else {
            // V tile: thread owns 8 keys (one MFMA k-chunk) x 8 dv; transpose, store rows of V^T
            const int c = tid >> 3, kgp = tid & 7;
            const int gam = kgp >> 1, hh = kgp & 1;
            u32x4 r[8], w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = kb + vkey(gam, hh, e);
                r[e] = key < p.L ? ldg16(vg_base + (size_t)key * kDv + 8 * c) : u32x4{0, 0, 0, 0};
            }
            transpose8x8_b16(r, w);
#pragma unroll
            for (int d = 0; d < 8; ++d) *reinterpret_cast<u32x4 *>(&Vt[vt_off(8 * c + d, kgp)]) = w[d];
        }
        __syncthreads();

        if (!wave_live) continue;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int k0 = kb + 32 * sb;
            const bool skip = k0 > qpos0 + kBQ - 1 || k0 >= p.L || (p.swa && k0 + 31 < qpos0 - p.window + 1);
            if (skip) continue;
            const bool need_mask = (k0 + 31 > qpos0) || (k0 + 31 >= p.L) ||
                                   (p.swa && k0 < qpos0 + kBQ - 1 - p.window + 1);
            f32x16 s = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 12; ++kk) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&Ks[ks_off(32 * sb + lq, 2 * kk + g)]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s, 0, 0, 0);
            }
            float x[16];
            float mx = m_run;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                x[r] = s[r] * p.scale_log2;
                if (need_mask) {
                    const int kj = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool ok = kj <= qi && kj < p.L && (!p.swa || kj > qi - p.window);
                    x[r] = ok ? x[r] : -INFINITY;
                }
                mx = fmaxf(mx, x[r]);
            }
            mx = max_xor32(mx);
            const float mu = (mx == -INFINITY) ? 0.f : mx;
            const float alpha = exp2f_fast(m_run - mu);
            m_run = mx;
            float ps = 0.f;
            uint32_t pk[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float p0 = exp2f_fast(x[2 * r] - mu), p1 = exp2f_fast(x[2 * r + 1] - mu);
                ps += p0 + p1;
                pk[r] = pack_bf16x2(p0, p1);
            }
            l_run = l_run * alpha + ps;
#pragma unroll
            for (int db = 0; db < 4; ++db) acc[db] *= alpha;
            const bf16x8 pf0 = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
            const bf16x8 pf1 = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const bf16x8 v0 = *reinterpret_cast<const bf16x8 *>(&Vt[vt_off(32 * db + lq, 4 * sb + g)]);
                const bf16x8 v1 = *reinterpret_cast<const bf16x8 *>(&Vt[vt_off(32 * db + lq, 4 * sb + 2 + g)]);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pf0, acc[db], 0, 0, 0);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pf1, acc[db], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: O = acc / l; lane holds dv 32db + 8i + 4g + j of query qi
    const float lt = sum_xor32(l_run);
    if (!wave_live || qi >= p.L) return;
    const float inv = 1.f / lt;
    uint16_t *orow = p.out + ((((size_t)b * p.Hq + h) * p.L) + qi) * kDv + 4 * g;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float o0 = acc[db][4 * i] * inv, o1 = acc[db][4 * i + 1] * inv;
            float o2 = acc[db][4 * i + 2] * inv, o3 = acc[db][4 * i + 3] * inv;
            if (sink_inf) o0 = o1 = o2 = o3 = 0.f;
            *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * i) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        }
    }
}

}  // namespace

int launch_prefill(const PrefillParams &prm, hipStream_t stream) {
    PrefillParams p = prm;
    const int grid = ((p.n_items + 8 * p.hgroups - 1) / (8 * p.hgroups)) * 8 * p.hgroups;
    void *args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_kernel), dim3(grid), dim3(256), args, 0,
                           stream) == hipSuccess ? 0 : -1;
}

}  // namespace sinkattn
