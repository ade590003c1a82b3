// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

struct PrefillParams {
    const uint16_t *q, *k, *v;
    uint16_t *vt;      // workspace: V^T [B][Hkv][lpad/64][kDv][64], keys in MFMA k-order
    int lpad;          // L rounded up to a multiple of 64
    const float *sink;  // [Hq] or nullptr
    uint16_t *out;
    int B, L, Hq, Hkv, G;  // L: keys per sequence (positions 0..L-1)
    int Lq, q0;            // query rows in q and out, at positions q0 .. q0 + Lq - 1 (q0 = L - Lq)
    float out_scale;       // multiplies the output
    float *lse;            // optional: natural-log log-sum-exp per row [B][Hq][Lq], or nullptr
    int swa, window;
    float scale_log2;  // logit scale * log2(e)
    // work layout, filled by plan_prefill
    int hpw;           // query heads per wave
    int hw;            // query heads per workgroup (a multiple of hpw dividing G)
    int pw;            // 32-position blocks per workgroup
    int n_pbw;         // position groups per (batch, kv head)
    int hgroups;       // head groups per kv head (G / hw)
    int n_items;       // n_pbw * B * Hkv * hgroups
    int ring;          // 1: the sliding-window ring kernel (then n_items = workgroups)
    int chunk;         // ring kernel: 32-position blocks per workgroup
    int reverse;       // 1: workgroups take their work items in reverse order (grid_reversed())
    // Ring kernel over a prefix held in a ring cache, read in place: rows below q0 (positions
    // prefix_base + row) come from prefix_k / prefix_v ([B][Hkv][prefix_w][d], position p in
    // slot p mod prefix_w), and k / v then hold only the chunk's Lq rows.  nullptr otherwise.
    const uint16_t *prefix_k, *prefix_v;
    int prefix_w, prefix_base;
};

// Keys per decode split at most: each of the 4 waves of a split walks 32-key slices, and
// holds the page ids of up to 64 of them per register.
constexpr int kDecodeMaxChunk = 16384;

struct DecodeParams {
    const uint16_t *q, *k, *v;
    const uint16_t *k_new, *v_new;  // the new tokens' keys and values beside the cache, or nullptr
    const int32_t *block_table;  // paged layout only
    const int32_t *seq_lens;
    const float *sink;  // [Hq] or nullptr
    uint16_t *out;
    float *ws;  // partials [B][Hq][q_len][nsplit][kDv + 4] when nsplit > 1
    int B, Hq, Hkv, G;
    int q_len;         // new tokens per sequence (positions seq_len - q_len .. seq_len - 1)
    int ncb, hchunks;  // 16-column blocks per workgroup; workgroups per KV head
    int swa, window, paged, page_size, max_pages, num_pages, max_seq_len;
    float scale_log2;  // logit scale * log2(e) (8-bit cache: times the K scale)
    int fp8;           // K and V are E4M3 codes (paged, page_size a multiple of 32)
    float out_scale;   // multiplies the output (8-bit cache: times the V scale)
    float *lse;        // optional: natural-log log-sum-exp per row [B][Hq][q_len], or nullptr
    int nsplit, chunk;  // splits per sequence; keys per split (multiple of 128)
    int reverse;        // 1: workgroups take their work items in reverse order (grid_reversed())
    // Fused decode step (a ring, one new token): q holds the new token's queries before
    // rotation; its key (before rotation) and value rows k_step, v_step [B][Hkv][kDqk or kDv]
    // are rotated (key) and written to ring slot (n - 1) mod window, and the attention uses them
    // there.  nullptr otherwise.
    const uint16_t *k_step, *v_step;
    double inv_freq[32];  // theta^(-2i/64)
};

// Partial rotary embedding of x [batch][heads][rows][kDqk] in place; row r of sequence b sits
// at position (seq_lens ? seq_lens[b] - rows : pos0) + r.
struct RopeParams {
    uint16_t *x;
    const int32_t *seq_lens;
    int batch, heads, rows, pos0;
    double inv_freq[32];  // theta^(-2i/64)
};

// New tokens -> KV cache: token t of sequence b (position seq_lens[b] - n_new + t).
struct AppendParams {
    const uint16_t *k_new, *v_new;  // [batch][hkv][n_new][kDqk or kDv]
    uint16_t *k_cache, *v_cache;    // bf16 caches
    uint8_t *k_cache8, *v_cache8;   // E4M3 caches (fp8)
    const int32_t *block_table, *seq_lens;
    int batch, hkv, n_new, paged, window, page_size, max_pages, num_pages, fp8;
    float k_scale, v_scale;  // fp8: codes of value / scale
};

// The decode prologue fused: RoPE of q (into q_out) and of the new keys, and the cache write.
struct PrologueParams {
    AppendParams a;          // the new keys and values and the cache they go to
    const uint16_t *q_in;    // [batch][hq][n_new][kDqk]
    uint16_t *q_out;         // the same shape; may be q_in (rotated in place)
    int hq;
    double inv_freq[32];     // theta^(-2i/64)
};
int launch_decode_prologue(const PrologueParams &p, hipStream_t stream);

// Backward of prefill (q, k, v, out, dout bf16; lse, delta, gradients float32).
struct BwdParams {
    const uint16_t *q, *k, *v, *out, *dout;
    const float *lse;   // [B][Hq][L] from the forward (natural log)
    const float *sink;  // [Hq] or nullptr
    float *dq, *dk, *dv;  // [B][Hq][L][kDqk], [B][Hkv][L][kDqk], [B][Hkv][L][kDv]
    float *dsink;         // [Hq] (sink given)
    float *delta;         // workspace [B][Hq][L]: dO . O
    float *nlse2;         // workspace [B][Hq][L]: -lse log2(e), the exponent offset of P
    float *dsink_part;    // workspace [B][Hq][ceil(L / 16)]
    int B, L, Hq, Hkv, G, swa, window;
    float scale, scale_log2;
    int reverse;  // workgroups take their work in reverse order (race check)
};
size_t backward_workspace_bytes(int B, int Hq, int L);
int launch_backward(const BwdParams &p, hipStream_t stream);

// Chunked prefill over a cached prefix: the keys and values of positions base .. base + Lc - 1
// gathered into contiguous rows, the prefix (positions below q0) from a ring or pages, the
// chunk (q0 .. q0 + Lq - 1) from its own rows.
struct GatherParams {
    const uint16_t *k_chunk, *v_chunk;  // [B][Hkv][Lq][kDqk], [B][Hkv][Lq][kDv]
    const uint16_t *k_cache, *v_cache;  // ring [B][Hkv][window][d] or pages [num_pages][Hkv][page_size][d]
    const int32_t *block_table;         // [B][max_pages] (paged)
    uint16_t *k_out, *v_out;            // [B][Hkv][Lc][kDqk], [B][Hkv][Lc][kDv]
    int B, Hkv, Lq, Lc, base, q0;
    int paged, window, page_size, max_pages, num_pages;
};
int launch_gather_prefix(const GatherParams &g, hipStream_t stream);

size_t prefill_workspace_bytes(int B, int Hkv, int L);
// Fills the work layout of p from B, L, Hkv, G and swa; returns the number of workgroups to
// launch (the caller rejects counts that do not fit a grid).
int64_t plan_prefill(PrefillParams &p);
int launch_prefill(const PrefillParams &p, hipStream_t stream);
// Race check: with SINKATTN_GRID_ORDER=reversed in the environment the attention kernels map
// workgroup ids to their work in reverse order, so work runs in a different order and next to
// different neighbours; every output must come out bit-identical.  Read at each launch.
int grid_reversed();
int launch_decode(const DecodeParams &p, hipStream_t stream);
// The decode scratch array of this device (nullptr if its address cannot be found) and its size.
float *decode_scratch();
size_t decode_scratch_bytes();
int launch_rope(const RopeParams &p, hipStream_t stream);
int launch_kv_append(const AppendParams &p, hipStream_t stream);

}  // namespace sinkattn
