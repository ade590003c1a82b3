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
    int swa, window;
    float scale_log2;  // logit scale * log2(e)
    // work layout, filled by plan_prefill
    int hpw;           // query heads per wave
    int hw;            // query heads per workgroup (a multiple of hpw dividing G)
    int pw;            // 32-position blocks per workgroup
    int n_pbw;         // position groups per (batch, kv head)
    int hgroups;       // head groups per kv head (G / hw)
    int n_items;       // n_pbw * B * Hkv * hgroups
};

struct DecodeParams {
    const uint16_t *q, *k, *v;
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
    float v_scale;     // 8-bit cache: V element = v_scale * code value
    int nsplit, chunk;  // splits per sequence; keys per split (multiple of 128)
};

size_t prefill_workspace_bytes(int B, int Hkv, int L);
// Fills the work layout of p from B, L, Hkv, G and swa; returns the number of workgroups to
// launch (the caller rejects counts that do not fit a grid).
int64_t plan_prefill(PrefillParams &p);
int launch_prefill(const PrefillParams &p, hipStream_t stream);
int launch_decode(const DecodeParams &p, hipStream_t stream);

}  // namespace sinkattn
