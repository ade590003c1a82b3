// C-ABI entry points of libsinkattn.so: argument validation, work planning and kernel
// launches.  Every check here runs on the host before anything touches the device, so
// argument errors are reported synchronously and nothing is enqueued.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "launch.h"
#include "sinkattn.h"

namespace {

using namespace sinkattn;

constexpr int kDqkSupported = 192;
constexpr int kDvSupported = 128;
// Decode workgroups to aim for: two rounds of the bf16 split kernel on a 256-CU MI355X (one
// workgroup per CU, 160 KB of LDS), one round of the E4M3 kernel (two per CU).  Every
// workgroup pays its first loads and its merge once, so fewer, longer splits win (8 x 256K
// GA decode: 853 us at 2048 workgroups, 818 at 1024, 794 at 512; 256 leaves half of the
// CUs idle for the E4M3 kernel).
constexpr int64_t kDecodeTargetWorkgroups = 512;
constexpr int kDecodeKeyBlock = 128;                // keys per decode workgroup iteration
constexpr int kDecodeSingleSplit = 1024;            // key ranges this short are not split
constexpr double kLog2eD = 1.4426950408889634;
constexpr int kDecodeStepMaxSlots = 128;  // the fused decode step's single-slice kernel: 4 waves x 32 keys

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Optional epilogue: a finite output scale and a 4-byte aligned LSE buffer.
int check_epilogue(const sinkattn_epilogue *ep) {
    if (!ep) return SINKATTN_OK;
    if (!isfinite(ep->out_scale)) return SINKATTN_E_SHAPE;
    if (ep->lse && (reinterpret_cast<uintptr_t>(ep->lse) & 3u)) return SINKATTN_E_ALIGN;
    return SINKATTN_OK;
}

int check_dims(int mode, int window, const sinkattn_dims *d) {
    if (!d) return SINKATTN_E_NULL;
    if (mode != SINKATTN_GLOBAL && mode != SINKATTN_SWA) return SINKATTN_E_UNSUPPORTED;
    if (d->d_qk != kDqkSupported || d->d_v != kDvSupported) return SINKATTN_E_UNSUPPORTED;
    if (d->batch < 0 || d->hq <= 0 || d->hkv <= 0 || d->hq % d->hkv != 0) return SINKATTN_E_SHAPE;
    if (mode == SINKATTN_SWA && window < 1) return SINKATTN_E_SHAPE;
    if (!isfinite(d->scale) || !(d->scale > 0.f)) return SINKATTN_E_SHAPE;
    return SINKATTN_OK;
}

constexpr int kMaxQLen = 256;  // new tokens per sequence at most (multi-token decode)

struct DecodePlan {
    int nsplit, chunk, ncb, hchunks;
    size_t ws_bytes;
};

// Columns: the G * q_len (query head, new token) pairs of a KV head, in blocks of 16; a
// workgroup takes ncb blocks (up to 4), so one pass over a KV head's cache serves them all.
// Keys per split: enough splits that B * Hkv * column-chunks * splits reaches about
// kDecodeTargetWorkgroups, in whole 128-key blocks.  The kernel walks keys in 32-key
// slices aligned to absolute positions, so a sliding window of W keys seen from q_len
// consecutive positions spans up to W + q_len - 1 + 31 aligned keys; short ranges (up to
// kDecodeSingleSplit keys) stay in one split.
DecodePlan plan_decode(int mode, int window, const sinkattn_dims *d, int32_t q_len, int32_t max_seq_len) {
    const int64_t G = d->hq / d->hkv;
    const int64_t rows = G * q_len;
    const int64_t ncb = rows <= 16 ? 1 : rows <= 32 ? 2 : 4;
    const int64_t hchunks = (rows + 16 * ncb - 1) / (16 * ncb);
    const int64_t span = (int64_t)window + q_len - 1;
    const int64_t kmax = mode == SINKATTN_SWA ? (span < max_seq_len ? span : max_seq_len) + 31 : max_seq_len;
    const int64_t units = (int64_t)d->batch * d->hkv * hchunks;
    int64_t chunk = units > 0 ? (kmax * units + kDecodeTargetWorkgroups - 1) / kDecodeTargetWorkgroups : kmax;
    if (kmax <= kDecodeSingleSplit) chunk = kmax;
    chunk = ((chunk + kDecodeKeyBlock - 1) / kDecodeKeyBlock) * kDecodeKeyBlock;
    if (chunk < kDecodeKeyBlock) chunk = kDecodeKeyBlock;
    if (chunk > kDecodeMaxChunk) chunk = kDecodeMaxChunk;
    const int64_t nsplit = (kmax + chunk - 1) / chunk;
    DecodePlan pl;
    pl.nsplit = (int)(nsplit < 1 ? 1 : nsplit);
    pl.chunk = (int)chunk;
    pl.ncb = (int)ncb;
    pl.hchunks = (int)hchunks;
    pl.ws_bytes =
        pl.nsplit > 1 ? (size_t)d->batch * d->hq * q_len * pl.nsplit * (kDvSupported + 4) * sizeof(float) : 0;
    return pl;
}

}  // namespace

extern "C" {

const char *sinkattn_status_string(int status) {
    switch (status) {
        case SINKATTN_OK: return "ok";
        case SINKATTN_E_NULL: return "a required pointer is NULL";
        case SINKATTN_E_SHAPE: return "invalid sizes";
        case SINKATTN_E_UNSUPPORTED: return "unsupported head size, mode or cache layout";
        case SINKATTN_E_ALIGN: return "a pointer is not 16-byte aligned";
        case SINKATTN_E_WORKSPACE: return "decode workspace missing or too small";
        case SINKATTN_E_DEVICE: return "kernel launch failed";
        default: return "unknown status";
    }
}

size_t sinkattn_prefill_workspace_bytes(const sinkattn_dims *d) {
    if (!d || d->batch < 0 || d->seqlen < 0 || d->hkv <= 0) return (size_t)-1;
    return prefill_workspace_bytes(d->batch, d->hkv, d->seqlen);
}

size_t sinkattn_prefill_chunk_workspace_bytes(const sinkattn_dims *d, int32_t kv_len) {
    if (!d || d->batch < 0 || d->seqlen < 0 || d->hkv <= 0 || kv_len < d->seqlen) return (size_t)-1;
    return prefill_workspace_bytes(d->batch, d->hkv, kv_len);
}

int sinkattn_prefill(int mode, int window, const sinkattn_dims *d, const void *q, const void *k, const void *v,
                     const float *sink, void *out, void *workspace, size_t workspace_bytes, void *stream) {
    return sinkattn_prefill_chunk(mode, window, d, d ? d->seqlen : 0, q, k, v, sink, out, workspace,
                                  workspace_bytes, stream);
}

int sinkattn_prefill_chunk(int mode, int window, const sinkattn_dims *d, int32_t kv_len, const void *q,
                           const void *k, const void *v, const float *sink, void *out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return sinkattn_prefill_ex(mode, window, d, kv_len, q, k, v, sink, nullptr, out, workspace, workspace_bytes,
                               stream);
}

int sinkattn_prefill_ex(int mode, int window, const sinkattn_dims *d, int32_t kv_len, const void *q, const void *k,
                        const void *v, const float *sink, const sinkattn_epilogue *ep, void *out, void *workspace,
                        size_t workspace_bytes, void *stream) {
    int st = check_dims(mode, window, d);
    if (st) return st;
    st = check_epilogue(ep);
    if (st) return st;
    if (d->seqlen < 0 || kv_len < d->seqlen) return SINKATTN_E_SHAPE;
    if ((int64_t)kv_len * kDqkSupported * 2 > INT32_MAX) return SINKATTN_E_SHAPE;  // 32-bit row offsets
    if (d->batch == 0 || d->seqlen == 0) return SINKATTN_OK;
    if (!q || !k || !v || !out) return SINKATTN_E_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || (sink && misaligned(sink)))
        return SINKATTN_E_ALIGN;
    const size_t need = prefill_workspace_bytes(d->batch, d->hkv, kv_len);
    if (!workspace || workspace_bytes < need) return SINKATTN_E_WORKSPACE;
    if (misaligned(workspace)) return SINKATTN_E_ALIGN;

    PrefillParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.sink = sink;
    p.out = static_cast<uint16_t *>(out);
    p.vt = static_cast<uint16_t *>(workspace);
    p.lpad = (kv_len + 63) / 64 * 64;
    p.B = d->batch;
    p.L = kv_len;
    p.Lq = d->seqlen;
    p.q0 = kv_len - d->seqlen;
    p.Hq = d->hq;
    p.Hkv = d->hkv;
    p.G = d->hq / d->hkv;
    p.swa = mode == SINKATTN_SWA;
    p.window = p.swa ? window : 0;
    p.scale_log2 = (float)((double)d->scale * kLog2eD);
    p.out_scale = ep ? ep->out_scale : 1.f;
    p.lse = ep ? ep->lse : nullptr;
    if (plan_prefill(p) > INT32_MAX) return SINKATTN_E_SHAPE;
    return launch_prefill(p, static_cast<hipStream_t>(stream)) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}

}  // extern "C"

namespace {
// Chunked prefill over a cached prefix: the rows gathered for the attention kernels are
// positions base .. kv_len - 1 (global: from 0; sliding window: from the first key the chunk's
// first query sees), then the workspace holds K and V of those rows and the V^T copy.
struct CachedLayout {
    int base, Lc;
    size_t k_off, v_off, vt_off, bytes;
};
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
CachedLayout cached_layout(int mode, int window, const sinkattn_dims *d, int32_t kv_len) {
    CachedLayout c{};
    const int q0 = kv_len - d->seqlen;
    c.base = mode == SINKATTN_SWA ? std::max(0, q0 - window + 1) : 0;
    c.Lc = kv_len - c.base;
    const size_t rows = (size_t)d->batch * d->hkv * c.Lc;
    c.k_off = 0;
    c.v_off = round256(rows * kDqkSupported * 2);
    c.vt_off = c.v_off + round256(rows * kDvSupported * 2);
    c.bytes = c.vt_off + prefill_workspace_bytes(d->batch, d->hkv, c.Lc);
    return c;
}
}  // namespace

extern "C" {

size_t sinkattn_prefill_cached_workspace_bytes(int mode, int window, const sinkattn_dims *d, int32_t kv_len) {
    if (check_dims(mode, window, d) || d->seqlen < 0 || kv_len < d->seqlen) return (size_t)-1;
    return cached_layout(mode, window, d, kv_len).bytes;
}

int sinkattn_prefill_cached(int mode, int window, const sinkattn_dims *d, int32_t kv_len, const void *q, const void *k,
                            const void *v, const sinkattn_kv *prefix, const float *sink, const sinkattn_epilogue *ep,
                            void *out, void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_dims(mode, window, d);
    if (st) return st;
    st = check_epilogue(ep);
    if (st) return st;
    if (d->seqlen < 0 || kv_len < d->seqlen) return SINKATTN_E_SHAPE;
    if ((int64_t)kv_len * kDqkSupported * 2 > INT32_MAX) return SINKATTN_E_SHAPE;  // 32-bit row offsets
    if (!prefix) return SINKATTN_E_NULL;
    if (prefix->layout != SINKATTN_KV_RING && prefix->layout != SINKATTN_KV_PAGED) return SINKATTN_E_UNSUPPORTED;
    if (prefix->layout == SINKATTN_KV_RING && mode != SINKATTN_SWA) return SINKATTN_E_UNSUPPORTED;
    const int q0 = kv_len - d->seqlen;
    if (prefix->layout == SINKATTN_KV_PAGED &&
        (prefix->page_size <= 0 || prefix->max_pages <= 0 || prefix->num_pages <= 0 ||
         (int64_t)prefix->max_pages * prefix->page_size < q0))
        return SINKATTN_E_SHAPE;
    if (d->batch > 65535 || (int64_t)d->batch * d->hkv > 65535) return SINKATTN_E_SHAPE;
    if (d->batch == 0 || d->seqlen == 0) return SINKATTN_OK;
    if (!q || !k || !v || !out) return SINKATTN_E_NULL;
    if (q0 > 0 && (!prefix->k || !prefix->v || (prefix->layout == SINKATTN_KV_PAGED && !prefix->block_table)))
        return SINKATTN_E_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || (sink && misaligned(sink)) ||
        (q0 > 0 && (misaligned(prefix->k) || misaligned(prefix->v))))
        return SINKATTN_E_ALIGN;
    const CachedLayout c = cached_layout(mode, window, d, kv_len);
    if (!workspace || workspace_bytes < c.bytes) return SINKATTN_E_WORKSPACE;
    if (misaligned(workspace)) return SINKATTN_E_ALIGN;
    char *ws = static_cast<char *>(workspace);

    GatherParams g{};
    g.k_chunk = static_cast<const uint16_t *>(k);
    g.v_chunk = static_cast<const uint16_t *>(v);
    g.k_cache = static_cast<const uint16_t *>(prefix->k);
    g.v_cache = static_cast<const uint16_t *>(prefix->v);
    g.block_table = prefix->layout == SINKATTN_KV_PAGED ? prefix->block_table : nullptr;
    g.k_out = reinterpret_cast<uint16_t *>(ws + c.k_off);
    g.v_out = reinterpret_cast<uint16_t *>(ws + c.v_off);
    g.B = d->batch;
    g.Hkv = d->hkv;
    g.Lq = d->seqlen;
    g.Lc = c.Lc;
    g.base = c.base;
    g.q0 = q0;
    g.paged = prefix->layout == SINKATTN_KV_PAGED;
    g.window = window;
    g.page_size = g.paged ? prefix->page_size : 0;
    g.max_pages = g.paged ? prefix->max_pages : 0;
    g.num_pages = g.paged ? prefix->num_pages : 0;

    PrefillParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = g.k_out;
    p.v = g.v_out;
    p.sink = sink;
    p.out = static_cast<uint16_t *>(out);
    p.vt = reinterpret_cast<uint16_t *>(ws + c.vt_off);
    p.lpad = (c.Lc + 63) / 64 * 64;
    p.B = d->batch;
    p.L = c.Lc;
    p.Lq = d->seqlen;
    p.q0 = q0 - c.base;  // positions relative to the first gathered row: masks depend on differences only
    p.Hq = d->hq;
    p.Hkv = d->hkv;
    p.G = d->hq / d->hkv;
    p.swa = mode == SINKATTN_SWA;
    p.window = p.swa ? window : 0;
    p.scale_log2 = (float)((double)d->scale * kLog2eD);
    p.out_scale = ep ? ep->out_scale : 1.f;
    p.lse = ep ? ep->lse : nullptr;
    if (plan_prefill(p) > INT32_MAX) return SINKATTN_E_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.ring && !g.paged) {
        // the ring kernel reads a ring prefix in place and the chunk's own rows: no gather
        p.k = g.k_chunk;
        p.v = g.v_chunk;
        p.prefix_k = g.k_cache;
        p.prefix_v = g.v_cache;
        p.prefix_w = window;
        p.prefix_base = c.base;
    } else if (launch_gather_prefix(g, s)) {
        return SINKATTN_E_DEVICE;
    }
    return launch_prefill(p, s) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}

size_t sinkattn_decode_workspace_bytes(int mode, int window, const sinkattn_dims *d, int32_t max_seq_len) {
    if (check_dims(mode, window, d) || max_seq_len < 1) return (size_t)-1;
    return plan_decode(mode, window, d, 1, max_seq_len).ws_bytes;
}

size_t sinkattn_decode_multi_workspace_bytes(int mode, int window, const sinkattn_dims *d, int32_t q_len,
                                             int32_t max_seq_len) {
    if (check_dims(mode, window, d) || max_seq_len < 1 || q_len < 1 || q_len > kMaxQLen) return (size_t)-1;
    return plan_decode(mode, window, d, q_len, max_seq_len).ws_bytes;
}

}  // extern "C"

namespace {
// Decode from a bf16 cache (fp8 = 0) or an E4M3 cache with per-tensor scales (fp8 = 1).
// use_scratch: the split partials go to the library's own device scratch array instead of
// the caller's workspace (which is then ignored).
// k_new / v_new: the new tokens' keys and values beside the cache (both NULL: they are in it).
// The fused decode step's extra inputs: the new token's key and value rows (before rotation)
// and the RoPE base.
struct StepArgs {
    const void *k_step, *v_step;
    double theta;
};

int decode_common(int mode, int window, const sinkattn_dims *d, int32_t q_len, const void *q, const sinkattn_kv *kv,
                  const void *k_new, const void *v_new, const int32_t *seq_lens, int32_t max_seq_len,
                  const float *sink, int fp8, float k_scale, float v_scale, const sinkattn_epilogue *ep, void *out,
                  void *workspace, size_t workspace_bytes, void *stream, bool use_scratch = false,
                  const StepArgs *step = nullptr) {
    int st = check_dims(mode, window, d);
    if (st) return st;
    st = check_epilogue(ep);
    if (st) return st;
    if (fp8) {
        if (!kv) return SINKATTN_E_NULL;
        if (kv->layout != SINKATTN_KV_PAGED || kv->page_size <= 0 || kv->page_size % 32) return SINKATTN_E_UNSUPPORTED;
        if (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale)) return SINKATTN_E_SHAPE;
    }
    const bool side = k_new || v_new;
    if (side && fp8) return SINKATTN_E_UNSUPPORTED;
    if (q_len < 1 || q_len > kMaxQLen) return SINKATTN_E_SHAPE;
    if (!kv) return SINKATTN_E_NULL;
    if (kv->layout != SINKATTN_KV_RING && kv->layout != SINKATTN_KV_PAGED) return SINKATTN_E_UNSUPPORTED;
    if (kv->layout == SINKATTN_KV_RING && (mode != SINKATTN_SWA || (q_len != 1 && !side)))
        return SINKATTN_E_UNSUPPORTED;
    if (max_seq_len < 1) return SINKATTN_E_SHAPE;
    if (kv->layout == SINKATTN_KV_PAGED) {
        if (kv->page_size <= 0 || kv->max_pages <= 0 || kv->num_pages <= 0) return SINKATTN_E_SHAPE;
        // the page table covers the cached positions: all of them, or all but the new tokens
        if ((int64_t)max_seq_len - (side ? q_len : 0) > (int64_t)kv->max_pages * kv->page_size)
            return SINKATTN_E_SHAPE;
    }
    if (d->batch == 0) return SINKATTN_OK;
    if (!q || !out || !seq_lens || !kv->k || !kv->v || (side && (!k_new || !v_new))) return SINKATTN_E_NULL;
    if (side && (misaligned(k_new) || misaligned(v_new))) return SINKATTN_E_ALIGN;
    if (kv->layout == SINKATTN_KV_PAGED && !kv->block_table) return SINKATTN_E_NULL;
    if (misaligned(q) || misaligned(out) || misaligned(seq_lens) || misaligned(kv->k) || misaligned(kv->v) ||
        (sink && misaligned(sink)) || (kv->layout == SINKATTN_KV_PAGED && misaligned(kv->block_table)))
        return SINKATTN_E_ALIGN;
    const DecodePlan pl = plan_decode(mode, window, d, q_len, max_seq_len);
    if (step) {
        // one kernel: a ring of at most 128 visible slots, one block of 16 query columns
        if (kv->layout != SINKATTN_KV_RING || q_len != 1 || fp8 || side || pl.nsplit != 1 || pl.ncb != 1 ||
            std::min(window, max_seq_len) > kDecodeStepMaxSlots)
            return SINKATTN_E_UNSUPPORTED;
        if (!step->k_step || !step->v_step) return SINKATTN_E_NULL;
        if (misaligned(step->k_step) || misaligned(step->v_step)) return SINKATTN_E_ALIGN;
    }
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
        if (pl.ws_bytes > decode_scratch_bytes()) return SINKATTN_E_WORKSPACE;
        if (pl.ws_bytes > 0) {
            workspace = decode_scratch();
            if (!workspace) return SINKATTN_E_DEVICE;
            workspace_bytes = decode_scratch_bytes();
        }
    }
    if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return SINKATTN_E_WORKSPACE;
        if (misaligned(workspace)) return SINKATTN_E_ALIGN;
    }

    DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(kv->k);
    p.v = static_cast<const uint16_t *>(kv->v);
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    p.block_table = kv->layout == SINKATTN_KV_PAGED ? kv->block_table : nullptr;
    p.seq_lens = seq_lens;
    p.sink = sink;
    p.out = static_cast<uint16_t *>(out);
    p.ws = static_cast<float *>(workspace);
    p.B = d->batch;
    p.Hq = d->hq;
    p.Hkv = d->hkv;
    p.G = d->hq / d->hkv;
    p.q_len = q_len;
    p.ncb = pl.ncb;
    p.hchunks = pl.hchunks;
    p.swa = mode == SINKATTN_SWA;
    p.window = p.swa ? window : 0;
    p.paged = kv->layout == SINKATTN_KV_PAGED;
    p.page_size = p.paged ? kv->page_size : 0;
    p.max_pages = p.paged ? kv->max_pages : 0;
    p.num_pages = p.paged ? kv->num_pages : 0;
    p.max_seq_len = max_seq_len;
    p.scale_log2 = (float)((double)d->scale * kLog2eD * (fp8 ? (double)k_scale : 1.0));
    p.fp8 = fp8;
    p.out_scale = (fp8 ? v_scale : 1.f) * (ep ? ep->out_scale : 1.f);
    p.lse = ep ? ep->lse : nullptr;
    p.nsplit = pl.nsplit;
    p.chunk = pl.chunk;
    if (step) {
        p.k_step = static_cast<const uint16_t *>(step->k_step);
        p.v_step = static_cast<const uint16_t *>(step->v_step);
        for (int i = 0; i < 32; ++i) p.inv_freq[i] = pow(step->theta, -2.0 * i / 64.0);
    }
    if ((int64_t)p.Hkv * p.hchunks > 65535 || p.B > 65535 || (int64_t)p.B * p.Hq * p.q_len > INT32_MAX)
        return SINKATTN_E_SHAPE;
    return launch_decode(p, static_cast<hipStream_t>(stream)) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}
}  // namespace

extern "C" {

int sinkattn_decode_multi(int mode, int window, const sinkattn_dims *d, int32_t q_len, const void *q,
                          const sinkattn_kv *kv, const int32_t *seq_lens, int32_t max_seq_len, const float *sink,
                          void *out, void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(mode, window, d, q_len, q, kv, nullptr, nullptr, seq_lens, max_seq_len, sink, 0, 1.f, 1.f,
                         nullptr, out, workspace, workspace_bytes, stream);
}

int sinkattn_decode_ex(int mode, int window, const sinkattn_dims *d, int32_t q_len, const void *q,
                       const sinkattn_kv *kv, int kv_fp8, float k_scale, float v_scale, const int32_t *seq_lens,
                       int32_t max_seq_len, const float *sink, const sinkattn_epilogue *ep, void *out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(mode, window, d, q_len, q, kv, nullptr, nullptr, seq_lens, max_seq_len, sink, kv_fp8 ? 1 : 0,
                         k_scale, v_scale, ep, out, workspace, workspace_bytes, stream);
}

int sinkattn_decode_ex_noalloc(int mode, int window, const sinkattn_dims *d, int32_t q_len, const void *q,
                               const sinkattn_kv *kv, int kv_fp8, float k_scale, float v_scale,
                               const int32_t *seq_lens, int32_t max_seq_len, const float *sink,
                               const sinkattn_epilogue *ep, void *out, void *stream) {
    return decode_common(mode, window, d, q_len, q, kv, nullptr, nullptr, seq_lens, max_seq_len, sink, kv_fp8 ? 1 : 0,
                         k_scale, v_scale, ep, out, nullptr, 0, stream, true);
}

int sinkattn_decode_verify(int mode, int window, const sinkattn_dims *d, int32_t q_len, const void *q,
                           const sinkattn_kv *kv, const void *k_new, const void *v_new, const int32_t *seq_lens,
                           int32_t max_seq_len, const float *sink, const sinkattn_epilogue *ep, void *out,
                           void *workspace, size_t workspace_bytes, void *stream) {
    if (!k_new || !v_new) return SINKATTN_E_NULL;
    return decode_common(mode, window, d, q_len, q, kv, k_new, v_new, seq_lens, max_seq_len, sink, 0, 1.f, 1.f, ep,
                         out, workspace, workspace_bytes, stream);
}

int sinkattn_decode_fp8(int mode, int window, const sinkattn_dims *d, int32_t q_len, const void *q,
                        const sinkattn_kv *kv, const int32_t *seq_lens, int32_t max_seq_len, const float *sink,
                        float k_scale, float v_scale, void *out, void *workspace, size_t workspace_bytes,
                        void *stream) {
    return decode_common(mode, window, d, q_len, q, kv, nullptr, nullptr, seq_lens, max_seq_len, sink, 1, k_scale,
                         v_scale, nullptr, out, workspace, workspace_bytes, stream);
}

size_t sinkattn_prefill_backward_workspace_bytes(const sinkattn_dims *d) {
    if (!d || d->batch < 0 || d->seqlen < 0 || d->hq <= 0) return (size_t)-1;
    return backward_workspace_bytes(d->batch, d->hq, d->seqlen);
}

int sinkattn_prefill_backward(int mode, int window, const sinkattn_dims *d, const void *q, const void *k,
                              const void *v, const float *sink, const void *out, const void *dout, const float *lse,
                              float *dq, float *dk, float *dv, float *dsink, void *workspace, size_t workspace_bytes,
                              void *stream) {
    int st = check_dims(mode, window, d);
    if (st) return st;
    if (d->seqlen < 0) return SINKATTN_E_SHAPE;
    if ((d->hq / d->hkv) % 4) return SINKATTN_E_UNSUPPORTED;
    if (d->batch > 65535 || d->hq / 4 > 65535 || (int64_t)d->seqlen * kDqkSupported * 2 > INT32_MAX)
        return SINKATTN_E_SHAPE;
    if (d->batch == 0 || d->seqlen == 0) return SINKATTN_OK;
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || (sink && !dsink)) return SINKATTN_E_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(dout) || misaligned(lse) ||
        misaligned(dq) || misaligned(dk) || misaligned(dv) || (sink && (misaligned(sink) || misaligned(dsink))))
        return SINKATTN_E_ALIGN;
    const size_t need = backward_workspace_bytes(d->batch, d->hq, d->seqlen);
    if (!workspace || workspace_bytes < need) return SINKATTN_E_WORKSPACE;
    if (misaligned(workspace)) return SINKATTN_E_ALIGN;
    BwdParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.out = static_cast<const uint16_t *>(out);
    p.dout = static_cast<const uint16_t *>(dout);
    p.lse = lse;
    p.sink = sink;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dsink = dsink;
    p.delta = static_cast<float *>(workspace);
    p.nlse2 = p.delta + (size_t)d->batch * d->hq * d->seqlen;
    p.dsink_part = p.nlse2 + (size_t)d->batch * d->hq * d->seqlen;
    p.B = d->batch;
    p.L = d->seqlen;
    p.Hq = d->hq;
    p.Hkv = d->hkv;
    p.G = d->hq / d->hkv;
    p.swa = mode == SINKATTN_SWA;
    p.window = p.swa ? window : 0;
    p.scale = d->scale;
    p.scale_log2 = (float)((double)d->scale * kLog2eD);
    return launch_backward(p, static_cast<hipStream_t>(stream)) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}

int sinkattn_rope(double theta, int32_t batch, int32_t heads, int32_t rows, void *x, const int32_t *seq_lens,
                  int32_t pos0, void *stream) {
    if (!(theta > 0.0) || !isfinite(theta)) return SINKATTN_E_SHAPE;
    if (batch < 0 || heads < 0 || rows < 0 || batch > 65535) return SINKATTN_E_SHAPE;
    if (batch == 0 || heads == 0 || rows == 0) return SINKATTN_OK;
    if (!x) return SINKATTN_E_NULL;
    if (misaligned(x) || (seq_lens && misaligned(seq_lens))) return SINKATTN_E_ALIGN;
    RopeParams p{};
    p.x = static_cast<uint16_t *>(x);
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.heads = heads;
    p.rows = rows;
    p.pos0 = pos0;
    for (int i = 0; i < 32; ++i) p.inv_freq[i] = pow(theta, -2.0 * i / 64.0);
    return launch_rope(p, static_cast<hipStream_t>(stream)) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}

}  // extern "C"

namespace {
// Checks of a cache write (shared by the append and the fused prologue) and its parameters.
int append_params(const sinkattn_kv *kv, int window, int32_t batch, int32_t hkv, int32_t n_new, const void *k_new,
                  const void *v_new, const int32_t *seq_lens, int kv_fp8, float k_scale, float v_scale,
                  AppendParams &p) {
    if (!kv) return SINKATTN_E_NULL;
    if (kv->layout != SINKATTN_KV_RING && kv->layout != SINKATTN_KV_PAGED) return SINKATTN_E_UNSUPPORTED;
    if (batch < 0 || hkv < 1 || n_new < 0 || batch > 65535) return SINKATTN_E_SHAPE;
    if (kv->layout == SINKATTN_KV_RING && window < 1) return SINKATTN_E_SHAPE;
    if (kv->layout == SINKATTN_KV_PAGED && (kv->page_size <= 0 || kv->max_pages <= 0 || kv->num_pages <= 0))
        return SINKATTN_E_SHAPE;
    if (kv_fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale)))
        return SINKATTN_E_SHAPE;
    if (batch == 0 || n_new == 0) return -1;  // nothing to do (not an error)
    if (!kv->k || !kv->v || !k_new || !v_new || !seq_lens) return SINKATTN_E_NULL;
    if (kv->layout == SINKATTN_KV_PAGED && !kv->block_table) return SINKATTN_E_NULL;
    if (misaligned(kv->k) || misaligned(kv->v) || misaligned(k_new) || misaligned(v_new) || misaligned(seq_lens) ||
        (kv->layout == SINKATTN_KV_PAGED && misaligned(kv->block_table)))
        return SINKATTN_E_ALIGN;
    p = AppendParams{};
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    // the descriptor is shared with decode, which only reads; appending writes the cache
    p.k_cache = static_cast<uint16_t *>(const_cast<void *>(kv->k));
    p.v_cache = static_cast<uint16_t *>(const_cast<void *>(kv->v));
    p.k_cache8 = static_cast<uint8_t *>(const_cast<void *>(kv->k));
    p.v_cache8 = static_cast<uint8_t *>(const_cast<void *>(kv->v));
    p.paged = kv->layout == SINKATTN_KV_PAGED;
    p.block_table = p.paged ? kv->block_table : nullptr;
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.hkv = hkv;
    p.n_new = n_new;
    p.window = p.paged ? 0 : window;
    p.page_size = p.paged ? kv->page_size : 0;
    p.max_pages = p.paged ? kv->max_pages : 0;
    p.num_pages = p.paged ? kv->num_pages : 0;
    p.fp8 = kv_fp8 ? 1 : 0;
    p.k_scale = kv_fp8 ? k_scale : 1.f;
    p.v_scale = kv_fp8 ? v_scale : 1.f;
    return SINKATTN_OK;
}
}  // namespace

extern "C" {

int sinkattn_kv_append(const sinkattn_kv *kv, int window, int32_t batch, int32_t hkv, int32_t n_new,
                       const void *k_new, const void *v_new, const int32_t *seq_lens, int kv_fp8, float k_scale,
                       float v_scale, void *stream) {
    AppendParams p;
    const int st = append_params(kv, window, batch, hkv, n_new, k_new, v_new, seq_lens, kv_fp8, k_scale, v_scale, p);
    if (st) return st < 0 ? SINKATTN_OK : st;
    return launch_kv_append(p, static_cast<hipStream_t>(stream)) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}

int sinkattn_decode_prologue(double theta, int window, const sinkattn_dims *d, int32_t n_new, const void *q_in,
                             void *q_out, const void *k_new, const void *v_new, const sinkattn_kv *kv, int kv_fp8,
                             float k_scale, float v_scale, const int32_t *seq_lens, void *stream) {
    if (!d) return SINKATTN_E_NULL;
    if (d->d_qk != kDqkSupported || d->d_v != kDvSupported) return SINKATTN_E_UNSUPPORTED;
    if (d->hq <= 0 || d->hkv <= 0 || d->hq % d->hkv || d->hkv > 65535) return SINKATTN_E_SHAPE;
    if (!(theta > 0.0) || !isfinite(theta)) return SINKATTN_E_SHAPE;
    PrologueParams pp{};
    const int st =
        append_params(kv, window, d->batch, d->hkv, n_new, k_new, v_new, seq_lens, kv_fp8, k_scale, v_scale, pp.a);
    if (st) return st < 0 ? SINKATTN_OK : st;
    if (!q_in || !q_out) return SINKATTN_E_NULL;
    if (misaligned(q_in) || misaligned(q_out)) return SINKATTN_E_ALIGN;
    pp.q_in = static_cast<const uint16_t *>(q_in);
    pp.q_out = static_cast<uint16_t *>(q_out);
    pp.hq = d->hq;
    for (int i = 0; i < 32; ++i) pp.inv_freq[i] = pow(theta, -2.0 * i / 64.0);
    return launch_decode_prologue(pp, static_cast<hipStream_t>(stream)) ? SINKATTN_E_DEVICE : SINKATTN_OK;
}

int sinkattn_decode_step(double theta, int window, const sinkattn_dims *d, const void *q_in, const void *k_new,
                         const void *v_new, const sinkattn_kv *kv, const int32_t *seq_lens, int32_t max_seq_len,
                         const float *sink, const sinkattn_epilogue *ep, void *out, void *stream) {
    if (!d) return SINKATTN_E_NULL;
    if (!(theta > 0.0) || !isfinite(theta)) return SINKATTN_E_SHAPE;
    const StepArgs step{k_new, v_new, theta};
    return decode_common(SINKATTN_SWA, window, d, 1, q_in, kv, nullptr, nullptr, seq_lens, max_seq_len, sink, 0, 1.f,
                         1.f, ep, out, nullptr, 0, stream, false, &step);
}

int sinkattn_decode(int mode, int window, const sinkattn_dims *d, const void *q, const sinkattn_kv *kv,
                    const int32_t *seq_lens, int32_t max_seq_len, const float *sink, void *out, void *workspace,
                    size_t workspace_bytes, void *stream) {
    return sinkattn_decode_multi(mode, window, d, 1, q, kv, seq_lens, max_seq_len, sink, out, workspace,
                                 workspace_bytes, stream);
}

}  // extern "C"
