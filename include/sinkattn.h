/*
 * sinkattn.h -- C ABI of libsinkattn.so: causal grouped-query softmax attention with a
 * learnable per-query-head sink term in the softmax denominator, for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (the sink softmax of "MiMo-V2-Flash 架构 QA", Q3.7 and Q3.8; the sink is
 * described on the paper-notes page "MiMo-V2-Flash Technical Report", §4.1 and §4.3, and
 * its eager form on "MiMo-V2-Flash 模型架构深度拆解", CH 10.1):
 *
 *   a_ij = scale * q_i . k_j
 *   m_i  = max(max_{j in J(i)} a_ij, sink_h)
 *   o_i  = sum_{j in J(i)} exp(a_ij - m_i) v_j / (exp(sink_h - m_i) + sum_{j in J(i)} exp(a_ij - m_i))
 *
 *   J(i) = { 0 <= j <= i }                      SINKATTN_GLOBAL (causal)
 *        = { max(0, i - window + 1) <= j <= i } SINKATTN_SWA    (the `window` most recent
 *                                                               keys, the query's own included)
 *
 * The sink has no value vector: it only enlarges the denominator, so the weights of a row
 * sum to less than one.  It is given per QUERY head (the model declares it with
 * num_attention_heads entries, deep-dive page CH 10.3) and in the units of the scaled
 * logits (it is not multiplied by `scale`).  A NULL sink pointer means no sink term
 * (standard softmax attention).  sink = +inf gives an all-zero output row; NaN is a caller
 * error and is not checked.  GQA: query head h reads KV head h / (hq / hkv).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or synchronises, and keeps no mutable global state (thread-safe).
 *    The one exception is sinkattn_decode_ex_noalloc, which keeps its partial results in a
 *    scratch array of its own on each device (see there).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 *    asynchronously.  Results are valid once the stream has reached that point.
 *  - Tensors are dense, row-major, in the index order written next to each argument.
 *    bf16 means IEEE bfloat16 (raw 16-bit storage); sink is float32.
 *  - Every pointer must be 16-byte aligned.
 *  - Argument errors return a nonzero status at once and enqueue nothing.  A failed
 *    kernel launch returns SINKATTN_E_DEVICE.  Faults during execution surface on the
 *    stream like any other HIP error.
 *  - Supported head sizes: d_qk = 192 and d_v = 128 (the model's qk/v head dims,
 *    deep-dive page CH 8.1 and CH 10.3).  Other sizes return SINKATTN_E_UNSUPPORTED.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SINKATTN_GLOBAL = 0, SINKATTN_SWA = 1 } sinkattn_mode;
typedef enum { SINKATTN_KV_RING = 0, SINKATTN_KV_PAGED = 1 } sinkattn_kv_layout;

enum {
    SINKATTN_OK = 0,
    SINKATTN_E_NULL = 1,        /* a required pointer is NULL                         */
    SINKATTN_E_SHAPE = 2,       /* a size is negative/zero where it must not be, or    */
                                /* hq % hkv != 0, or a cache is too small for a length */
    SINKATTN_E_UNSUPPORTED = 3, /* head sizes other than 192/128, unknown mode/layout, */
                                /* a ring cache in global mode                         */
    SINKATTN_E_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
    SINKATTN_E_WORKSPACE = 5,   /* workspace NULL or smaller than required             */
    SINKATTN_E_DEVICE = 6       /* the kernel launch failed                            */
};

/* Problem sizes.  seqlen: prefill length L (ignored by decode).  scale: logit scale,
 * normally 1/sqrt(d_qk) (deep-dive page CH 10.3: scaling = head_dim ** -0.5); it must be a
 * positive finite number. */
typedef struct {
    int32_t batch, seqlen, hq, hkv, d_qk, d_v;
    float scale;
} sinkattn_dims;

/*
 * KV cache descriptor for decode.
 *  RING  (sliding-window mode only; deep-dive page CH 2.6: sliding layers keep only the
 *        last `window` tokens): k bf16 [batch][hkv][window][d_qk], v bf16
 *        [batch][hkv][window][d_v]; the token at position p is in slot p mod window.
 *        block_table must be NULL; page_size, max_pages, num_pages are ignored.
 *  PAGED (either mode; global layers keep every token): k bf16
 *        [num_pages][hkv][page_size][d_qk], v bf16 [num_pages][hkv][page_size][d_v];
 *        the token at position p of sequence b is in page block_table[b][p / page_size]
 *        at offset p mod page_size.  block_table int32 [batch][max_pages].  A contiguous
 *        cache is the identity table.  A page id outside [0, num_pages) is never read:
 *        that sequence's output row becomes NaN.
 */
typedef struct {
    int32_t layout;
    const void *k;
    const void *v;
    const int32_t *block_table;
    int32_t page_size, max_pages, num_pages;
} sinkattn_kv;

/*
 * Optional work at the end of the attention (the *_ex entry points; a NULL pointer means
 * out_scale = 1 and no lse).
 *   out_scale  multiplies every output element; must be finite.  The attention layer scales
 *              the values by 0.707 before attention ("MiMo-V2-Flash 模型架构深度拆解", CH 10.3
 *              forward step 2; "MiMo-V2-Flash 架构 QA", Q2.10); the output is linear in the
 *              values, so passing that factor here gives the same result without a pass
 *              over V.
 *   lse        device float32, 4-byte aligned, one value per output row laid out like the
 *              output without its last axis, or NULL: the row's log-sum-exp in natural
 *              log, log(exp(sink) + sum over the visible keys of exp(scale * q.k)), the
 *              log of the sink softmax denominator ("MiMo-V2-Flash 架构 QA", Q3.8).  No
 *              sink and no visible key: -inf; a row before its sequence (decode): the
 *              sink; sink +inf: +inf; a row whose output is NaN: NaN.
 */
typedef struct {
    float out_scale;
    float *lse;
} sinkattn_epilogue;

/*
 * Bytes of device workspace sinkattn_prefill needs for these sizes (batch, seqlen, hkv are
 * read): a transposed copy of V, 2 * batch * hkv * 128 * roundup(seqlen, 64) bytes.
 * Returns (size_t)-1 for invalid sizes.
 */
size_t sinkattn_prefill_workspace_bytes(const sinkattn_dims *d);

/*
 * Prefill: every position of every sequence attends causally (GLOBAL) or within the
 * sliding window (SWA) over the same sequence.
 *   mode      SINKATTN_GLOBAL or SINKATTN_SWA
 *   window    window size W >= 1 (SWA; ignored by GLOBAL).  W >= seqlen equals GLOBAL.
 *   d         sizes; batch >= 0, seqlen >= 0 (zero-sized work is a no-op), hq % hkv == 0,
 *             seqlen * 384 < 2^31
 *   q         bf16 [batch][hq][seqlen][d_qk]
 *   k         bf16 [batch][hkv][seqlen][d_qk]
 *   v         bf16 [batch][hkv][seqlen][d_v]
 *   sink      float32 [hq], or NULL for no sink
 *   out       bf16 [batch][hq][seqlen][d_v]  (written; may not alias the inputs)
 *   workspace device scratch of at least sinkattn_prefill_workspace_bytes(d) bytes; its
 *             contents need no initialisation and are overwritten.  Concurrent calls need
 *             separate workspaces.
 * Two kernels run on `stream`: one writes V transposed into the workspace, the second
 * computes attention.  Accumulation is float32; the probabilities enter the value product
 * as bf16; out is rounded to nearest even.
 */
int sinkattn_prefill(int mode, int window, const sinkattn_dims *d, const void *q, const void *k,
                     const void *v, const float *sink, void *out, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace sinkattn_prefill_chunk needs: the transposed copy of V over all
 * kv_len keys, 2 * batch * hkv * 128 * roundup(kv_len, 64) bytes (batch, seqlen, hkv are
 * read; seqlen <= kv_len).  Returns (size_t)-1 for invalid sizes.
 */
size_t sinkattn_prefill_chunk_workspace_bytes(const sinkattn_dims *d, int32_t kv_len);

/*
 * Chunked prefill over a cached prefix: the last d->seqlen positions of sequences that are
 * kv_len tokens long.  The serving set-up on the model card ("MiMo-V2-Flash-Base", SGLang
 * quick start) prefills long prompts in chunks of 16384 tokens; each chunk's queries attend
 * to the keys of the earlier chunks and causally within the chunk, which is the prefill
 * definition above restricted to rows kv_len - seqlen .. kv_len - 1.
 *   d         sizes as for sinkattn_prefill; d->seqlen = Lq, the new tokens (0 <= Lq <= kv_len)
 *   kv_len    keys per sequence, the prefix and the chunk together; kv_len * 384 < 2^31
 *   q         bf16 [batch][hq][Lq][d_qk]: query row r is position kv_len - Lq + r
 *   k         bf16 [batch][hkv][kv_len][d_qk]
 *   v         bf16 [batch][hkv][kv_len][d_v]
 *   sink      float32 [hq], or NULL
 *   out       bf16 [batch][hq][Lq][d_v]
 *   workspace at least sinkattn_prefill_chunk_workspace_bytes(d, kv_len) bytes
 * With kv_len == d->seqlen this is sinkattn_prefill.  Errors as sinkattn_prefill; kv_len <
 * d->seqlen is SINKATTN_E_SHAPE.
 */
int sinkattn_prefill_chunk(int mode, int window, const sinkattn_dims *d, int32_t kv_len,
                           const void *q, const void *k, const void *v, const float *sink,
                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace sinkattn_prefill_cached needs: the gathered keys and values of
 * the rows the chunk sees (global: all kv_len positions; sliding window: the chunk and the
 * window - 1 positions before it) and their V^T copy.  (size_t)-1 for invalid arguments.
 */
size_t sinkattn_prefill_cached_workspace_bytes(int mode, int window, const sinkattn_dims *d,
                                               int32_t kv_len);

/*
 * Chunked prefill over a prefix that is already in a KV cache: the chunk's d->seqlen = Lq
 * queries at positions kv_len - Lq .. kv_len - 1 attend causally (or within the window) to the
 * prefix, read from the cache, and to the chunk's own keys, given contiguously.  The model
 * card's serving set-up prefills long prompts in chunks of 16384 tokens over a paged cache
 * ("MiMo-V2-Flash", SGLang quick start: chunked prefill size, page size); the result is the
 * prefill definition's rows kv_len - Lq .. kv_len - 1.
 *   q          bf16 [batch][hq][Lq][d_qk]
 *   k, v       bf16 [batch][hkv][Lq][d_qk], [batch][hkv][Lq][d_v]: the chunk's keys and values
 *   prefix     the cache holding positions 0 .. kv_len - Lq - 1: PAGED (either mode; the
 *              table covers them) or RING (sliding-window mode; it holds the prefix's last
 *              `window` positions, position p in slot p mod window).  Only read.
 *   sink, ep, out (bf16 [batch][hq][Lq][d_v]), stream as sinkattn_prefill_ex
 *   workspace  at least sinkattn_prefill_cached_workspace_bytes(mode, window, d, kv_len)
 * A first kernel gathers the visible prefix rows and the chunk into the workspace (one pass
 * over the keys the chunk sees); the prefill kernels then run on them.  A ring prefix with a
 * window of at most 128 and a multiple of 8 query heads per KV head is read in place by the
 * sliding-window kernel instead, and the workspace is not touched.  A prefix page id
 * outside [0, num_pages) is never read: every output row that sees that page is NaN, and so
 * may be rows that share a 32-key block with it.  Errors as
 * sinkattn_prefill_ex; a ring in global mode is SINKATTN_E_UNSUPPORTED; a page table too short
 * for the prefix is SINKATTN_E_SHAPE.
 */
int sinkattn_prefill_cached(int mode, int window, const sinkattn_dims *d, int32_t kv_len,
                            const void *q, const void *k, const void *v, const sinkattn_kv *prefix,
                            const float *sink, const sinkattn_epilogue *ep, void *out,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * sinkattn_prefill_chunk with an epilogue (lse: float32 [batch][hq][seqlen]).  Errors as
 * sinkattn_prefill_chunk; a non-finite out_scale is SINKATTN_E_SHAPE, a misaligned lse
 * SINKATTN_E_ALIGN.
 */
int sinkattn_prefill_ex(int mode, int window, const sinkattn_dims *d, int32_t kv_len,
                        const void *q, const void *k, const void *v, const float *sink,
                        const sinkattn_epilogue *ep, void *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace sinkattn_decode needs for these arguments (0 when none).
 * max_seq_len is the host-side upper bound on seq_lens used to plan the key splits; pass
 * the same value to sinkattn_decode.  Returns (size_t)-1 for invalid sizes.
 */
size_t sinkattn_decode_workspace_bytes(int mode, int window, const sinkattn_dims *d,
                                       int32_t max_seq_len);

/*
 * Decode: one new query per sequence, at position seq_lens[b] - 1; its own key and value
 * must already be in the cache (the cache update precedes attention, deep-dive page
 * CH 10.3 forward steps 6-7).
 *   q            bf16 [batch][hq][d_qk]
 *   kv           cache descriptor (above)
 *   seq_lens     device int32 [batch]: tokens in each sequence INCLUDING the new one.
 *                1 <= seq_lens[b] <= max_seq_len (PAGED: also <= max_pages * page_size).
 *                A value <= 0 yields a zero output row; one above max_seq_len yields NaN.
 *   max_seq_len  host upper bound on seq_lens (>= 1), used for split planning only
 *   sink         float32 [hq], or NULL
 *   out          bf16 [batch][hq][d_v]
 *   workspace    device scratch of at least sinkattn_decode_workspace_bytes(...) bytes
 *                (may be NULL when that is 0); its contents need no initialisation.
 * Long contexts are split across workgroups; the per-split partial results are merged
 * in a second kernel on the same stream, where the sink term enters exactly once.
 */
int sinkattn_decode(int mode, int window, const sinkattn_dims *d, const void *q,
                    const sinkattn_kv *kv, const int32_t *seq_lens, int32_t max_seq_len,
                    const float *sink, void *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Bytes of device workspace sinkattn_decode_multi needs (0 when none); (size_t)-1 for
 * invalid arguments.  Pass the same max_seq_len to sinkattn_decode_multi.
 */
size_t sinkattn_decode_multi_workspace_bytes(int mode, int window, const sinkattn_dims *d,
                                             int32_t q_len, int32_t max_seq_len);

/*
 * Multi-token decode: q_len new queries per sequence, at positions seq_lens[b] - q_len ..
 * seq_lens[b] - 1, as when the model checks several draft tokens in one forward pass
 * (deep-dive page CH 4.4: the main model verifies the MTP drafts in parallel; paper-notes
 * page §6.4 walks through one such step with four tokens).  The new tokens' keys and values
 * must already be in the cache.  Query i attends to the keys j <= its own position p_i
 * (causal among the new tokens) and, in SWA mode, only to j > p_i - window; each gets the
 * sink term of its head.  q_len = 1 is sinkattn_decode.
 *   q_len        1 .. 256
 *   q            bf16 [batch][hq][q_len][d_qk]
 *   kv           PAGED (either mode).  A RING cache holds only the last `window` tokens,
 *                too few for the earlier new tokens' windows: RING needs q_len = 1
 *                (SINKATTN_E_UNSUPPORTED otherwise).
 *   seq_lens     device int32 [batch]: tokens in each sequence INCLUDING the q_len new
 *                ones.  A query whose position is negative (seq_lens[b] < q_len) gets a zero
 *                row; seq_lens[b] above max_seq_len makes the sequence's rows NaN.
 *   out          bf16 [batch][hq][q_len][d_v]
 *   everything else as sinkattn_decode.  All q_len * (hq / hkv) queries of a KV head read
 * its cache once.
 */
int sinkattn_decode_multi(int mode, int window, const sinkattn_dims *d, int32_t q_len,
                          const void *q, const sinkattn_kv *kv, const int32_t *seq_lens,
                          int32_t max_seq_len, const float *sink, void *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Verification of drafted tokens whose keys and values are NOT in the cache: the q_len new
 * tokens (positions seq_lens[b] - q_len .. seq_lens[b] - 1) attend causally, as in
 * sinkattn_decode_multi, to the cached positions before them and to the new tokens up to
 * their own position, whose keys and values are read from k_new / v_new.  The main model
 * checks the drafts of its multi-token-prediction head in one parallel pass ("MiMo-V2-Flash
 * 模型架构深度拆解", CH 4.4), and the drafts after the first mismatch are rejected (paper-notes
 * page "MiMo-V2-Flash Technical Report", §6.4): writing them into a sliding-window ring first
 * would overwrite committed keys that a rejection cannot restore, so the cache is only read
 * here and the caller appends the accepted tokens afterwards (sinkattn_kv_append).
 *   kv         RING (sliding-window mode; it holds the last `window` committed positions,
 *              position p in slot p mod window) or PAGED (either mode; the table covers the
 *              committed positions 0 .. seq_lens[b] - q_len - 1).  bf16 only.
 *   k_new      bf16 [batch][hkv][q_len][d_qk], v_new bf16 [batch][hkv][q_len][d_v]: token t at
 *              position seq_lens[b] - q_len + t (already rotated, as the cache's keys)
 *   q_len      1 .. 256; seq_lens counts the committed tokens plus the q_len new ones
 *   q, out, seq_lens, max_seq_len, sink, ep, workspace (sinkattn_decode_multi_workspace_bytes),
 *   stream     as sinkattn_decode_ex.
 * Errors as sinkattn_decode_ex; k_new or v_new NULL is SINKATTN_E_NULL.  The cache and the
 * new tokens' rows are read with a row lookup per key (no page-aligned fast path).
 */
int sinkattn_decode_verify(int mode, int window, const sinkattn_dims *d, int32_t q_len,
                           const void *q, const sinkattn_kv *kv, const void *k_new,
                           const void *v_new, const int32_t *seq_lens, int32_t max_seq_len,
                           const float *sink, const sinkattn_epilogue *ep, void *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode (q_len >= 1 new tokens, as sinkattn_decode_multi) from a KV cache held in 8-bit
 * floating point: the pages size the cache with one byte per element (paper notes "MiMo-
 * V2-Flash Technical Report", §3.2), which halves the bytes that bound decode.
 *   kv         PAGED only, page_size a multiple of 32 (else SINKATTN_E_UNSUPPORTED);
 *              kv->k: uint8 [num_pages][hkv][page_size][d_qk], kv->v: uint8 [num_pages][hkv]
 *              [page_size][d_v], each byte an OCP E4M3 code (sign, 4 exponent bits with bias
 *              7, 3 mantissa bits; no infinities, code 0x7F / 0xFF is NaN)
 *   k_scale    K element = k_scale * value(code); v_scale likewise for V; both finite and
 *              > 0 (else SINKATTN_E_SHAPE)
 *   q, out, seq_lens, sink, workspace, stream: as sinkattn_decode_multi (q and out bf16); the
 *              workspace size is sinkattn_decode_multi_workspace_bytes(mode, window, d, q_len,
 *              max_seq_len).
 * The codes are widened to bf16 exactly after they reach LDS; k_scale joins the logit
 * scale and v_scale multiplies the output, so the result is attention over the scaled
 * values.
 */
int sinkattn_decode_fp8(int mode, int window, const sinkattn_dims *d, int32_t q_len,
                        const void *q, const sinkattn_kv *kv, const int32_t *seq_lens,
                        int32_t max_seq_len, const float *sink, float k_scale, float v_scale,
                        void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace sinkattn_prefill_backward needs: 4 * batch * hq * (2 * seqlen +
 * ceil(seqlen / 16)).  Returns (size_t)-1 for invalid sizes.
 */
size_t sinkattn_prefill_backward_workspace_bytes(const sinkattn_dims *d);

/*
 * Backward of prefill attention, including the gradient of the sink.  The sink is a
 * learnable per-head scalar ("MiMo-V2-Flash 模型架构深度拆解", CH 10.1) that enters the
 * outputs only through the softmax denominator ("MiMo-V2-Flash 架构 QA", Q3.8); with P the
 * forward weights, D_i = dO_i . O_i and dS = P (dO v^T - D):
 *   dq = scale dS k,  dk = scale dS^T q,  dv = P^T dO,  dsink_h = -sum_i exp(sink_h - LSE_i) D_i
 * (dsink summed over the batch).
 *   mode, window, d   as for sinkattn_prefill; hq / hkv must be a multiple of 4 (else
 *                     SINKATTN_E_UNSUPPORTED)
 *   q, k, v, sink     the forward's inputs
 *   out, lse          the forward's output (bf16 [batch][hq][seqlen][d_v]) and its per-row
 *                     log-sum-exp (float32 [batch][hq][seqlen], from sinkattn_prefill_ex)
 *   dout              bf16 [batch][hq][seqlen][d_v], the gradient of out
 *   dq, dk, dv        float32 [batch][hq][seqlen][d_qk], [batch][hkv][seqlen][d_qk],
 *                     [batch][hkv][seqlen][d_v]: written (not accumulated into)
 *   dsink             float32 [hq], written; required when sink is given, ignored otherwise
 *   workspace         at least sinkattn_prefill_backward_workspace_bytes(d) bytes
 * The products run on bf16 matrix cores with float32 accumulation (the weights and dS enter
 * them rounded to bf16); the sink gradient is summed in a fixed order (deterministic).
 */
int sinkattn_prefill_backward(int mode, int window, const sinkattn_dims *d, const void *q,
                              const void *k, const void *v, const float *sink, const void *out,
                              const void *dout, const float *lse, float *dq, float *dk, float *dv,
                              float *dsink, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Partial rotary position embedding, in place ("MiMo-V2-Flash 模型架构深度拆解", CH 3.5 and
 * CH 10.5; "MiMo-V2-Flash 架构 QA", Q2.7): of each row's 192 q or k dimensions only the first
 * 64 turn, pair i (dimensions i and i + 32) by the angle pos * theta^(-2i/64); the other 128
 * carry content only.  theta is 10 000 in sliding-window layers and 5 000 000 in global
 * ones.  Apply it to q and to the new keys before attention and before sinkattn_kv_append.
 *   theta     > 0, finite (else SINKATTN_E_SHAPE)
 *   x         bf16 [batch][heads][rows][192], rotated in place
 *   seq_lens  device int32 [batch] or NULL: with it, row r of sequence b is at position
 *             seq_lens[b] - rows + r (the new tokens of a decode step); without it at
 *             pos0 + r (a prefill chunk starting at pos0)
 * The angle is formed in double precision and reduced before its sine and cosine are taken
 * in float, so positions up to 256K keep their accuracy.  Zero sizes are a no-op.
 */
int sinkattn_rope(double theta, int32_t batch, int32_t heads, int32_t rows, void *x,
                  const int32_t *seq_lens, int32_t pos0, void *stream);

/*
 * Write new tokens' keys and values into a KV cache (the cache update that precedes
 * attention, deep-dive CH 10.3 forward step 6).
 *   kv        descriptor of the cache to write (RING or PAGED, as for decode; the library
 *             writes through its k and v pointers)
 *   window    ring slots (RING)
 *   batch, hkv, n_new  sizes; n_new tokens per sequence
 *   k_new     bf16 [batch][hkv][n_new][192] (already rotated), v_new bf16 [batch][hkv][n_new][128]
 *   seq_lens  device int32 [batch]: tokens per sequence INCLUDING the new ones; token t
 *             goes to position seq_lens[b] - n_new + t
 *   kv_fp8    0: bf16 cache; 1: E4M3 cache, codes of value / k_scale (or v_scale), rounded
 *             to nearest even and clamped to +-448
 * Positions below 0, ring positions older than the last `window` of the sequence, and page
 * ids outside [0, num_pages) are skipped.  Errors: SINKATTN_E_NULL, _SHAPE, _ALIGN,
 * _UNSUPPORTED as for decode.
 */
int sinkattn_kv_append(const sinkattn_kv *kv, int window, int32_t batch, int32_t hkv, int32_t n_new,
                       const void *k_new, const void *v_new, const int32_t *seq_lens, int kv_fp8,
                       float k_scale, float v_scale, void *stream);

/*
 * The steps before decode attention in one kernel ("MiMo-V2-Flash 模型架构深度拆解", CH 10.3
 * forward steps 3-6): the partial RoPE of the new tokens' queries and keys (as sinkattn_rope,
 * at positions seq_lens[b] - n_new + t) and the cache write of the rotated keys and the values
 * (as sinkattn_kv_append), reading each input once.  The results are bit-identical to
 * sinkattn_rope on q, sinkattn_rope on k_new and sinkattn_kv_append in turn (the rotated keys
 * are rounded to bf16 before an 8-bit cache encodes them), except that k_new is not modified.
 *   theta        10 000 (sliding-window layers) or 5 000 000 (global layers); > 0, finite
 *   window       ring slots (RING caches)
 *   d            batch, hq, hkv (d_qk = 192, d_v = 128; seqlen and scale are not read)
 *   n_new        new tokens per sequence
 *   q_in         bf16 [batch][hq][n_new][192]: the new queries before rotation
 *   q_out        bf16 [batch][hq][n_new][192]: written, rotated; may be q_in (in place)
 *   k_new, v_new bf16 [batch][hkv][n_new][192 / 128]: the new keys (before rotation), values
 *   kv, kv_fp8, k_scale, v_scale, seq_lens  as sinkattn_kv_append
 * Then call the decode entry point on q_out.  Errors as sinkattn_rope and sinkattn_kv_append.
 */
int sinkattn_decode_prologue(double theta, int window, const sinkattn_dims *d, int32_t n_new,
                             const void *q_in, void *q_out, const void *k_new, const void *v_new,
                             const sinkattn_kv *kv, int kv_fp8, float k_scale, float v_scale,
                             const int32_t *seq_lens, void *stream);

/*
 * One whole sliding-window decode step in a single kernel ("MiMo-V2-Flash 模型架构深度拆解",
 * CH 10.3 forward steps 3-6 and the attention): the partial RoPE of the new token's queries
 * and key at position seq_lens[b] - 1, the write of the rotated key and the value into ring
 * slot (seq_lens[b] - 1) mod window, and the sink attention of the new token over the ring.
 * The output and the ring contents are bit-identical to sinkattn_decode_prologue (n_new = 1)
 * followed by sinkattn_decode_ex on its rotated queries.
 *   theta        10 000 for the sliding-window layers; > 0, finite
 *   window       ring slots W (<= 128), the window of the attention
 *   d            batch, hq, hkv (hq / hkv <= 16), scale (d_qk = 192, d_v = 128)
 *   q_in         bf16 [batch][hq][1][192]: the new token's queries before rotation (not modified)
 *   k_new, v_new bf16 [batch][hkv][1][192 / 128]: its key (before rotation) and value (not modified)
 *   kv           a RING bf16 cache, [batch][hkv][W][192] and [batch][hkv][W][128]: written
 *                at the new token's slot, read at every slot of the window
 *   seq_lens     device int32 [batch]: tokens per sequence including the new one; a length
 *                <= 0 writes nothing and gives a zero row; above max_seq_len, a NaN row
 *   max_seq_len  an upper bound of seq_lens (>= 1)
 *   sink, ep, out (bf16 [batch][hq][1][128]), stream  as sinkattn_decode_ex
 * No workspace (one split).  Errors: SINKATTN_E_UNSUPPORTED for any other cache layout, a ring
 * of more than 128 visible slots or more than 16 query heads per KV head (use
 * sinkattn_decode_prologue and sinkattn_decode_ex there); otherwise as sinkattn_decode_ex.
 */
int sinkattn_decode_step(double theta, int window, const sinkattn_dims *d, const void *q_in, const void *k_new,
                         const void *v_new, const sinkattn_kv *kv, const int32_t *seq_lens, int32_t max_seq_len,
                         const float *sink, const sinkattn_epilogue *ep, void *out, void *stream);

/*
 * Decode with every option: q_len new tokens (as sinkattn_decode_multi), a bf16 cache
 * (kv_fp8 = 0; k_scale and v_scale ignored) or an E4M3 cache (kv_fp8 = 1, as
 * sinkattn_decode_fp8), and an epilogue (lse: float32 [batch][hq][q_len]).  Errors as those
 * entry points; a non-finite out_scale is SINKATTN_E_SHAPE, a misaligned lse
 * SINKATTN_E_ALIGN.
 */
int sinkattn_decode_ex(int mode, int window, const sinkattn_dims *d, int32_t q_len,
                       const void *q, const sinkattn_kv *kv, int kv_fp8, float k_scale,
                       float v_scale, const int32_t *seq_lens, int32_t max_seq_len,
                       const float *sink, const sinkattn_epilogue *ep, void *out, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * sinkattn_decode_ex for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and the
 * same kernels, but no workspace argument.  The split partials go to a scratch array inside
 * the library, SINKATTN_NOALLOC_SCRATCH_BYTES of device memory that each GPU the library runs
 * on holds until the process ends (located on the first call on each device).  The call
 * allocates and frees nothing.
 *   Errors as sinkattn_decode_ex; SINKATTN_E_WORKSPACE when the partials these arguments
 *   need (sinkattn_decode_multi_workspace_bytes(mode, window, d, q_len, max_seq_len)) exceed
 *   SINKATTN_NOALLOC_SCRATCH_BYTES (decode of 8 sequences x 256K over 64 query heads needs
 *   4.3 MB with one token, 17.3 MB with 4 drafted tokens, 69 MB with 16); SINKATTN_E_DEVICE
 *   when the scratch array cannot be located.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (on
 *   different streams, or from different threads) race and give wrong results.
 *   Serialise them.
 */
#define SINKATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int sinkattn_decode_ex_noalloc(int mode, int window, const sinkattn_dims *d, int32_t q_len,
                               const void *q, const sinkattn_kv *kv, int kv_fp8, float k_scale,
                               float v_scale, const int32_t *seq_lens, int32_t max_seq_len,
                               const float *sink, const sinkattn_epilogue *ep, void *out,
                               void *stream);

/* Static, human-readable name of a status code. */
const char *sinkattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */
