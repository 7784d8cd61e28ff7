/*
 * vc.h - C ABI of the VeriCache draft/verify hot path for AMD MI355X (gfx950).
 *
 * Method (VeriCache: Turning Lossy KV Cache into Lossless LLM Inference,
 * technical summary, section "Core algorithm"): a lossy compressed KV cache
 * drafts a run of k tokens with the same model; one forward pass over the
 * full cache verifies all k in parallel; tokens are accepted greedily up to
 * the first mismatch, plus a bonus token when every draft matches.
 *
 * Conventions for every call:
 *  - Pointers are device memory unless stated otherwise. fp16 / bf16 data is
 *    passed as `const void *` holding IEEE binary16 / bfloat16 bit patterns.
 *  - Calls are asynchronous on the given stream and never allocate, free or
 *    synchronise. The caller owns every buffer (including workspaces and
 *    pinned host memory) and keeps it alive until the stream has passed the
 *    call. No pointer is retained after return.
 *  - Argument checks (shapes, null pointers, alignment, supported modes,
 *    workspace size) run on the host before anything is enqueued; a failed
 *    check returns a negative status and enqueues nothing. Launch and copy
 *    failures return VC_ERR_HIP. Device-side faults surface at the caller's
 *    next synchronisation. vc_last_error() gives the text of the last
 *    failure on the calling thread.
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs (fixed split and merge order, no floating-point atomics).
 *  - Lengths that change while decoding (context, body, tail) are device
 *    int32 arrays indexed by sequence, so a batch may be ragged.
 */
#ifndef VC_H
#define VC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vc_status;
enum {
  VC_OK = 0,
  VC_ERR_INVALID_ARG = -1, /* null pointer, bad shape or alignment */
  VC_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim 96) */
  VC_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  VC_ERR_HIP = -4          /* a HIP launch or copy reported an error */
};

/* Library version string, and the text of the last non-OK status returned on
 * this thread ("" if none). */
const char *vc_version(void);
const char *vc_last_error(void);

/* Kernel timing without extra queue packets (for callers that measure the
 * calls). The next call made on this thread has its own kernel dispatches
 * record the given events: with VC_TIME_CALL, start_event when the call's
 * first kernel starts and stop_event when its last kernel ends; with
 * VC_TIME_MAIN_KERNEL, both around the call's main kernel (the verification
 * kernel before its split merge, the vocab product before its argmax
 * reduction; draft attention is one kernel, so both scopes time it). Recording events around a call from the host instead adds a
 * marker to the queue before and after it, which idles the GPU for a few
 * microseconds each time. Calls that take part: vc_draft_decode_attn,
 * vc_verify_attn, vc_vocab_logits; any other call discards the setting.
 * The events are hipEvent_t handles created by the caller on the device of
 * the call (passed as void *); either may be NULL. The setting is consumed by
 * the next call whatever its outcome. Returns VC_ERR_INVALID_ARG for an
 * unknown scope. */
enum { VC_TIME_CALL = 0, VC_TIME_MAIN_KERNEL = 1 };
vc_status vc_time_next_call(void *start_event, void *stop_event, int32_t scope);

/* Attention shape. head_dim is 64 or 128; n_q_heads % n_kv_heads == 0 and the
 * group g = n_q_heads / n_kv_heads is at most 16. Query head h reads KV head
 * h / g (contiguous groups). batch <= 255, n_kv_heads <= 255. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
} vc_attn_shape;

/* ------------------------------------------------------------------------- */
/* Compressed (draft) cache                                                   */
/* ------------------------------------------------------------------------- */
/* One descriptor covers every compressor (VeriCache summary, "Architecture
 * support": a single compressor interface over token dropping and
 * quantisation). The draft-visible token set of sequence b is
 *   body tokens [0, body_len[b])  followed by  tail tokens [0, tail_len[b]).
 *
 * VC_DRAFT_KIVI: the body is quantised (bits 2 or 4): keys per channel over
 *   groups of 32 tokens, values per token over groups of 32 channels, each
 *   group with an fp16 scale and zero point (x = code * scale + zero). The
 *   tail holds the most recent tokens unquantised, as fp16. body_len[b] must
 *   be a multiple of 32.
 *   Key scales: the kernel multiplies each query value (taken as fp16, exact
 *   for bf16 values of magnitude 2^-17 .. 65504) by the key scale of its
 *   channel in fp16. A key scale with at most three significant bits (what
 *   vc_kivi_quantize writes) makes that product exact, and the result is then
 *   within the attention tolerance of exact attention over the dequantised
 *   cache. Any other finite fp16 key scale is accepted, but each product is
 *   rounded to fp16: a score s_t = q . k_t / sqrt(D) gains an error of at most
 *   eps_t = sum_d (2^-11 |q_d scale_d| + 2^-25) code_td / sqrt(D), and each
 *   output channel d moves by at most (exp(2 eps) - 1) sum_t p_t |v_td - o_d|
 *   more (eps the largest eps_t of the row, p the exact softmax weights, o the
 *   exact output).
 *   Stored layout: the body is block-major, one record of
 *   BLK = 8 * D * (bits + 1) bytes (vc_kivi_block_bytes) per 32-token block,
 *   kivi_blocks [u][body_cap/32][BLK] with u = b * n_kv_heads + h, so that a
 *   block is one contiguous read. A record holds, at byte offsets:
 *     0          key codes uint32 [32][D*bits/32]: token-major; channel d of
 *                a token in word floor(d*bits/32) at bit (d*bits) % 32, LSB
 *                first.
 *     4*D*bits   value codes uint32 [64][D*bits/64]: lanes L = 16*q + c
 *                (q 0..3, c 0..15); lane L holds channels 16*m + c
 *                (m 0..D/16-1) of the tokens tau(q,s) = 4*q + s/2 + 16*(s%2)
 *                (s 0..7); code (m, s) in word (m*bits)/4 at bit
 *                8*(s/2) + 4*(s%2) + 2*(m%2)             for bits = 2,
 *                16*(s/4) + 8*(s%2) + 4*((s/2)%2)        for bits = 4.
 *     8*D*bits   key scale fp16 [D] (per channel, over the block's tokens),
 *                then key zero fp16 [D]; both in runs of 8 channels whose
 *                positions 0..7 hold channels 0, 2, 1, 3, 4, 6, 5, 7 of
 *                the run.
 *     8*D*bits + 4*D
 *                value scale fp16 [D/32][32], then value zero fp16
 *                [D/32][32]: entry 8*q + s of channel group j is the
 *                parameter of token tau(q,s) of the block.
 * VC_DRAFT_TOKDROP: the body is a sorted list of kept token positions
 *   kept_idx int32 [u][body_cap] (ascending, each < src_t_cap) into the bf16
 *   source rows src_k / src_v [u][src_t_cap][D]; the tail is bf16.
 * VC_DRAFT_DENSE: the identity compressor; body tokens are src rows
 *   [0, body_len[b]); the tail is bf16.
 * Tail arrays: [u][tail_cap][D], tail_cap a multiple of 32. */
enum { VC_DRAFT_DENSE = 0, VC_DRAFT_KIVI = 1, VC_DRAFT_TOKDROP = 2 };

typedef struct {
  int32_t kind;
  int32_t bits;       /* KIVI: 2 or 4; ignored otherwise */
  int32_t body_cap;   /* body capacity in tokens (KIVI: multiple of 32, and one
                         (sequence, KV head)'s records, body_cap / 32 records of
                         8 * head_dim * (bits + 1) bytes, below 2^31 bytes;
                         VC_ERR_UNSUPPORTED otherwise) */
  int32_t tail_cap;   /* tail capacity in tokens (multiple of 32) */
  const int32_t *body_len; /* [B] */
  const int32_t *tail_len; /* [B], >= 1 when attending */
  const void *kivi_blocks; /* KIVI body records, 256-byte aligned */
  const int32_t *kept_idx;
  const void *src_k, *src_v;
  int32_t src_t_cap;
  const void *tail_k, *tail_v;
} vc_draft_kv;

/* Bytes of one KIVI block record: 8 * head_dim * (bits + 1). */
vc_status vc_kivi_block_bytes(int32_t head_dim, int32_t bits, size_t *bytes);

/* Workspace size for vc_draft_decode_attn with this shape and cache. The
 * workspace starts with one 32-bit split counter per (sequence, KV head): it
 * must be all zero before its first use (e.g. hipMemset once after
 * allocation), and every completed call leaves those words zero again, so a
 * workspace is zeroed once and then reused. Calls that share a workspace
 * must not run concurrently. */
vc_status vc_draft_workspace_bytes(const vc_attn_shape *shape, const vc_draft_kv *kv, size_t *bytes);

/* Draft decode attention (VeriCache summary, "Core algorithm", drafting with
 * KV_comp; "P1": drafting is bound by HBM bandwidth). For every sequence b
 * and query head h: out[b][h] = softmax(K q / sqrt(D)) V over the draft-visible
 * set of KV head h / g, with K, V dequantised in registers (KIVI) or gathered
 * (token drop). q: bf16 [B][Hq][D]. out: fp32 [B][Hq][D]. */
vc_status vc_draft_decode_attn(const vc_attn_shape *shape, const void *q, const vc_draft_kv *kv,
                               float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of vc_draft_decode_attn, for callers that cannot
 * allocate (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation and kernels, with the workspace
 * taken from an 8 MiB device array inside the library instead of a caller
 * buffer (one copy per GPU the library runs on, held until the process
 * ends): a 260,352-byte region of split counters, then room for
 * 8,128,256 bytes of split partials, i.e. a call whose
 * vc_draft_workspace_bytes, less its counter words
 * (B * n_kv_heads * 4 rounded up to 256), exceeds that returns
 * VC_ERR_WORKSPACE and enqueues nothing (about B * n_q_heads * splits <=
 * 15,000 rows at head_dim 128). The caller still owns q, the cache and out.
 * The first call on a device also enqueues one small kernel on `stream` that
 * clears the counters; every completed call leaves them zero. All calls on
 * one GPU share the array: calls that may overlap on one GPU (different
 * streams, or graphs replayed concurrently) race and must be serialised by
 * the caller. Allocates and frees nothing. */
vc_status vc_draft_decode_attn_noalloc(const vc_attn_shape *shape, const void *q, const vc_draft_kv *kv, float *out,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Verification attention over the full cache                                 */
/* ------------------------------------------------------------------------- */
/* VeriCache summary, "Core algorithm" (verification: one forward pass over
 * KV_full checks the drafted tokens in parallel) and "Architecture support"
 * (long-context decoding keeps KV_full in host memory and loads it over
 * PCIe for verification). Row j (0..n_rows-1) of sequence b is the query of
 * token x_j; it sees context positions [0, ctx_len[b]) and block rows 0..j
 * (causal inside the block).
 *
 * The context may arrive in chunks: a chunk holds positions
 * [tok_begin, tok_begin + tok_count) at rows 0.. of k / v (bf16
 * [u][t_cap][D]). The first call of a verification passes VC_VERIFY_BEGIN,
 * the last VC_VERIFY_END (resident context: one call with both, tok_begin 0);
 * the calls must cover [0, max ctx_len) exactly once, in any grouping, with
 * the same ws. Partial results are merged in a fixed order (call order, then
 * split order). */
enum { VC_VERIFY_BEGIN = 1, VC_VERIFY_END = 2 };

typedef struct {
  const void *k, *v;
  int32_t t_cap;
  int32_t tok_begin;
  int32_t tok_count;
} vc_kv_chunk;

/* Workspace for vc_verify_attn; max_chunk_tokens bounds tok_count. */
vc_status vc_verify_workspace_bytes(const vc_attn_shape *shape, int32_t n_rows, int32_t max_chunk_tokens,
                                    size_t *bytes);

/* Position-major block arrays: q: bf16 [n_rows][B][Hq][D]; k_new, v_new:
 * bf16 [n_rows][B][Hkv][D] (the block tokens' keys/values); ctx_len: [B];
 * out: fp32 [n_rows][B][Hq][D], written by the END call. n_rows <= 64 and
 * n_rows * g <= 288.
 * Arithmetic: scores q.k from the exact bf16 operands in fp32; the softmax
 * probabilities are rounded to fp16 (11 significant bits) for P x V and for
 * the row sums alike, and the values are taken to fp16 for that product,
 * which is exact for |v| in [2^-17, 65504] (smaller values round to
 * multiples of 2^-24); values must not exceed 65504 in magnitude. The
 * relative error of a row is then of order 2^-12 (measured rel-L2 about
 * 2e-4 against fp64 on random data, for any context length). */
vc_status vc_verify_attn(const vc_attn_shape *shape, int32_t n_rows, const void *q, const void *k_new,
                         const void *v_new, const vc_kv_chunk *ctx, const int32_t *ctx_len, int32_t flags,
                         float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Vocabulary projection + greedy argmax                                      */
/* ------------------------------------------------------------------------- */
/* Greedy decoding picks the largest logit (VeriCache summary, "Experimental
 * results": identical output under greedy decoding). h: fp32 [m_rows][hidden],
 * rounded to bf16 (nearest even) on load; w: bf16 [vocab][hidden].
 * argmax [m_rows]: first index of the largest fp32 logit (-0 == +0; NaN
 * logits are not ordered: a row that holds one has no defined argmax).
 * max_logit [m_rows] (optional, may be NULL): that logit.
 * logits [m_rows][vocab] (optional, may be NULL): all logits.
 * hidden must be a multiple of 128; m_rows <= 448; vocab < 2^31. */
vc_status vc_vocab_workspace_bytes(int32_t m_rows, int32_t hidden, int32_t vocab, size_t *bytes);
vc_status vc_vocab_logits(int32_t m_rows, int32_t hidden, int32_t vocab, const float *h, const void *w,
                          int32_t *argmax, float *max_logit, float *logits, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Greedy acceptance                                                          */
/* ------------------------------------------------------------------------- */
/* VeriCache summary, "Core algorithm" (acceptance). Position-major arrays:
 * x [k+1][B] holds x_0..x_k (x_0 the pending token, x_1..x_k the drafts);
 * y [k+1][B] holds y_1..y_{k+1}, y_{j+1} the full-cache argmax after
 * x_0..x_j. Writes n_accept[b] = m (first j < k with x_{j+1} != y_{j+1},
 * else k), next_token[b] = y_{m+1} (the correction, or the bonus when
 * m == k), and optionally committed [k+1][B] = x_1..x_m, y_{m+1}, then -1.
 * next_token may alias row 0 of x (the next round's pending token). k <= 1024. */
vc_status vc_greedy_accept(int32_t batch, int32_t k, const int32_t *x, const int32_t *y, int32_t *n_accept,
                           int32_t *next_token, int32_t *committed, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Commit / restart                                                           */
/* ------------------------------------------------------------------------- */
/* Mutable view of the draft cache for vc_commit_round (same layout as
 * vc_draft_kv). */
typedef struct {
  int32_t kind, bits, body_cap, tail_cap;
  int32_t *body_len, *tail_len;
  void *kivi_blocks;
  void *tail_k, *tail_v;
  int32_t residual; /* KIVI: recent-token window R kept unquantised */
} vc_draft_cache;

/* Applies an accepted round (VeriCache summary, "Core algorithm": restart
 * from the last accepted token). For each sequence b with m = n_accept[b]:
 * block rows 0..m of k_new / v_new (bf16 [k+1][B][Hkv][D], the keys/values
 * of x_0..x_m) are appended to the full cache at ctx_len[b] (ctx_len += m+1);
 * the draft tail, which holds tail_start = tail_len[b] - k rows from before
 * the round plus the k drafted inputs, keeps tail_start + m + 1 rows (rows
 * x_0..x_m rewritten from the block); DENSE: body_len[b] = ctx_len[b] and
 * the tail empties; KIVI: while the tail holds >= residual + 32 tokens its
 * oldest 32 are quantised into the body and removed from the tail.
 * Sequences whose full cache would exceed full_t_cap (or tail/body caps)
 * are left unchanged and flagged in status_flags[b] (nonzero), [B].
 * The calls that follow must not run before this one (same stream). */
vc_status vc_commit_workspace_bytes(const vc_attn_shape *shape, size_t *bytes);
vc_status vc_commit_round(const vc_attn_shape *shape, int32_t k, const int32_t *n_accept, const void *k_new,
                          const void *v_new, void *full_k, void *full_v, int32_t full_t_cap, int32_t *ctx_len,
                          const vc_draft_cache *draft, int32_t *status_flags, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Compressor builders                                                        */
/* ------------------------------------------------------------------------- */
/* KIVI compression of a context: rows [0, n_body) of bf16 src_k / src_v
 * [u][src_t_cap][D] become body blocks [0, n_body/32) with the min/max rule
 * zero = fp16(min); value scale = fp16(rne((max - min) / (2^bits - 1)));
 * key scale = (max - min) / (2^bits - 1) rounded up to three significant
 * bits (stored as fp16: a bf16 query value times it is exact in fp16),
 * code = clamp(rint((x - zero) / scale), 0, 2^bits - 1) in fp64 (0 when
 * scale == 0); rows [n_body, n_body + n_tail) become the fp16 tail (the
 * recent-token residual). Sets body_len[b] = n_body, tail_len[b] = n_tail. */
vc_status vc_kivi_quantize(const vc_attn_shape *shape, const void *src_k, const void *src_v, int32_t src_t_cap,
                           int32_t n_body, int32_t n_tail, const vc_draft_cache *draft, hipStream_t stream);

/* Token-drop selection: kept_idx [u][n_keep] = the n_keep positions with the
 * largest fp32 score (scores [u][T]), ties to the lower position, ascending.
 * n_keep <= T <= 2^24. Workspace from vc_tokdrop_workspace_bytes. */
vc_status vc_tokdrop_workspace_bytes(const vc_attn_shape *shape, int32_t T, size_t *bytes);
vc_status vc_tokdrop_select(const vc_attn_shape *shape, const float *scores, int32_t T, int32_t n_keep,
                            int32_t *kept_idx, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Full-cache staging (host -> device)                                        */
/* ------------------------------------------------------------------------- */
/* VeriCache summary, "P1" (verification is bound by the interconnect that
 * brings the full cache from host memory; drafting by HBM; the scheduler
 * overlaps them) and "Architecture support" (long-context decoding keeps
 * KV_full in CPU memory). Copies positions [tok_begin, tok_begin + tok_count)
 * of the pinned host cache host_k / host_v (bf16 [u][t_host][D]) to rows
 * 0..tok_count-1 of dev_k / dev_v ([u][chunk_cap][D]) with one 2-D async
 * copy per tensor on copy_stream, then records `done` (if not NULL) on it.
 * host_k / host_v are HOST pointers (pinned, e.g. hipHostMalloc). */
vc_status vc_stage_full_kv(const vc_attn_shape *shape, const void *host_k, const void *host_v, int64_t t_host,
                           int32_t tok_begin, int32_t tok_count, void *dev_k, void *dev_v, int32_t chunk_cap,
                           hipStream_t copy_stream, hipEvent_t done);

#ifdef __cplusplus
}
#endif
#endif /* VC_H */
