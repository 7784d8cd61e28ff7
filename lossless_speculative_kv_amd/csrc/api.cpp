// C ABI of libvc: argument checks on the host, then the kernel launchers.
// Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/vc.h"
#include "vc_internal.h"

namespace vc {

// launchers (defined with their kernels)
size_t draft_ws_bytes(const vc_attn_shape& sh, const vc_draft_kv& kv);
vc_status draft_launch(const vc_attn_shape& sh, const void* q, const vc_draft_kv& kv, float* out, void* ws,
                       hipStream_t stream);
size_t draft_partial_bytes(const vc_attn_shape& sh, const vc_draft_kv& kv);
size_t draft_noalloc_max_partial_bytes();
vc_status draft_launch_noalloc(const vc_attn_shape& sh, const void* q, const vc_draft_kv& kv, float* out,
                               hipStream_t stream);
size_t verify_ws_bytes(const vc_attn_shape& sh, int n_rows, int max_chunk_tokens);
vc_status verify_launch(const vc_attn_shape& sh, int n_rows, const void* q, const void* k_new, const void* v_new,
                        const vc_kv_chunk& ctx, const int32_t* ctx_len, int flags, float* out, void* ws,
                        size_t ws_bytes, hipStream_t stream);
int verify_max_rows();
size_t vocab_ws_bytes(int M, int K, int V);
int vocab_max_rows();
vc_status vocab_launch(int M, int K, int V, const float* h, const void* w, int32_t* argmax, float* max_logit,
                       float* logits, void* ws, hipStream_t stream);
vc_status accept_launch(int B, int k, const int32_t* x, const int32_t* y, int32_t* n_accept, int32_t* next_token,
                        int32_t* committed, hipStream_t stream);
vc_status kivi_quantize_launch(const vc_attn_shape& sh, int bits, const void* src_k, const void* src_v, int src_fp16,
                               int src_t_cap, int grid_blocks, int nblk_const, const int32_t* nblk_dev,
                               const int32_t* dst_tok_dev, const int32_t* skip, const vc_draft_cache& dc,
                               hipStream_t stream);
vc_status fill_i32_launch(int32_t* p, int n, int32_t value, hipStream_t stream);
vc_status tail_from_rows_launch(const vc_attn_shape& sh, const void* src_k, const void* src_v, int src_t_cap,
                                int row0, int n, const vc_draft_cache& dc, hipStream_t stream);
vc_status commit_launch(const vc_attn_shape& sh, int k, const int32_t* n_accept, const void* k_new,
                        const void* v_new, void* full_k, void* full_v, int full_t_cap, int32_t* ctx_len,
                        const vc_draft_cache& dc, int32_t* status, int32_t* scratch_nf, hipStream_t stream);
vc_status tokdrop_launch(const vc_attn_shape& sh, const float* scores, int T, int n_keep, int32_t* kept,
                         hipStream_t stream);

static thread_local std::string g_last_error;
static thread_local Timing g_timing;

Timing take_timing() {
  const Timing t = g_timing;
  g_timing = Timing{};
  return t;
}

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

vc_status fail(vc_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

vc_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return VC_OK;
}

}  // namespace vc

using vc::fail;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

vc_status check_shape(const vc_attn_shape* sh) {
  if (sh == nullptr) return fail(VC_ERR_INVALID_ARG, "shape is NULL");
  if (sh->batch < 1 || sh->batch > 255) return fail(VC_ERR_INVALID_ARG, "batch %d not in [1, 255]", sh->batch);
  if (sh->n_kv_heads < 1 || sh->n_kv_heads > 255)
    return fail(VC_ERR_INVALID_ARG, "n_kv_heads %d not in [1, 255]", sh->n_kv_heads);
  if (sh->n_q_heads < 1 || sh->n_q_heads % sh->n_kv_heads != 0)
    return fail(VC_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d", sh->n_q_heads, sh->n_kv_heads);
  if (sh->n_q_heads / sh->n_kv_heads > 16)
    return fail(VC_ERR_UNSUPPORTED, "query group %d > 16", sh->n_q_heads / sh->n_kv_heads);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(VC_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", sh->head_dim);
  return VC_OK;
}

#define VC_REQ(p, al, name)                                                                 \
  do {                                                                                      \
    if ((p) == nullptr) return fail(VC_ERR_INVALID_ARG, "%s is NULL", name);                \
    if (!aligned((p), (al))) return fail(VC_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, (int)(al)); \
  } while (0)

vc_status check_draft_kv(const vc_attn_shape* sh, const vc_draft_kv* kv) {
  if (kv == nullptr) return fail(VC_ERR_INVALID_ARG, "draft kv is NULL");
  if (kv->tail_cap <= 0 || kv->tail_cap % 32) return fail(VC_ERR_INVALID_ARG, "tail_cap %d must be a positive multiple of 32", kv->tail_cap);
  if (kv->body_cap < 0) return fail(VC_ERR_INVALID_ARG, "body_cap %d < 0", kv->body_cap);
  VC_REQ(kv->body_len, 4, "body_len");
  VC_REQ(kv->tail_len, 4, "tail_len");
  VC_REQ(kv->tail_k, 16, "tail_k");
  VC_REQ(kv->tail_v, 16, "tail_v");
  switch (kv->kind) {
    case VC_DRAFT_KIVI:
      if (kv->bits != 2 && kv->bits != 4) return fail(VC_ERR_UNSUPPORTED, "KIVI bits %d (supported: 2, 4)", kv->bits);
      if (kv->body_cap % 32) return fail(VC_ERR_INVALID_ARG, "KIVI body_cap %d must be a multiple of 32", kv->body_cap);
      VC_REQ(kv->kivi_blocks, 256, "kivi_blocks");
      // one (sequence, KV head)'s records are addressed with 32-bit byte offsets
      if (sh != nullptr && (int64_t)(kv->body_cap / 32) * 8 * sh->head_dim * (kv->bits + 1) > INT32_MAX)
        return fail(VC_ERR_UNSUPPORTED, "KIVI body_cap %d: one KV head's records exceed 2^31 bytes", kv->body_cap);
      break;
    case VC_DRAFT_TOKDROP:
      VC_REQ(kv->kept_idx, 4, "kept_idx");
      /* fall through */
    case VC_DRAFT_DENSE:
      VC_REQ(kv->src_k, 16, "src_k");
      VC_REQ(kv->src_v, 16, "src_v");
      if (kv->src_t_cap <= 0) return fail(VC_ERR_INVALID_ARG, "src_t_cap %d <= 0", kv->src_t_cap);
      if (kv->kind == VC_DRAFT_DENSE && kv->body_cap > kv->src_t_cap)
        return fail(VC_ERR_INVALID_ARG, "dense body_cap %d > src_t_cap %d", kv->body_cap, kv->src_t_cap);
      break;
    default:
      return fail(VC_ERR_UNSUPPORTED, "draft kind %d", kv->kind);
  }
  return VC_OK;
}

vc_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return VC_OK;
  if (ws == nullptr) return fail(VC_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(VC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (have < need) return fail(VC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
  return VC_OK;
}

// Clears a pending vc_time_next_call setting when an entry point returns,
// whether or not a launcher consumed it.
struct TimingClear {
  ~TimingClear() { (void)vc::take_timing(); }
};

}  // namespace

extern "C" {

const char* vc_version(void) { return "vericache-mi355x 0.1 (gfx950)"; }
const char* vc_last_error(void) { return vc::g_last_error.c_str(); }

vc_status vc_time_next_call(void* start_event, void* stop_event, int32_t scope) {
  if (scope != VC_TIME_CALL && scope != VC_TIME_MAIN_KERNEL)
    return fail(VC_ERR_INVALID_ARG, "scope %d is neither VC_TIME_CALL nor VC_TIME_MAIN_KERNEL", scope);
  vc::g_timing.start = static_cast<hipEvent_t>(start_event);
  vc::g_timing.stop = static_cast<hipEvent_t>(stop_event);
  vc::g_timing.scope = scope;
  return VC_OK;
}

vc_status vc_kivi_block_bytes(int32_t head_dim, int32_t bits, size_t* bytes) {
  TimingClear timing_clear;
  if (head_dim != 64 && head_dim != 128) return fail(VC_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (bits != 2 && bits != 4) return fail(VC_ERR_UNSUPPORTED, "KIVI bits %d (supported: 2, 4)", bits);
  if (bytes == nullptr) return fail(VC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (size_t)8 * head_dim * (bits + 1);
  return VC_OK;
}

vc_status vc_draft_workspace_bytes(const vc_attn_shape* shape, const vc_draft_kv* kv, size_t* bytes) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if ((st = check_draft_kv(shape, kv)) != VC_OK) return st;
  if (bytes == nullptr) return fail(VC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = vc::draft_ws_bytes(*shape, *kv);
  return VC_OK;
}

vc_status vc_draft_decode_attn(const vc_attn_shape* shape, const void* q, const vc_draft_kv* kv, float* out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if ((st = check_draft_kv(shape, kv)) != VC_OK) return st;
  VC_REQ(q, 16, "q");
  VC_REQ(out, 16, "out");
  if ((st = check_ws(ws, ws_bytes, vc::draft_ws_bytes(*shape, *kv))) != VC_OK) return st;
  return vc::draft_launch(*shape, q, *kv, out, ws, stream);
}

vc_status vc_draft_decode_attn_noalloc(const vc_attn_shape* shape, const void* q, const vc_draft_kv* kv, float* out,
                                       hipStream_t stream) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if ((st = check_draft_kv(shape, kv)) != VC_OK) return st;
  VC_REQ(q, 16, "q");
  VC_REQ(out, 16, "out");
  const size_t need = vc::draft_partial_bytes(*shape, *kv), have = vc::draft_noalloc_max_partial_bytes();
  if (need > have)
    return fail(VC_ERR_WORKSPACE, "this call needs %zu bytes of split partials; the allocation-free entry point "
                "holds %zu (use vc_draft_decode_attn with a workspace)", need, have);
  return vc::draft_launch_noalloc(*shape, q, *kv, out, stream);
}

vc_status vc_verify_workspace_bytes(const vc_attn_shape* shape, int32_t n_rows, int32_t max_chunk_tokens,
                                    size_t* bytes) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (n_rows < 1 || n_rows > 64) return fail(VC_ERR_INVALID_ARG, "n_rows %d not in [1, 64]", n_rows);
  if (n_rows * (shape->n_q_heads / shape->n_kv_heads) > vc::verify_max_rows())
    return fail(VC_ERR_UNSUPPORTED, "n_rows * group = %d > %d", n_rows * (shape->n_q_heads / shape->n_kv_heads),
                vc::verify_max_rows());
  if (max_chunk_tokens < 0) return fail(VC_ERR_INVALID_ARG, "max_chunk_tokens %d < 0", max_chunk_tokens);
  if (bytes == nullptr) return fail(VC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = vc::verify_ws_bytes(*shape, n_rows, max_chunk_tokens);
  return VC_OK;
}

vc_status vc_verify_attn(const vc_attn_shape* shape, int32_t n_rows, const void* q, const void* k_new,
                         const void* v_new, const vc_kv_chunk* ctx, const int32_t* ctx_len, int32_t flags, float* out,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (n_rows < 1 || n_rows > 64) return fail(VC_ERR_INVALID_ARG, "n_rows %d not in [1, 64]", n_rows);
  if (n_rows * (shape->n_q_heads / shape->n_kv_heads) > vc::verify_max_rows())
    return fail(VC_ERR_UNSUPPORTED, "n_rows * group > %d", vc::verify_max_rows());
  VC_REQ(q, 16, "q");
  VC_REQ(k_new, 16, "k_new");
  VC_REQ(v_new, 16, "v_new");
  VC_REQ(ctx_len, 4, "ctx_len");
  if (ctx == nullptr) return fail(VC_ERR_INVALID_ARG, "ctx is NULL");
  if (ctx->tok_count < 0 || ctx->tok_begin < 0 || ctx->tok_count > ctx->t_cap)
    return fail(VC_ERR_INVALID_ARG, "chunk tok_begin %d tok_count %d t_cap %d", ctx->tok_begin, ctx->tok_count,
                ctx->t_cap);
  if (ctx->tok_count > 0) {
    VC_REQ(ctx->k, 16, "ctx.k");
    VC_REQ(ctx->v, 16, "ctx.v");
  }
  if ((flags & ~(VC_VERIFY_BEGIN | VC_VERIFY_END)) != 0) return fail(VC_ERR_INVALID_ARG, "flags 0x%x", flags);
  if ((flags & VC_VERIFY_END) != 0) VC_REQ(out, 16, "out");
  if ((st = check_ws(ws, ws_bytes, vc::verify_ws_bytes(*shape, n_rows, ctx->tok_count))) != VC_OK) return st;
  return vc::verify_launch(*shape, n_rows, q, k_new, v_new, *ctx, ctx_len, flags, out, ws, ws_bytes, stream);
}

// Argument checks and sizes behind the *_workspace_bytes entry points; the
// launching calls use these directly, so that no entry point calls another
// (each one consumes a pending vc_time_next_call setting when it returns).
static vc_status vocab_ws_query(int32_t m_rows, int32_t hidden, int32_t vocab, size_t* bytes) {
  if (m_rows < 1 || m_rows > vc::vocab_max_rows())
    return fail(VC_ERR_UNSUPPORTED, "m_rows %d not in [1, %d]", m_rows, vc::vocab_max_rows());
  if (hidden < 128 || hidden % 128) return fail(VC_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128", hidden);
  if (vocab < 1) return fail(VC_ERR_INVALID_ARG, "vocab %d < 1", vocab);
  if (bytes == nullptr) return fail(VC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = vc::vocab_ws_bytes(m_rows, hidden, vocab);
  return VC_OK;
}

vc_status vc_vocab_workspace_bytes(int32_t m_rows, int32_t hidden, int32_t vocab, size_t* bytes) {
  TimingClear timing_clear;
  return vocab_ws_query(m_rows, hidden, vocab, bytes);
}

vc_status vc_vocab_logits(int32_t m_rows, int32_t hidden, int32_t vocab, const float* h, const void* w,
                          int32_t* argmax, float* max_logit, float* logits, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  TimingClear timing_clear;
  size_t need = 0;
  vc_status st = vocab_ws_query(m_rows, hidden, vocab, &need);
  if (st != VC_OK) return st;
  VC_REQ(h, 16, "h");
  VC_REQ(w, 16, "w");
  VC_REQ(argmax, 4, "argmax");
  if (max_logit != nullptr && !aligned(max_logit, 4)) return fail(VC_ERR_INVALID_ARG, "max_logit misaligned");
  if (logits != nullptr && !aligned(logits, 16)) return fail(VC_ERR_INVALID_ARG, "logits is not 16-byte aligned");
  if ((st = check_ws(ws, ws_bytes, need)) != VC_OK) return st;
  return vc::vocab_launch(m_rows, hidden, vocab, h, w, argmax, max_logit, logits, ws, stream);
}

vc_status vc_greedy_accept(int32_t batch, int32_t k, const int32_t* x, const int32_t* y, int32_t* n_accept,
                           int32_t* next_token, int32_t* committed, hipStream_t stream) {
  TimingClear timing_clear;
  if (batch < 1) return fail(VC_ERR_INVALID_ARG, "batch %d < 1", batch);
  if (k < 0 || k > 1024) return fail(VC_ERR_INVALID_ARG, "k %d not in [0, 1024]", k);
  VC_REQ(x, 4, "x");
  VC_REQ(y, 4, "y");
  VC_REQ(n_accept, 4, "n_accept");
  VC_REQ(next_token, 4, "next_token");
  if (committed != nullptr && !aligned(committed, 4)) return fail(VC_ERR_INVALID_ARG, "committed misaligned");
  return vc::accept_launch(batch, k, x, y, n_accept, next_token, committed, stream);
}

static size_t commit_ws_bytes(const vc_attn_shape& sh) { return ((size_t)sh.batch * 4 + 255) / 256 * 256; }

vc_status vc_commit_workspace_bytes(const vc_attn_shape* shape, size_t* bytes) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (bytes == nullptr) return fail(VC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = commit_ws_bytes(*shape);
  return VC_OK;
}

vc_status vc_commit_round(const vc_attn_shape* shape, int32_t k, const int32_t* n_accept, const void* k_new,
                          const void* v_new, void* full_k, void* full_v, int32_t full_t_cap, int32_t* ctx_len,
                          const vc_draft_cache* draft, int32_t* status_flags, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (k < 0 || k > 63) return fail(VC_ERR_INVALID_ARG, "k %d not in [0, 63]", k);
  VC_REQ(n_accept, 4, "n_accept");
  VC_REQ(k_new, 16, "k_new");
  VC_REQ(v_new, 16, "v_new");
  VC_REQ(full_k, 16, "full_k");
  VC_REQ(full_v, 16, "full_v");
  VC_REQ(ctx_len, 4, "ctx_len");
  VC_REQ(status_flags, 4, "status_flags");
  if (full_t_cap <= 0) return fail(VC_ERR_INVALID_ARG, "full_t_cap %d", full_t_cap);
  if (draft == nullptr) return fail(VC_ERR_INVALID_ARG, "draft is NULL");
  VC_REQ(draft->body_len, 4, "draft.body_len");
  VC_REQ(draft->tail_len, 4, "draft.tail_len");
  if (draft->kind != VC_DRAFT_DENSE) {
    VC_REQ(draft->tail_k, 16, "draft.tail_k");
    VC_REQ(draft->tail_v, 16, "draft.tail_v");
    if (draft->tail_cap <= 0 || draft->tail_cap % 32) return fail(VC_ERR_INVALID_ARG, "tail_cap %d", draft->tail_cap);
  }
  if (draft->kind == VC_DRAFT_KIVI) {
    if (draft->bits != 2 && draft->bits != 4) return fail(VC_ERR_UNSUPPORTED, "KIVI bits %d", draft->bits);
    if (draft->body_cap % 32) return fail(VC_ERR_INVALID_ARG, "body_cap %d", draft->body_cap);
    if (draft->residual < 0 || draft->residual % 32)
      return fail(VC_ERR_INVALID_ARG, "residual %d must be a non-negative multiple of 32", draft->residual);
    VC_REQ(draft->kivi_blocks, 256, "draft.kivi_blocks");
  } else if (draft->kind != VC_DRAFT_TOKDROP && draft->kind != VC_DRAFT_DENSE) {
    return fail(VC_ERR_UNSUPPORTED, "draft kind %d", draft->kind);
  }
  if ((st = check_ws(ws, ws_bytes, commit_ws_bytes(*shape))) != VC_OK) return st;
  return vc::commit_launch(*shape, k, n_accept, k_new, v_new, full_k, full_v, full_t_cap, ctx_len, *draft, status_flags,
                           static_cast<int32_t*>(ws), stream);
}

vc_status vc_kivi_quantize(const vc_attn_shape* shape, const void* src_k, const void* src_v, int32_t src_t_cap,
                           int32_t n_body, int32_t n_tail, const vc_draft_cache* draft, hipStream_t stream) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (draft == nullptr || draft->kind != VC_DRAFT_KIVI) return fail(VC_ERR_INVALID_ARG, "draft must be a KIVI cache");
  if (draft->bits != 2 && draft->bits != 4) return fail(VC_ERR_UNSUPPORTED, "KIVI bits %d", draft->bits);
  if (draft->body_cap % 32) return fail(VC_ERR_INVALID_ARG, "body_cap %d", draft->body_cap);
  if (n_body < 0 || n_body % 32 || n_body > draft->body_cap)
    return fail(VC_ERR_INVALID_ARG, "n_body %d (multiple of 32, <= body_cap %d)", n_body, draft->body_cap);
  if (n_tail < 0 || n_tail > draft->tail_cap || (int64_t)n_body + n_tail > src_t_cap)
    return fail(VC_ERR_INVALID_ARG, "n_tail %d (tail_cap %d, src_t_cap %d)", n_tail, draft->tail_cap, src_t_cap);
  VC_REQ(src_k, 16, "src_k");
  VC_REQ(src_v, 16, "src_v");
  VC_REQ(draft->body_len, 4, "draft.body_len");
  VC_REQ(draft->tail_len, 4, "draft.tail_len");
  VC_REQ(draft->kivi_blocks, 256, "draft.kivi_blocks");
  if (n_tail > 0) {
    VC_REQ(draft->tail_k, 16, "draft.tail_k");
    VC_REQ(draft->tail_v, 16, "draft.tail_v");
  }
  st = vc::kivi_quantize_launch(*shape, draft->bits, src_k, src_v, 0, src_t_cap, n_body / 32, n_body / 32, nullptr,
                                nullptr, nullptr, *draft, stream);
  if (st != VC_OK) return st;
  if ((st = vc::tail_from_rows_launch(*shape, src_k, src_v, src_t_cap, n_body, n_tail, *draft, stream)) != VC_OK)
    return st;
  if ((st = vc::fill_i32_launch(draft->body_len, shape->batch, n_body, stream)) != VC_OK) return st;
  return vc::fill_i32_launch(draft->tail_len, shape->batch, n_tail, stream);
}

static vc_status tokdrop_ws_query(const vc_attn_shape* shape, int32_t T, size_t* bytes) {
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (T < 1 || T > (1 << 24)) return fail(VC_ERR_INVALID_ARG, "T %d not in [1, 2^24]", T);
  if (bytes == nullptr) return fail(VC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  return VC_OK;
}

vc_status vc_tokdrop_workspace_bytes(const vc_attn_shape* shape, int32_t T, size_t* bytes) {
  TimingClear timing_clear;
  return tokdrop_ws_query(shape, T, bytes);
}

vc_status vc_tokdrop_select(const vc_attn_shape* shape, const float* scores, int32_t T, int32_t n_keep,
                            int32_t* kept_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  TimingClear timing_clear;
  size_t need = 0;
  vc_status st = tokdrop_ws_query(shape, T, &need);
  if (st != VC_OK) return st;
  (void)ws;
  (void)ws_bytes;
  if (n_keep < 0 || n_keep > T) return fail(VC_ERR_INVALID_ARG, "n_keep %d not in [0, T=%d]", n_keep, T);
  VC_REQ(scores, 4, "scores");
  VC_REQ(kept_idx, 4, "kept_idx");
  return vc::tokdrop_launch(*shape, scores, T, n_keep, kept_idx, stream);
}

vc_status vc_stage_full_kv(const vc_attn_shape* shape, const void* host_k, const void* host_v, int64_t t_host,
                           int32_t tok_begin, int32_t tok_count, void* dev_k, void* dev_v, int32_t chunk_cap,
                           hipStream_t copy_stream, hipEvent_t done) {
  TimingClear timing_clear;
  vc_status st;
  if ((st = check_shape(shape)) != VC_OK) return st;
  if (host_k == nullptr || host_v == nullptr || dev_k == nullptr || dev_v == nullptr)
    return fail(VC_ERR_INVALID_ARG, "NULL buffer");
  if (tok_begin < 0 || tok_count < 0 || (int64_t)tok_begin + tok_count > t_host || tok_count > chunk_cap)
    return fail(VC_ERR_INVALID_ARG, "tok_begin %d tok_count %d t_host %lld chunk_cap %d", tok_begin, tok_count,
                (long long)t_host, chunk_cap);
  const size_t row = (size_t)shape->head_dim * 2;
  const size_t rows = (size_t)shape->batch * shape->n_kv_heads;
  if (tok_count > 0) {
    const void* srcs[2] = {host_k, host_v};
    void* dsts[2] = {dev_k, dev_v};
    for (int i = 0; i < 2; ++i) {
      const char* src = static_cast<const char*>(srcs[i]) + (size_t)tok_begin * row;
      const hipError_t e = hipMemcpy2DAsync(dsts[i], (size_t)chunk_cap * row, src, (size_t)t_host * row,
                                            (size_t)tok_count * row, rows, hipMemcpyHostToDevice, copy_stream);
      if (e != hipSuccess) return fail(VC_ERR_HIP, "stage copy: %s", hipGetErrorString(e));
    }
  }
  if (done != nullptr) {
    const hipError_t e = hipEventRecord(done, copy_stream);
    if (e != hipSuccess) return fail(VC_ERR_HIP, "stage event: %s", hipGetErrorString(e));
  }
  return VC_OK;
}

}  // extern "C"
