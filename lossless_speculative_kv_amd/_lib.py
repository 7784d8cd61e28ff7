"""ctypes binding of libvc (include/vc.h): the same entry points, argument
marshalling only. Pointers are plain integers (device addresses, or host
addresses for the staging source); streams and events are raw handles.

Importing this module loads the in-tree libvc.so and fails loudly when it is
missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvc.so")

VC_OK, VC_ERR_INVALID_ARG, VC_ERR_UNSUPPORTED, VC_ERR_WORKSPACE, VC_ERR_HIP = 0, -1, -2, -3, -4
VC_DRAFT_DENSE, VC_DRAFT_KIVI, VC_DRAFT_TOKDROP = 0, 1, 2
VC_VERIFY_BEGIN, VC_VERIFY_END = 1, 2
VC_TIME_CALL, VC_TIME_MAIN_KERNEL = 0, 1

EXPORTS = [
    "vc_version", "vc_last_error", "vc_time_next_call", "vc_kivi_block_bytes", "vc_draft_workspace_bytes", "vc_draft_decode_attn",
    "vc_draft_decode_attn_noalloc",
    "vc_verify_workspace_bytes", "vc_verify_attn", "vc_vocab_workspace_bytes", "vc_vocab_logits",
    "vc_greedy_accept", "vc_commit_workspace_bytes", "vc_commit_round", "vc_kivi_quantize",
    "vc_tokdrop_workspace_bytes", "vc_tokdrop_select", "vc_stage_full_kv",
]


class VCError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class vc_attn_shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32)]


class vc_draft_kv(C.Structure):
    _fields_ = [("kind", C.c_int32), ("bits", C.c_int32), ("body_cap", C.c_int32), ("tail_cap", C.c_int32),
                ("body_len", C.c_void_p), ("tail_len", C.c_void_p),
                ("kivi_blocks", C.c_void_p),
                ("kept_idx", C.c_void_p), ("src_k", C.c_void_p), ("src_v", C.c_void_p),
                ("src_t_cap", C.c_int32), ("tail_k", C.c_void_p), ("tail_v", C.c_void_p)]


class vc_kv_chunk(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("t_cap", C.c_int32), ("tok_begin", C.c_int32),
                ("tok_count", C.c_int32)]


class vc_draft_cache(C.Structure):
    _fields_ = [("kind", C.c_int32), ("bits", C.c_int32), ("body_cap", C.c_int32), ("tail_cap", C.c_int32),
                ("body_len", C.c_void_p), ("tail_len", C.c_void_p),
                ("kivi_blocks", C.c_void_p),
                ("tail_k", C.c_void_p), ("tail_v", C.c_void_p), ("residual", C.c_int32)]


def _load() -> C.CDLL:
    # libvc.so needs the HIP runtime (soname libamdhip64.so.7). PyTorch ships its
    # own copy and a process must hold exactly one runtime, so torch is loaded
    # first: the dynamic linker then binds libvc.so to the runtime torch uses.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lossless_speculative_kv_amd.build`")
    return C.CDLL(LIB_PATH)


lib = _load()

_P = C.c_void_p
_S = C.POINTER(vc_attn_shape)
_sigs = {
    "vc_version": ([], C.c_char_p),
    "vc_last_error": ([], C.c_char_p),
    "vc_time_next_call": ([_P, _P, C.c_int32], C.c_int32),
    "vc_kivi_block_bytes": ([C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "vc_draft_workspace_bytes": ([_S, C.POINTER(vc_draft_kv), C.POINTER(C.c_size_t)], C.c_int32),
    "vc_draft_decode_attn": ([_S, _P, C.POINTER(vc_draft_kv), _P, _P, C.c_size_t, _P], C.c_int32),
    "vc_draft_decode_attn_noalloc": ([_S, _P, C.POINTER(vc_draft_kv), _P, _P], C.c_int32),
    "vc_verify_workspace_bytes": ([_S, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "vc_verify_attn": ([_S, C.c_int32, _P, _P, _P, C.POINTER(vc_kv_chunk), _P, C.c_int32, _P, _P, C.c_size_t, _P],
                       C.c_int32),
    "vc_vocab_workspace_bytes": ([C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "vc_vocab_logits": ([C.c_int32, C.c_int32, C.c_int32, _P, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int32),
    "vc_greedy_accept": ([C.c_int32, C.c_int32, _P, _P, _P, _P, _P, _P], C.c_int32),
    "vc_commit_workspace_bytes": ([_S, C.POINTER(C.c_size_t)], C.c_int32),
    "vc_commit_round": ([_S, C.c_int32, _P, _P, _P, _P, _P, C.c_int32, _P, C.POINTER(vc_draft_cache), _P, _P,
                         C.c_size_t, _P], C.c_int32),
    "vc_kivi_quantize": ([_S, _P, _P, C.c_int32, C.c_int32, C.c_int32, C.POINTER(vc_draft_cache), _P], C.c_int32),
    "vc_tokdrop_workspace_bytes": ([_S, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "vc_tokdrop_select": ([_S, _P, C.c_int32, C.c_int32, _P, _P, C.c_size_t, _P], C.c_int32),
    "vc_stage_full_kv": ([_S, _P, _P, C.c_int64, C.c_int32, C.c_int32, _P, _P, C.c_int32, _P, _P], C.c_int32),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def last_error() -> str:
    return lib.vc_last_error().decode()


def version() -> str:
    return lib.vc_version().decode()


def vc_time_next_call(start_event, stop_event, scope=VC_TIME_CALL):
    """The next call on this thread records these hipEvent_t handles (ints or
    None) from its own kernel dispatches; see include/vc.h."""
    check(lib.vc_time_next_call(start_event, stop_event, scope), "vc_time_next_call")


def check(status: int, where: str) -> None:
    if status != VC_OK:
        raise VCError(status, where, last_error())


def _size(fn, *args) -> int:
    out = C.c_size_t(0)
    check(fn(*args, C.byref(out)), fn.__name__)
    return int(out.value)


# --- entry points with the C names (raise VCError on a non-OK status) -------

def vc_kivi_block_bytes(head_dim: int, bits: int) -> int:
    return _size(lib.vc_kivi_block_bytes, head_dim, bits)


def vc_draft_workspace_bytes(shape: vc_attn_shape, kv: vc_draft_kv) -> int:
    return _size(lib.vc_draft_workspace_bytes, C.byref(shape), C.byref(kv))


def vc_draft_decode_attn(shape, q, kv, out, ws, ws_bytes, stream):
    check(lib.vc_draft_decode_attn(C.byref(shape), q, C.byref(kv), out, ws, ws_bytes, stream), "vc_draft_decode_attn")


def vc_draft_decode_attn_noalloc(shape, q, kv, out, stream):
    check(lib.vc_draft_decode_attn_noalloc(C.byref(shape), q, C.byref(kv), out, stream),
          "vc_draft_decode_attn_noalloc")


def vc_verify_workspace_bytes(shape, n_rows, max_chunk_tokens) -> int:
    return _size(lib.vc_verify_workspace_bytes, C.byref(shape), n_rows, max_chunk_tokens)


def vc_verify_attn(shape, n_rows, q, k_new, v_new, ctx: vc_kv_chunk, ctx_len, flags, out, ws, ws_bytes, stream):
    check(lib.vc_verify_attn(C.byref(shape), n_rows, q, k_new, v_new, C.byref(ctx), ctx_len, flags, out, ws,
                             ws_bytes, stream), "vc_verify_attn")


def vc_vocab_workspace_bytes(m_rows, hidden, vocab) -> int:
    return _size(lib.vc_vocab_workspace_bytes, m_rows, hidden, vocab)


def vc_vocab_logits(m_rows, hidden, vocab, h, w, argmax, max_logit, logits, ws, ws_bytes, stream):
    check(lib.vc_vocab_logits(m_rows, hidden, vocab, h, w, argmax, max_logit, logits, ws, ws_bytes, stream),
          "vc_vocab_logits")


def vc_greedy_accept(batch, k, x, y, n_accept, next_token, committed, stream):
    check(lib.vc_greedy_accept(batch, k, x, y, n_accept, next_token, committed, stream), "vc_greedy_accept")


def vc_commit_workspace_bytes(shape) -> int:
    return _size(lib.vc_commit_workspace_bytes, C.byref(shape))


def vc_commit_round(shape, k, n_accept, k_new, v_new, full_k, full_v, full_t_cap, ctx_len, draft: vc_draft_cache,
                    status_flags, ws, ws_bytes, stream):
    check(lib.vc_commit_round(C.byref(shape), k, n_accept, k_new, v_new, full_k, full_v, full_t_cap, ctx_len,
                              C.byref(draft), status_flags, ws, ws_bytes, stream), "vc_commit_round")


def vc_kivi_quantize(shape, src_k, src_v, src_t_cap, n_body, n_tail, draft: vc_draft_cache, stream):
    check(lib.vc_kivi_quantize(C.byref(shape), src_k, src_v, src_t_cap, n_body, n_tail, C.byref(draft), stream),
          "vc_kivi_quantize")


def vc_tokdrop_workspace_bytes(shape, T) -> int:
    return _size(lib.vc_tokdrop_workspace_bytes, C.byref(shape), T)


def vc_tokdrop_select(shape, scores, T, n_keep, kept_idx, ws, ws_bytes, stream):
    check(lib.vc_tokdrop_select(C.byref(shape), scores, T, n_keep, kept_idx, ws, ws_bytes, stream),
          "vc_tokdrop_select")


def vc_stage_full_kv(shape, host_k, host_v, t_host, tok_begin, tok_count, dev_k, dev_v, chunk_cap, copy_stream,
                     done_event):
    check(lib.vc_stage_full_kv(C.byref(shape), host_k, host_v, t_host, tok_begin, tok_count, dev_k, dev_v,
                               chunk_cap, copy_stream, done_event), "vc_stage_full_kv")
