"""ctypes binding of synth/libvcsynth.so, the device copy of the generator in
synth/__init__.py. Pointers are device addresses; stream is a raw handle."""
from __future__ import annotations

import ctypes as C
import os

try:  # bind to the HIP runtime torch already uses (one runtime per process)
    import torch  # noqa: F401
except ImportError:
    pass

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvcsynth.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lossless_speculative_kv_amd.build`")
lib = C.CDLL(LIB_PATH)
_P, _I, _U = C.c_void_p, C.c_int, C.c_uint64
lib.vcs_fill_ctx.argtypes = [_U, _I, _I, _I, _I, _I, _I, _P, _P, _P]
lib.vcs_fill_w.argtypes = [_U, _I, _I, _P, _P]
lib.vcs_fill_scores.argtypes = [_U, _I, _I, _I, _P, _P]
lib.vcs_embed.argtypes = [_U, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
lib.vcs_embed_draft.argtypes = [_U, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P]
for f in (lib.vcs_fill_ctx, lib.vcs_fill_w, lib.vcs_fill_scores, lib.vcs_embed, lib.vcs_embed_draft):
    f.restype = C.c_int


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def fill_ctx(seed, which_v, B, Hkv, T, D, t_cap, key_mult, out, stream):
    _ok(lib.vcs_fill_ctx(seed, 1 if which_v else 0, B, Hkv, T, D, t_cap, key_mult, out, stream), "vcs_fill_ctx")


def fill_w(seed, V, H, out, stream):
    _ok(lib.vcs_fill_w(seed, V, H, out, stream), "vcs_fill_w")


def fill_scores(seed, B, Hkv, T, out, stream):
    _ok(lib.vcs_fill_scores(seed, B, Hkv, T, out, stream), "vcs_fill_scores")


def embed(seed, tokens, n, Hq, Hkv, D, key_mult, q, k, v, stream):
    _ok(lib.vcs_embed(seed, tokens, n, Hq, Hkv, D, key_mult, q, k, v, stream), "vcs_embed")


def embed_draft(seed, tokens, stride, B, Hq, Hkv, D, key_mult, q, tail_k, tail_v, tail_cap, tail_fp16, tail_len,
                stream):
    _ok(lib.vcs_embed_draft(seed, tokens, stride, B, Hq, Hkv, D, key_mult, q, tail_k, tail_v, tail_cap,
                            1 if tail_fp16 else 0, tail_len, stream), "vcs_embed_draft")
