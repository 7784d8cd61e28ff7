"""The C ABI without a GPU: the library loads, exports every entry point that
include/vc.h declares, and rejects bad arguments on the host (nothing is
launched, so these run anywhere)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc.h")

L = pytest.importorskip("lossless_speculative_kv_amd._lib", reason="libvc.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:vc_status|const char \*)\s*(vc_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L.lib, n), n
    assert sorted(L.EXPORTS) == names


def test_version_string():
    assert "gfx950" in L.version()


def shape(B=2, Hq=8, Hkv=2, D=128):
    return L.vc_attn_shape(B, Hq, Hkv, D)


def kivi_kv(**kw):
    kv = L.vc_draft_kv()
    kv.kind, kv.bits, kv.body_cap, kv.tail_cap = L.VC_DRAFT_KIVI, 2, 1024, 64
    fake = 0x10000  # never dereferenced: every test below fails before any launch
    for f in ("body_len", "tail_len", "tail_k", "tail_v"):
        setattr(kv, f, fake)
    kv.kivi_blocks = 0x100000
    for k, v in kw.items():
        setattr(kv, k, v)
    return kv


def status(fn, *args):
    return fn(*args)


def test_bad_shapes_rejected():
    out = C.c_size_t()
    for sh, code in [(shape(B=0), L.VC_ERR_INVALID_ARG), (shape(Hq=6, Hkv=4), L.VC_ERR_INVALID_ARG),
                     (shape(D=96), L.VC_ERR_UNSUPPORTED), (shape(Hq=64, Hkv=2), L.VC_ERR_UNSUPPORTED)]:
        assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(kivi_kv()), C.byref(out)) == code
        assert "batch" in L.last_error() or "head" in L.last_error() or "group" in L.last_error()


def test_draft_argument_checks():
    sh = shape()
    out = C.c_size_t()
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(kivi_kv(bits=3)), C.byref(out)) == L.VC_ERR_UNSUPPORTED
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(kivi_kv(kivi_blocks=None)), C.byref(out)) == L.VC_ERR_INVALID_ARG
    assert "kivi_blocks" in L.last_error()
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(kivi_kv(tail_cap=40)), C.byref(out)) == L.VC_ERR_INVALID_ARG
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(kivi_kv(kivi_blocks=0x100010)), C.byref(out)) == L.VC_ERR_INVALID_ARG
    assert "aligned" in L.last_error()
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(kivi_kv()), C.byref(out)) == L.VC_OK


def test_kivi_records_within_32_bit_offsets():
    # one (sequence, KV head)'s records are addressed with 32-bit byte offsets:
    # at D = 128, 2-bit, a record is 3072 bytes, so 699050 records fit below
    # 2^31 bytes and 699051 do not
    sh = shape()
    out = C.c_size_t()
    rec = 8 * 128 * 3
    assert (2**31 - 1) // rec == 699050
    ok = kivi_kv(body_cap=699050 * 32)
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(ok), C.byref(out)) == L.VC_OK
    big = kivi_kv(body_cap=699051 * 32)
    assert L.lib.vc_draft_workspace_bytes(C.byref(sh), C.byref(big), C.byref(out)) == L.VC_ERR_UNSUPPORTED
    assert "2^31" in L.last_error()
    assert out.value > 0
    # workspace too small
    rc = L.lib.vc_draft_decode_attn(C.byref(sh), 0x10000, C.byref(kivi_kv()), 0x10000, 0x10000, 16, None)
    assert rc == L.VC_ERR_WORKSPACE
    rc = L.lib.vc_draft_decode_attn(C.byref(sh), None, C.byref(kivi_kv()), 0x10000, 0x10000, 1 << 30, None)
    assert rc == L.VC_ERR_INVALID_ARG


def test_verify_vocab_accept_checks():
    sh = shape()
    out = C.c_size_t()
    assert L.lib.vc_verify_workspace_bytes(C.byref(sh), 0, 1024, C.byref(out)) == L.VC_ERR_INVALID_ARG
    assert L.lib.vc_verify_workspace_bytes(C.byref(sh), 65, 1024, C.byref(out)) == L.VC_ERR_INVALID_ARG
    assert L.lib.vc_verify_workspace_bytes(C.byref(sh), 33, 1024, C.byref(out)) == L.VC_OK
    sh16 = shape(Hq=32, Hkv=2)  # g = 16, 33 * 16 rows > 288
    assert L.lib.vc_verify_workspace_bytes(C.byref(sh16), 33, 1024, C.byref(out)) == L.VC_ERR_UNSUPPORTED
    ctx = L.vc_kv_chunk(0x10000, 0x10000, 100, 0, 200)  # tok_count > t_cap
    rc = L.lib.vc_verify_attn(C.byref(sh), 4, 0x10000, 0x10000, 0x10000, C.byref(ctx), 0x10000, 3, 0x10000, 0x10000,
                              1 << 30, None)
    assert rc == L.VC_ERR_INVALID_ARG
    assert L.lib.vc_vocab_workspace_bytes(8, 100, 1000, C.byref(out)) == L.VC_ERR_UNSUPPORTED
    assert L.lib.vc_vocab_workspace_bytes(0, 128, 1000, C.byref(out)) == L.VC_ERR_UNSUPPORTED
    assert L.lib.vc_vocab_workspace_bytes(8, 4096, 128256, C.byref(out)) == L.VC_OK
    assert L.lib.vc_greedy_accept(0, 4, 0x10000, 0x10000, 0x10000, 0x10000, None, None) == L.VC_ERR_INVALID_ARG
    assert L.lib.vc_greedy_accept(2, 4, None, 0x10000, 0x10000, 0x10000, None, None) == L.VC_ERR_INVALID_ARG


def _ring_plan(M, K, V):
    """The ring kernel's plan, restated: row tiles per row group and vocab
    groups per row-tile count, then the k split of the last round of 256
    CUs (at least 8 k slices per part, only when that round would leave half
    of the CUs or more idle)."""
    mt = (M + 15) // 16
    nt, vg = (max(2, (mt + 1) // 2), 4) if mt <= 18 else \
        (5, 2) if mt <= 20 else (13, 4) if mt <= 26 else (7, 2)
    nwg = -(-V // (64 * vg))
    left, full, split = nwg % 256, nwg, 1
    if left and 2 * left <= 256 and min(256 // left, K // 32 // 8) >= 2:
        split, full = min(256 // left, K // 32 // 8), nwg - left
    return nt, vg, nwg, full, split


def _align(x):
    return -(-x // 256) * 256


@pytest.mark.parametrize("M,K,V", [(416, 5120, 152064), (264, 4096, 128256), (164, 5120, 32768), (33, 8192, 128256),
                                   (48, 1024, 65948), (448, 256, 1000), (300, 1024, 3000), (90, 512, 3001),
                                   (200, 512, 2500), (250, 1024, 4001)])
def test_vocab_ring_workspace(M, K, V):
    """Workspace of the ring path: the bf16 hidden copy, a 64-bit key per row
    and key slot (whole slices one slot, a k-split slice one per vocab group),
    and the k parts' fp32 products (8 waves x 4 vocab tiles x NT row tiles x
    64 lanes x 16 bytes per part)."""
    nt, vg, nwg, full, split = _ring_plan(M, K, V)
    Mp = (M + 15) // 16 * 16
    nkeys = full + (nwg - full) * vg if split > 1 else nwg
    parts = (nwg - full) * split * 8 * 4 * nt * 64 * 16 if split > 1 else 0
    out = C.c_size_t()
    assert L.lib.vc_vocab_workspace_bytes(M, K, V, C.byref(out)) == L.VC_OK
    assert out.value == _align(Mp * K * 2) + _align(nkeys * M * 8) + _align(parts)
    if (M, K, V) == (416, 5120, 152064):
        assert (nwg, full, split, nkeys) == (594, 512, 3, 840)  # 82 leftover slices in 3 k parts


def test_stage_and_compressor_checks():
    sh = shape()
    rc = L.lib.vc_stage_full_kv(C.byref(sh), 0x10000, 0x10000, 1000, 900, 200, 0x10000, 0x10000, 4096, None, None)
    assert rc == L.VC_ERR_INVALID_ARG
    dc = L.vc_draft_cache()
    dc.kind = L.VC_DRAFT_TOKDROP
    assert L.lib.vc_kivi_quantize(C.byref(sh), 0x10000, 0x10000, 1024, 64, 32, C.byref(dc), None) == L.VC_ERR_INVALID_ARG
    out = C.c_size_t()
    assert L.lib.vc_tokdrop_workspace_bytes(C.byref(sh), 0, C.byref(out)) == L.VC_ERR_INVALID_ARG
    assert L.lib.vc_tokdrop_select(C.byref(sh), 0x10000, 100, 101, 0x10000, None, 0, None) == L.VC_ERR_INVALID_ARG


def test_time_next_call_scope():
    """The timing hook validates its scope without touching a GPU."""
    from lossless_speculative_kv_amd import _lib as L
    L.vc_time_next_call(None, None, L.VC_TIME_CALL)
    L.vc_time_next_call(None, None, L.VC_TIME_MAIN_KERNEL)
    with pytest.raises(L.VCError) as e:
        L.vc_time_next_call(None, None, 7)
    assert e.value.status == L.VC_ERR_INVALID_ARG


def test_kivi_block_bytes():
    assert L.vc_kivi_block_bytes(128, 2) == 3072
    assert L.vc_kivi_block_bytes(64, 4) == 2560
    out = C.c_size_t()
    assert L.lib.vc_kivi_block_bytes(96, 2, C.byref(out)) == L.VC_ERR_UNSUPPORTED
    assert L.lib.vc_kivi_block_bytes(128, 3, C.byref(out)) == L.VC_ERR_UNSUPPORTED
    assert L.lib.vc_kivi_block_bytes(128, 2, None) == L.VC_ERR_INVALID_ARG


def test_noalloc_rejects_oversized_calls():
    """The allocation-free draft call rejects, on the host, a call whose split
    partials exceed its fixed scratch (255 sequences x 4080 query heads at
    head_dim 128 need far more than 8 MiB), and checks its arguments like the
    workspace call."""
    sh = L.vc_attn_shape(255, 4080, 255, 128)
    rc = L.lib.vc_draft_decode_attn_noalloc(C.byref(sh), 0x10000, C.byref(kivi_kv()), 0x10000, None)
    assert rc == L.VC_ERR_WORKSPACE
    assert "partials" in L.last_error()
    rc = L.lib.vc_draft_decode_attn_noalloc(C.byref(shape()), None, C.byref(kivi_kv()), 0x10000, None)
    assert rc == L.VC_ERR_INVALID_ARG
    rc = L.lib.vc_draft_decode_attn_noalloc(C.byref(shape()), 0x10000, C.byref(kivi_kv(bits=3)), 0x10000, None)
    assert rc == L.VC_ERR_UNSUPPORTED
