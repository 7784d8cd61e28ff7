"""vc_time_next_call on the GPU: the events a timed call records must fall
inside a pair of host-recorded markers around that call, in the order start,
stop, for every call that takes part and both scopes (a call that left an
event unrecorded keeps the timestamp of its creation, which precedes the
first marker)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from tests.gpu_util import bf16_tensor, ctx_rows, f16_dev, log, to_dev  # noqa: E402
from tests.test_gpu_kernels import build_kivi, draft_queries  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import _lib
    return _lib


def recorded_events(n, s):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record(s)
    torch.cuda.synchronize()
    return ev


def check_timed(L, fn, what):
    s = torch.cuda.current_stream()
    for scope in (L.VC_TIME_CALL, L.VC_TIME_MAIN_KERNEL):
        before, start, stop, after = recorded_events(4, s)
        before.record(s)
        L.vc_time_next_call(start.cuda_event, stop.cuda_event, scope)
        fn()
        after.record(s)
        torch.cuda.synchronize()
        lead = before.elapsed_time(start) * 1e3
        span = start.elapsed_time(stop) * 1e3
        trail = stop.elapsed_time(after) * 1e3
        log(f"  {what} scope {scope}: lead {lead:.1f} us, span {span:.1f} us, trail {trail:.1f} us")
        assert lead >= 0 and span > 0 and trail >= 0, (what, scope, lead, span, trail)
    # the setting is consumed: an untimed call afterwards leaves the events alone
    before, start, stop = recorded_events(3, s)
    t0 = before.elapsed_time(stop)
    fn()
    torch.cuda.synchronize()
    assert before.elapsed_time(stop) == t0


@pytest.mark.parametrize("M,K,V", [(4, 512, 4096), (72, 1024, 6000)], ids=["stream", "staged"])
def test_vocab_call_records_events(L, M, K, V):
    log(f"timing vocab M={M} K={K} V={V}")
    rng = np.random.default_rng(M)
    dh = to_dev((rng.standard_normal((M, K)) * 0.05).astype(np.float32))
    dW = bf16_tensor(synth.w_vocab_rows(M, 0, V, K))
    am = torch.empty((M,), dtype=torch.int32, device="cuda")
    ws = torch.empty(L.vc_vocab_workspace_bytes(M, K, V), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    check_timed(L, lambda: L.vc_vocab_logits(M, K, V, dh.data_ptr(), dW.data_ptr(), am.data_ptr(), None, None,
                                             ws.data_ptr(), ws.numel(), s), "vocab")


def test_draft_call_records_events(L):
    B, Hq, Hkv, D, bits, body, tail = 2, 32, 8, 128, 2, [2048, 1024], [130, 129]
    log("timing draft kivi")
    arr, _, body_cap, tail_cap = build_kivi(B, Hq, Hkv, D, bits, body, tail, 7)
    dev = {k: (f16_dev(v) if v.dtype == np.float16 else to_dev(v)) for k, v in arr.items()}
    bl, tl = to_dev(np.array(body, np.int32)), to_dev(np.array(tail, np.int32))
    sh = L.vc_attn_shape(B, Hq, Hkv, D)
    kv = L.vc_draft_kv()
    kv.kind, kv.bits, kv.body_cap, kv.tail_cap = L.VC_DRAFT_KIVI, bits, body_cap, tail_cap
    kv.body_len, kv.tail_len = bl.data_ptr(), tl.data_ptr()
    for f in ("kivi_blocks", "tail_k", "tail_v"):
        setattr(kv, f, dev[f].data_ptr())
    q = bf16_tensor(draft_queries(7, B, Hq, D))
    ws = torch.empty(L.vc_draft_workspace_bytes(sh, kv), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    check_timed(L, lambda: L.vc_draft_decode_attn(sh, q.data_ptr(), kv, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                                  s), "draft")


def test_verify_call_records_events(L):
    B, Hq, Hkv, D, NR, T = 2, 32, 8, 128, 33, 1500
    log("timing verify")
    t_cap = (T + 31) // 32 * 32
    K, V = ctx_rows(9, B, Hkv, T, D)
    fk = np.zeros((B, Hkv, t_cap, D), np.float32)
    fv = np.zeros_like(fk)
    fk[:, :, :T], fv[:, :, :T] = K, V
    toks = (np.arange(NR * B).reshape(NR, B) * 37 + 5) % 4096
    q, kn, vn = synth.embed(9, toks, Hq, Hkv, D)
    sh = L.vc_attn_shape(B, Hq, Hkv, D)
    dq, dkn, dvn, dk, dv = (bf16_tensor(x) for x in (q, kn, vn, fk, fv))
    cl = to_dev(np.array([T, T - 300], np.int32))
    ws = torch.empty(L.vc_verify_workspace_bytes(sh, NR, t_cap), dtype=torch.uint8, device="cuda")
    out = torch.empty((NR, B, Hq, D), dtype=torch.float32, device="cuda")
    ctxd = L.vc_kv_chunk(dk.data_ptr(), dv.data_ptr(), t_cap, 0, t_cap)
    s = torch.cuda.current_stream().cuda_stream
    check_timed(L, lambda: L.vc_verify_attn(sh, NR, dq.data_ptr(), dkn.data_ptr(), dvn.data_ptr(), ctxd,
                                            cl.data_ptr(), L.VC_VERIFY_BEGIN | L.VC_VERIFY_END, out.data_ptr(),
                                            ws.data_ptr(), ws.numel(), s), "verify")
