"""vc_draft_decode_attn_noalloc (the allocation-free draft call, for callers
that cannot allocate) against vc_draft_decode_attn with a caller workspace,
through the C ABI: several calls in a row on the library's own scratch
array, the second with a smaller input and a later one larger again, each
bit for bit equal to the existing entry point (same kernels and split plan)
and within the attention tolerance of the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.gpu_util import assert_attention_close, bf16_tensor, f16_dev, log, to_dev  # noqa: E402
from tests.test_gpu_kernels import build_kivi, draft_queries  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import _lib
    return _lib


# B, Hq, Hkv, D, bits, body lens, tail lens
CALLS = [
    (2, 32, 8, 128, 2, [2048, 1024], [130, 129]),   # Llama-3-8B layer shape, short context
    (1, 8, 2, 64, 4, [512], [40]),                   # smaller: fewer units, other kernel
    (4, 40, 8, 128, 2, [1024, 2048, 512, 1536], [128, 3, 77, 129]),  # larger again (more counters)
]


def test_noalloc_matches_workspace_entry_point(L):
    s = torch.cuda.current_stream().cuda_stream
    for i, (B, Hq, Hkv, D, bits, body, tail) in enumerate(CALLS):
        log(f"no-alloc draft call {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} bits={bits} body={body} tail={tail}")
        seed = 950 + i
        arr, vis, body_cap, tail_cap = build_kivi(B, Hq, Hkv, D, bits, body, tail, seed)
        dev = {k: (f16_dev(v) if v.dtype == np.float16 else to_dev(v)) for k, v in arr.items()}
        bl, tl = to_dev(np.array(body, np.int32)), to_dev(np.array(tail, np.int32))
        sh = L.vc_attn_shape(B, Hq, Hkv, D)
        kv = L.vc_draft_kv()
        kv.kind, kv.bits, kv.body_cap, kv.tail_cap = L.VC_DRAFT_KIVI, bits, body_cap, tail_cap
        kv.body_len, kv.tail_len = bl.data_ptr(), tl.data_ptr()
        for f in ("kivi_blocks", "tail_k", "tail_v"):
            setattr(kv, f, dev[f].data_ptr())
        q = draft_queries(seed, B, Hq, D)
        dq = bf16_tensor(q)
        ws = torch.zeros(L.vc_draft_workspace_bytes(sh, kv), dtype=torch.uint8, device="cuda")
        ref = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        L.vc_draft_decode_attn(sh, dq.data_ptr(), kv, ref.data_ptr(), ws.data_ptr(), ws.numel(), s)
        got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        L.vc_draft_decode_attn_noalloc(sh, dq.data_ptr(), kv, got.data_ptr(), s)
        got2 = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        L.vc_draft_decode_attn_noalloc(sh, dq.data_ptr(), kv, got2.data_ptr(), s)
        torch.cuda.synchronize()
        ref, got, got2 = ref.cpu().numpy(), got.cpu().numpy(), got2.cpu().numpy()
        assert np.array_equal(got, ref), f"call {i}: differs from the workspace entry point"
        assert np.array_equal(got2, ref), f"call {i} (repeated): differs from the workspace entry point"
        g = Hq // Hkv
        want = np.stack([np.stack([oracle.attend(q[b, h], *vis[b, h // g]) for h in range(Hq)]) for b in range(B)])
        mad, rl2 = assert_attention_close(got, want, f"no-alloc call {i}")
        log(f"  bit-identical to the workspace call; vs oracle max|d| {mad:.2e} rel-L2 {rl2:.2e}")
