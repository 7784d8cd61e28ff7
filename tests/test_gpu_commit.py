"""vc_commit_round on a KIVI cache with planted accept lengths, so that the
residual flush really runs: sequences whose tail crosses R + 32 (one and two
32-token blocks), one that stays below it, and one that would overflow the
full cache (left unchanged, flagged). Checked against the oracle:

* the new body records, byte for byte, against the oracle quantiser applied
  to the oldest 32 rows of the tail as it stood after the accepted rows were
  written (the fp16 values the GPU quantises);
* the records before and after them untouched;
* the tail after the flush (the remaining rows moved to the front, in order);
* the full cache rows appended, and the context, body and tail lengths.

VeriCache summary, "Core algorithm": decoding restarts from the last
accepted token; the KIVI residual keeps the most recent tokens unquantised
and the oldest ones join the quantised body."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.gpu_util import bf16_tensor, f16_dev, log, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import _lib
    return _lib


def bf16_values(rng, shape, scale=1.0):
    """bf16 values kept away from zero (|x| >= 2^-10), so that their fp16 copies
    in the tail are exact."""
    x = rng.standard_normal(shape) * scale
    x = np.where(np.abs(x) < 2.0 ** -10, np.copysign(2.0 ** -10, x), x).astype(np.float32)
    return oracle.to_bf16(x).astype(np.float32)


# D, bits, residual, k, per sequence: (body_len, tail_start, n_accept, ctx_len)
COMMIT_CASES = [
    (128, 2, 32, 8, [(64, 56, 8, 700),     # new tail 65 >= 64: one block, 33 rows kept (shift in two chunks)
                     (32, 32, 0, 300),     # new tail 33: no flush
                     (0, 90, 8, 512),      # new tail 99: two blocks from an empty body
                     (96, 40, 8, 1020)]),  # would overflow the full cache (cap 1024): unchanged, flagged
    (64, 4, 64, 20, [(32, 80, 20, 128),    # new tail 101 >= 96: one block, 69 kept
                     (0, 64, 0, 64)]),     # new tail 65: no flush
]


@pytest.mark.parametrize("case", COMMIT_CASES, ids=[f"commit{i}" for i in range(len(COMMIT_CASES))])
def test_commit_flush_parity(L, case):
    D, bits, R, k, seqs = case
    B, Hkv, Hq = len(seqs), 2, 4
    log(f"commit flush D={D} bits={bits} R={R} k={k} seqs={seqs}")
    rng = np.random.default_rng(700 + D + bits)
    full_cap = 1024
    body_cap, tail_cap = 256, 192
    nbc = body_cap // 32
    rec = L.vc_kivi_block_bytes(D, bits)
    # caches before the commit
    blocks = rng.integers(0, 256, size=(B, Hkv, nbc, rec), dtype=np.uint8)   # sentinel bytes
    tail_k = np.zeros((B, Hkv, tail_cap, D), np.float16)
    tail_v = np.zeros_like(tail_k)
    full_k = np.zeros((B, Hkv, full_cap, D), np.float32)
    full_v = np.zeros_like(full_k)
    for b, (nb, ts, m, ctx) in enumerate(seqs):
        # the tail holds its round-start rows plus the k drafted inputs
        tail_k[b, :, :ts + k] = rng.standard_normal((Hkv, ts + k, D)).astype(np.float16)
        tail_v[b, :, :ts + k] = rng.standard_normal((Hkv, ts + k, D)).astype(np.float16)
        full_k[b, :, :ctx] = bf16_values(rng, (Hkv, ctx, D))
        full_v[b, :, :ctx] = bf16_values(rng, (Hkv, ctx, D))
    k_new = bf16_values(rng, (k + 1, B, Hkv, D), 2.0)
    v_new = bf16_values(rng, (k + 1, B, Hkv, D))
    n_accept = np.array([s[2] for s in seqs], np.int32)

    d_blocks = to_dev(blocks)
    d_tk, d_tv = f16_dev(tail_k), f16_dev(tail_v)
    d_fk, d_fv = bf16_tensor(full_k), bf16_tensor(full_v)
    d_kn, d_vn = bf16_tensor(k_new), bf16_tensor(v_new)
    body_len = to_dev(np.array([s[0] for s in seqs], np.int32))
    tail_len = to_dev(np.array([s[1] + k for s in seqs], np.int32))
    ctx_len = to_dev(np.array([s[3] for s in seqs], np.int32))
    d_na = to_dev(n_accept)
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    sh = L.vc_attn_shape(B, Hq, Hkv, D)
    dc = L.vc_draft_cache()
    dc.kind, dc.bits, dc.body_cap, dc.tail_cap, dc.residual = L.VC_DRAFT_KIVI, bits, body_cap, tail_cap, R
    dc.body_len, dc.tail_len = body_len.data_ptr(), tail_len.data_ptr()
    dc.kivi_blocks, dc.tail_k, dc.tail_v = d_blocks.data_ptr(), d_tk.data_ptr(), d_tv.data_ptr()
    ws = torch.empty(L.vc_commit_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    L.vc_commit_round(sh, k, d_na.data_ptr(), d_kn.data_ptr(), d_vn.data_ptr(), d_fk.data_ptr(), d_fv.data_ptr(),
                      full_cap, ctx_len.data_ptr(), dc, status.data_ptr(), ws.data_ptr(), ws.numel(),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g_blocks = d_blocks.cpu().numpy()
    g_tk, g_tv = d_tk.cpu().numpy(), d_tv.cpu().numpy()
    g_fk, g_fv = d_fk.float().cpu().numpy(), d_fv.float().cpu().numpy()
    g_body, g_tail, g_ctx = body_len.cpu().numpy(), tail_len.cpu().numpy(), ctx_len.cpu().numpy()
    g_status = status.cpu().numpy()
    flushed = 0
    for b, (nb, ts, m, ctx) in enumerate(seqs):
        if ctx + m + 1 > full_cap:
            assert g_status[b] != 0, f"seq {b}: overflow not flagged"
            assert (g_body[b], g_tail[b], g_ctx[b]) == (nb, ts + k, ctx), f"seq {b}: lengths changed"
            assert np.array_equal(g_blocks[b], blocks[b]) and np.array_equal(g_tk[b], tail_k[b])
            assert np.array_equal(g_fk[b], full_k[b])
            continue
        assert g_status[b] == 0, f"seq {b}: status {g_status[b]}"
        # the tail as the oracle's commit builds it: round-start rows, then x_0..x_m
        pre_k = np.concatenate([tail_k[b, :, :ts].astype(np.float64),
                                k_new[:m + 1, b].transpose(1, 0, 2).astype(np.float64)], axis=1)
        pre_v = np.concatenate([tail_v[b, :, :ts].astype(np.float64),
                                v_new[:m + 1, b].transpose(1, 0, 2).astype(np.float64)], axis=1)
        new_tail = ts + m + 1
        nf = (new_tail - R) // 32 if new_tail >= R + 32 else 0
        flushed += nf
        log(f"  seq {b}: tail {ts}+{m + 1} -> flush {nf} block(s), keep {new_tail - 32 * nf}")
        assert g_body[b] == nb + 32 * nf and g_tail[b] == new_tail - 32 * nf and g_ctx[b] == ctx + m + 1
        for h in range(Hkv):
            if nf:
                kc, ks, kz = oracle.quantize_keys(pre_k[h, :32 * nf], bits)
                vc, vs, vz = oracle.quantize_values(pre_v[h, :32 * nf], bits)
                want = oracle.pack_blocks(kc, ks, kz, vc, vs, vz, bits)
                got = g_blocks[b, h, nb // 32:nb // 32 + nf]
                assert np.array_equal(got, want), f"seq {b} head {h}: flushed records"
            assert np.array_equal(g_blocks[b, h, :nb // 32], blocks[b, h, :nb // 32]), "older records changed"
            assert np.array_equal(g_blocks[b, h, nb // 32 + nf:], blocks[b, h, nb // 32 + nf:]), "records past"
            keep = new_tail - 32 * nf
            assert np.array_equal(g_tk[b, h, :keep].astype(np.float64), pre_k[h, 32 * nf:new_tail])
            assert np.array_equal(g_tv[b, h, :keep].astype(np.float64), pre_v[h, 32 * nf:new_tail])
            assert np.array_equal(g_fk[b, h, ctx:ctx + m + 1], k_new[:m + 1, b, h])
            assert np.array_equal(g_fv[b, h, ctx:ctx + m + 1], v_new[:m + 1, b, h])
            assert np.array_equal(g_fk[b, h, :ctx], full_k[b, h, :ctx])
    assert flushed >= 1
