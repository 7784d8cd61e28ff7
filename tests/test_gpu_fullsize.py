"""Parity at full size, in the launch configuration bench.py times: the
Llama-3-8B layer (B = 8, 32 q / 8 KV heads, D = 128, context 32768, KIVI-2,
k = 32, vocab 128256 x 4096) driven through the same engine, split plans and
kernels. The oracle computes sampled outputs one by one:

* the KIVI body records of sampled KV heads, byte for byte, against the
  oracle quantiser applied to the GPU's own full-cache rows;
* draft attention of every query head of those KV heads against fp64
  attention over the dequantised body and the fp16 tail;
* verification attention of every row of two whole (sequence, KV head)
  units, and sampled rows of a third, over the full context plus the causal
  draft block;
* the draft-step argmax of every sequence against fp64 logits (exact except
  within the near-tie bound).
Tolerances as in the kernel tests: attention max |d| <= 1e-2 and rel-L2 <=
2e-3; records and argmax bit-exact."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.gpu_util import (FP16P_RL2, assert_attention_close, check_argmax_chunked, check_verify_unit,  # noqa: E402
                            log)

pytestmark = pytest.mark.gpu

UNITS = [(0, 0), (3, 5), (7, 7)]  # (sequence, KV head)


@pytest.fixture(scope="module")
def eng():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import configs, engine
    cfg = configs.BY_NAME["llama3-8b-layer"]
    log("full size: building the Llama-3-8B layer engine")
    e = engine.Engine(cfg, rounds_cap=1)
    e.begin_round()
    e.draft_step(0)
    torch.cuda.synchronize()
    return e


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_records_and_draft_attention(eng):
    c = eng.cfg
    D, g = c.head_dim, c.n_q_heads // c.n_kv_heads
    body = eng.body_len.cpu().numpy()
    tail = eng.tail_len.cpu().numpy()
    out = eng.o_draft.cpu().numpy()
    for b, hk in UNITS:
        log(f"full size draft: sequence {b} KV head {hk}, body {body[b]}, tail {tail[b]}")
        nb = int(body[b])
        rec = eng.kivi_blocks[b, hk, :nb // 32].cpu().numpy()
        K = bf16_to_f64(eng.full_k[b, hk, :nb])
        V = bf16_to_f64(eng.full_v[b, hk, :nb])
        kc, ks, kz = oracle.quantize_keys(K, c.bits)
        vc, vs, vz = oracle.quantize_values(V, c.bits)
        want = oracle.pack_blocks(kc, ks, kz, vc, vs, vz, c.bits)
        assert np.array_equal(rec, want), f"records of unit ({b}, {hk})"
        Kv = np.concatenate([oracle.dequantize_keys(kc, ks, kz),
                             eng.tail_k[b, hk, :tail[b]].float().cpu().numpy().astype(np.float64)])
        Vv = np.concatenate([oracle.dequantize_values(vc, vs, vz),
                             eng.tail_v[b, hk, :tail[b]].float().cpu().numpy().astype(np.float64)])
        q = bf16_to_f64(eng.q_draft[b, hk * g:(hk + 1) * g])
        ref = np.stack([oracle.attend(q[i], Kv, Vv) for i in range(g)])
        mad, rl2 = assert_attention_close(out[b, hk * g:(hk + 1) * g], ref, f"draft unit ({b}, {hk})")
        log(f"  max|d| {mad:.2e} rel-L2 {rl2:.2e}")


def test_verify_attention(eng):
    """Every verification row of two whole KV-head units, then sampled rows of
    a third."""
    c = eng.cfg
    eng.embed_block()
    eng.verify_attention()
    torch.cuda.synchronize()
    for b, hk in UNITS[:2]:
        log(f"full size verify: whole unit (sequence {b}, KV head {hk}), {(c.k + 1) * (c.n_q_heads // c.n_kv_heads)} rows")
        mad, rl2, worst = check_verify_unit(eng, b, hk)
        log(f"  max|d| {mad:.2e} rel-L2 {rl2:.2e} (worst row {worst:.2e})")
    g = c.n_q_heads // c.n_kv_heads
    ctx = eng.ctx_len.cpu().numpy()
    o = eng.o_ver.cpu().numpy()
    b, hk = UNITS[2]
    n = int(ctx[b])
    K = bf16_to_f64(eng.full_k[b, hk, :n])
    V = bf16_to_f64(eng.full_v[b, hk, :n])
    kn = bf16_to_f64(eng.kn[:, b, hk])
    vn = bf16_to_f64(eng.vn[:, b, hk])
    for j in (0, 17, c.k):
        h = hk * g + (j % g)
        log(f"full size verify: sequence {b} head {h} row {j}, context {n}")
        Ka, Va = np.concatenate([K, kn[:j + 1]]), np.concatenate([V, vn[:j + 1]])
        ref = oracle.attend(bf16_to_f64(eng.qv[j, b, h]), Ka, Va)
        assert_attention_close(o[j, b, h], ref, f"verify ({b}, {h}, row {j})", rl2_max=FP16P_RL2)


def test_draft_vocab_argmax(eng):
    c = eng.cfg
    h = oracle.to_bf16(eng.o_draft.reshape(c.batch, -1).cpu().numpy())
    got = eng.xs[1].cpu().numpy()
    log(f"full size vocab: {c.batch} rows x {c.vocab} x {c.hidden}")
    excused = check_argmax_chunked(eng.W, h, got)
    log(f"  near-tie excused rows: {excused}/{c.batch}")
