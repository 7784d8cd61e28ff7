"""Draft parity at full size for the other layer shapes, driven through the
bench's engine, split plans and kernels (one draft step each), with sampled
outputs computed one by one by the oracle:

* Mistral-24B layer (B = 4, 32 q / 8 KV heads, context 131072, token drop
  keeping 25%): the kept positions of sampled KV heads bit for bit against the
  oracle dropper on the GPU's own scores, then draft attention of their query
  heads over the gathered rows and the bf16 tail;
* Qwen-32B layer (B = 16, 40 q / 8 KV heads, context 65536, KIVI-2, g = 5):
  body records byte for byte against the oracle quantiser on the GPU's own
  full-cache rows, then draft attention over the dequantised body and fp16
  tail;
* Llama-70B layer with a 1M-token context (B = 1, 64 q / 8 KV heads, KIVI-2,
  g = 8, full cache in pinned host memory): the same for one KV head.

Each test then runs the layer's verification pass and checks every row of
two whole (sequence, KV head) units, plus sampled (sequence, head, draft row)
outputs, over the whole context plus the causal draft block: on the Mistral-24B layer (eleven row tiles) the wave pairs that
issue their own loads, on the Qwen-32B layer the wave pairs with producer
waves, on the 1M-token layer the chunked pass staged from host memory.

Tolerances as in the kernel tests: attention max |d| <= 1e-2 and rel-L2 <=
2e-3; kept positions and records bit-exact."""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.gpu_util import (FP16P_RL2, assert_attention_close, check_argmax_chunked, check_verify_unit,  # noqa: E402
                            log)

pytestmark = pytest.mark.gpu


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def build(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import configs, engine
    cfg = configs.BY_NAME[name]
    log(f"full size: building the {name} engine")
    e = engine.Engine(cfg, rounds_cap=1)
    e.begin_round()
    e.draft_step(0)
    torch.cuda.synchronize()
    return e


def release(e):
    del e
    gc.collect()
    torch.cuda.empty_cache()


def check_verify(eng, samples, units=()):
    """Verification pass of the round's block, then the oracle on every row of
    the whole (sequence, KV head) units given, and on sampled (sequence, KV
    head, draft rows): row j sees the context and block rows 0..j (query head
    hk * g + j mod g)."""
    c = eng.cfg
    g = c.n_q_heads // c.n_kv_heads
    eng.embed_block()
    eng.verify_attention()
    torch.cuda.synchronize()
    for b, hk in units:
        log(f"full size verify ({c.name}): whole unit (sequence {b}, KV head {hk}), {(c.k + 1) * g} rows")
        mad, rl2, worst = check_verify_unit(eng, b, hk)
        log(f"  max|d| {mad:.2e} rel-L2 {rl2:.2e} (worst row {worst:.2e})")
    ctx = eng.ctx_len.cpu().numpy()
    o = eng.o_ver.cpu().numpy()
    for b, hk, rows in samples:
        n = int(ctx[b])
        K = f64(eng.full_k[b, hk, :n])
        V = f64(eng.full_v[b, hk, :n])
        kn = f64(eng.kn[:, b, hk])
        vn = f64(eng.vn[:, b, hk])
        for j in rows:
            h = hk * g + (j % g)
            log(f"full size verify ({c.name}): sequence {b} head {h} row {j}, context {n}")
            ref = oracle.attend(f64(eng.qv[j, b, h]), np.concatenate([K, kn[:j + 1]]), np.concatenate([V, vn[:j + 1]]))
            mad, rl2 = assert_attention_close(o[j, b, h], ref, f"verify ({b}, {h}, row {j})", rl2_max=FP16P_RL2)
            log(f"  max|d| {mad:.2e} rel-L2 {rl2:.2e}")


def check_kivi_unit(eng, b, hk):
    c = eng.cfg
    g = c.n_q_heads // c.n_kv_heads
    nb = int(eng.body_len[b])
    nt = int(eng.tail_len[b])
    log(f"full size draft ({c.name}): sequence {b} KV head {hk}, body {nb}, tail {nt}")
    rec = eng.kivi_blocks[b, hk, :nb // 32].cpu().numpy()
    K = f64(eng.full_k[b, hk, :nb])
    V = f64(eng.full_v[b, hk, :nb])
    kc, ks, kz = oracle.quantize_keys(K, c.bits)
    vc, vs, vz = oracle.quantize_values(V, c.bits)
    assert np.array_equal(rec, oracle.pack_blocks(kc, ks, kz, vc, vs, vz, c.bits)), f"records of ({b}, {hk})"
    del K, V, rec
    Kv = np.concatenate([oracle.dequantize_keys(kc, ks, kz), f64(eng.tail_k[b, hk, :nt])])
    Vv = np.concatenate([oracle.dequantize_values(vc, vs, vz), f64(eng.tail_v[b, hk, :nt])])
    q = f64(eng.q_draft[b, hk * g:(hk + 1) * g])
    ref = np.stack([oracle.attend(q[i], Kv, Vv) for i in range(g)])
    got = eng.o_draft[b, hk * g:(hk + 1) * g].cpu().numpy()
    mad, rl2 = assert_attention_close(got, ref, f"draft unit ({b}, {hk})")
    log(f"  max|d| {mad:.2e} rel-L2 {rl2:.2e}")


def test_mistral_tokdrop_draft():
    eng = build("mistral-24b-layer")
    c = eng.cfg
    g = c.n_q_heads // c.n_kv_heads
    out = eng.o_draft.cpu().numpy()
    for b, hk in [(0, 0), (c.batch - 1, c.n_kv_heads - 1), (2, 3)]:
        kept = eng.kept[b, hk, :eng.n_keep].cpu().numpy()
        want = oracle.select_kept(eng.scores[b, hk].cpu().numpy(), c.keep)
        assert np.array_equal(kept, want), f"kept positions of ({b}, {hk})"
        nt = int(eng.tail_len[b])
        log(f"full size draft ({c.name}): sequence {b} KV head {hk}, kept {len(kept)}, tail {nt}")
        K = np.concatenate([f64(eng.full_k[b, hk])[kept], f64(eng.tail_k[b, hk, :nt])])
        V = np.concatenate([f64(eng.full_v[b, hk])[kept], f64(eng.tail_v[b, hk, :nt])])
        q = f64(eng.q_draft[b, hk * g:(hk + 1) * g])
        ref = np.stack([oracle.attend(q[i], K, V) for i in range(g)])
        mad, rl2 = assert_attention_close(out[b, hk * g:(hk + 1) * g], ref, f"draft unit ({b}, {hk})",
                                          rl2_max=FP16P_RL2)
        log(f"  max|d| {mad:.2e} rel-L2 {rl2:.2e}")
    check_verify(eng, [(1, 5, (0, 21, c.k))], units=[(0, 0), (c.batch - 1, c.n_kv_heads - 1)])
    release(eng)


def test_qwen_kivi_draft():
    eng = build("qwen-32b-layer")
    c = eng.cfg
    for b, hk in [(0, 0), (c.batch - 1, c.n_kv_heads - 1), (9, 4)]:
        check_kivi_unit(eng, b, hk)
    check_verify(eng, [(5, 2, (0, 12, c.k))], units=[(0, 0), (c.batch - 1, c.n_kv_heads - 1)])
    # the verification argmax over the 152064-entry vocabulary (M = 416 rows:
    # 512 whole ring slices, the last 82 in k parts summed by the fixup
    # kernel) on sampled rows
    eng.verify_vocab()
    torch.cuda.synchronize()
    M = (c.k + 1) * c.batch
    rows = [0, 1, 100, 207, 208, 333, M - 2, M - 1]
    h = oracle.to_bf16(eng.o_ver.reshape(M, -1)[rows].cpu().numpy())
    got = eng.y.reshape(-1)[rows].cpu().numpy()
    log(f"full size verify vocab ({c.name}): rows {rows} of {M} x {c.vocab} x {c.hidden}")
    excused = check_argmax_chunked(eng.W, h, got)
    log(f"  near-tie excused rows: {excused}/{len(rows)}")
    release(eng)


def test_llama70b_1m_kivi_draft():
    eng = build("llama-70b-layer-1m")
    c = eng.cfg
    check_kivi_unit(eng, 0, c.n_kv_heads - 1)
    # the draft step's argmax over the 128256-entry vocabulary at hidden 8192
    h = oracle.to_bf16(eng.o_draft.reshape(1, -1).cpu().numpy())
    log(f"full size vocab ({c.name}): 1 row x {c.vocab} x {c.hidden}")
    excused = check_argmax_chunked(eng.W, h, eng.xs[1].cpu().numpy())
    log(f"  near-tie excused rows: {excused}/1")
    check_verify(eng, [(0, 5, (0, c.k))], units=[(0, 3), (0, c.n_kv_heads - 1)])
    release(eng)
