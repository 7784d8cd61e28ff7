"""Method-level pins of the oracle: the invariants the pages fix.

* identity compressor (dense draft cache, i.e. "16-bit quantisation") and
  keep-all token dropping: draft and full paths agree, every round accepts
  all k drafts plus the bonus;
* drafts taken from full-cache greedy decoding are always accepted;
* lossless: the committed stream equals full-cache greedy decoding for every
  compressor (VeriCache summary, "Experimental results": identical output
  under greedy decoding);
* a planted wrong draft at position j gives accept length j.
"""
import numpy as np
import pytest

from oracle.model import ModelConfig, full_kv_greedy, make_states


def small_cfg(**kw):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, context=96, vocab=256, k=5,
                kind="kivi", bits=2, residual=32, keep=0.25, seed=11)
    base.update(kw)
    return ModelConfig(**base)


def run(cfg, rounds):
    model, states = make_states(cfg)
    res = [[st.run_round() for _ in range(rounds)] for st in states]
    return model, states, res


@pytest.mark.parametrize("kind,extra", [("dense", {}), ("tokdrop", {"keep": 1.0})])
def test_identity_compressor_accepts_everything(kind, extra):
    cfg = small_cfg(kind=kind, **extra)
    _, _, res = run(cfg, 3)
    for per_seq in res:
        for r in per_seq:
            assert r["m"] == cfg.k
            assert r["committed"][-1] == r["y"][-1]   # the bonus token


def test_drafts_from_full_cache_always_accepted():
    cfg = small_cfg(kind="kivi", bits=2, k=6)
    model, states = make_states(cfg)
    for b, st in enumerate(states):
        ref = full_kv_greedy(cfg, b, 3 * (cfg.k + 1), model)
        pos = 0
        for _ in range(3):
            r = st.run_round(forced_drafts=ref[pos:pos + cfg.k])
            assert r["m"] == cfg.k
            pos += cfg.k + 1


@pytest.mark.parametrize("kind,bits,keep,seed", [
    ("kivi", 2, 0.25, 1), ("kivi", 4, 0.25, 2), ("tokdrop", 2, 0.25, 3), ("tokdrop", 2, 0.5, 4),
    ("dense", 2, 0.25, 5)])
def test_lossless_stream_equals_full_cache_greedy(kind, bits, keep, seed):
    cfg = small_cfg(kind=kind, bits=bits, keep=keep, seed=seed, k=7, residual=32)
    model, states, res = run(cfg, 6)
    for b in range(cfg.batch):
        stream = [int(t) for r in res[b] for t in r["committed"] if t >= 0]
        assert stream == full_kv_greedy(cfg, b, len(stream), model)


def test_kivi_flush_moves_tail_into_body():
    cfg = small_cfg(kind="kivi", k=40, residual=32, batch=1)
    model, states = make_states(cfg)
    st = states[0]
    assert st.body_len() == 64 and st.tail_k.shape[1] == 32
    r = st.run_round()
    n_tail = 32 + r["m"] + 1
    flushed = 32 * ((n_tail - 32) // 32)
    assert st.body_len() == 64 + flushed
    assert st.tail_k.shape[1] == n_tail - flushed
    assert st.tail_k.shape[1] < 32 + 32


@pytest.mark.parametrize("j", [0, 2, 4])
def test_planted_wrong_draft_gives_accept_length_j(j):
    cfg = small_cfg(kind="dense", batch=1, k=5)
    model, states = make_states(cfg)
    ref = full_kv_greedy(cfg, 0, cfg.k, model)
    forced = list(ref)
    forced[j] = (forced[j] + 1) % cfg.vocab
    r = states[0].run_round(forced_drafts=forced)
    assert r["m"] == j
    assert r["committed"][j] == ref[j]      # the correction is the full-cache token
    assert states[0].x0 == ref[j]
