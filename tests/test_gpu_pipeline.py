"""Pipelined drafting during verification (Engine with pipeline = J): while a
staged verification waits for the host-resident full cache, the drafter
continues from x_k on a side stream; the continued drafts are reused as the
next round's first drafts when every draft was accepted and the bonus token
equals the first continued draft, and discarded otherwise.

Checked on a host-resident configuration whose drafter is nearly exact (the
whole context is the unquantised residual window, so almost every draft is
accepted and reuse happens): the committed stream equals full-cache greedy
decoding (the oracle), drafts were reused, and the cache lengths follow the
committed tokens; and on a lossy KIVI-2 drafter (discards) the stream also
equals full-cache greedy decoding."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.model import ModelConfig, SynthModel, full_kv_greedy  # noqa: E402
from tests.gpu_util import log  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "exact-drafter": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, context=1024, vocab=512, k=6,
                          kind="kivi", bits=4, residual=1024, staged=True, chunk=256, stage_buffers=2, pipeline=7,
                          seed=51),
    "kivi2": dict(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128, context=2048, vocab=1024, k=6, kind="kivi",
                  bits=2, residual=128, staged=True, chunk=512, pipeline=4, seed=52),
}


@pytest.mark.parametrize("name", list(CASES))
def test_pipelined_drafting_is_lossless(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import configs, engine
    cfg = configs.RoundConfig(name=f"pipe-{name}", **CASES[name])
    rounds = 8
    eng = engine.Engine(cfg, rounds_cap=rounds)
    streams = [[] for _ in range(cfg.batch)]
    for r in range(rounds):
        eng.round()
        torch.cuda.synchronize()
        cm = eng.committed[r].cpu().numpy()
        for b in range(cfg.batch):
            streams[b] += [int(t) for t in cm[:, b] if t >= 0]
        log(f"  {name} round {r}: accept {eng.n_accept[r].cpu().tolist()}, reuse next {eng.reuse}")
    assert (eng.status.cpu().numpy() == 0).all()
    ocfg = ModelConfig(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                       context=cfg.context, vocab=cfg.vocab, k=cfg.k, kind=cfg.kind, bits=cfg.bits,
                       residual=cfg.residual, seed=cfg.seed)
    model = SynthModel(ocfg)
    for b in range(cfg.batch):
        assert streams[b] == full_kv_greedy(ocfg, b, len(streams[b]), model), f"{name}: stream of sequence {b}"
    ctx = eng.ctx_len.cpu().numpy()
    assert all(ctx[b] == cfg.context + len(streams[b]) for b in range(cfg.batch))
    log(f"  {name}: {eng.reused_drafts} drafts reused over {rounds} rounds")
    if name == "exact-drafter":
        assert eng.reused_drafts > 0, "no continued draft was ever reused"
