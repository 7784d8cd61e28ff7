"""A whole VeriCache round captured in a HIP graph (Engine.capture_round):
replayed round after round, with eager work and synchronisations between the
replays, every replay's results equal, bit for bit, those of the same round
run eagerly on a second engine (the eager rounds are the ones the
teacher-forced round tests check against the oracle): drafted and verified
tokens, accept lengths, committed tokens, cache lengths, verification
outputs, and the caches themselves. Covers a KIVI cache whose residual
flushes during the replays, token drop and the identity compressor."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.gpu_util import log  # noqa: E402

pytestmark = pytest.mark.gpu

# (config, rounds): kivi4 runs enough rounds for its tail (R = 32, one or more
# committed tokens per round) to reach R + 32 and flush during the replays
GRAPH_CASES = {
    "kivi4": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, context=256, vocab=1024, k=6, kind="kivi",
                  bits=4, residual=32, seed=31),
    "kivi2": dict(batch=3, n_q_heads=16, n_kv_heads=4, head_dim=128, context=512, vocab=2048, k=12, kind="kivi",
                  bits=2, residual=32, outliers=True, seed=32),
    "tokdrop": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, context=1024, vocab=1024, k=5,
                    kind="tokdrop", keep=0.25, seed=33),
    "dense": dict(batch=2, n_q_heads=8, n_kv_heads=4, head_dim=64, context=300, vocab=512, k=7, kind="dense",
                  seed=34),
}


def snapshot(eng, slot):
    t = {"xs": eng.xs, "y": eng.y, "n_accept": eng.n_accept[slot], "committed": eng.committed[slot],
         "ctx": eng.ctx_len, "body": eng.body_len, "tail": eng.tail_len, "o_ver": eng.o_ver,
         "tail_k": eng.tail_k, "status": eng.status}
    if eng.cfg.kind == "kivi":
        t["blocks"] = eng.kivi_blocks
    # bf16 tensors are compared as their 16-bit patterns
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy().copy() for k, v in t.items()}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_round_replays_match_eager_rounds(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import configs, engine
    cfg = configs.RoundConfig(name=f"graph-{name}", **GRAPH_CASES[name])
    rounds = 34 if name == "kivi4" else 6
    log(f"graph round {name}: eager reference, {rounds} rounds")
    ref = engine.Engine(cfg, rounds_cap=rounds)
    want = []
    for r in range(rounds):
        ref.round()
        torch.cuda.synchronize()
        want.append(snapshot(ref, r))
    log(f"graph round {name}: capture and {rounds} replays")
    eng = engine.Engine(cfg, rounds_cap=rounds)
    g = eng.capture_round()
    slot = eng.graph_slot
    body0 = int(eng.body_len.sum())
    for r in range(rounds):
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(eng, slot)
        for key, w in want[r].items():
            assert np.array_equal(got[key], w), f"{name}: replay {r}: {key} differs from the eager round"
        # eager work and a synchronisation between replays
        junk = torch.arange(4096, device="cuda", dtype=torch.float32)
        assert float(junk.sum().item()) == 4096 * 4095 / 2
        log(f"  replay {r}: accept lengths {got['n_accept'].tolist()}, context {got['ctx'].tolist()}")
    if cfg.kind == "kivi":
        grew = int(eng.body_len.sum()) - body0
        log(f"  body grew by {grew} tokens over the replays")
        if name == "kivi4":
            assert grew >= 32 * cfg.batch, "the residual flush did not run during the replays"
