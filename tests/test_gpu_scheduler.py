"""The P1 scheduler (two request groups, host-resident full caches, each on
its own compute and copy streams, drafting staggered across the groups)
gives every group exactly the results of running that group alone on one
stream: drafted and verified tokens, accept lengths, committed tokens, cache
lengths and verification outputs, bit for bit. The interleaving changes only
when work runs, never what it computes (the eager rounds are the ones the
teacher-forced round tests check against the oracle)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.gpu_util import log  # noqa: E402

pytestmark = pytest.mark.gpu


def snap(e, rounds):
    return {"xs": e.xs.cpu().numpy().copy(), "n_accept": e.n_accept[:rounds].cpu().numpy().copy(),
            "committed": e.committed[:rounds].cpu().numpy().copy(), "ctx": e.ctx_len.cpu().numpy().copy(),
            "body": e.body_len.cpu().numpy().copy(), "tail": e.tail_len.cpu().numpy().copy(),
            "o_ver": e.o_ver.cpu().numpy().copy()}


def test_staggered_groups_match_groups_run_alone():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import configs, engine
    from lossless_speculative_kv_amd.scheduler import StaggeredGroups
    cfg = configs.RoundConfig("p1-small", batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128, context=2048,
                              vocab=1024, k=6, kind="kivi", bits=2, residual=128, staged=True, chunk=512,
                              stage_buffers=1, seed=41)
    rounds = 3
    log("p1 scheduler: two staggered groups")
    sched = StaggeredGroups(cfg, 2, rounds_cap=rounds)
    stats = sched.run(rounds, trace=True)
    log(f"  {stats.as_dict()}")
    got = [snap(e, rounds) for e in sched.groups]
    assert stats.committed_tokens == sum(int(g["n_accept"].sum()) + rounds * cfg.batch for g in got)
    assert stats.link_busy_s > 0 and stats.draft_busy_s > 0
    for g in range(2):
        log(f"p1 scheduler: group {g} alone")
        alone = engine.Engine(cfg.scaled(name=f"{cfg.name}-g{g}", seed=cfg.seed + 1000 * g), rounds_cap=rounds)
        for _ in range(rounds):
            alone.round()
        torch.cuda.synchronize()
        want = snap(alone, rounds)
        for key, w in want.items():
            assert np.array_equal(got[g][key], w), f"group {g}: {key} differs from the group run alone"
        del alone
