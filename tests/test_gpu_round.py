"""Teacher-forced round parity: the GPU engine runs whole VeriCache rounds; the
oracle replays every step on the GPU's token history and checks

* each draft-step and verify attention output (tolerance of the fp64 oracle),
* each drafted / verified token: the argmax of the oracle's fp64 logits on the
  GPU's own bf16 hidden vector, bit-exact unless within the near-tie bound,
* accept length, committed tokens and next token (bit-exact),
* the cache lengths after commit (context, tail, body),
* the identity compressor (dense) and the staged (host-resident) full cache,
* the committed stream against full-cache greedy decoding.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from oracle.model import ModelConfig, SequenceState, SynthModel, full_kv_greedy  # noqa: E402
from tests.gpu_util import assert_attention_close, log  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eng_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_speculative_kv_amd import configs, engine
    return configs, engine


def oracle_cfg(c):
    return ModelConfig(batch=c.batch, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                       context=c.context, vocab=c.vocab, k=c.k, kind=c.kind, bits=c.bits, residual=c.residual,
                       keep=c.keep, outliers=c.outliers, seed=c.seed)


def check_token(model, o_gpu_row, tok_gpu, what):
    """Oracle argmax on the GPU's own hidden vector; returns 1 if excused."""
    hid = oracle.to_bf16(np.asarray(o_gpu_row, np.float32).reshape(1, -1))
    lg = oracle.logits(hid, model.W)[0]
    want = int(oracle.argmax_first(lg))
    if want == tok_gpu:
        return 0
    gap = lg[want] - lg[tok_gpu]
    bound = oracle.tie_bound(hid, model.W, [want])[0]
    assert gap <= bound, f"{what}: GPU token {tok_gpu} vs oracle {want}, gap {gap:.3e} > {bound:.3e}"
    return 1


def run_case(configs, engine, cfg, rounds):
    eng = engine.Engine(cfg, rounds_cap=rounds)
    ocfg = oracle_cfg(cfg)
    model = SynthModel(ocfg)
    states = [SequenceState(model, b, int(eng.xs[0, b].item())) for b in range(cfg.batch)]
    k, B = cfg.k, cfg.batch
    excused = 0
    streams = [[] for _ in range(B)]
    for r in range(rounds):
        log(f"{cfg.name} round {r}")
        tail_start = [st.tail_k.shape[1] for st in states]
        for j in range(k):
            eng.draft_step(j)
            torch.cuda.synchronize()
            o = eng.o_draft.cpu().numpy()
            xs = eng.xs.cpu().numpy()
            for b, st in enumerate(states):
                o_ref, _, _, _ = st.draft_step(int(xs[j, b]))
                assert_attention_close(o[b], o_ref, f"{cfg.name} r{r} draft step {j} seq {b}")
                excused += check_token(model, o[b], int(xs[j + 1, b]), f"draft r{r} j{j} b{b}")
        eng.embed_block()
        eng.verify_attention()
        eng.verify_vocab()
        torch.cuda.synchronize()
        ov = eng.o_ver.cpu().numpy()
        y = eng.y.cpu().numpy()
        xs = eng.xs.cpu().numpy().copy()
        for b, st in enumerate(states):
            o_ref, _, _, _ = st.verify([int(t) for t in xs[:, b]])
            assert_attention_close(ov[:, b], o_ref, f"{cfg.name} r{r} verify seq {b}")
            for j in range(k + 1):
                excused += check_token(model, ov[j, b], int(y[j, b]), f"verify r{r} row {j} b{b}")
        eng.accept_commit()
        torch.cuda.synchronize()
        na = eng.n_accept[r].cpu().numpy()
        cm = eng.committed[r].cpu().numpy()
        nxt = eng.xs[0].cpu().numpy()
        assert (eng.status.cpu().numpy() == 0).all()
        for b, st in enumerate(states):
            m, n, c = oracle.greedy_accept(xs[1:, b], y[:, b])
            assert na[b] == m and nxt[b] == n and np.array_equal(cm[:, b], c), f"accept r{r} b{b}"
            st.commit([int(t) for t in xs[:, b]], m, tail_start[b], n)
            streams[b] += [int(t) for t in c if t >= 0]
        ctx = eng.ctx_len.cpu().numpy()
        tl = eng.tail_len.cpu().numpy()
        bl = eng.body_len.cpu().numpy()
        for b, st in enumerate(states):
            assert ctx[b] == st.k_full.shape[1]
            if cfg.kind != "dense":
                assert tl[b] == st.tail_k.shape[1], (r, b, tl[b], st.tail_k.shape[1])
            if cfg.kind == "kivi":
                assert bl[b] == st.body_len()
            if cfg.kind == "dense":
                assert bl[b] == ctx[b] and tl[b] == 0
        log(f"  accept lengths {na.tolist()}")
    return eng, states, streams, excused, model


ROUND_CASES = {
    "kivi4": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, context=256, vocab=1024, k=6, kind="kivi",
                  bits=4, residual=32, seed=11),
    "kivi2-flush": dict(batch=2, n_q_heads=16, n_kv_heads=4, head_dim=128, context=512, vocab=2048, k=40,
                        kind="kivi", bits=2, residual=32, outliers=True, seed=12),
    "tokdrop": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, context=1024, vocab=1024, k=5,
                    kind="tokdrop", keep=0.25, seed=13),
    "dense": dict(batch=2, n_q_heads=8, n_kv_heads=4, head_dim=64, context=300, vocab=512, k=7, kind="dense",
                  seed=14),
    "staged-kivi": dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, context=2048, vocab=1024, k=6,
                        kind="kivi", bits=2, residual=128, staged=True, chunk=512, seed=15),
}


@pytest.mark.parametrize("name", list(ROUND_CASES))
def test_round_teacher_forced(eng_mod, name):
    configs, engine = eng_mod
    cfg = configs.RoundConfig(name=f"round-{name}", **ROUND_CASES[name])
    rounds = 3
    eng, states, streams, excused, model = run_case(configs, engine, cfg, rounds)
    log(f"  near-tie excused tokens: {excused}")
    if name == "dense" and excused == 0:
        # identity compressor: every round accepts all k drafts plus the bonus
        assert (eng.n_accept.cpu().numpy() == cfg.k).all()
    if excused == 0:
        ocfg = oracle_cfg(cfg)
        for b in range(cfg.batch):
            assert streams[b] == full_kv_greedy(ocfg, b, len(streams[b]), model), f"lossless stream b{b}"
