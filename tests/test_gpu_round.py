"""Teacher-forced round parity: the GPU engine runs whole VeriCache rounds; the
oracle replays every step on the GPU's token history and checks

* each draft-step and verify attention output (tolerance of the fp64 oracle),
* each drafted / verified token: the argmax of the oracle's fp64 logits on the
  GPU's own bf16 hidden vector, bit-exact unless within the near-tie bound,
* accept length, committed tokens and next token (bit-exact),
* the cache lengths after commit (context, tail, body),
* the identity compressor (dense): every draft is accepted unless the draft
  and verification tokens are a near-tie at the fp64 reference (two kernels
  round differently, so a tie can fall either way),
* the staged (host-resident) full cache,
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


def ref_tie(model, o_gpu_row, o_ref_row, tok_gpu, what):
    """0 if tok_gpu is also the argmax at the fp64 reference hidden o_ref;
    else assert that the two tokens are a near-tie there (within the logit
    change that the GPU hidden's deviation and bf16 rounding allow) and
    return 1: past such a tie the greedy streams may part."""
    ref = np.asarray(o_ref_row, np.float64).reshape(1, -1)
    h_ref = oracle.to_bf16(ref.astype(np.float32))
    want = int(oracle.argmax_first(oracle.logits(h_ref, model.W)[0]))
    if want == tok_gpu:
        return 0
    W = np.asarray(model.W, np.float64)
    h_gpu = oracle.to_bf16(np.asarray(o_gpu_row, np.float32).reshape(1, -1))[0].astype(np.float64)
    dev = np.abs(h_gpu - h_ref[0]).max() + np.abs(h_ref[0] - ref[0]).max()
    gap = abs(float((W[want] - W[tok_gpu]) @ ref[0]))
    bound = float(np.abs(W[want] - W[tok_gpu]).sum()) * dev
    log(f"  {what}: reference near-tie {tok_gpu} vs {want}, gap {gap:.3e} <= {bound:.3e}")
    assert gap <= bound, f"{what}: token {tok_gpu} vs reference {want} is not a near-tie ({gap} > {bound})"
    return 1


def check_kivi_records(eng, states, cfg, what):
    """The GPU's body records, byte for byte, against the oracle's body
    (quantised by the oracle from its own fp64 rows) in the stored layout."""
    blocks = eng.kivi_blocks.cpu().numpy()
    for b, st in enumerate(states):
        nb = st.body_len()
        for h in range(cfg.n_kv_heads):
            bd = st.body[h]
            want = oracle.pack_blocks(bd["kc"], bd["ks"], bd["kz"], bd["vc"], bd["vs"], bd["vz"], cfg.bits)
            assert np.array_equal(blocks[b, h, :nb // 32], want), f"{what}: records of ({b}, {h})"


def run_case(configs, engine, cfg, rounds, forced=False):
    """forced: after each draft step is checked, the drafted token is replaced
    by the full-cache greedy token (teacher forcing as in the oracle's
    run_round(forced_drafts=...)), so every round accepts all k drafts unless
    verification meets a near-tie; the KIVI tail then crosses R + 32 and the
    residual flush runs."""
    eng = engine.Engine(cfg, rounds_cap=rounds)
    ocfg = oracle_cfg(cfg)
    model = SynthModel(ocfg)
    states = [SequenceState(model, b, int(eng.xs[0, b].item())) for b in range(cfg.batch)]
    k, B = cfg.k, cfg.batch
    excused = 0
    streams = [[] for _ in range(B)]
    greedy = [full_kv_greedy(ocfg, b, rounds * (k + 1), model) for b in range(B)] if forced else None
    hist = []  # per round: draft hiddens [k][B], verify hiddens [k+1][B], references, tokens
    flush_total = 0
    for r in range(rounds):
        log(f"{cfg.name} round {r}")
        tail_start = [st.tail_k.shape[1] for st in states]
        body_before = [int(x) for x in eng.body_len.cpu().numpy()]
        rec = {"draft": [], "draft_ref": []}
        eng.begin_round()
        for j in range(k):
            eng.draft_step(j)
            torch.cuda.synchronize()
            o = eng.o_draft.cpu().numpy()
            xs = eng.xs.cpu().numpy()
            refs = []
            for b, st in enumerate(states):
                o_ref, _, _, _ = st.draft_step(int(xs[j, b]))
                assert_attention_close(o[b], o_ref, f"{cfg.name} r{r} draft step {j} seq {b}")
                excused += check_token(model, o[b], int(xs[j + 1, b]), f"draft r{r} j{j} b{b}")
                refs.append(o_ref)
            if forced:
                # force only while the committed stream follows full-cache greedy
                # decoding (a near-tie in verification may part them)
                row = [greedy[b][len(streams[b]) + j] if streams[b] == greedy[b][:len(streams[b])]
                       else int(xs[j + 1, b]) for b in range(B)]
                eng.xs[j + 1] = torch.tensor(row, dtype=torch.int32, device=eng.xs.device)
            rec["draft"].append(o.copy())
            rec["draft_ref"].append(refs)
        eng.embed_block()
        eng.verify_attention()
        eng.verify_vocab()
        torch.cuda.synchronize()
        ov = eng.o_ver.cpu().numpy()
        y = eng.y.cpu().numpy()
        xs = eng.xs.cpu().numpy().copy()
        rec["verify"], rec["verify_ref"], rec["xs"], rec["y"] = ov.copy(), [], xs.copy(), y.copy()
        for b, st in enumerate(states):
            o_ref, _, _, _ = st.verify([int(t) for t in xs[:, b]])
            assert_attention_close(ov[:, b], o_ref, f"{cfg.name} r{r} verify seq {b}")
            for j in range(k + 1):
                excused += check_token(model, ov[j, b], int(y[j, b]), f"verify r{r} row {j} b{b}")
            rec["verify_ref"].append(o_ref)
        hist.append(rec)
        eng.accept_commit()
        torch.cuda.synchronize()
        na = eng.n_accept[r].cpu().numpy()
        cm = eng.committed[r].cpu().numpy()
        nxt = eng.xs[0].cpu().numpy()
        assert (eng.status.cpu().numpy() == 0).all()
        for b, st in enumerate(states):
            m, n, c = oracle.greedy_accept(xs[1:, b], y[:, b])
            # committed tokens come from verification rows 0..m
            for j in range(m + 1):
                excused += ref_tie(model, ov[j, b], rec["verify_ref"][b][j], int(y[j, b]), f"r{r} row {j} b{b}")
            assert na[b] == m and nxt[b] == n and np.array_equal(cm[:, b], c), f"accept r{r} b{b}"
            st.commit([int(t) for t in xs[:, b]], m, tail_start[b], n)
            streams[b] += [int(t) for t in c if t >= 0]
        ctx = eng.ctx_len.cpu().numpy()
        tl = eng.tail_len.cpu().numpy()
        bl = eng.body_len.cpu().numpy()
        if cfg.kind == "kivi":
            check_kivi_records(eng, states, cfg, f"{cfg.name} r{r}")
            flushes = [int(bl[b]) - body_before[b] for b in range(B)]
            log(f"  body growth {flushes}")
            flush_total += sum(flushes)
        for b, st in enumerate(states):
            assert ctx[b] == st.k_full.shape[1]
            if cfg.kind != "dense":
                assert tl[b] == st.tail_k.shape[1], (r, b, tl[b], st.tail_k.shape[1])
            if cfg.kind == "kivi":
                assert bl[b] == st.body_len()
            if cfg.kind == "dense":
                assert bl[b] == ctx[b] and tl[b] == 0
        log(f"  accept lengths {na.tolist()}")
    eng.flushed_tokens = flush_total
    return eng, states, streams, excused, model, hist


def check_dense_acceptance(eng, cfg, model, hist):
    """Identity compressor: a draft is rejected only at a near-tie. At the
    first mismatch m the draft token x (from the draft hidden hd) and the
    verification token y (from the verify hidden hv) are both exact argmaxes
    of their own hiddens; both hiddens are within the attention tolerance of
    the same fp64 reference o_ref, so at o_ref the logits of x and y may differ
    by at most sum_c |W_y,c - W_x,c| * (|hd - o_ref|_inf + |hv - o_ref|_inf +
    the bf16 rounding of the hidden)."""
    na = eng.n_accept.cpu().numpy()
    W = np.asarray(model.W, np.float64)
    flips = 0
    for r, rec in enumerate(hist):
        for b in range(cfg.batch):
            m = int(na[r, b])
            if m == cfg.k:
                continue
            flips += 1
            x, yv = int(rec["xs"][m + 1, b]), int(rec["y"][m, b])
            assert x != yv
            ref = np.asarray(rec["verify_ref"][b][m], np.float64).reshape(-1)
            ref_d = np.asarray(rec["draft_ref"][m][b], np.float64).reshape(-1)
            np.testing.assert_allclose(ref_d, ref, rtol=0, atol=1e-9)  # same KV, same query in dense mode
            hd = oracle.to_bf16(np.asarray(rec["draft"][m][b], np.float32).reshape(1, -1))[0].astype(np.float64)
            hv = oracle.to_bf16(np.asarray(rec["verify"][m, b], np.float32).reshape(1, -1))[0].astype(np.float64)
            dev = np.abs(hd - ref).max() + np.abs(hv - ref).max()
            gap = abs(float((W[yv] - W[x]) @ ref))
            bound = float(np.abs(W[yv] - W[x]).sum()) * dev
            log(f"  dense round {r} seq {b}: rejected at {m}, reference gap {gap:.3e} <= bound {bound:.3e}")
            assert gap <= bound, f"dense r{r} b{b}: draft {x} vs verify {yv} is not a near-tie ({gap} > {bound})"
    return flips


ROUND_CASES = {
    "kivi4": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, context=256, vocab=1024, k=6, kind="kivi",
                  bits=4, residual=32, seed=11),
    "kivi2-flush": dict(batch=2, n_q_heads=16, n_kv_heads=4, head_dim=128, context=512, vocab=2048, k=40,
                        kind="kivi", bits=2, residual=32, outliers=True, seed=12),
    "kivi4-flush-d64": dict(batch=3, n_q_heads=8, n_kv_heads=4, head_dim=64, context=320, vocab=1024, k=20,
                            kind="kivi", bits=4, residual=64, seed=16),
    "tokdrop": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, context=1024, vocab=1024, k=5,
                    kind="tokdrop", keep=0.25, seed=13),
    "dense": dict(batch=2, n_q_heads=8, n_kv_heads=4, head_dim=64, context=300, vocab=512, k=7, kind="dense",
                  seed=14),
    "staged-kivi": dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, context=2048, vocab=1024, k=6,
                        kind="kivi", bits=2, residual=128, staged=True, chunk=512, seed=15),
}


# cases whose drafts are forced to the full-cache greedy tokens: every round
# accepts all k, so the KIVI tail crosses R + 32 and flushes each round
FORCED = {"kivi2-flush", "kivi4-flush-d64"}


@pytest.mark.parametrize("name", list(ROUND_CASES))
def test_round_teacher_forced(eng_mod, name):
    configs, engine = eng_mod
    cfg = configs.RoundConfig(name=f"round-{name}", **ROUND_CASES[name])
    rounds = 3
    forced = name in FORCED
    eng, states, streams, excused, model, hist = run_case(configs, engine, cfg, rounds, forced=forced)
    if forced:
        # at least one 32-token block per sequence joined the body over the rounds
        assert eng.flushed_tokens >= 32 * cfg.batch, f"flushed {eng.flushed_tokens} tokens"
    log(f"  near-tie excused tokens: {excused}")
    if name == "dense":
        flips = check_dense_acceptance(eng, cfg, model, hist)
        assert flips <= rounds * cfg.batch // 2, f"dense: {flips} rejections in {rounds * cfg.batch} rounds"
    if excused == 0:
        ocfg = oracle_cfg(cfg)
        for b in range(cfg.batch):
            assert streams[b] == full_kv_greedy(ocfg, b, len(streams[b]), model), f"lossless stream b{b}"
