"""Benchmark: VeriCache rounds on one MI355X, one JSON line on stdout.

A step is one whole round of the hot path on one batch of synthetic input:
k draft steps (embedding, draft decode attention over the compressed cache,
vocab projection + argmax), the verification pass over the full cache (verify
attention, vocab projection + argmax), greedy acceptance and commit (full
cache append, tail rewrite, residual flush). Inputs are resident in HBM when
the timed region starts. The default workload is the Qwen-32B-shaped layer
(B = 16, 40 q / 8 KV heads, context 65536, KIVI-2, k = 25), the largest whose
full cache and compressed cache both live in HBM; the 1M-token Llama-70B
layer (full cache in pinned host memory, staged over the host link) is
measured after it as an extra block.

metric (per decoder layer): accepted tokens per second per layer,
    value = sum over timed rounds and sequences of (m + 1)
            / (timed rounds * (k * t_draft_attn + t_verify_attn)),
with t_draft_attn / t_verify_attn the median duration of a whole draft /
verification attention call (attention kernel + split merge), measured inside
the timed region by HIP events that the calls' own kernel dispatches record
(vc_time_next_call: no queue markers, so timing does not idle the GPU); p10
and p90 of the same formula are reported beside it. A real model projects to
the vocabulary once per token, not once per layer, so the vocab projection is
outside the per-layer metric; the whole-round wall clock is ms_per_step and
round_tok_s.

Comparator: full-KV decoding per layer, B / t(dense draft kernel over the
whole committed context plus the new token), measured in the same run; the
ratio value / comparator is reported, and the same time model at the pages'
25 and 40 accepted tokens per round (derived figures).

roofline: the draft decode attention kernel (the dominant term of the
metric): algorithmic bytes per launch (compressed body + fp16 tail + q + out)
over the kernel's own median duration (events around the attention kernel
alone, on alternate draft steps), against 8 TB/s; `traffic` is the HBM bytes
per launch from the committed FETCH_SIZE / WRITE_SIZE measurement when the
kernel source has not changed since. The same figures for the verification
kernel are under verify_attn.
cpu_baseline: the fp64 CPU oracle timed by the same formula (its draft-step
and verification attention, on one sequence and one KV-head group, scaled
by batch x KV heads).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen-32b-layer")
    ap.add_argument("--extra", default="llama-70b-layer-1m",
                    help="comma-separated workloads measured after the main one (3 rounds each) and reported "
                         "under extra_workloads; 'none' for none")
    ap.add_argument("--p1", default="llama-70b-layer-1m,llama-70b-layer-256k,llama-70b-layer-256k-1buf",
                    help="host-resident workloads on which the P1 scheduler's two staggered request groups are "
                         "measured against one group (3 rounds each); 'none' for none")
    ap.add_argument("--pipeline", default="llama-70b-layer-1m",
                    help="host-resident workload on which pipelined drafting is timed against plain rounds; 'none' "
                         "for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-states", action="store_true",
                    help="skip the cold / warm calls timed alone (kernel profiles then hold the round's calls only)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (5 times) and print its byte counts; the "
                         "HBM counters of this run calibrate the traffic figures of the hot-path kernels")
    return ap.parse_args()


def copy_calibration(mb: int):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mb * 1024 * 1024
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": 5}}))


def log(msg, quiet=False):
    if not quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


def draft_bytes_per_launch(cfg, body_len, tail_len):
    """Algorithmic bytes of one draft attention launch: what the method must
    read for each (sequence, KV head) plus the query and output vectors."""
    B, Hq, Hkv, D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    qo = B * Hq * D * (2 + 4)
    if cfg.kind == "kivi":
        per_tok = 2 * D * cfg.bits // 8 + 4 * D // 32 + 4 * D // 32   # K,V codes + K scale/zero per token + V scale/zero
        tail_tok = 4 * D                                            # fp16 K and V
        return sum(Hkv * (body_len[b] * per_tok + tail_len[b] * tail_tok) for b in range(B)) + qo
    if cfg.kind == "tokdrop":
        return sum(Hkv * (body_len[b] * (4 * D + 4) + tail_len[b] * 4 * D) for b in range(B)) + qo
    return sum(Hkv * (body_len[b] + tail_len[b]) * 4 * D for b in range(B)) + qo


def verify_bytes_per_launch(cfg, ctx_len):
    B, Hq, Hkv, D, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.k + 1
    return sum(Hkv * (ctx_len[b] + n) * 4 * D for b in range(B)) + n * B * Hq * D * (2 + 4)


def verify_flops_per_launch(cfg, ctx_len):
    """Algorithmic MFMA work of one verification launch: QK^T and PV (2 * 2 * D
    flops per query row and visible key); row j of the block sees the context
    and block rows 0..j."""
    B, Hq, D, n = cfg.batch, cfg.n_q_heads, cfg.head_dim, cfg.k + 1
    return sum(Hq * (n * ctx_len[b] + n * (n + 1) / 2) * 4 * D for b in range(B))


def mfma_entry(kernel, flops, seconds):
    tflops = flops / seconds / 1e12 if seconds > 0 else 0.0
    return {"kernel": kernel, "flops_per_launch": flops, "avg_launch_us": seconds * 1e6, "achieved_TFLOPs": tflops,
            "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "frac": tflops / MFMA_BF16_PEAK_TFLOPS}


def draft_kernel_name(cfg):
    return {"kivi": "draft_kivi_kernel", "tokdrop": "draft_rows_kernel"}.get(cfg.kind, "draft_rows_kernel")


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter measurement (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE,
    scaled by a plain copy of known size), or None when no measurement exists
    or the kernel's source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    entry = table.get("kernels", {}).get(f"{kernel}@{workload}")
    if not entry:
        return None
    src = os.path.join(ROOT, entry["source"])
    try:
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if digest != entry["source_sha256"]:
        return None
    return entry["fetch_bytes"] + entry["write_bytes"]


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v, dtype=np.float64), q)) if len(v) else 0.0


def dist_us(v):
    """Median, p10, p90 of a list of seconds, in microseconds."""
    return {"median": pct(v, 50) * 1e6, "p10": pct(v, 10) * 1e6, "p90": pct(v, 90) * 1e6, "n": len(v)}


def cpu_baseline(cfg, accepted_per_round, quiet, budget_s=18.0):
    """The CPU oracle (fp64 numpy) timed by the metric's own formula.

    On one sequence and one KV-head group of the layer (the g query heads of
    KV head 0), the oracle's draft step (SequenceState.draft_step: tail
    append, attention of the g heads over the dequantised body or kept rows
    plus the tail) and its verification (SequenceState.verify: the round's
    rows over the full context plus the causal block) are timed separately,
    each scaled by B * Hkv (attention work is linear in it), and
        value = accepted tokens per round / (k * t_draft + t_verify),
    with the accepted tokens per round of the GPU run (identical by parity).
    The sample's vocabulary has 256 entries, so the projection inside
    draft_step / verify is negligible beside attention. A verification sample
    that would exceed the budget covers the block's first r rows and is
    scaled by (k + 1) / r (row j costs the context plus j + 1 block rows).
    Median, p10 and p90 over repetitions."""
    import numpy as np

    from oracle.model import ModelConfig, make_states
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    g, k = cfg.group, cfg.k
    ocfg = ModelConfig(batch=1, n_q_heads=g, n_kv_heads=1, head_dim=cfg.head_dim, context=cfg.context,
                       vocab=256, k=k, kind=cfg.kind, bits=cfg.bits, residual=cfg.residual, keep=cfg.keep,
                       outliers=cfg.outliers, seed=cfg.seed)
    log("cpu baseline: building the oracle sample", quiet)
    _, states = make_states(ocfg)
    st = states[0]
    xs = [st.x0]
    d_times = []
    t_begin = time.perf_counter()
    while len(d_times) < k and (len(d_times) < 2 or time.perf_counter() - t_begin < budget_s / 3):
        t0 = time.perf_counter()
        _, _, _, nxt = st.draft_step(xs[-1])
        d_times.append(time.perf_counter() - t0)
        xs.append(int(nxt))
    while len(xs) < k + 1:
        xs.append((xs[-1] * 7 + 1) % 256)   # tokens for the verification rows the sample did not draft
    t0 = time.perf_counter()
    st.verify(xs[:1])
    t_row = time.perf_counter() - t0
    rows = int(max(1, min(k + 1, (budget_s * 2 / 3) / (3 * t_row * 1.05))))
    v_times = []
    for _ in range(3):
        t0 = time.perf_counter()
        st.verify(xs[:rows])
        v_times.append((time.perf_counter() - t0) * (k + 1) / rows)
    spent = time.perf_counter() - t_begin
    scale = cfg.batch * cfg.n_kv_heads
    td = np.array(d_times) * scale
    tv = np.array(v_times) * scale

    def val(a, b):
        return accepted_per_round / (k * a + b)
    value = val(pct(td, 50), pct(tv, 50))
    log(f"cpu baseline: {len(d_times)} draft steps, {rows}-row verification x3 in {spent:.1f} s", quiet)
    return {
        "value": value, "unit": "accepted tok/s/layer", "cores": threads, "kind": "oracle",
        "p10": val(pct(td, 90), pct(tv, 90)), "p90": val(pct(td, 10), pct(tv, 10)),
        "sample": (f"the oracle's draft step (x{len(d_times)}) and verification ({rows} of {k + 1} rows, x3) on 1 "
                   f"sequence x 1 KV-head group ({g} q heads) of the {cfg.name} shape (context {cfg.context}), "
                   f"{spent:.1f} s of CPU work; each time scaled x{scale} (batch x KV heads) and, for "
                   f"verification, x{(k + 1) / rows:.2f} (rows); value = accepted tokens per round of the GPU "
                   f"run / (k * t_draft + t_verify), medians (p10/p90 from the slow/fast ends)"),
        "t_draft_step_s": {"median": pct(td, 50), "p10": pct(td, 10), "p90": pct(td, 90)},
        "t_verify_s": {"median": pct(tv, 50), "p10": pct(tv, 10), "p90": pct(tv, 90)},
        "sample_seconds": spent, "host_cpus": os.cpu_count(),
    }


def full_kv_decode(eng, n_calls=12):
    """Full-KV decoding per layer, the comparator of the metric: the dense
    (identity) draft kernel over each sequence's whole committed context plus
    one new token, timed by the call's own dispatches. Returns (durations in
    seconds, algorithmic bytes per launch)."""
    import torch

    from lossless_speculative_kv_amd import _lib as L
    c = eng.cfg
    B, Hq, Hkv, D = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim
    kv = L.vc_draft_kv()
    kv.kind, kv.body_cap, kv.tail_cap = L.VC_DRAFT_DENSE, eng.full_cap, 32
    body = eng.ctx_len.clone()
    tail = torch.ones((B,), dtype=torch.int32, device=eng.dev)
    tk = torch.zeros((B, Hkv, 32, D), dtype=torch.bfloat16, device=eng.dev)
    tv = torch.zeros_like(tk)
    tk[:, :, 0] = eng.kn[0]
    tv[:, :, 0] = eng.vn[0]
    kv.body_len, kv.tail_len = body.data_ptr(), tail.data_ptr()
    kv.src_k, kv.src_v, kv.src_t_cap = eng.full_k.data_ptr(), eng.full_v.data_ptr(), eng.full_cap
    kv.tail_k, kv.tail_v = tk.data_ptr(), tv.data_ptr()
    ws = torch.zeros(L.vc_draft_workspace_bytes(eng.shape, kv), dtype=torch.uint8, device=eng.dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=eng.dev)
    s = eng.stream
    ev = []
    for _ in range(n_calls):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        b.record(s)
        ev.append((a, b))
    torch.cuda.synchronize(eng.dev)
    for i in range(n_calls + 2):
        if i >= 2:
            a, b = ev[i - 2]
            L.vc_time_next_call(a.cuda_event, b.cuda_event, L.VC_TIME_CALL)
        L.vc_draft_decode_attn(eng.shape, eng.q_draft.data_ptr(), kv, out.data_ptr(), ws.data_ptr(), ws.numel(),
                               s.cuda_stream)
    torch.cuda.synchronize(eng.dev)
    times = [a.elapsed_time(b) * 1e-3 for a, b in ev]
    ctx = eng.ctx_len.cpu().numpy()
    nbytes = sum(Hkv * (int(ctx[b]) + 1) * 4 * D for b in range(B)) + B * Hq * D * 6
    return times, nbytes


def cache_states(eng, reps=10):
    """Draft and verify attention calls timed alone, cold and warm: "cold"
    writes a 1 GiB scratch buffer on the engine's stream before each call
    (evicting the per-XCD L2s and the 256 MB memory-side cache), "warm"
    repeats the call. Each call follows an idle gap of 2 ms (back-to-back
    heavy calls run at lower clocks: verification calls took about 25%
    longer), so both modes start from the same power state. The round above
    times the calls inside the round, where the 1-1.6 GB vocabulary read of
    each draft step sits between two draft calls. Calls are timed by their
    own dispatches (vc_time_next_call); their outputs and workspaces are the
    engine's, and nothing they write is read by a later round."""
    import torch

    import lossless_speculative_kv_amd._lib as L

    s = eng.stream
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=eng.dev)
    c = eng.cfg

    def draft():
        L.vc_draft_decode_attn(eng.shape, eng.q_draft.data_ptr(), eng.kv, eng.o_draft.data_ptr(),
                               eng.ws_draft.data_ptr(), eng.ws_draft.numel(), s.cuda_stream)

    def verify():
        ctx = L.vc_kv_chunk(eng.full_k.data_ptr(), eng.full_v.data_ptr(), eng.full_cap, 0, eng.full_cap)
        L.vc_verify_attn(eng.shape, c.k + 1, eng.qv.data_ptr(), eng.kn.data_ptr(), eng.vn.data_ptr(), ctx,
                         eng.ctx_len.data_ptr(), L.VC_VERIFY_BEGIN | L.VC_VERIFY_END, eng.o_ver.data_ptr(),
                         eng.ws_verify.data_ptr(), eng.ws_verify.numel(), s.cuda_stream)

    out = {}
    for name, fn in (("draft_attn_call_us", draft), ("verify_attn_call_us", verify)):
        res = {}
        for mode in ("cold", "warm"):
            ev = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(s)
                b.record(s)
                ev.append((a, b))
            torch.cuda.synchronize(eng.dev)
            fn()  # warms the call itself (and, for "warm", the caches)
            for i, (a, b) in enumerate(ev):
                if mode == "cold":
                    with torch.cuda.stream(s):
                        scratch.fill_(i & 0xFF)
                torch.cuda.synchronize(eng.dev)
                time.sleep(0.002)
                L.vc_time_next_call(a.cuda_event, b.cuda_event, L.VC_TIME_CALL)
                fn()
            torch.cuda.synchronize(eng.dev)
            res[mode] = dist_us([a.elapsed_time(b) * 1e-3 for a, b in ev])
        out[name] = res
    del scratch
    out["note"] = ("calls timed alone after a 2 ms idle gap: cold = a 1 GiB scratch write before each call (L2 and "
                   "memory-side cache evicted), warm = the call repeated; the headline uses the calls as timed "
                   "inside the round")
    return out


def measure(cfg, steps, warmup, q, comparator=True, graph_reps=0, cache=True):
    """Warm-up rounds, then `steps` timed rounds of one workload; returns the
    figures of the JSON line (without the CPU baseline). With graph_reps, a
    round is then captured in a HIP graph and replayed that many times
    (wall clock per replay, next to the eager round's)."""
    import numpy as np
    import torch

    from lossless_speculative_kv_amd import engine

    log(f"workload {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} D={cfg.head_dim} "
        f"T={cfg.context} k={cfg.k} V={cfg.vocab} kind={cfg.kind}", q)
    t_setup = time.perf_counter()
    eng = engine.Engine(cfg, rounds_cap=warmup + steps + (graph_reps + 2 if graph_reps else 0))
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s", q)
    for _ in range(warmup):
        eng.round()
    torch.cuda.synchronize()
    body0, tail0, ctx0 = (eng.body_len.cpu().numpy(), eng.tail_len.cpu().numpy(), eng.ctx_len.cpu().numpy())
    eng.prepare_timing(steps * (2 * cfg.k + 2) + 4)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        eng.round()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"{steps} timed rounds in {wall * 1e3:.1f} ms", q)
    body1, tail1, ctx1 = (eng.body_len.cpu().numpy(), eng.tail_len.cpu().numpy(), eng.ctx_len.cpu().numpy())
    ev = eng.events
    eng.events = None

    times = {}
    for name, a, b in ev:
        times.setdefault(name, []).append(a.elapsed_time(b) * 1e-3)
    n_acc = eng.n_accept[warmup:warmup + steps].cpu().numpy()
    accepted = float((n_acc + 1).sum())
    acc_round = accepted / steps
    # whole calls (attention kernel + split merge) were timed on even draft
    # steps / even rounds, the attention kernel alone on odd ones; the events
    # are recorded by the kernels' own dispatches (vc_time_next_call)
    med = {name: pct(v, 50) for name, v in times.items()}
    get = lambda name: med.get(name, 0.0)  # noqa: E731
    t_draft, t_draft_main = get("draft_attn"), get("draft_attn_main")
    t_verify, t_verify_main = get("verify_attn"), get("verify_attn_main")
    k, B = cfg.k, cfg.batch
    per_round = k * t_draft + t_verify
    value = acc_round / per_round if per_round > 0 else 0.0
    d10, d90 = pct(times.get("draft_attn", []), 10), pct(times.get("draft_attn", []), 90)
    v10, v90 = pct(times.get("verify_attn", []), 10), pct(times.get("verify_attn", []), 90)

    mid_body = [(int(a) + int(b)) / 2 for a, b in zip(body0, body1)]
    mid_tail = [(int(a) + int(b)) / 2 + k / 2 for a, b in zip(tail0, tail1)]  # tail grows by 1 per draft step
    mid_ctx = [(int(a) + int(b)) / 2 for a, b in zip(ctx0, ctx1)]
    draft_bytes = draft_bytes_per_launch(cfg, mid_body, mid_tail)
    verify_bytes = verify_bytes_per_launch(cfg, mid_ctx)
    draft_gbs = draft_bytes / t_draft_main / 1e9 if t_draft_main > 0 else 0.0
    t_vmain = t_verify_main if t_verify_main > 0 else t_verify   # staged: whole chunked pass only
    verify_gbs = verify_bytes / t_vmain / 1e9 if t_vmain > 0 else 0.0

    # MFMA utilisation: algorithmic flops over the main kernel's own duration
    mfma = {
        "verify_attn": mfma_entry("verify_kernel", verify_flops_per_launch(cfg, mid_ctx), t_vmain),
        "draft_vocab": mfma_entry("vocab product, M = batch", 2.0 * B * cfg.hidden * cfg.vocab, get("draft_vocab_main")),
        "verify_vocab": mfma_entry("vocab product, M = (k+1) * batch", 2.0 * (k + 1) * B * cfg.hidden * cfg.vocab,
                                   get("verify_vocab_main")),
    }
    w_bytes = 2.0 * cfg.hidden * cfg.vocab
    for key in ("draft_vocab", "verify_vocab"):
        t = mfma[key]["avg_launch_us"] * 1e-6
        mfma[key]["weight_GBs"] = w_bytes / t / 1e9 if t > 0 else 0.0
        mfma[key]["median_launch_us"] = mfma[key].pop("avg_launch_us")

    # comparator: full-KV decoding per layer
    if comparator and not cfg.staged:
        d_times, d_bytes = full_kv_decode(eng)
        t_full = pct(d_times, 50)
        full = {"tok_s_layer": B / t_full, "t_call": dist_us(d_times), "kernel": "draft_rows_kernel (dense)",
                "bytes_per_launch": d_bytes, "achieved_GBs": d_bytes / t_full / 1e9,
                "frac": d_bytes / t_full / 1e9 / HBM_PEAK_GBS,
                "definition": "B / t(dense draft attention over the committed context plus the new token)"}
    elif comparator:
        full = {"tok_s_layer": B / t_verify if t_verify > 0 else 0.0,
                "definition": ("full cache in host memory: every decoded token needs a pass over it across the host "
                               "link, as one verification pass does; B / t(verification pass, staged)")}
    else:
        full = None
    graph = None
    if graph_reps and not cfg.staged:
        g = eng.capture_round()
        g.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(graph_reps):
            g.replay()
        torch.cuda.synchronize()
        graph = {"round_ms": (time.perf_counter() - tg) / graph_reps * 1e3, "replays": graph_reps,
                 "eager_round_ms": wall / steps * 1e3,
                 "note": "one HIP graph launch per round (Engine.capture_round) against the eager round of the "
                         "timed region (one host call per kernel, timing events on)"}
        log(f"graph replay {graph['round_ms']:.3f} ms per round (eager {graph['eager_round_ms']:.3f} ms)", q)
        del g
    cache = cache_states(eng) if cache and not cfg.staged else None
    what_if = {str(a): B * a / ((a - 1) * t_draft + t_verify) for a in (25, 40)}
    ceiling = B * (k + 1) / per_round if per_round > 0 else 0.0
    out = {
        "cfg": cfg, "value": value, "ms_per_step": wall / steps * 1e3, "round_tok_s": accepted / wall,
        "value_p10": acc_round / (k * d90 + v90) if d90 + v90 > 0 else 0.0,
        "value_p90": acc_round / (k * d10 + v10) if d10 + v10 > 0 else 0.0,
        "t_draft_call": dist_us(times.get("draft_attn", [])), "t_draft_kernel": dist_us(times.get("draft_attn_main", [])),
        "t_verify_call": dist_us(times.get("verify_attn", [])),
        "t_verify_kernel": dist_us(times.get("verify_attn_main", [])),
        "draft_bytes": draft_bytes, "draft_gbs": draft_gbs, "t_draft_main": t_draft_main, "t_draft": t_draft,
        "verify_bytes": verify_bytes, "verify_gbs": verify_gbs, "t_vmain": t_vmain, "t_verify": t_verify,
        "mfma": mfma, "full": full, "graph": graph, "cache": cache,
        "what_if": {"all_accepted_m_eq_k": ceiling, "accepted_25_per_round": what_if["25"],
                    "accepted_40_per_round": what_if["40"],
                    "note": ("derived from the measured call times: B * a / ((a - 1) * t_draft + t_verify) for a "
                             "accepted tokens per round (a - 1 drafts all accepted plus the bonus); a = k + 1 is "
                             "this configuration's ceiling, 25 and 40 are the pages' range")},
        "accept": {"mean_m": float(n_acc.mean()), "accepted_per_round": acc_round,
                   "histogram_m": np.bincount(n_acc.ravel(), minlength=k + 1).tolist()},
        "kernels": {name: {"median_us": pct(v, 50) * 1e6, "calls": len(v)} for name, v in times.items()},
    }
    del eng
    return out


def p1_staggering(cfg, rounds, q):
    """Two request groups of a host-resident layer under the P1 scheduler
    (drafting staggered across groups, each group's full cache crossing the
    host link on its own copy stream) against one group alone: committed
    tokens per second, and the busy fractions of the host link and of
    drafting over the run."""
    from lossless_speculative_kv_amd.scheduler import StaggeredGroups
    log(f"p1 scheduler on {cfg.name}: two groups", q)
    sched = StaggeredGroups(cfg, 2, rounds_cap=1 + 2 * rounds)
    sched.run(1)  # warm-up round of both groups
    one = sched.run(rounds, trace=True, n_groups=1)
    two = sched.run(rounds, trace=True)
    log(f"p1 scheduler on {cfg.name}: one group {one.group_rounds_s:.2f} rounds/s, two groups "
        f"{two.group_rounds_s:.2f} group-rounds/s", q)
    del sched
    return {"one_group": one.as_dict(), "two_groups": two.as_dict(),
            "speedup": two.group_rounds_s / one.group_rounds_s,
            "context": cfg.context, "chunk_tokens": cfg.chunk, "device_chunk_buffers": cfg.stage_buffers,
            "draft_k": cfg.k,
            "note": "speedup = group-rounds per second with two staggered groups / rounds per second of one group "
                    "(committed tokens also depend on each group's acceptance, so they are reported but not "
                    "compared); link = host-to-device chunk copies (union of their intervals), draft = the "
                    "groups' draft-step phases"}


def pipelined_drafting(cfg, rounds, q):
    """Rounds of a host-resident layer with pipelined drafting (the drafter
    continues k + 1 steps on a side stream while verification waits for the
    full cache) against the same rounds without: wall time per round, and
    how many continued drafts the next rounds could use."""
    import torch

    from lossless_speculative_kv_amd import engine
    out = {}
    for label, pipe in (("off", 0), ("on", cfg.k + 1)):
        log(f"pipelined drafting on {cfg.name}: {label}", q)
        e = engine.Engine(cfg.scaled(pipeline=pipe), rounds_cap=rounds + 1)
        e.round()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(rounds):
            e.round()
        torch.cuda.synchronize()
        out[label] = {"round_ms": (time.perf_counter() - t0) / rounds * 1e3, "drafts_reused": e.reused_drafts,
                      "mean_m": float(e.n_accept[1:rounds + 1].float().mean())}
        del e
        torch.cuda.empty_cache()
    out["note"] = ("continued drafts are reused only after a round that accepted all k drafts whose bonus token "
                   "equals the first continued draft; with the synthetic data's low acceptance none is, so this "
                   "measures the cost of drafting during verification")
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the hot path is measured on a single "
              "MI355X. Across GPUs it would shard by sequence (draft and verify attention need no exchange) and, "
              "for one long sequence, by context, merging (max, sum, output) partials; the vocabulary shards by "
              "columns with one 64-bit argmax key per row.", file=sys.stderr)
        sys.exit(2)
    import gc

    import torch

    from lossless_speculative_kv_amd import configs

    cfg = configs.BY_NAME[args.workload]
    q = args.quiet
    r = measure(cfg, args.steps, args.warmup, q, graph_reps=args.steps, cache=not args.no_cache_states)
    full = r["full"]
    result = {
        "metric": "accepted tok/s/layer; draft & verify attn HBM GB/s as % of 8 TB/s peak",
        "value": r["value"],
        "unit": "accepted tok/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16 MFMA, fp32 accumulate (KIVI-2 codes)",
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "context": cfg.context,
                   "draft_k": cfg.k, "compressor": cfg.kind if cfg.kind != "kivi" else f"kivi-{cfg.bits}",
                   "residual": cfg.residual, "vocab": cfg.vocab, "hidden": cfg.hidden},
        "value_p10": r["value_p10"], "value_p90": r["value_p90"],
        "roofline": {"bound": "hbm", "kernel": draft_kernel_name(cfg),
                     "achieved": r["draft_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["draft_gbs"] / HBM_PEAK_GBS, "traffic": traffic_for(draft_kernel_name(cfg), cfg.name),
                     "bytes_per_launch": r["draft_bytes"], "median_launch_us": r["t_draft_main"] * 1e6,
                     "call_us": r["t_draft"] * 1e6, "launch_us": r["t_draft_kernel"], "call": r["t_draft_call"]},
        "verify_attn": {"kernel": "verify_kernel", "achieved_GBs": r["verify_gbs"],
                        "frac": r["verify_gbs"] / HBM_PEAK_GBS, "traffic": traffic_for("verify_kernel", cfg.name),
                        "bytes_per_launch": r["verify_bytes"], "median_launch_us": r["t_vmain"] * 1e6,
                        "call_us": r["t_verify"] * 1e6, "launch_us": r["t_verify_kernel"],
                        "call": r["t_verify_call"]},
        "full_kv_decode": full,
        "vs_full_kv_decode": (r["value"] / full["tok_s_layer"]) if full and full["tok_s_layer"] > 0 else None,
        "what_if": r["what_if"],
        "mfma": r["mfma"],
        "accept": r["accept"],
        "round_tok_s": r["round_tok_s"],
        "graph_round": r["graph"],
        "cache_states": r["cache"],
        "kernels": r["kernels"],
    }
    r = None
    gc.collect()
    torch.cuda.empty_cache()
    extras = {}
    for name in [x for x in args.extra.split(",") if x and x not in (cfg.name, "none")]:
        e = measure(configs.BY_NAME[name], 3, 1, q)
        ec = e["cfg"]
        extras[name] = {
            "value": e["value"], "unit": "accepted tok/s/layer", "ms_per_step": e["ms_per_step"], "steps": 3,
            "draft_attn": {"kernel": draft_kernel_name(ec), "achieved_GBs": e["draft_gbs"],
                           "frac": e["draft_gbs"] / HBM_PEAK_GBS, "bytes_per_launch": e["draft_bytes"],
                           "median_launch_us": e["t_draft_main"] * 1e6, "call": e["t_draft_call"]},
            "verify_pass": {"t_call": e["t_verify_call"], "bytes": e["verify_bytes"],
                            "GBs": e["verify_gbs"],
                            **({"note": "PCIe-inclusive: the pass streams the host-resident full cache in chunks"}
                               if ec.staged else {})},
            "full_kv_decode": e["full"], "what_if": e["what_if"], "accept": e["accept"],
            "vs_full_kv_decode": (e["value"] / e["full"]["tok_s_layer"]) if e["full"] else None,
        }
        e = None
        gc.collect()
        torch.cuda.empty_cache()
    result["extra_workloads"] = extras
    p1 = {}
    for name in [x for x in args.p1.split(",") if x and x != "none"]:
        p1[name] = p1_staggering(configs.BY_NAME[name], 3, q)
        gc.collect()
        torch.cuda.empty_cache()
    result["p1_scheduler"] = p1
    if args.pipeline != "none":
        result["pipelined_drafting"] = {args.pipeline: pipelined_drafting(configs.BY_NAME[args.pipeline], 3, q)}
        gc.collect()
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, result["accept"]["accepted_per_round"], q)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
