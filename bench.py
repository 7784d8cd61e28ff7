"""Benchmark: VeriCache rounds on one MI355X, one JSON line on stdout.

A step is one whole round of the hot path on one batch of synthetic input:
k draft steps (embedding, draft decode attention over the compressed cache,
vocab projection + argmax), the verification pass over the full cache (verify
attention, vocab projection + argmax), greedy acceptance and commit (full
cache append, tail rewrite, residual flush). Inputs are resident in HBM when
the timed region starts.

metric (per decoder layer): accepted tokens per second per layer,
    value = sum over timed rounds and sequences of (m + 1)
            / (timed rounds * (k * t_draft_attn + t_verify_attn)),
with t_draft_attn / t_verify_attn the average duration of a whole draft /
verification attention call (attention kernel + split merge), measured inside
the timed region by HIP events that the calls' own kernel dispatches record
(vc_time_next_call: no queue markers, so timing does not idle the GPU). A
real model projects to the vocabulary once per token, not once per layer,
so the vocab projection is outside the per-layer metric; the whole-round
wall clock is reported as ms_per_step and round_tok_s.

roofline: the draft decode attention kernel (the dominant term of the
metric): algorithmic bytes per launch (compressed body + fp16 tail + q + out)
over the kernel's own average duration (events around the attention kernel
alone, on alternate draft steps), against 8 TB/s; `traffic` is the HBM bytes
per launch from the committed FETCH_SIZE / WRITE_SIZE measurement when the
kernel source has not changed since. The same figures for the verification
kernel are under verify_attn.
cpu_baseline: the fp64 CPU oracle on a bounded sample of the same workload.
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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3-8b-layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def cpu_baseline(cfg, accepted_per_round, quiet):
    """The CPU oracle (fp64 numpy) on a bounded sample: one sequence and one
    KV-head group (its g query heads) of the same layer, one whole round
    (k draft steps + verify + accept + commit), projected to the batch by
    B * Hkv (attention work is linear in it)."""
    import numpy as np

    from oracle.model import ModelConfig, make_states
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    g = cfg.group
    ocfg = ModelConfig(batch=1, n_q_heads=g, n_kv_heads=1, head_dim=cfg.head_dim, context=cfg.context,
                       vocab=8192, k=cfg.k, kind=cfg.kind, bits=cfg.bits, residual=cfg.residual, keep=cfg.keep,
                       outliers=cfg.outliers, seed=cfg.seed)
    log("cpu baseline: building the oracle sample", quiet)
    _, states = make_states(ocfg)
    # consecutive rounds of the sample until about 12 s of CPU work (at least
    # one round, at most eight), averaged per round
    t0 = time.perf_counter()
    rounds = 0
    while True:
        states[0].run_round()
        rounds += 1
        spent = time.perf_counter() - t0
        if spent >= 12.0 or rounds >= 8:
            break
    dt = spent / rounds
    scale = cfg.batch * cfg.n_kv_heads
    projected = dt * scale
    value = accepted_per_round / projected
    log(f"cpu baseline: {rounds} sample rounds in {spent:.2f} s, projected round {projected:.1f} s", quiet)
    return {
        "value": value, "unit": "accepted tok/s/layer", "cores": threads, "kind": "oracle",
        "sample": (f"1 sequence x 1 KV-head group ({g} q heads) of the {cfg.name} shape, {rounds} consecutive whole "
                   f"oracle rounds (each k={cfg.k} draft steps + verify + accept + commit, vocab 8192 x "
                   f"{g * cfg.head_dim}) in {spent:.2f} s, {dt:.2f} s per round, scaled x{scale} (batch x KV heads) "
                   f"to {projected:.1f} s per round; accepted tokens per round taken from the GPU run (identical by "
                   f"parity)"),
        "sample_seconds": spent, "sample_rounds": rounds, "host_cpus": os.cpu_count(),
    }


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
    import numpy as np
    import torch

    from lossless_speculative_kv_amd import configs, engine

    cfg = configs.BY_NAME[args.workload]
    q = args.quiet
    log(f"workload {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} D={cfg.head_dim} "
        f"T={cfg.context} k={cfg.k} V={cfg.vocab} kind={cfg.kind}", q)
    t_setup = time.perf_counter()
    eng = engine.Engine(cfg, rounds_cap=args.warmup + args.steps)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s", q)

    for _ in range(args.warmup):
        eng.round()
    torch.cuda.synchronize()
    body0, tail0, ctx0 = (eng.body_len.cpu().numpy(), eng.tail_len.cpu().numpy(), eng.ctx_len.cpu().numpy())
    eng.prepare_timing(args.steps * (2 * cfg.k + 2) + 4)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        eng.round()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    body1, tail1, ctx1 = (eng.body_len.cpu().numpy(), eng.tail_len.cpu().numpy(), eng.ctx_len.cpu().numpy())
    ev = eng.events
    eng.events = None

    times = {}
    for name, a, b in ev:
        times.setdefault(name, []).append(a.elapsed_time(b) * 1e-3)
    n_acc = eng.n_accept[args.warmup:args.warmup + args.steps].cpu().numpy()
    accepted = float((n_acc + 1).sum())
    # whole calls (attention kernel + split merge) were timed on even draft
    # steps / even rounds, the attention kernel alone on odd ones; the events
    # are recorded by the kernels' own dispatches (vc_time_next_call)
    def avg(name):
        v = times.get(name, [])
        return float(np.mean(v)) if v else 0.0
    t_draft_avg, t_draft_main = avg("draft_attn"), avg("draft_attn_main")
    t_verify_avg, t_verify_main = avg("verify_attn"), avg("verify_attn_main")
    attn_time = args.steps * (cfg.k * t_draft_avg + t_verify_avg)
    value = accepted / attn_time if attn_time > 0 else 0.0

    mid_body = [(int(a) + int(b)) / 2 for a, b in zip(body0, body1)]
    mid_tail = [(int(a) + int(b)) / 2 + cfg.k / 2 for a, b in zip(tail0, tail1)]  # tail grows by 1 per draft step
    draft_bytes = draft_bytes_per_launch(cfg, mid_body, mid_tail)
    verify_bytes = verify_bytes_per_launch(cfg, [(int(a) + int(b)) / 2 for a, b in zip(ctx0, ctx1)])
    draft_gbs = draft_bytes / t_draft_main / 1e9 if t_draft_main > 0 else 0.0
    t_vmain = t_verify_main if t_verify_main > 0 else t_verify_avg   # staged: whole chunked pass only
    verify_gbs = verify_bytes / t_vmain / 1e9 if t_vmain > 0 else 0.0

    B, k = cfg.batch, cfg.k
    # MFMA utilisation: algorithmic flops over the main kernel's own duration
    mid_ctx = [(int(a) + int(b)) / 2 for a, b in zip(ctx0, ctx1)]
    mfma = {
        "verify_attn": mfma_entry("verify_kernel", verify_flops_per_launch(cfg, mid_ctx), t_vmain),
        "draft_vocab": mfma_entry("vocab product, M = batch", 2.0 * B * cfg.hidden * cfg.vocab,
                                  avg("draft_vocab_main")),
        "verify_vocab": mfma_entry("vocab product, M = (k+1) * batch", 2.0 * (k + 1) * B * cfg.hidden * cfg.vocab,
                                   avg("verify_vocab_main")),
    }
    w_bytes = 2.0 * cfg.hidden * cfg.vocab
    for key in ("draft_vocab", "verify_vocab"):
        t = mfma[key]["avg_launch_us"] * 1e-6
        mfma[key]["weight_GBs"] = w_bytes / t / 1e9 if t > 0 else 0.0
    ceiling = B * (k + 1) / (k * t_draft_avg + t_verify_avg) if (k * t_draft_avg + t_verify_avg) > 0 else 0.0
    breakdown = {name: {"avg_us": float(np.mean(v)) * 1e6, "calls": len(v)} for name, v in times.items()}
    result = {
        "metric": "accepted tok/s/layer; draft & verify attn HBM GB/s as % of 8 TB/s peak",
        "value": value,
        "unit": "accepted tok/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16 MFMA, fp32 accumulate (KIVI-2 codes)",
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "context": cfg.context,
                   "draft_k": cfg.k, "compressor": cfg.kind if cfg.kind != "kivi" else f"kivi-{cfg.bits}",
                   "residual": cfg.residual, "vocab": cfg.vocab, "hidden": cfg.hidden},
        "roofline": {"bound": "hbm", "kernel": draft_kernel_name(cfg),
                     "achieved": draft_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": draft_gbs / HBM_PEAK_GBS, "traffic": traffic_for(draft_kernel_name(cfg), cfg.name),
                     "bytes_per_launch": draft_bytes, "avg_launch_us": t_draft_main * 1e6,
                     "call_us": t_draft_avg * 1e6},
        "verify_attn": {"kernel": "verify_kernel", "achieved_GBs": verify_gbs, "frac": verify_gbs / HBM_PEAK_GBS,
                        "traffic": traffic_for("verify_kernel", cfg.name),
                        "bytes_per_launch": verify_bytes, "avg_launch_us": t_vmain * 1e6,
                        "call_us": t_verify_avg * 1e6},
        "mfma": mfma,
        **({"staging": {"host_resident_full_cache": True, "chunk_tokens": cfg.chunk,
                        "device_chunk_buffers": cfg.stage_buffers,
                        "verify_host_link_GBs": verify_gbs,
                        "note": "verify time covers the whole chunked pass with its host-to-device copies "
                                "(PCIe-inclusive); the first chunks are copied while the round drafts"}}
           if cfg.staged else {}),
        "accept": {"mean_m": float(n_acc.mean()), "accepted_per_round": accepted / args.steps,
                   "histogram_m": np.bincount(n_acc.ravel(), minlength=k + 1).tolist()},
        "round_tok_s": accepted / wall,
        "what_if_all_accepted_tok_s_layer": ceiling,
        "kernels": breakdown,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, accepted / args.steps, q)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
