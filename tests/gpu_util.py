"""Helpers for the GPU parity tests: host-side inputs (seeded, via synth),
oracle-side references, and uploads. Imported only by tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth


def log(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_tensor(values_f32: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 array holding bf16 values -> torch bfloat16 on the device (exact)."""
    bits = synth.fp32_to_bf16_bits(np.ascontiguousarray(values_f32, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def f16_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(device)


def ctx_rows(seed, B, Hkv, T, D, key_mult=None):
    """Context K, V float32 [B][Hkv][T][D] (bf16 values)."""
    K = np.stack([np.stack([synth.ctx_kv(seed, "k", b, h, 0, T, D, key_mult) for h in range(Hkv)]) for b in range(B)])
    V = np.stack([np.stack([synth.ctx_kv(seed, "v", b, h, 0, T, D) for h in range(Hkv)]) for b in range(B)])
    return K.astype(np.float32), V.astype(np.float32)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# Verification attention and the draft over bf16 rows (token drop, dense)
# round their probabilities to fp16 (11 significant bits) and take bf16
# values to fp16 exactly, so their rel-L2 error is of order 2^-12 (about
# 1.5e-4 .. 2.3e-4 measured at every size); their checks use half the
# general bound.
FP16P_RL2 = 1e-3


def assert_attention_close(gpu, ref, what="", rl2_max=2e-3):
    """Tolerance of the attention outputs: max |d| <= 1e-2 and rel-L2 <= 2e-3
    (rl2_max) against the fp64 oracle (bf16 inputs, fp32 accumulation)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    mad = float(np.abs(gpu - ref).max())
    rl2 = rel_l2(gpu, ref)
    assert mad <= 1e-2 and rl2 <= rl2_max, f"{what}: max|d| {mad:.3e} rel-L2 {rl2:.3e}"
    return mad, rl2


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_argmax_chunked(W_dev: torch.Tensor, h_bf16: np.ndarray, got: np.ndarray, step: int = 16384) -> int:
    """GPU argmax tokens `got` [M] against the first-index argmax of the
    oracle's fp64 logits of the bf16 hidden rows h_bf16 [M][H] over the whole
    vocabulary W_dev [V][H] (read in row chunks); a differing token is
    excused only within the near-tie bound. Returns the number excused."""
    import oracle
    M = h_bf16.shape[0]
    V = W_dev.shape[0]
    best = np.full(M, -np.inf)
    arg = np.zeros(M, np.int64)
    lg_got = np.zeros(M)
    for v0 in range(0, V, step):
        Wc = f64(W_dev[v0:v0 + step])
        lg = oracle.logits(h_bf16, Wc)
        am = oracle.argmax_first(lg)
        m = lg[np.arange(M), am]
        upd = m > best
        best[upd], arg[upd] = m[upd], am[upd] + v0
        inside = (got >= v0) & (got < v0 + Wc.shape[0])
        lg_got[inside] = lg[np.arange(M)[inside], got[inside] - v0]
    excused = 0
    for r in range(M):
        if got[r] != arg[r]:
            W2 = f64(W_dev[int(arg[r])])[None, :]
            bound = oracle.tie_bound(h_bf16[r:r + 1], W2, [0])[0]
            assert best[r] - lg_got[r] <= bound, f"row {r}: gap {best[r] - lg_got[r]} > {bound}"
            excused += 1
    return excused


def check_verify_unit(eng, b: int, hk: int, rows_per_pass: int = 32):
    """Every verification row of one (sequence, KV head) unit: the (k+1) * g
    query rows (draft row j, query head hk*g + i) against the oracle's
    prefix attention over the full context followed by the block rows (row j
    sees the context and block rows 0..j). Tolerance on the whole unit's
    output, as for a call; returns (max |d|, rel-L2, worst row rel-L2)."""
    import oracle
    c = eng.cfg
    g = c.n_q_heads // c.n_kv_heads
    n = int(eng.ctx_len[b])
    K = np.concatenate([f64(eng.full_k[b, hk, :n]), f64(eng.kn[:, b, hk])])
    V = np.concatenate([f64(eng.full_v[b, hk, :n]), f64(eng.vn[:, b, hk])])
    Q = f64(eng.qv[:, b, hk * g:(hk + 1) * g]).reshape(-1, c.head_dim)       # rows (j, i)
    nvis = n + 1 + np.repeat(np.arange(c.k + 1), g)
    got = eng.o_ver[:, b, hk * g:(hk + 1) * g].cpu().numpy().reshape(-1, c.head_dim)
    ref = np.concatenate([oracle.attend_prefix(Q[r0:r0 + rows_per_pass], K, V, nvis[r0:r0 + rows_per_pass])
                          for r0 in range(0, Q.shape[0], rows_per_pass)])
    worst = max(rel_l2(got[r], ref[r]) for r in range(Q.shape[0]))
    mad, rl2 = assert_attention_close(got, ref, f"verify unit ({b}, {hk}) of {c.name}", rl2_max=FP16P_RL2)
    return mad, rl2, worst
