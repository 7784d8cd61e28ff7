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


def assert_attention_close(gpu, ref, what=""):
    """Tolerance of the attention outputs: max |d| <= 1e-2 and rel-L2 <= 2e-3
    against the fp64 oracle (bf16 inputs, fp32 accumulation)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    mad = float(np.abs(gpu - ref).max())
    rl2 = rel_l2(gpu, ref)
    assert mad <= 1e-2 and rl2 <= 2e-3, f"{what}: max|d| {mad:.3e} rel-L2 {rl2:.3e}"
    return mad, rl2
