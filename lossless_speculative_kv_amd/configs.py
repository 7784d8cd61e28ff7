"""Workload shapes: one decoder layer of each model family the VeriCache
evaluation names (VeriCache summary, "Experimental results": Mistral-24B,
Qwen-32B, Llama-70B), plus a tiny layer and a Llama-3-8B layer. Inputs are
seeded synthetic data; see synth/."""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class RoundConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int
    vocab: int
    k: int
    kind: str = "kivi"        # "kivi" | "tokdrop" | "dense"
    bits: int = 2
    residual: int = 32
    keep: float = 0.25
    outliers: bool = False
    staged: bool = False      # full cache in pinned host memory, streamed in chunks
    chunk: int = 65536
    stage_buffers: int = 4    # device chunk buffers (>= 1); the first ones fill while the round drafts
    pipeline: int = 0         # staged only: draft steps continued on a side stream during verification (<= k + 1)
    seed: int = 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def hidden(self) -> int:
        return self.n_q_heads * self.head_dim

    def scaled(self, **kw) -> "RoundConfig":
        return dataclasses.replace(self, **kw)


TINY = RoundConfig("tiny-layer", 1, 8, 8, 64, 2048, 4096, 8, "kivi", bits=4, residual=32, seed=1)
LLAMA3_8B = RoundConfig("llama3-8b-layer", 8, 32, 8, 128, 32768, 128256, 32, "kivi", bits=2, residual=128,
                        outliers=True, seed=2)
MISTRAL_24B = RoundConfig("mistral-24b-layer", 4, 32, 8, 128, 131072, 32768, 40, "tokdrop", keep=0.25, seed=3)
QWEN_32B = RoundConfig("qwen-32b-layer", 16, 40, 8, 128, 65536, 152064, 25, "kivi", bits=2, residual=128, seed=4)
LLAMA_70B = RoundConfig("llama-70b-layer-1m", 1, 64, 8, 128, 1048576, 128256, 32, "kivi", bits=2, residual=128,
                        staged=True, chunk=65536, seed=5)

ALL = [TINY, LLAMA3_8B, MISTRAL_24B, QWEN_32B, LLAMA_70B]
# the Llama-70B layer with a 256K-token host-resident context: its drafting
# and its staging take similar time, the case where staggering two request
# groups can pay off
LLAMA_70B_256K = LLAMA_70B.scaled(name="llama-70b-layer-256k", context=262144)
# the same with one device chunk buffer (device memory for staging scarce):
# one group cannot keep the link busy while it drafts
LLAMA_70B_256K_1BUF = LLAMA_70B_256K.scaled(name="llama-70b-layer-256k-1buf", stage_buffers=1)
BY_NAME = {c.name: c for c in ALL + [LLAMA_70B_256K, LLAMA_70B_256K_1BUF]}
