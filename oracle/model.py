"""The synthetic one-layer model and the VeriCache round, in fp64.

VeriCache summary, "Core algorithm": (1) drafting - the same target model
produces a run of candidate tokens x using the compressed cache KV_comp;
(2) verification - one forward pass over the full cache KV_full checks the
drafted tokens in parallel; (3) acceptance - tokens are accepted up to the
first mismatch, plus a bonus token when all match, and decoding restarts
from the last accepted token. "Experimental results": the output equals
full-cache greedy decoding.

Synthetic model (stand-in for weights and datasets the pages do not give):
a token t has q, k, v = synth.embed(t) (per head, bf16 values); the hidden
vector is the attention output rounded to bf16, flattened head-major; the
next token is the first-index argmax of hidden . W^T. Query head h reads KV
head h // g (g = Hq / Hkv, contiguous groups).

Round with draft length k, for one sequence with pending token x_0:
  draft step j = 0..k-1: append k/v of x_j to the draft tail, attend over the
      draft-visible set, x_{j+1} = argmax;
  verify: rows j = 0..k with queries of x_0..x_k; row j sees the full
      context and block rows 0..j; y_{j+1} = argmax of row j;
  accept: m = first j with x_{j+1} != y_{j+1} (else k); commit x_1..x_m and
      y_{m+1}; the KV rows of x_0..x_m join the full context; the draft tail
      keeps x_0..x_m; the new pending token is y_{m+1};
  KIVI only: while the tail holds at least R + 32 tokens, its oldest 32
      tokens are quantised into the body (one key group, 32 value rows).

Draft-visible set: KIVI - dequantised body plus tail; token drop - kept
context tokens plus tail; dense (identity compressor) - the whole initial
context plus tail.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

import synth
from . import attention, kivi, tokdrop, vocab
from .accept import greedy_accept


@dataclasses.dataclass
class ModelConfig:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int
    vocab: int
    k: int
    kind: str = "kivi"          # "kivi" | "tokdrop" | "dense"
    bits: int = 2
    residual: int = 32          # KIVI recent-token window R (T - R must be a multiple of 32)
    keep: float = 0.25          # token-drop keep ratio
    outliers: bool = False      # x8 key outliers on 4 channels per KV head
    seed: int = 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def hidden(self) -> int:
        return self.n_q_heads * self.head_dim


class SynthModel:
    """Synthetic weights: embedding via ``synth`` and the vocab matrix W."""

    def __init__(self, cfg: ModelConfig, W: np.ndarray | None = None):
        self.cfg = cfg
        self.key_mult = synth.outlier_multiplier(cfg.seed, cfg.n_kv_heads, cfg.head_dim, cfg.outliers)
        self.W = W if W is not None else synth.w_vocab_rows(cfg.seed, 0, cfg.vocab, cfg.hidden).astype(np.float64)

    def embed(self, tokens):
        c = self.cfg
        q, k, v = synth.embed(c.seed, tokens, c.n_q_heads, c.n_kv_heads, c.head_dim, self.key_mult)
        return q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)

    def project(self, o_rows):
        """o_rows: [M][Hq][D] attention outputs -> (bf16 hidden [M][H], logits [M][V])."""
        h = vocab.to_bf16(np.asarray(o_rows).reshape(len(o_rows), -1))
        return h, vocab.logits(h, self.W)


def attend_heads(cfg: ModelConfig, q, K, V):
    """q [Hq][D]; K, V [Hkv][T][D] -> o [Hq][D] (each q head over its KV head)."""
    g = cfg.group
    return np.stack([attention.attend(q[h], K[h // g], V[h // g]) for h in range(cfg.n_q_heads)])


class SequenceState:
    """Full cache, draft cache and pending token of one sequence (fp64 values)."""

    def __init__(self, model: SynthModel, b: int, x0: int):
        c = model.cfg
        self.model, self.b, self.cfg = model, b, c
        T = c.context
        self.k_full = np.stack([synth.ctx_kv(c.seed, "k", b, h, 0, T, c.head_dim, model.key_mult)
                                for h in range(c.n_kv_heads)]).astype(np.float64)
        self.v_full = np.stack([synth.ctx_kv(c.seed, "v", b, h, 0, T, c.head_dim)
                                for h in range(c.n_kv_heads)]).astype(np.float64)
        self.x0 = int(x0)
        Hkv, D = c.n_kv_heads, c.head_dim
        if c.kind == "kivi":
            n_body = T - c.residual
            if n_body < 0 or n_body % kivi.GROUP:
                raise ValueError("context - residual must be a non-negative multiple of 32")
            self.body = [self._quantize_block(h, self.k_full[h, :n_body], self.v_full[h, :n_body])
                         for h in range(Hkv)]
            self.tail_k = self.k_full[:, n_body:].copy()
            self.tail_v = self.v_full[:, n_body:].copy()
        elif c.kind == "tokdrop":
            self.kept = [tokdrop.select_kept(synth.scores(c.seed, b, h, 0, T), c.keep) for h in range(Hkv)]
            self.tail_k = np.zeros((Hkv, 0, D))
            self.tail_v = np.zeros((Hkv, 0, D))
        elif c.kind == "dense":
            self.n_dense = T
            self.tail_k = np.zeros((Hkv, 0, D))
            self.tail_v = np.zeros((Hkv, 0, D))
        else:
            raise ValueError(c.kind)

    # -- KIVI body: list per KV head of dicts with codes and parameters --
    def _quantize_block(self, h, K, V):
        b = self.cfg.bits
        kc, ks, kz = kivi.quantize_keys(K, b)
        vc, vs, vz = kivi.quantize_values(V, b)
        return {"kc": kc, "ks": ks, "kz": kz, "vc": vc, "vs": vs, "vz": vz}

    def body_len(self) -> int:
        return self.body[0]["kc"].shape[0] if self.cfg.kind == "kivi" else 0

    def draft_kv(self, h):
        """(K, V) of the draft-visible set of KV head h, in attention order."""
        c = self.cfg
        if c.kind == "kivi":
            bd = self.body[h]
            K = np.concatenate([kivi.dequantize_keys(bd["kc"], bd["ks"], bd["kz"]), self.tail_k[h]])
            V = np.concatenate([kivi.dequantize_values(bd["vc"], bd["vs"], bd["vz"]), self.tail_v[h]])
        elif c.kind == "tokdrop":
            idx = self.kept[h]
            K = np.concatenate([self.k_full[h, idx], self.tail_k[h]])
            V = np.concatenate([self.v_full[h, idx], self.tail_v[h]])
        else:
            K = np.concatenate([self.k_full[h, :self.n_dense], self.tail_k[h]])
            V = np.concatenate([self.v_full[h, :self.n_dense], self.tail_v[h]])
        return K, V

    # -- the three steps --
    def draft_step(self, x_j: int):
        """Append x_j to the tail, attend over the draft set.

        Returns (o [Hq][D], hidden bf16 [H], logits [V], argmax)."""
        q, k, v = self.model.embed([x_j])
        self.tail_k = np.concatenate([self.tail_k, k[0][:, None, :]], axis=1)
        self.tail_v = np.concatenate([self.tail_v, v[0][:, None, :]], axis=1)
        g = self.cfg.group
        o = np.stack([attention.attend(q[0][h], *self.draft_kv(h // g)) for h in range(self.cfg.n_q_heads)])
        hid, lg = self.model.project(o[None])
        return o, hid[0], lg[0], int(vocab.argmax_first(lg[0]))

    def verify(self, xs):
        """xs = x_0..x_k. Returns (o [k+1][Hq][D], hidden, logits [k+1][V], y [k+1])."""
        q, k, v = self.model.embed(list(xs))
        n = len(xs)
        g = self.cfg.group
        T = self.k_full.shape[1]
        o = np.empty((n, self.cfg.n_q_heads, self.cfg.head_dim))
        for j in range(n):
            for h in range(self.cfg.n_q_heads):
                hk = h // g
                K = np.concatenate([self.k_full[hk, :T], k[:j + 1, hk]])
                V = np.concatenate([self.v_full[hk, :T], v[:j + 1, hk]])
                o[j, h] = attention.attend(q[j, h], K, V)
        hid, lg = self.model.project(o)
        return o, hid, lg, vocab.argmax_first(lg)

    def commit(self, xs, m: int, tail_start: int, next_token: int):
        """Apply an accepted round: context gains x_0..x_m; the tail keeps
        its round-start part plus x_0..x_m; pending token <- next_token."""
        _, k, v = self.model.embed(list(xs[:m + 1]))
        self.k_full = np.concatenate([self.k_full, k.transpose(1, 0, 2)], axis=1)
        self.v_full = np.concatenate([self.v_full, v.transpose(1, 0, 2)], axis=1)
        self.tail_k = np.concatenate([self.tail_k[:, :tail_start], k.transpose(1, 0, 2)], axis=1)
        self.tail_v = np.concatenate([self.tail_v[:, :tail_start], v.transpose(1, 0, 2)], axis=1)
        if self.cfg.kind == "kivi":
            self.flush()
        elif self.cfg.kind == "dense":
            # identity compressor: the drafter's cache is the whole committed context
            self.n_dense = self.k_full.shape[1]
            self.tail_k = self.tail_k[:, :0]
            self.tail_v = self.tail_v[:, :0]
        self.x0 = int(next_token)

    def flush(self):
        R = self.cfg.residual
        while self.tail_k.shape[1] >= R + kivi.GROUP:
            G = kivi.GROUP
            for h in range(self.cfg.n_kv_heads):
                blk = self._quantize_block(h, self.tail_k[h, :G], self.tail_v[h, :G])
                bd = self.body[h]
                for key in ("kc", "ks", "kz", "vc", "vs", "vz"):
                    bd[key] = np.concatenate([bd[key], blk[key]])
            self.tail_k = self.tail_k[:, G:]
            self.tail_v = self.tail_v[:, G:]

    def run_round(self, forced_drafts=None):
        """One round. Returns dict(x=[x_0..x_k], y=[y_1..y_{k+1}], m, committed).

        forced_drafts: optional list of k tokens overriding the drafted
        x_1..x_k (teacher forcing / planted mismatches); the draft steps still
        run so the tail is built exactly as the drafter would."""
        kd = self.cfg.k
        tail_start = self.tail_k.shape[1]
        xs = [self.x0]
        for j in range(kd):
            _, _, _, nxt = self.draft_step(xs[j])
            xs.append(int(forced_drafts[j]) if forced_drafts is not None else nxt)
        _, _, _, y = self.verify(xs)
        m, nxt, committed = greedy_accept(xs[1:], y)
        self.commit(xs, m, tail_start, nxt)
        return {"x": xs, "y": [int(t) for t in y], "m": m, "committed": committed}


def make_states(cfg: ModelConfig, W: np.ndarray | None = None):
    model = SynthModel(cfg, W)
    x0 = synth.start_tokens(cfg.seed, cfg.batch, cfg.vocab)
    return model, [SequenceState(model, b, int(x0[b])) for b in range(cfg.batch)]


def full_kv_greedy(cfg: ModelConfig, b: int, n_tokens: int, model: SynthModel | None = None):
    """Plain greedy decoding with the full cache: the stream VeriCache must equal.

    Starting from the pending start token x_0, each step appends its k/v to
    the context and emits the argmax over that context; returns the emitted
    tokens in order."""
    model = model or SynthModel(cfg)
    c = cfg
    T = c.context
    K = np.stack([synth.ctx_kv(c.seed, "k", b, h, 0, T, c.head_dim, model.key_mult)
                  for h in range(c.n_kv_heads)]).astype(np.float64)
    V = np.stack([synth.ctx_kv(c.seed, "v", b, h, 0, T, c.head_dim)
                  for h in range(c.n_kv_heads)]).astype(np.float64)
    x = int(synth.start_tokens(c.seed, c.batch, c.vocab)[b])
    out = []
    for _ in range(n_tokens):
        q, k, v = model.embed([x])
        K = np.concatenate([K, k[0][:, None, :]], axis=1)
        V = np.concatenate([V, v[0][:, None, :]], axis=1)
        o = attend_heads(c, q[0], K, V)
        _, lg = model.project(o[None])
        x = int(vocab.argmax_first(lg[0]))
        out.append(x)
    return out
