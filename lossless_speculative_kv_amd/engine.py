"""Round driver: device buffers from PyTorch, every step in libvc kernels.

One VeriCache round (VeriCache summary, "Core algorithm"), all launches on
the current stream with no host synchronisation:

  for j in 0..k-1:   embed(x_j) -> q, append k/v to the draft tail
                     vc_draft_decode_attn   (compressed cache)
                     vc_vocab_logits(M=B)   -> x_{j+1}
  embed(x_0..x_k)    -> verify queries and block keys/values
  vc_verify_attn     (full cache; staged from pinned host memory in chunks on
                      a side stream when the cache lives on the host)
  vc_vocab_logits(M=(k+1)B) -> y_1..y_{k+1}
  vc_greedy_accept   -> m, next token (written into row 0 of the token array)
  vc_commit_round    -> full cache grows by m+1 rows; tail / body updated

The synthetic model below attention (embedding of a token, vocab matrix) is
drawn by the device copy of the seeded generator in synth/.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

import synth
import synth.dev as sdev

from . import _lib as L
from .configs import RoundConfig

KIND = {"dense": L.VC_DRAFT_DENSE, "kivi": L.VC_DRAFT_KIVI, "tokdrop": L.VC_DRAFT_TOKDROP}


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _round32(x: int) -> int:
    return (x + 31) // 32 * 32


class Engine:
    """Owns the caches and round buffers of one batch of sequences."""

    def __init__(self, cfg: RoundConfig, rounds_cap: int = 4, device: str = "cuda",
                 stream: "torch.cuda.Stream | None" = None):
        """stream: the compute stream of this engine's calls (default: the
        current stream); set-up work runs on it too."""
        self.dev = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.dev)
        with torch.cuda.stream(self.stream):
            self._setup(cfg, rounds_cap)

    def _setup(self, cfg: RoundConfig, rounds_cap: int):
        self.cfg = c = cfg
        sh = self.shape = L.vc_attn_shape(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim)
        B, Hq, Hkv, D, k = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.k
        self.rounds_cap = rounds_cap
        self.round_idx = 0
        # optional timing: when a list (see prepare_timing), (name, start, end)
        # torch events recorded by the timed calls' own kernel dispatches
        self.events = None
        self._ev_pool = []
        # optional copy tracing (staged caches): when a list, (start, end,
        # bytes) of every chunk copy, events recorded on the copy stream
        self.copy_events = None
        s = self.stream.cuda_stream
        bf = torch.bfloat16

        # synthetic model
        km = synth.outlier_multiplier(c.seed, Hkv, D, c.outliers)
        self.key_mult = torch.from_numpy(km).to(self.dev) if c.outliers else None
        self.W = torch.empty((c.vocab, c.hidden), dtype=bf, device=self.dev)
        sdev.fill_w(c.seed, c.vocab, c.hidden, self.W.data_ptr(), s)

        # full cache (context + room for committed rows)
        self.full_cap = _round32(c.context + rounds_cap * (k + 1))
        self.ctx_len = torch.full((B,), c.context, dtype=torch.int32, device=self.dev)
        if c.staged:
            self._init_staged()
        else:
            self.full_k = torch.empty((B, Hkv, self.full_cap, D), dtype=bf, device=self.dev)
            self.full_v = torch.empty_like(self.full_k)
            self._fill_context(self.full_k, self.full_v, self.full_cap)

        # draft cache
        if c.pipeline and (not c.staged or c.pipeline > k + 1):
            raise ValueError("pipelined drafting needs a staged configuration and at most k + 1 steps")
        # (pipelined drafting appends up to `pipeline` more rows before commit)
        self.tail_cap = _round32(max(c.residual, 0) + rounds_cap * (k + 1) + 32 + c.pipeline)
        self.body_len = torch.zeros((B,), dtype=torch.int32, device=self.dev)
        self.tail_len = torch.zeros((B,), dtype=torch.int32, device=self.dev)
        self.kv = L.vc_draft_kv()
        self.kv.kind = KIND[c.kind]
        self.kv.tail_cap = self.tail_cap
        self.kv.body_len = self.body_len.data_ptr()
        self.kv.tail_len = self.tail_len.data_ptr()
        tail_dtype = torch.float16 if c.kind == "kivi" else bf
        self.tail_k = torch.zeros((B, Hkv, self.tail_cap, D), dtype=tail_dtype, device=self.dev)
        self.tail_v = torch.zeros_like(self.tail_k)
        self.kv.tail_k = self.tail_k.data_ptr()
        self.kv.tail_v = self.tail_v.data_ptr()
        self.dc = L.vc_draft_cache()
        self.dc.kind = self.kv.kind
        self.dc.tail_cap = self.tail_cap
        self.dc.body_len = self.kv.body_len
        self.dc.tail_len = self.kv.tail_len
        self.dc.tail_k = self.kv.tail_k
        self.dc.tail_v = self.kv.tail_v
        self.dc.residual = c.residual
        if c.kind == "kivi":
            self._init_kivi()
        elif c.kind == "tokdrop":
            self._init_tokdrop()
        else:
            if c.staged:
                raise ValueError("the dense draft cache needs the full cache on the device")
            self.kv.body_cap = self.dc.body_cap = self.full_cap
            self.kv.src_k, self.kv.src_v = self.full_k.data_ptr(), self.full_v.data_ptr()
            self.kv.src_t_cap = self.full_cap
            self.body_len.fill_(c.context)

        # round buffers (position-major [k+1][B])
        self.xs = torch.zeros((k + 1, B), dtype=torch.int32, device=self.dev)
        # pipelined drafting: continued drafts s_1..s_J in rows 1..J
        self.xs_spec = torch.zeros((c.pipeline + 1, B), dtype=torch.int32, device=self.dev)
        self.reuse = 0            # leading drafts of the next round already known
        self.reused_drafts = 0    # drafts reused over all rounds
        self.xs[0] = torch.from_numpy(synth.start_tokens(c.seed, B, c.vocab).astype(np.int32)).to(self.dev)
        self.y = torch.zeros((k + 1, B), dtype=torch.int32, device=self.dev)
        self.n_accept = torch.zeros((rounds_cap, B), dtype=torch.int32, device=self.dev)
        self.committed = torch.full((rounds_cap, k + 1, B), -1, dtype=torch.int32, device=self.dev)
        self.status = torch.zeros((B,), dtype=torch.int32, device=self.dev)
        self.q_draft = torch.empty((B, Hq, D), dtype=bf, device=self.dev)
        self.o_draft = torch.empty((B, Hq, D), dtype=torch.float32, device=self.dev)
        self.qv = torch.empty((k + 1, B, Hq, D), dtype=bf, device=self.dev)
        self.kn = torch.empty((k + 1, B, Hkv, D), dtype=bf, device=self.dev)
        self.vn = torch.empty_like(self.kn)
        self.o_ver = torch.empty((k + 1, B, Hq, D), dtype=torch.float32, device=self.dev)

        # workspaces
        # the draft workspace starts with split counters that must be zero
        # before the first call (every call leaves them zero)
        self.ws_draft = self._ws(L.vc_draft_workspace_bytes(sh, self.kv)).zero_()
        max_chunk = c.chunk if c.staged else self.full_cap
        self.ws_verify = self._ws(L.vc_verify_workspace_bytes(sh, k + 1, max_chunk))
        self.ws_vocab_d = self._ws(L.vc_vocab_workspace_bytes(B, c.hidden, c.vocab))
        self.ws_vocab_v = self._ws(L.vc_vocab_workspace_bytes((k + 1) * B, c.hidden, c.vocab))
        self.ws_commit = self._ws(L.vc_commit_workspace_bytes(sh))

    # ---------------------------------------------------------------- setup
    def _ws(self, n: int) -> torch.Tensor:
        return torch.empty((max(n, 256) + 255) // 256 * 256, dtype=torch.uint8, device=self.dev)

    def _fill_context(self, K, V, t_cap):
        c = self.cfg
        s = self.stream.cuda_stream
        sdev.fill_ctx(c.seed, False, c.batch, c.n_kv_heads, c.context, c.head_dim, t_cap, _ptr(self.key_mult),
                      K.data_ptr(), s)
        sdev.fill_ctx(c.seed, True, c.batch, c.n_kv_heads, c.context, c.head_dim, t_cap, None, V.data_ptr(), s)

    def _init_staged(self):
        """Full cache in pinned host memory. The context is drawn on the device,
        copied to the host cache, and kept on the device only until the
        compressed cache has been built from it."""
        c = self.cfg
        B, Hkv, D, T = c.batch, c.n_kv_heads, c.head_dim, c.context
        self.full_k = torch.empty((B, Hkv, self.full_cap, D), dtype=torch.bfloat16, pin_memory=True)
        self.full_v = torch.empty((B, Hkv, self.full_cap, D), dtype=torch.bfloat16, pin_memory=True)
        big_k = torch.empty((B, Hkv, T, D), dtype=torch.bfloat16, device=self.dev)
        big_v = torch.empty_like(big_k)
        s = self.stream.cuda_stream
        sdev.fill_ctx(c.seed, False, B, Hkv, T, D, T, _ptr(self.key_mult), big_k.data_ptr(), s)
        sdev.fill_ctx(c.seed, True, B, Hkv, T, D, T, None, big_v.data_ptr(), s)
        self.full_k[:, :, :T].copy_(big_k)
        self.full_v[:, :, :T].copy_(big_v)
        torch.cuda.synchronize(self.dev)
        self._big = (big_k, big_v)
        nbuf = max(1, c.stage_buffers)
        self.chunk_k = [torch.empty((B, Hkv, c.chunk, D), dtype=torch.bfloat16, device=self.dev) for _ in range(nbuf)]
        self.chunk_v = [torch.empty_like(self.chunk_k[0]) for _ in range(nbuf)]
        self.copy_stream = torch.cuda.Stream(self.dev)
        self._staged_ready = {}

    def _init_kivi(self):
        c = self.cfg
        B, Hkv, D, bits = c.batch, c.n_kv_heads, c.head_dim, c.bits
        n_body = c.context - c.residual
        if n_body < 0 or n_body % 32:
            raise ValueError("context - residual must be a non-negative multiple of 32")
        self.body_cap = _round32(n_body + self.rounds_cap * (c.k + 1) + 32)
        nb = self.body_cap // 32
        dev = self.dev
        rec = L.vc_kivi_block_bytes(D, bits)
        self.kivi_blocks = torch.zeros((B, Hkv, nb, rec), dtype=torch.uint8, device=dev)
        for o in (self.kv, self.dc):
            o.bits = bits
            o.body_cap = self.body_cap
            o.kivi_blocks = self.kivi_blocks.data_ptr()
        if c.staged:
            src_k, src_v = self._big
            t_cap = c.context
        else:
            src_k, src_v, t_cap = self.full_k, self.full_v, self.full_cap
        L.vc_kivi_quantize(self.shape, src_k.data_ptr(), src_v.data_ptr(), t_cap, n_body, c.residual, self.dc,
                           self.stream.cuda_stream)
        if c.staged:
            torch.cuda.synchronize(self.dev)
            del self._big

    def _init_tokdrop(self):
        c = self.cfg
        B, Hkv, T = c.batch, c.n_kv_heads, c.context
        n_keep = int(np.ceil(c.keep * T - 1e-12)) if c.keep < 1.0 else T
        self.n_keep = n_keep
        scores = torch.empty((B, Hkv, T), dtype=torch.float32, device=self.dev)
        sdev.fill_scores(c.seed, B, Hkv, T, scores.data_ptr(), self.stream.cuda_stream)
        self.kept = torch.empty((B, Hkv, max(n_keep, 1)), dtype=torch.int32, device=self.dev)
        L.vc_tokdrop_select(self.shape, scores.data_ptr(), T, n_keep, self.kept.data_ptr(), None, 0,
                            self.stream.cuda_stream)
        self.kv.body_cap = self.dc.body_cap = max(n_keep, 1)
        self.kv.kept_idx = self.kept.data_ptr()
        if self.cfg.staged:
            raise ValueError("token drop gathers from the full cache and needs it on the device")
        self.kv.src_k, self.kv.src_v = self.full_k.data_ptr(), self.full_v.data_ptr()
        self.kv.src_t_cap = self.full_cap
        self.body_len.fill_(n_keep)
        self.scores = scores

    # --------------------------------------------------------------- steps
    def _embed_draft(self, tok_ptr: int, stream: int):
        """Query of the given tokens, and their keys / values appended to the
        draft tail (tail_len grows by one)."""
        c = self.cfg
        sdev.embed_draft(c.seed, tok_ptr, 1, c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim,
                         _ptr(self.key_mult), self.q_draft.data_ptr(), self.tail_k.data_ptr(),
                         self.tail_v.data_ptr(), self.tail_cap, c.kind == "kivi", self.tail_len.data_ptr(), stream)

    def draft_step(self, j: int):
        c = self.cfg
        s = self.stream.cuda_stream
        self._embed_draft(self.xs[j].data_ptr(), s)
        self.draft_attention(j)
        # even steps time the whole call, odd steps the vocab product alone
        name, scope = ("draft_vocab", L.VC_TIME_CALL) if j % 2 == 0 else ("draft_vocab_main", L.VC_TIME_MAIN_KERNEL)
        self._timed(name, lambda: L.vc_vocab_logits(
            c.batch, c.hidden, c.vocab, self.o_draft.data_ptr(), self.W.data_ptr(), self.xs[j + 1].data_ptr(),
            None, None, self.ws_vocab_d.data_ptr(), self.ws_vocab_d.numel(), s), scope)

    def prepare_timing(self, n_calls: int):
        """Create the events of n_calls timed calls before a timed region and
        switch timing on. The events are materialised here (one host record
        each), so inside the region the library records them from its own
        kernel dispatches (vc_time_next_call) and nothing is added to the
        queue."""
        pool = []
        for _ in range(n_calls):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            b.record(self.stream)
            pool.append((a, b))
        torch.cuda.synchronize(self.dev)
        self._ev_pool = pool
        self.events = []

    def _timed(self, name, fn, scope=L.VC_TIME_CALL):
        if self.events is None:
            fn()
            return
        if not self._ev_pool:
            raise RuntimeError("prepare_timing() was given too few calls for this timed region")
        a, b = self._ev_pool.pop()
        L.vc_time_next_call(a.cuda_event, b.cuda_event, scope)
        fn()
        self.events.append((name, a, b))

    def draft_attention(self, j: int = 0):
        # even steps time the whole call (attention kernel + split merge), odd
        # steps the attention kernel alone
        name, scope = ("draft_attn", L.VC_TIME_CALL) if j % 2 == 0 else ("draft_attn_main", L.VC_TIME_MAIN_KERNEL)
        self._timed(name, lambda: L.vc_draft_decode_attn(
            self.shape, self.q_draft.data_ptr(), self.kv, self.o_draft.data_ptr(), self.ws_draft.data_ptr(),
            self.ws_draft.numel(), self.stream.cuda_stream), scope)

    def embed_block(self):
        c = self.cfg
        sdev.embed(c.seed, self.xs.data_ptr(), (c.k + 1) * c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim,
                   _ptr(self.key_mult), self.qv.data_ptr(), self.kn.data_ptr(), self.vn.data_ptr(),
                   self.stream.cuda_stream)

    def verify_attention(self):
        c = self.cfg
        s = self.stream.cuda_stream
        if not c.staged:
            ctx = L.vc_kv_chunk(self.full_k.data_ptr(), self.full_v.data_ptr(), self.full_cap, 0, self.full_cap)
            # even rounds time the whole call, odd rounds the attention kernel alone
            name, scope = (("verify_attn", L.VC_TIME_CALL) if self.round_idx % 2 == 0
                           else ("verify_attn_main", L.VC_TIME_MAIN_KERNEL))
            self._timed(name, lambda: L.vc_verify_attn(
                self.shape, c.k + 1, self.qv.data_ptr(), self.kn.data_ptr(), self.vn.data_ptr(), ctx,
                self.ctx_len.data_ptr(), L.VC_VERIFY_BEGIN | L.VC_VERIFY_END, self.o_ver.data_ptr(),
                self.ws_verify.data_ptr(), self.ws_verify.numel(), s), scope)
            return
        self.verify_staged()

    def stage_plan(self):
        """Chunks covering every position that may hold context this round."""
        c = self.cfg
        upper = min(self.full_cap, c.context + self.round_idx * (c.k + 1))
        return [(t0, min(c.chunk, upper - t0)) for t0 in range(0, upper, c.chunk)]

    def stage_ahead(self):
        """P1 staggering ("P1 cross-resource staggering"): copy the first chunks
        of the host-resident full cache into the device chunk buffers on the
        side stream at the start of the round, so the transfer runs while the
        compute stream drafts (HBM-bound) instead of after it."""
        cs, comp = self.copy_stream, self.stream
        cs.wait_stream(comp)  # the previous round's commit wrote the host cache
        plan = self.stage_plan()
        self._staged_ready = {}
        for i, (t0, n) in enumerate(plan[:len(self.chunk_k)]):
            self._stage_chunk(i, t0, n)

    def _stage_chunk(self, i, t0, n):
        cs = self.copy_stream
        buf = i % len(self.chunk_k)
        tracing = self.copy_events is not None
        if tracing:
            a = torch.cuda.Event(enable_timing=True)
            a.record(cs)
        L.vc_stage_full_kv(self.shape, self.full_k.data_ptr(), self.full_v.data_ptr(), self.full_cap, t0, n,
                           self.chunk_k[buf].data_ptr(), self.chunk_v[buf].data_ptr(), self.cfg.chunk,
                           cs.cuda_stream, None)
        ev = torch.cuda.Event(enable_timing=tracing)
        ev.record(cs)
        if tracing:
            c = self.cfg
            self.copy_events.append((a, ev, 2 * c.batch * c.n_kv_heads * n * c.head_dim * 2))
        self._staged_ready[i] = ev

    def verify_staged(self, after_chunk=None):
        """Stream the host-resident full cache through the device chunk buffers:
        chunks not already staged ahead are copied on the side stream once
        their buffer is free, overlapping the verification of earlier chunks
        on the compute stream. after_chunk(i, n_chunks), if given, enqueues
        more work on the compute stream after chunk i's verification."""
        c = self.cfg
        comp = self.stream
        cs = self.copy_stream
        plan = self.stage_plan()
        nbuf = len(self.chunk_k)
        free = [None] * nbuf
        if not self._staged_ready:
            cs.wait_stream(comp)  # committed rows of the previous round are in host memory
        # timed: from the first chunk's verify kernel start to the last chunk's end
        timing = None
        if self.events is not None:
            if not self._ev_pool:
                raise RuntimeError("prepare_timing() was given too few calls for this timed region")
            timing = self._ev_pool.pop()
            self.events.append(("verify_attn",) + timing)
        for i, (t0, n) in enumerate(plan):
            buf = i % nbuf
            if i not in self._staged_ready:
                if free[buf] is not None:
                    cs.wait_event(free[buf])
                self._stage_chunk(i, t0, n)
            comp.wait_event(self._staged_ready[i])
            flags = (L.VC_VERIFY_BEGIN if i == 0 else 0) | (L.VC_VERIFY_END if i == len(plan) - 1 else 0)
            ctx = L.vc_kv_chunk(self.chunk_k[buf].data_ptr(), self.chunk_v[buf].data_ptr(), c.chunk, t0, n)
            if timing is not None and (i == 0 or i == len(plan) - 1):
                L.vc_time_next_call(timing[0].cuda_event if i == 0 else None,
                                    timing[1].cuda_event if i == len(plan) - 1 else None, L.VC_TIME_CALL)
            L.vc_verify_attn(self.shape, c.k + 1, self.qv.data_ptr(), self.kn.data_ptr(), self.vn.data_ptr(), ctx,
                             self.ctx_len.data_ptr(), flags, self.o_ver.data_ptr(), self.ws_verify.data_ptr(),
                             self.ws_verify.numel(), comp.cuda_stream)
            free[buf] = torch.cuda.Event()
            free[buf].record(comp)
            if after_chunk is not None:
                after_chunk(i, len(plan))
        self._staged_ready = {}

    def verify_vocab(self):
        c = self.cfg
        name, scope = (("verify_vocab", L.VC_TIME_CALL) if self.round_idx % 2 == 0
                       else ("verify_vocab_main", L.VC_TIME_MAIN_KERNEL))
        self._timed(name, lambda: L.vc_vocab_logits(
            (c.k + 1) * c.batch, c.hidden, c.vocab, self.o_ver.data_ptr(), self.W.data_ptr(), self.y.data_ptr(),
            None, None, self.ws_vocab_v.data_ptr(), self.ws_vocab_v.numel(), self.stream.cuda_stream), scope)

    def accept_commit(self):
        c = self.cfg
        r = self.round_idx
        if r >= self.rounds_cap:
            raise RuntimeError("round capacity exhausted; raise rounds_cap")
        s = self.stream.cuda_stream
        na = self.n_accept[r]
        L.vc_greedy_accept(c.batch, c.k, self.xs.data_ptr(), self.y.data_ptr(), na.data_ptr(), self.xs[0].data_ptr(),
                           self.committed[r].data_ptr(), s)
        full_k = self.full_k.data_ptr()
        full_v = self.full_v.data_ptr()
        L.vc_commit_round(self.shape, c.k, na.data_ptr(), self.kn.data_ptr(), self.vn.data_ptr(), full_k, full_v,
                          self.full_cap, self.ctx_len.data_ptr(), self.dc, self.status.data_ptr(),
                          self.ws_commit.data_ptr(), self.ws_commit.numel(), s)
        self.round_idx += 1

    def begin_round(self):
        """Work issued before the draft steps (the staged cache's first chunk copies)."""
        if self.cfg.staged:
            self.stage_ahead()

    def round(self):
        c = self.cfg
        self.begin_round()
        for j in range(c.k):
            if j < self.reuse:
                # x_{j+1} was drafted during the previous verification: only
                # x_j's keys and values join the tail
                self._embed_draft(self.xs[j].data_ptr(), self.stream.cuda_stream)
            else:
                self.draft_step(j)
        self.embed_block()
        if c.pipeline:
            self.verify_staged(after_chunk=self._speculate_between)
        else:
            self.verify_attention()
        self.verify_vocab()
        if c.pipeline:
            # the continued drafts' tail rows are dropped again before commit
            with torch.cuda.stream(self.stream):
                self.tail_len.sub_(c.pipeline)
        self.accept_commit()
        if c.pipeline:
            self.reuse = self.decide_reuse()

    def _speculate_between(self, i: int, n_chunks: int):
        """Pipelined drafting (the drafter keeps writing while the verifier
        fetches the full cache, then is corrected): the drafter continues
        from x_k, s_1 = draft(x_k), s_{i+1} = draft(s_i), for `pipeline`
        steps in all, a share of them after the verification of each chunk
        but the last, on the compute stream. A chunk's verification has then
        released its buffer, and the steps run while the next chunk is still
        crossing the host link. (On a stream of their own they took the
        compute units from the chunk verifications, which delayed the buffer
        releases the copies wait for.) The steps append their inputs to the
        draft tail like any draft step; round() drops those rows before
        commit."""
        c = self.cfg
        parts = max(1, n_chunks - 1)
        if i >= parts:
            return
        lo, hi = i * c.pipeline // parts, (i + 1) * c.pipeline // parts
        s = self.stream.cuda_stream
        for st in range(lo, hi):
            tok_in = self.xs[c.k] if st == 0 else self.xs_spec[st]
            self._embed_draft(tok_in.data_ptr(), s)
            L.vc_draft_decode_attn(self.shape, self.q_draft.data_ptr(), self.kv, self.o_draft.data_ptr(),
                                   self.ws_draft.data_ptr(), self.ws_draft.numel(), s)
            L.vc_vocab_logits(c.batch, c.hidden, c.vocab, self.o_draft.data_ptr(), self.W.data_ptr(),
                              self.xs_spec[st + 1].data_ptr(), None, None, self.ws_vocab_d.data_ptr(),
                              self.ws_vocab_d.numel(), s)

    def decide_reuse(self) -> int:
        """After commit (host synchronisation): when every sequence accepted all
        k drafts and its bonus token y_{k+1} equals the first continued draft
        s_1, the continued drafts s_2..s_J are the drafter's proposals after
        the new pending token, so they become x_1..x_{J-1} of the next round;
        otherwise they are discarded. Returns the number reused. Whatever the
        drafts, verification keeps the committed stream equal to full-cache
        greedy decoding."""
        c = self.cfg
        r = self.round_idx - 1
        with torch.cuda.stream(self.stream):
            ok = bool(((self.n_accept[r] == c.k) & (self.y[c.k] == self.xs_spec[1])).all().item())
            if not ok:
                return 0
            n = min(c.pipeline - 1, c.k)
            if n > 0:
                self.xs[1:n + 1].copy_(self.xs_spec[2:n + 2])
        self.reused_drafts += n
        return n

    def capture_round(self) -> "torch.cuda.CUDAGraph":
        """Capture one whole round (k draft steps with their embeddings and
        vocab projections, the verification pass and its projection, accept
        and commit) into a HIP graph. Every replay runs the next round from
        the device-resident state (tokens, cache lengths, caches) with a
        single launch from the host; nothing in the round reads the host, so
        the replays chain like eager rounds. The accept lengths and committed
        tokens of every replay land in round slot `graph_slot` (the round
        index at capture time). Needs the full cache on the device (staging
        waits on events across streams) and timing switched off."""
        if self.cfg.staged:
            raise ValueError("graph capture needs the full cache on the device")
        if self.events is not None:
            raise ValueError("switch timing off before capturing a round")
        if self.round_idx >= self.rounds_cap:
            raise RuntimeError("round capacity exhausted; raise rounds_cap")
        g = torch.cuda.CUDAGraph()
        saved = self.stream
        slot = self.round_idx
        torch.cuda.synchronize(self.dev)
        try:
            with torch.cuda.graph(g):
                # the capture runs on torch's side stream: every call of the
                # round goes there
                self.stream = torch.cuda.current_stream(self.dev)
                self.round()
        finally:
            self.stream = saved
            self.round_idx = slot + 1
        self.graph_slot = slot
        return g
