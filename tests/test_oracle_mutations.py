"""The pins have teeth: plant a plausible mistake in the oracle (CPU only,
via monkeypatch) and check that at least one pin fails."""
import numpy as np
import pytest

import oracle
import oracle.accept
import oracle.attention
import oracle.kivi
import oracle.model
import tests.test_oracle_attention as ta
import tests.test_oracle_kivi_tokdrop as tk
import tests.test_oracle_round as tr
import tests.test_oracle_vocab_accept as tv


def _fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def test_missing_scale_is_caught(monkeypatch):
    def bad(q, K, V):
        q, K, V = (np.asarray(x, dtype=np.float64) for x in (q, K, V))
        s = K @ q                        # forgot 1/sqrt(D)
        p = np.exp(s - s.max())
        return (p @ V) / p.sum()
    monkeypatch.setattr(ta, "attend", bad)
    assert _fails(ta.test_matches_torch_sdpa, 64, 64)


def test_off_by_one_causal_block_is_caught(monkeypatch):
    orig = oracle.model.SequenceState.verify

    def bad_verify(self, xs):
        o, hid, lg, y = orig(self, xs)
        # pretend row j saw only block rows 0..j-1: shift predictions by one
        return o, hid, lg, np.concatenate([y[1:], y[-1:]])
    monkeypatch.setattr(oracle.model.SequenceState, "verify", bad_verify)
    assert _fails(tr.test_identity_compressor_accepts_everything, "dense", {})


def test_accept_off_by_one_is_caught(monkeypatch):
    def bad(draft, verify):
        m, nxt, c = oracle.accept.greedy_accept(draft, verify)
        m2 = min(m + 1, len(draft))
        return m2, verify[m2], c
    monkeypatch.setattr(tv, "greedy_accept", bad)
    assert _fails(tv.test_acceptor_exhaustive_small_vocab)


def test_floor_instead_of_round_is_caught(monkeypatch):
    def bad_groups(x, bits, axis, key_scale=False):
        qmax = float((1 << bits) - 1)
        mn = x.min(axis=axis, keepdims=True)
        mx = x.max(axis=axis, keepdims=True)
        raw = (mx - mn) / qmax
        scale = oracle.kivi.round_up_3sig(raw) if key_scale else oracle.kivi.fp16_round(raw)
        zero = oracle.kivi.fp16_round(mn)
        safe = np.where(scale == 0.0, 1.0, scale)
        codes = np.clip(np.floor((x - zero) / safe), 0.0, qmax)
        return codes.astype(np.int64), scale, zero
    monkeypatch.setattr(oracle.kivi, "_quantize_groups", bad_groups)
    assert _fails(tk.test_codes_nearest_level_brute_force, 2)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    orig = oracle.model.SequenceState.draft_step

    def bad_draft(self, x_j):
        # query head h reading KV head h % Hkv instead of h // g
        c = self.cfg
        q, k, v = self.model.embed([x_j])
        self.tail_k = np.concatenate([self.tail_k, k[0][:, None, :]], axis=1)
        self.tail_v = np.concatenate([self.tail_v, v[0][:, None, :]], axis=1)
        o = np.stack([oracle.attention.attend(q[0][h], *self.draft_kv(h % c.n_kv_heads))
                      for h in range(c.n_q_heads)])
        hid, lg = self.model.project(o[None])
        return o, hid[0], lg[0], int(np.argmax(lg[0]))
    monkeypatch.setattr(oracle.model.SequenceState, "draft_step", bad_draft)
    assert _fails(tr.test_identity_compressor_accepts_everything, "dense", {})


def test_flushing_the_newest_rows_is_caught(monkeypatch):
    def bad_flush(self):
        R, G = self.cfg.residual, oracle.kivi.GROUP
        while self.tail_k.shape[1] >= R + G:
            for h in range(self.cfg.n_kv_heads):
                blk = self._quantize_block(h, self.tail_k[h, -G:], self.tail_v[h, -G:])
                bd = self.body[h]
                for key in ("kc", "ks", "kz", "vc", "vs", "vz"):
                    bd[key] = np.concatenate([bd[key], blk[key]])
            self.tail_k = self.tail_k[:, :-G]
            self.tail_v = self.tail_v[:, :-G]
    monkeypatch.setattr(oracle.model.SequenceState, "flush", bad_flush)
    assert _fails(tr.test_kivi_flush_quantises_the_oldest_tail_rows)


def test_key_dequantisation_with_tiled_parameters_is_caught(monkeypatch):
    def bad(codes, scale, zero):
        n = np.asarray(codes).shape[0] // oracle.kivi.GROUP
        return (np.asarray(codes, np.float64) * np.tile(np.asarray(scale), (oracle.kivi.GROUP, 1))[:n * 32]
                + np.tile(np.asarray(zero), (oracle.kivi.GROUP, 1))[:n * 32])
    monkeypatch.setattr(tk, "dequantize_keys", bad)
    assert _fails(tk.test_key_roundtrip_error_bound, 2)
