"""CPU oracle for the VeriCache draft/verify hot path.

TEST INFRASTRUCTURE. This package is the plain, slow, fp64 statement of what
the GPU path computes, written from the VeriCache technical summary ("VeriCache:
Turning Lossy KV Cache into Lossless LLM Inference", section "Core algorithm":
drafting with the compressed cache, one verification pass with the full
cache, acceptance up to the first mismatch plus a bonus token) and from the
plain definitions of softmax attention, min/max quantisation and top-k
selection. Only the test suite, the smoke entry point and the CPU-baseline
leg of the benchmark may import it; the GPU library never does, and the two
share no code: the only common module is ``synth`` (seeded inputs).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, brute force, a library routine, or the method's own
invariants (identity compressor => all drafts accepted; the committed
stream equals full-cache greedy decoding). Parity unpinned: nothing here
has absolute throughput or acceptance values to check against, because
the pages print none.
"""
from .attention import attend, attend_masked, attend_prefix
from .kivi import (quantize_keys, quantize_values, dequantize_keys, dequantize_values,
                   pack_key_codes, pack_value_codes, pack_value_side, unpack_key_codes,
                   unpack_value_codes, unpack_value_side, fp16_round, value_slot_token, pack_blocks,
                   unpack_blocks, record_bytes, record_offsets, key_side_channel, pack_key_side, unpack_key_side)
from .tokdrop import select_kept
from .vocab import to_bf16, logits, argmax_first, tie_bound
from .accept import greedy_accept

__all__ = [
    "attend", "attend_masked", "attend_prefix", "quantize_keys", "quantize_values", "dequantize_keys",
    "dequantize_values", "pack_key_codes", "pack_value_codes", "pack_value_side",
    "unpack_key_codes", "unpack_value_codes", "unpack_value_side", "fp16_round", "pack_blocks", "unpack_blocks",
    "record_bytes", "record_offsets", "key_side_channel", "pack_key_side", "unpack_key_side",
    "value_slot_token", "select_kept", "to_bf16", "logits", "argmax_first", "tie_bound",
    "greedy_accept",
]
