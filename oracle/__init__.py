"""CPU fp64 oracle for DiT sequence-parallel attention (test infrastructure).

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg
may import this package.  The HIP library and its Python binding never do.
"""
from .ref import (attention, attention_rows, probabilities, split_kv, merge,
                  attention_backward, attention_backward_rows, attention_backward_keys,
                  ring_attention, shard_tokens, seq2head, head2seq,
                  unshard_tokens, ulysses_attention, ulysses_send_bytes_per_rank,
                  default_scale, rope, round_bf16, joint_sequence,
                  joint_attention, E4M3_MAX, e4m3_decode, e4m3_round, e4m3_encode,
                  quantize_fp8, attention_fp8, LOG2E_F32, pow2_descale, quantize_fp8_mx,
                  attention_fp8_mx)

__all__ = ["attention", "attention_rows", "probabilities", "split_kv", "merge",
           "attention_backward", "attention_backward_rows", "attention_backward_keys",
           "ring_attention", "shard_tokens", "seq2head", "head2seq",
           "unshard_tokens", "ulysses_attention", "ulysses_send_bytes_per_rank",
           "default_scale", "rope", "round_bf16", "joint_sequence",
           "joint_attention", "E4M3_MAX", "e4m3_decode", "e4m3_round", "e4m3_encode",
           "quantize_fp8", "attention_fp8", "LOG2E_F32", "pow2_descale", "quantize_fp8_mx",
           "attention_fp8_mx"]
