"""CPU oracle (test infrastructure only; see cacheblend_oracle's header)."""
from .cacheblend_oracle import (rope_theta, rope_rotate, rmsnorm, silu, attention,
                                qkv_rows, finish_rows, prefill, schedule,
                                kv_deviation, topk_select, rerotate_chunks, blend,
                                kv_size_bytes, check_offsets, quantize_channels,
                                dequantize_channels, pack_codes, unpack_codes, load_time,
                                controller_ratio, lru_replay, lm_head, argmax_first,
                                decode_step, spearman, layer_rank_correlation,
                                attention_probs, attention_deviation)

__all__ = ["rope_theta", "rope_rotate", "rmsnorm", "silu", "attention", "qkv_rows",
           "finish_rows", "prefill", "schedule", "kv_deviation", "topk_select",
           "rerotate_chunks", "blend", "kv_size_bytes", "check_offsets",
           "quantize_channels", "dequantize_channels", "pack_codes", "unpack_codes",
           "load_time", "controller_ratio", "lru_replay", "lm_head", "argmax_first",
           "decode_step", "spearman", "layer_rank_correlation",
           "attention_probs", "attention_deviation"]
