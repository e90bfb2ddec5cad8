"""CPU float64 oracle for paged attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package; the HIP library never does, and the two share no
code.
"""
from .paged_attention import (NEG_INF, attend, bf16_to_f32, bf16_to_f64, combine, decode,
                              dequantize_int8, empty_pool, gather, kv_write, paged_attention,
                              quantize_int8, slot_of, smoothing_factors, split_partials, visible_mask)

from .tq3 import (codebook_f32, dequantize_tq3, fwht_f32, lloyd_max_normal, pack_codes,
                  quantize_tq3, sum_squares_f32, unpack_codes)

from .attn_input import (attention_input, attention_input_to_pool, f32_to_bf16, rms_norm_bf16,
                         rope_bf16, token_positions)

__all__ = ["attention_input", "attention_input_to_pool", "f32_to_bf16", "rms_norm_bf16", "rope_bf16",
           "token_positions", "NEG_INF", "attend", "bf16_to_f32", "bf16_to_f64", "combine", "decode",
           "dequantize_int8", "empty_pool", "gather", "kv_write", "paged_attention",
           "quantize_int8", "slot_of", "smoothing_factors", "split_partials", "visible_mask", "codebook_f32",
           "dequantize_tq3", "fwht_f32", "lloyd_max_normal", "pack_codes", "quantize_tq3",
           "sum_squares_f32", "unpack_codes"]
