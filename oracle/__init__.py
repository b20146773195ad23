"""CPU float64 oracle for segment attention — test infrastructure, never on the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. It shares no code with the HIP library.
"""
from .attention import (attend, attention, attention_rows, bf16_to_f64, decode_kv,
                        e4m3fn_to_f64, int8_to_f64, merge_partials, request_slots, split_merge,
                        visible_keys)
from .kv_append import (bf16_bits_to_f32, f32_to_e4m3fn, kv_append, quantize_rows,
                        quantize_rows_int8)
from .linear import linear_attention, linear_attention_closed_form

__all__ = ["attend", "attention", "attention_rows", "bf16_bits_to_f32", "bf16_to_f64", "decode_kv",
           "e4m3fn_to_f64", "f32_to_e4m3fn", "int8_to_f64", "kv_append", "linear_attention",
           "linear_attention_closed_form", "merge_partials",
           "quantize_rows", "quantize_rows_int8",
           "request_slots", "split_merge", "visible_keys"]
