"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .kvc_oracle import (  # noqa: F401
    FLAG_BAD_INDEX, FLAG_CACHE_FULL, FP8_E4M3_MAX, append, append_fp8,
    append_paged, bf16_to_f64, cache_bytes, decode, decode_fp8, decode_mla,
    decode_paged, decode_topk, paged_rows, paged_waste_fraction,
    decode_window, topk_select, f64_to_fp8_e4m3, fp8_e4m3_to_f64, full_causal,
    FP4_BLOCK, FP4_E2M1_MAX, append_fp4, decode_fp4, dequantize_fp4, f64_to_fp4_e2m1,
    fp4_e2m1_to_f64, quantize_fp4,
    merge_partials, mla_cache_bytes, quantize_fp8, to_f64, window_range,
)
