"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .kvc_oracle import (  # noqa: F401
    FLAG_BAD_INDEX, FLAG_CACHE_FULL, append, bf16_to_f64, cache_bytes,
    decode, decode_mla, decode_topk, full_causal, merge_partials,
    mla_cache_bytes, to_f64,
)
