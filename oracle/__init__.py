"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .lra_oracle import (  # noqa: F401
    adapter_term,
    attend,
    kv_head_of,
    lora_attention,
    lr_cache_build,
    lr_cache_build_multi,
    materialise_kv,
    rope_angles,
    rope_rotate,
)
