"""Shared-base + low-rank KV attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library liblra.so (C ABI in include/lra.h);
this package only marshals arguments to it.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    LRA_BF16,
    LRA_F32,
    LRA_L_KEY_CHUNKED,
    LRA_L_RANK_MAJOR,
    LRA_L_TOKEN_MAJOR,
    LraError,
    load,
    lora_attn_decode,
    lora_attn_decode_noalloc,
    lora_attn_decode_workspace_size,
    lora_attn_prefill,
    lora_attn_prefill_workspace_size,
    lora_attn_varlen,
    lora_attn_varlen_workspace_size,
    lr_cache_build,
    lr_cache_build_multi,
    lr_cache_build_workspace_size,
    lra_last_error,
    lra_version,
)
