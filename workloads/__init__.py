"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path."""
from .gen import (  # noqa: F401
    MLA_DIMS,
    Dims,
    PrefillWorkload,
    DecodeWorkload,
    make_prefill,
    make_decode,
    prefill_recipe,
    prefill_recipe_lengths,
    decode_recipe,
    PREFILL_RECIPES,
    DECODE_RECIPES,
    f32_to_bf16_bits,
    f32_to_e4m3fn_codes,
)
