"""CPU oracle for GQA decode and the GQLA latent path. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python binding)
never calls it, and it never calls the product path.
"""
from .gqa_oracle import (  # noqa: F401
    bf16_bits_to_float64,
    group_of_head,
    heads_of_group,
    visible_keys,
    kv_rows,
    gqa_decode,
    append_kv,
    kv_bytes,
    touched_kv_rows,
)
from .gqla_oracle import (  # noqa: F401
    latent_rows,
    expand_cache,
    gqla_decode,
    append_latent,
    latent_bytes,
    touched_latent_rows,
)
