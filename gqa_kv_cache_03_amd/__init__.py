"""MI355X (gfx950) grouped-query-attention decode: HIP kernels behind a C ABI.

    from gqa_kv_cache_03_amd import gqa_decode
    out = gqa_decode(q, k_cache, v_cache, seq_lens)            # contiguous cache
    out = gqa_decode(q, pool_k, pool_v, seq_lens, block_table)  # paged cache
    out = gqa_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens)  # append + decode
    out = gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, out=out)  # no workspace
    out = gqla_absorb_decode(q, latent, w_uk, w_uv, seq_lens)  # GQLA, absorbed form
"""
from .ops import gqa_decode, gqa_decode_append, gqa_decode_noalloc, plan, workspace_bytes, read_stream  # noqa: F401
from .ops import gqla_absorb_decode, gqla_absorb_decode_append, gqla_plan, check_inputs  # noqa: F401
from ._lib import GqaError, LIB_PATH  # noqa: F401
