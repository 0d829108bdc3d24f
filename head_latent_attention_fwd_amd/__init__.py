"""MI355X-native multi-head latent attention (MLA) forward.

The computation lives in ``libmla.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/mla.h``); this package is its Python binding.
"""
from ._lib import (  # noqa: F401
    BIAS_NAMES, BLOCK_NAMES, MLA_BF16, MLA_F32, W_NAMES, BlockWeights, Dims, MLAError, Weights,
    bias_shapes, block_workspace_size, chunk_workspace_size, mla_prefill_chunk_fullcache,
    mla_prefill_chunk_latentcache,
    decode_workspace_size, dense_block_fwd, load, make_dims, mla_decode_fullcache,
    mla_decode_fullcache_ragged, mla_decode_latentcache, mla_decode_latentcache_noalloc,
    mla_decode_latentcache_persistent, mla_decode_latentcache_persistent_status,
    mla_decode_latentcache_ragged, mla_prefill, NOALLOC_SCRATCH_BYTES,
    mla_profile_enable, mla_profile_summary, mla_read_sweep, mla_rope_table, prefill_workspace_size, weight_shapes,
)
