"""MLA chunked prefill over a paged, packed latent cache for MI355X (gfx950).

The compute lives in libmla.so (HIP kernels behind the C ABI of
include/mla.h); this package is its ctypes binding plus the host launch
order of the chunked prefill. Calls raise if the library is not built.
"""
from ._lib import (  # noqa: F401
    ARTIFACT_REASONS, ARTIFACT_VALID, DTYPE_BF16, DTYPE_FP32, DTYPE_FP8_E4M3, EXPORTS, LIB_PATH,
    ROPE_HALF, ROPE_INTERLEAVED, ArtifactMeta, MlaError, load, mla_absorb_out, mla_absorb_q,
    mla_absorbed_attn, mla_artifact_check, mla_cache_append, mla_decompress, mla_gather_context,
    mla_gather_context_fp8_raw,
    mla_head_partition_merge, mla_head_partition_merge_noalloc, mla_merge_states, mla_merge_states_n, mla_merge_states_sets, mla_pack_weight_t, mla_prefill_attn,
    mla_prefill_attn_merge, mla_prefill_attn_2seg, mla_prefill_attn_chunk, mla_rope_relocate_q, mla_token_hash,
    raise_on_device_status,
)
