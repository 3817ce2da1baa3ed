"""DSA decode hot path for MI355X (gfx950): lightning indexer, top-k and
sparse absorbed-MLA decode behind a C ABI (include/dsa.h, libdsa.so).

The Python names mirror the C entry points and only marshal arguments.
"""
from .binding import (  # noqa: F401
    DSA_MODE_FUSED, DSA_MODE_MLI, DSA_NUM_STAGES, DSA_OP_DECODE_STEP, DSA_OP_DENSE_MLA, DSA_OP_SPARSE_MLA, DSA_OP_TOPK, DSA_STAGE_ATTENTION,
    DSA_IDX_LOGICAL, DSA_IDX_PAGED, DSA_IDX_RAGGED, DSA_STAGE_INDEX_SCORE, DSA_STAGE_TOPK, EXPORTS,
    Batch, DsaError, dsa_cache_append, dsa_decode_layers, dsa_decode_step, dsa_decode_step_noalloc,
    dsa_dense_mla_decode, dsa_default_splits, dsa_index_score, dsa_sparse_mla_decode,
    dsa_sparse_mla_decode_paged, dsa_topk, dsa_topk_transform, dsa_workspace_size, lib,
    dsa_device_check, dsa_device_checks_enabled, DSA_CHECK_INDEX, DSA_CHECK_METADATA,
    DSA_CHECK_NAN_SCORE, DSA_CHECK_PAGE_ID, DSA_ERR_DEVICE_CHECK, checked,
    DSA_OP_MASKED_MHA, dsa_masked_mha_prefill)
