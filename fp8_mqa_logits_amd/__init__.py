"""fp8 MQA indexer (logits + top-k) for AMD Instinct MI355X (gfx950).

The computation lives in libfp8idx.so (HIP kernels behind the C ABI of
include/fp8idx.h); this package is its Python binding.  Importing it does
not load the library; the first call does, and raises if it is not built.
"""

from .binding import (  # noqa: F401
    Fp8idxError,
    TopkMap,
    MAP_NONE,
    MAP_TOKEN_TABLE,
    MAP_BLOCK_TABLE,
    OP_TOPK,
    OP_LOGITS_TOPK_RAGGED,
    OP_LOGITS_TOPK_RAGGED_OVERLAP,
    OP_LOGITS_RAGGED,
    ENTRY_LOGITS_RAGGED,
    ENTRY_LOGITS_PAGED,
    ENTRY_TOPK,
    ENTRY_LOGITS_TOPK_RAGGED,
    ENTRY_LOGITS_TOPK_RAGGED_OVERLAP,
    ENTRY_LOGITS_TOPK_PAGED,
    CallArgs,
    fp8idx_validate_only,
    LIB_PATH,
    load_library,
    indexer_logits_ragged,
    indexer_logits_ragged_noalloc,
    indexer_logits_paged,
    indexer_topk,
    indexer_logits_topk_ragged,
    indexer_logits_topk_ragged_overlap,
    indexer_logits_topk_paged,
    indexer_quant_fp8,
    indexer_prepare_ragged,
    indexer_prepare_decode,
    indexer_sparse_mla,
    fp8idx_sparse_mla_workspace_bytes,
    MLA_DQK,
    MLA_DV,
    fp8idx_workspace_bytes,
    fp8idx_workspace_bytes_paged,
    fp8idx_rows_per_chunk,
    fp8idx_version,
    fp8idx_probe_mfma_fp8,
    fp8idx_probe_logits_core,
)
