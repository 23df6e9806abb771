"""libdsa: DeepSeek-Sparse-Attention decode hot path for MI355X (gfx950).

The compute is in hand-written HIP kernels behind the C ABI of
``include/dsa.h``; this package is only the Python binding (argument
marshalling through ctypes) plus the synthetic-workload generator.
"""
from .binding import (  # noqa: F401
    DSAError, load, library_path, indexer_logits_paged, indexer_logits_prefill, topk,
    sparse_mla_decode, topk_workspace_bytes, sparse_mla_workspace_bytes, sparse_mla_pick_splits,
    indexer_q_quant_fp8, indexer_k_quant_and_cache, latent_cache_write, sparse_mla_decode_fp8,
    latent_cache_write_fp8, sparse_mla_decode_noalloc, Batch,
)
