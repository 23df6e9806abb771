"""Float64 CPU oracle of the DSA decode step -- test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py``; never by the library.
"""
from .dsa_oracle import (  # noqa: F401
    e4m3fn_decode, bf16_decode, row_extents, token_location, indexer_keys,
    indexer_logits, topk_row, topk, sparse_mla, sparse_mla_split, MASK_SENTINEL,
    E4M3_MAX, e4m3fn_encode, quantize_groups_fp8, indexer_q_quant, indexer_k_quant_and_cache,
    latent_cache_write, KV8_ROW_BYTES, KV8_SCALE_OFFSET, KV8_PAGE_BYTES, latent_cache_write_fp8, kv8_rows,
)
