// The C ABI of libdsa (include/dsa.h): host-side argument checks, status
// strings, workspace sizing and kernel dispatch.  Nothing here synchronises or
// allocates; every call only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.h"
#include "dsa.h"
#include "kernels.h"

namespace {

// MI355X has 256 compute units; the split heuristic and grid sizes are tuned
// for it and depend on host fields only, so workspace queries need no GPU.
constexpr int kTargetCUs = 256;

// Largest row / token count one quantiser or cache-writer call takes (keeps
// every grid far inside the 2^31 workgroup limit).
constexpr int kMaxWriteItems = DSA_MAX_WRITE_ITEMS;

// The fp8 sparse MLA keeps a token's cache slot (page * 64 + slot) in 32 bits.
constexpr int kMaxKv8Pages = 1 << 25;

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_batch(const dsa_batch_t* b) {
  if (!b) return fail(DSA_ERR_NULL, "batch is NULL");
  if (b->num_seqs < 0 || b->num_seqs > DSA_MAX_SEQS)
    return fail(DSA_ERR_UNSUPPORTED, "num_seqs=%d outside [0, %d]", b->num_seqs, DSA_MAX_SEQS);
  if (b->num_rows < 0) return fail(DSA_ERR_INVALID, "num_rows=%d < 0", b->num_rows);
  if (b->max_seq_len < 0) return fail(DSA_ERR_INVALID, "max_seq_len=%d < 0", b->max_seq_len);
  if (b->max_q_len < 0) return fail(DSA_ERR_INVALID, "max_q_len=%d < 0", b->max_q_len);
  if (b->num_pages < 0) return fail(DSA_ERR_INVALID, "num_pages=%d < 0", b->num_pages);
  if (b->bt_stride < 0 || (int64_t)b->bt_stride < ceil_div(b->max_seq_len, DSA_PAGE_SIZE))
    return fail(DSA_ERR_INVALID, "bt_stride=%d < ceil(max_seq_len=%d / 64)", b->bt_stride, b->max_seq_len);
  if (b->num_seqs > 0) {
    if (!b->seq_lens) return fail(DSA_ERR_NULL, "seq_lens is NULL");
    if (!b->query_start) return fail(DSA_ERR_NULL, "query_start is NULL");
    if (b->max_seq_len > 0 && !b->block_table) return fail(DSA_ERR_NULL, "block_table is NULL");
  }
  return DSA_OK;
}

dsa::BatchArgs to_args(const dsa_batch_t* b) {
  dsa::BatchArgs a{};
  a.num_seqs = b->num_seqs;
  a.num_rows = b->num_rows;
  a.max_seq_len = b->max_seq_len;
  a.max_q_len = b->max_q_len;
  a.bt_stride = b->bt_stride;
  a.num_pages = b->num_pages;
  a.seq_lens = b->seq_lens;
  a.query_start = b->query_start;
  a.block_table = b->block_table;
  return a;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_indexer(const dsa_batch_t* batch, const uint8_t* q, const float* w, const uint8_t* cache,
                  int64_t page_stride, float* logits, int64_t logits_stride, int clean) {
  int st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (page_stride < DSA_INDEXER_PAGE_BYTES || page_stride % 16 != 0)
    return fail(DSA_ERR_INVALID, "idx_page_stride=%lld must be >= 8448 and a multiple of 16", (long long)page_stride);
  if (logits_stride < batch->max_seq_len || logits_stride < 1 || logits_stride % 4 != 0)
    return fail(DSA_ERR_INVALID, "logits_stride=%lld must be >= max_seq_len=%d, >= 1 and a multiple of 4",
                (long long)logits_stride, batch->max_seq_len);
  if (clean != 0 && clean != 1) return fail(DSA_ERR_INVALID, "clean_logits=%d must be 0 or 1", clean);
  if (batch->num_rows > 0) {
    if (!q || !w || !logits) return fail(DSA_ERR_NULL, "q_fp8, weights and logits must not be NULL");
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(logits, 16))
      return fail(DSA_ERR_INVALID, "q_fp8, weights and logits must be 16-byte aligned");
    if (batch->max_seq_len > 0 && batch->num_pages > 0) {
      if (!cache) return fail(DSA_ERR_NULL, "idx_cache is NULL");
      if (!aligned(cache, 16)) return fail(DSA_ERR_INVALID, "idx_cache must be 16-byte aligned");
    }
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_INVALID: return "DSA_ERR_INVALID: a size, stride or alignment is out of contract";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape not supported by this build";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: the HIP runtime rejected a launch";
    default: return "unknown dsa_status";
  }
}

const char* dsa_last_error_message(void) { return g_last_error.c_str(); }

const char* dsa_version(void) { return "libdsa 0.1.0 gfx950"; }

int dsa_indexer_logits_paged(const dsa_batch_t* batch, const uint8_t* q_fp8, const float* weights,
                             const uint8_t* idx_cache, int64_t idx_page_stride, float* logits,
                             int64_t logits_stride, int clean_logits, void* stream) {
  int st = check_indexer(batch, q_fp8, weights, idx_cache, idx_page_stride, logits, logits_stride, clean_logits);
  if (st != DSA_OK) return st;
  if (batch->num_rows == 0) return ok();
  return hip_status(dsa::launch_indexer_paged(to_args(batch), q_fp8, weights, idx_cache, idx_page_stride, logits,
                                              logits_stride, clean_logits, kTargetCUs, (hipStream_t)stream),
                    "dsa_indexer_logits_paged launch");
}

int dsa_indexer_logits_prefill(const dsa_batch_t* batch, const uint8_t* q_fp8, const float* weights,
                               const uint8_t* idx_cache, int64_t idx_page_stride, float* logits,
                               int64_t logits_stride, int clean_logits, void* stream) {
  int st = check_indexer(batch, q_fp8, weights, idx_cache, idx_page_stride, logits, logits_stride, clean_logits);
  if (st != DSA_OK) return st;
  if (batch->num_rows == 0) return ok();
  return hip_status(dsa::launch_indexer_prefill(to_args(batch), q_fp8, weights, idx_cache, idx_page_stride, logits,
                                                logits_stride, clean_logits, kTargetCUs, (hipStream_t)stream),
                    "dsa_indexer_logits_prefill launch");
}

size_t dsa_topk_workspace_bytes(const dsa_batch_t* batch, int32_t k) {
  if (!batch || k < 1 || k > DSA_MAX_TOPK || batch->num_rows <= 0 || batch->max_seq_len <= 0) return 0;
  return dsa::topk_workspace_bytes(batch->num_rows, batch->max_seq_len, k);
}

int dsa_topk(const dsa_batch_t* batch, const float* logits, int64_t logits_stride, int32_t k, int32_t* indices,
             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k=%d outside [1, %d]", k, DSA_MAX_TOPK);
  if (logits_stride < batch->max_seq_len || logits_stride < 1 || logits_stride % 4 != 0)
    return fail(DSA_ERR_INVALID, "logits_stride=%lld must be >= max_seq_len=%d, >= 1 and a multiple of 4",
                (long long)logits_stride, batch->max_seq_len);
  if ((int64_t)batch->max_seq_len > dsa::topk_max_seq_len(k))
    return fail(DSA_ERR_UNSUPPORTED, "max_seq_len=%d exceeds the %lld keys per row dsa_topk handles for k=%d",
                batch->max_seq_len, (long long)dsa::topk_max_seq_len(k), k);
  if (batch->num_rows == 0) return ok();
  if (!logits || !indices) return fail(DSA_ERR_NULL, "logits and indices must not be NULL");
  if (!aligned(logits, 16)) return fail(DSA_ERR_INVALID, "logits must be 16-byte aligned");
  if (!aligned(indices, 4)) return fail(DSA_ERR_INVALID, "indices must be 4-byte aligned");
  const size_t need = dsa_topk_workspace_bytes(batch, k);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "dsa_topk needs %zu workspace bytes, got %zu", need, workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  return hip_status(dsa::launch_topk(to_args(batch), logits, logits_stride, k, indices, workspace, (hipStream_t)stream),
                    "dsa_topk launch");
}

static bool heads_supported(int32_t H) { return H >= 16 && H <= 1024 && H % 16 == 0; }

int32_t dsa_sparse_mla_pick_splits(const dsa_batch_t* batch, int32_t num_heads, int32_t k) {
  if (!batch || !heads_supported(num_heads) || k < 1 || k > DSA_MAX_TOPK) return 1;
  return dsa::plan_sparse_mla(batch->num_rows, batch->max_seq_len, num_heads, k, 0, kTargetCUs).splits;
}

size_t dsa_sparse_mla_workspace_bytes(const dsa_batch_t* batch, int32_t num_heads, int32_t k, int32_t num_splits) {
  if (!batch || !heads_supported(num_heads) || k < 1 || k > DSA_MAX_TOPK || num_splits < 0 || batch->num_rows <= 0)
    return 0;
  const dsa::MlaPlan p = dsa::plan_sparse_mla(batch->num_rows, batch->max_seq_len, num_heads, k, num_splits, kTargetCUs);
  return dsa::sparse_mla_workspace_bytes(batch->num_rows, num_heads, p);
}

// Argument checks shared by dsa_sparse_mla_decode and its no-allocation
// variant.  DSA_OK with *empty set means there is nothing to launch.
static int check_sparse_mla(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads, const uint16_t* kv_cache,
                            int64_t kv_page_stride, const int32_t* indices, int32_t k, float softmax_scale,
                            int32_t num_splits, uint16_t* out, float* lse, bool* empty) {
  *empty = true;
  int st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (!heads_supported(num_heads))
    return fail(DSA_ERR_UNSUPPORTED, "num_heads=%d: supported are multiples of 16 from 16 to 1024", num_heads);
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k=%d outside [1, %d]", k, DSA_MAX_TOPK);
  if (kv_page_stride < (int64_t)DSA_PAGE_SIZE * DSA_KV_DIM || kv_page_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "kv_page_stride=%lld must be >= 36864 elements and a multiple of 8",
                (long long)kv_page_stride);
  if (!std::isfinite(softmax_scale)) return fail(DSA_ERR_INVALID, "softmax_scale is not finite");
  if (num_splits < 0) return fail(DSA_ERR_INVALID, "num_splits=%d < 0", num_splits);
  if (batch->num_rows == 0) return ok();
  if (!q || !indices || !out || !lse) return fail(DSA_ERR_NULL, "q, indices, out and lse must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(DSA_ERR_INVALID, "q and out must be 16-byte aligned");
  if (!aligned(indices, 4) || !aligned(lse, 4)) return fail(DSA_ERR_INVALID, "indices and lse must be 4-byte aligned");
  if (batch->max_seq_len > 0 && batch->num_pages > 0) {
    if (!kv_cache) return fail(DSA_ERR_NULL, "kv_cache is NULL");
    if (!aligned(kv_cache, 16)) return fail(DSA_ERR_INVALID, "kv_cache must be 16-byte aligned");
  }
  *empty = false;
  return DSA_OK;
}

int dsa_sparse_mla_decode(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads, const uint16_t* kv_cache,
                          int64_t kv_page_stride, const int32_t* indices, int32_t k, float softmax_scale,
                          int32_t num_splits, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  bool empty = true;
  const int st = check_sparse_mla(batch, q, num_heads, kv_cache, kv_page_stride, indices, k, softmax_scale,
                                  num_splits, out, lse, &empty);
  if (st != DSA_OK || empty) return st;
  const dsa::MlaPlan p = dsa::plan_sparse_mla(batch->num_rows, batch->max_seq_len, num_heads, k, num_splits, kTargetCUs);
  const size_t need = dsa::sparse_mla_workspace_bytes(batch->num_rows, num_heads, p);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "dsa_sparse_mla_decode needs %zu workspace bytes, got %zu", need,
                  workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  return hip_status(dsa::launch_sparse_mla(to_args(batch), q, num_heads, kv_cache, kv_page_stride, indices, k,
                                           softmax_scale, p, out, lse, workspace, (hipStream_t)stream),
                    "dsa_sparse_mla_decode launch");
}

int dsa_sparse_mla_decode_noalloc(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads,
                                  const uint16_t* kv_cache, int64_t kv_page_stride, const int32_t* indices,
                                  int32_t k, float softmax_scale, int32_t num_splits, uint16_t* out, float* lse,
                                  void* stream) {
  bool empty = true;
  const int st = check_sparse_mla(batch, q, num_heads, kv_cache, kv_page_stride, indices, k, softmax_scale,
                                  num_splits, out, lse, &empty);
  if (st != DSA_OK || empty) return st;
  const size_t cap = dsa::static_scratch_bytes();
  dsa::MlaPlan p = dsa::plan_sparse_mla(batch->num_rows, batch->max_seq_len, num_heads, k, num_splits, kTargetCUs);
  size_t need = dsa::sparse_mla_workspace_bytes(batch->num_rows, num_heads, p);
  if (need > cap && num_splits == 0) {
    // the automatic count, lowered until the partials fit (one split needs none)
    for (int s = p.splits - 1; s >= 1 && need > cap; --s) {
      p = dsa::plan_sparse_mla(batch->num_rows, batch->max_seq_len, num_heads, k, s, kTargetCUs);
      need = dsa::sparse_mla_workspace_bytes(batch->num_rows, num_heads, p);
    }
  }
  if (need > cap)
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_sparse_mla_decode_noalloc: %d splits need %zu scratch bytes, above its %zu-byte device array "
                "(pass fewer splits, or use dsa_sparse_mla_decode with a workspace)",
                p.splits, need, cap);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = dsa::static_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "dsa_sparse_mla_decode_noalloc scratch address");
  }
  return hip_status(dsa::launch_sparse_mla(to_args(batch), q, num_heads, kv_cache, kv_page_stride, indices, k,
                                           softmax_scale, p, out, lse, scratch, (hipStream_t)stream),
                    "dsa_sparse_mla_decode_noalloc launch");
}

int dsa_sparse_mla_decode_fp8(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads,
                              const uint8_t* kv_cache_fp8, int64_t kv_page_stride_bytes, const int32_t* indices,
                              int32_t k, float softmax_scale, int32_t num_splits, uint16_t* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (!heads_supported(num_heads))
    return fail(DSA_ERR_UNSUPPORTED, "num_heads=%d: supported are multiples of 16 from 16 to 1024", num_heads);
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k=%d outside [1, %d]", k, DSA_MAX_TOPK);
  if (kv_page_stride_bytes < DSA_KV8_PAGE_BYTES || kv_page_stride_bytes % 16 != 0)
    return fail(DSA_ERR_INVALID, "kv_page_stride_bytes=%lld must be >= %d and a multiple of 16",
                (long long)kv_page_stride_bytes, DSA_KV8_PAGE_BYTES);
  if (!std::isfinite(softmax_scale)) return fail(DSA_ERR_INVALID, "softmax_scale is not finite");
  if (num_splits < 0) return fail(DSA_ERR_INVALID, "num_splits=%d < 0", num_splits);
  if (batch->num_pages > kMaxKv8Pages)
    return fail(DSA_ERR_UNSUPPORTED, "num_pages=%d above %d for the fp8 latent cache", batch->num_pages, kMaxKv8Pages);
  if (batch->num_rows == 0) return ok();
  if (!q || !indices || !out || !lse) return fail(DSA_ERR_NULL, "q, indices, out and lse must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(DSA_ERR_INVALID, "q and out must be 16-byte aligned");
  if (!aligned(indices, 4) || !aligned(lse, 4)) return fail(DSA_ERR_INVALID, "indices and lse must be 4-byte aligned");
  if (batch->max_seq_len > 0 && batch->num_pages > 0) {
    if (!kv_cache_fp8) return fail(DSA_ERR_NULL, "kv_cache_fp8 is NULL");
    if (!aligned(kv_cache_fp8, 16)) return fail(DSA_ERR_INVALID, "kv_cache_fp8 must be 16-byte aligned");
  }
  const dsa::MlaPlan p = dsa::plan_sparse_mla(batch->num_rows, batch->max_seq_len, num_heads, k, num_splits, kTargetCUs);
  const size_t need = dsa::sparse_mla_workspace_bytes(batch->num_rows, num_heads, p);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "dsa_sparse_mla_decode_fp8 needs %zu workspace bytes, got %zu", need,
                  workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 256)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  return hip_status(dsa::launch_sparse_mla_fp8(to_args(batch), q, num_heads, kv_cache_fp8, kv_page_stride_bytes,
                                               indices, k, softmax_scale, p, out, lse, workspace,
                                               (hipStream_t)stream),
                    "dsa_sparse_mla_decode_fp8 launch");
}

int dsa_latent_cache_write_fp8(int32_t num_tokens, const uint16_t* latent, int64_t latent_stride,
                               const uint16_t* rope, int64_t rope_stride, const int64_t* slot_mapping,
                               uint8_t* kv_cache_fp8, int64_t kv_page_stride_bytes, int32_t num_pages,
                               void* stream) {
  if (num_tokens < 0 || num_tokens > kMaxWriteItems)
    return fail(DSA_ERR_UNSUPPORTED, "num_tokens=%d outside [0, %d]", num_tokens, kMaxWriteItems);
  if (num_pages < 0) return fail(DSA_ERR_INVALID, "num_pages=%d < 0", num_pages);
  if (latent_stride < DSA_V_DIM || latent_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "latent_stride=%lld must be >= 512 elements and a multiple of 8",
                (long long)latent_stride);
  if (rope_stride < DSA_KV_DIM - DSA_V_DIM || rope_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "rope_stride=%lld must be >= 64 elements and a multiple of 8", (long long)rope_stride);
  if (kv_page_stride_bytes < DSA_KV8_PAGE_BYTES || kv_page_stride_bytes % 16 != 0)
    return fail(DSA_ERR_INVALID, "kv_page_stride_bytes=%lld must be >= %d and a multiple of 16",
                (long long)kv_page_stride_bytes, DSA_KV8_PAGE_BYTES);
  if (num_tokens == 0 || num_pages == 0) return ok();
  if (!latent || !rope || !slot_mapping || !kv_cache_fp8)
    return fail(DSA_ERR_NULL, "latent, rope, slot_mapping and kv_cache_fp8 must not be NULL");
  if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(kv_cache_fp8, 16))
    return fail(DSA_ERR_INVALID, "latent, rope and kv_cache_fp8 must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(DSA_ERR_INVALID, "slot_mapping must be 8-byte aligned");
  return hip_status(dsa::launch_latent_cache_write_fp8(num_tokens, latent, latent_stride, rope, rope_stride,
                                                       slot_mapping, kv_cache_fp8, kv_page_stride_bytes, num_pages,
                                                       (hipStream_t)stream),
                    "dsa_latent_cache_write_fp8 launch");
}

int dsa_indexer_q_quant_fp8(int32_t num_rows, const uint16_t* q, const float* weights, uint8_t* q_fp8,
                            float* weights_out, void* stream) {
  if (num_rows < 0 || num_rows > kMaxWriteItems)
    return fail(DSA_ERR_UNSUPPORTED, "num_rows=%d outside [0, %d]", num_rows, kMaxWriteItems);
  if (num_rows == 0) return ok();
  if (!q || !weights || !q_fp8 || !weights_out)
    return fail(DSA_ERR_NULL, "q, weights, q_fp8 and weights_out must not be NULL");
  if (!aligned(q, 16)) return fail(DSA_ERR_INVALID, "q must be 16-byte aligned");
  if (!aligned(q_fp8, 8)) return fail(DSA_ERR_INVALID, "q_fp8 must be 8-byte aligned");
  if (!aligned(weights, 4) || !aligned(weights_out, 4))
    return fail(DSA_ERR_INVALID, "weights and weights_out must be 4-byte aligned");
  return hip_status(dsa::launch_indexer_q_quant(num_rows, q, weights, q_fp8, weights_out, (hipStream_t)stream),
                    "dsa_indexer_q_quant_fp8 launch");
}

int dsa_indexer_k_quant_and_cache(int32_t num_tokens, const uint16_t* k, int64_t k_stride,
                                  const int64_t* slot_mapping, uint8_t* idx_cache, int64_t idx_page_stride,
                                  int32_t num_pages, void* stream) {
  if (num_tokens < 0 || num_tokens > kMaxWriteItems)
    return fail(DSA_ERR_UNSUPPORTED, "num_tokens=%d outside [0, %d]", num_tokens, kMaxWriteItems);
  if (num_pages < 0) return fail(DSA_ERR_INVALID, "num_pages=%d < 0", num_pages);
  if (k_stride < DSA_INDEXER_DIM || k_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "k_stride=%lld must be >= 128 elements and a multiple of 8", (long long)k_stride);
  if (idx_page_stride < DSA_INDEXER_PAGE_BYTES || idx_page_stride % 16 != 0)
    return fail(DSA_ERR_INVALID, "idx_page_stride=%lld must be >= 8448 bytes and a multiple of 16",
                (long long)idx_page_stride);
  if (num_tokens == 0 || num_pages == 0) return ok();
  if (!k || !slot_mapping || !idx_cache) return fail(DSA_ERR_NULL, "k, slot_mapping and idx_cache must not be NULL");
  if (!aligned(k, 16) || !aligned(idx_cache, 16))
    return fail(DSA_ERR_INVALID, "k and idx_cache must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(DSA_ERR_INVALID, "slot_mapping must be 8-byte aligned");
  return hip_status(dsa::launch_indexer_k_quant_cache(num_tokens, k, k_stride, slot_mapping, idx_cache,
                                                      idx_page_stride, num_pages, (hipStream_t)stream),
                    "dsa_indexer_k_quant_and_cache launch");
}

int dsa_latent_cache_write(int32_t num_tokens, const uint16_t* latent, int64_t latent_stride, const uint16_t* rope,
                           int64_t rope_stride, const int64_t* slot_mapping, uint16_t* kv_cache,
                           int64_t kv_page_stride, int32_t num_pages, void* stream) {
  if (num_tokens < 0 || num_tokens > kMaxWriteItems)
    return fail(DSA_ERR_UNSUPPORTED, "num_tokens=%d outside [0, %d]", num_tokens, kMaxWriteItems);
  if (num_pages < 0) return fail(DSA_ERR_INVALID, "num_pages=%d < 0", num_pages);
  if (latent_stride < DSA_V_DIM || latent_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "latent_stride=%lld must be >= 512 elements and a multiple of 8",
                (long long)latent_stride);
  if (rope_stride < DSA_KV_DIM - DSA_V_DIM || rope_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "rope_stride=%lld must be >= 64 elements and a multiple of 8", (long long)rope_stride);
  if (kv_page_stride < (int64_t)DSA_PAGE_SIZE * DSA_KV_DIM || kv_page_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "kv_page_stride=%lld must be >= 36864 elements and a multiple of 8",
                (long long)kv_page_stride);
  if (num_tokens == 0 || num_pages == 0) return ok();
  if (!latent || !rope || !slot_mapping || !kv_cache)
    return fail(DSA_ERR_NULL, "latent, rope, slot_mapping and kv_cache must not be NULL");
  if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(kv_cache, 16))
    return fail(DSA_ERR_INVALID, "latent, rope and kv_cache must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(DSA_ERR_INVALID, "slot_mapping must be 8-byte aligned");
  return hip_status(dsa::launch_latent_cache_write(num_tokens, latent, latent_stride, rope, rope_stride,
                                                   slot_mapping, kv_cache, kv_page_stride, num_pages,
                                                   (hipStream_t)stream),
                    "dsa_latent_cache_write launch");
}

}  // extern "C"
