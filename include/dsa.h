/*
 * dsa.h -- libdsa: the DeepSeek-Sparse-Attention (DSA) decode hot path on
 * AMD MI355X (gfx950), behind a plain C ABI.
 *
 * One DSA layer step runs three stages for every query row (the vLLM PR page
 * "[Feature] TRITON_MLA_SPARSE backend for SM8x/11x/12x DSA Sparse MLA
 * Support", section Changes, items 2 and 3):
 *   1. lightning-indexer MQA logits over a paged FP8 indexer-K cache
 *      (dsa_indexer_logits_paged for decode, dsa_indexer_logits_prefill for
 *      chunked prefill);
 *   2. per-row top-k of those logits, k = index_topk = 2048 (dsa_topk);
 *   3. sparse MLA attention over only the selected tokens of a paged bf16
 *      latent cache, split-KV partials merged by online softmax, with a
 *      single-pass fast path (dsa_sparse_mla_decode).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers unless the comment says [host].  The caller
 *    owns every buffer; the library never allocates, frees or keeps device
 *    memory and keeps no state between calls.  Outputs must not alias inputs.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on it and never synchronises, so a device fault
 *    surfaces at the caller's next synchronisation.  Launch geometry depends on
 *    host fields only, so a call can be captured into a HIP graph.
 *  - Return value: DSA_OK (0) or a negative dsa_status.  Argument checks run on
 *    the host before anything is launched; on failure nothing is enqueued and
 *    dsa_last_error_message() (thread-local) says what was wrong.
 *  - Device contents are validated only where a bad value could make a kernel
 *    touch memory it does not own: sequence lengths are clamped to max_seq_len,
 *    query rows to num_rows, block-table entries outside [0, num_pages) mark
 *    their tokens masked, and top-k indices outside a row's causal range are
 *    masked, never dereferenced.
 *  - Determinism: the same inputs give bit-identical outputs on every call
 *    (fixed reduction orders; the only atomics count integers).  Batch
 *    invariance: a row's logits over [0, e_r) and its top-k indices depend on
 *    that row's own inputs only; so do its sparse MLA out and lse when
 *    num_splits = 1.  The automatic split count follows the batch shape, which
 *    changes the summation order of the split merge (the pages' backend
 *    forces one split for batch-invariant runs: PR page, Limitations).
 *
 * Geometry of a step
 * ------------------
 *  Sequence b has L_b = seq_lens[b] cached tokens (this step's queries
 *  included) and q_len_b = query_start[b+1] - query_start[b] query rows.  Row
 *  r = query_start[b] + i (0 <= i < q_len_b) sees keys [0, e_r) with
 *      e_r = L_b - q_len_b + i + 1   (floored at 0)
 *  -- the per-row causal bound: a decode row sees the whole context, the two
 *  rows of a draft+verify (MTP) step see L-1 and L keys.
 *  Logical token s of sequence b lives in physical page
 *  block_table[b * bt_stride + s / 64], slot s % 64.  Block size is 64 (the
 *  indexer requires it; the pages' backend declares MultipleOf(64)).  One block
 *  table serves both caches: the same physical page id indexes the indexer
 *  cache and the latent cache, each with its own page stride (the KV unifier
 *  pads indexer pages, vllm-dsa-mtp-sm80 README, skew fix 0).
 *
 * Cache layouts
 * -------------
 *  Indexer K page (132 bytes per token, 64 tokens): bytes [0, 8192) hold
 *  [64 tokens][128] OCP e4m3 codes (e4m3fn, max 448), bytes [8192, 8448) hold
 *  the 64 fp32 per-token scales.  Pages are idx_page_stride bytes apart
 *  (>= 8448, a multiple of 16; padding is never read).
 *  Latent page: [64 tokens][576] bf16 (512 latent = V, then 64 rope), pages
 *  kv_page_stride ELEMENTS apart (>= 64*576, a multiple of 8).
 */
#ifndef LIBDSA_DSA_H
#define LIBDSA_DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  DSA_ERR_INVALID = -2,     /* a size, stride or alignment is out of contract    */
  DSA_ERR_UNSUPPORTED = -3, /* a valid shape this build has no kernel for       */
  DSA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required        */
  DSA_ERR_HIP = -5          /* the HIP runtime rejected a launch                 */
} dsa_status;

#define DSA_PAGE_SIZE 64
#define DSA_INDEXER_HEADS 64
#define DSA_INDEXER_DIM 128
#define DSA_INDEXER_PAGE_BYTES 8448
#define DSA_KV_DIM 576
#define DSA_V_DIM 512
#define DSA_MAX_TOPK 2048
#define DSA_MAX_SEQS 4096
#define DSA_KV8_PAGE_BYTES 41984      /* fp8 latent page: 64 x 640 B rows + 64 x 16 B scale records */
#define DSA_MAX_WRITE_ITEMS (1 << 24) /* rows / tokens per quantiser or cache-writer call */
#define DSA_NOALLOC_SCRATCH_BYTES (32u << 20) /* device scratch of dsa_sparse_mla_decode_noalloc */

/* One step's batch description, shared by all four calls. */
typedef struct {
  int32_t num_seqs;            /* B, 0 <= B <= DSA_MAX_SEQS                          [host] */
  int32_t num_rows;            /* R = total query rows = query_start[B]              [host] */
  int32_t max_seq_len;         /* >= every L_b; sizes grids and splits, clamps L_b   [host] */
  int32_t max_q_len;           /* >= every q_len_b (1 decode, 2 MTP, large prefill)  [host] */
  int32_t bt_stride;           /* block-table row length, >= ceil(max_seq_len / 64)  [host] */
  int32_t num_pages;           /* physical pages in each cache (ids 0..num_pages-1)  [host] */
  const int32_t* seq_lens;     /* [B]     L_b                                               */
  const int32_t* query_start;  /* [B+1]   non-decreasing row offsets, query_start[0] = 0    */
  const int32_t* block_table;  /* [B, bt_stride] physical page ids                          */
} dsa_batch_t;

/*
 * dsa_indexer_logits_paged -- lightning-indexer logits, decode shape.
 * (PR page, Changes item 2: "paged MQA logits" with in-kernel FP8 decode and
 * the K-side scale applied to the fp32 dot output.)
 *
 *   logits[r, s] = sum_h weights[r, h] * max(q[r, h, :] . k[s, :], 0) * kscale[s]
 *   for 0 <= s < e_r, with q and k decoded from e4m3 inside fp8 matrix
 *   instructions.  The products are exact; the matrix unit adds each aligned
 *   group of 8 of them (dims 8j..8j+7) in a narrow adder (a product 2^14 or
 *   more below the group's largest may be dropped), the group sums and the
 *   64-term head sum in fp32 -- errors near 3e-5 of
 *   sum_h |weights[r, h]| * max(q . k, 0) * kscale[s].
 *
 *  q_fp8         [R, 64, 128] e4m3 codes, 16-byte aligned.  Any q scale must be
 *                folded into `weights` by the caller.
 *  weights       [R, 64] fp32, 16-byte aligned.
 *  idx_cache     indexer pages, 16-byte aligned; idx_page_stride in bytes.
 *  logits        [R, logits_stride] fp32, 16-byte aligned;
 *                logits_stride >= max_seq_len and a multiple of 4.
 *  clean_logits  1: columns [e_r, logits_stride) of every row are set to -inf
 *                ("clean"); 0: they are left untouched ("dirty").  Tokens whose
 *                block maps outside [0, num_pages) get -inf either way.
 * Best for max_q_len <= 2 (decode, MTP); correct for any q_len.
 */
int dsa_indexer_logits_paged(const dsa_batch_t* batch, const uint8_t* q_fp8, const float* weights,
                             const uint8_t* idx_cache, int64_t idx_page_stride, float* logits,
                             int64_t logits_stride, int clean_logits, void* stream);

/*
 * dsa_indexer_logits_prefill -- the same logits for chunked prefill, where a
 * sequence has many query rows (PR page, Changes item 2: prefill MQA logits
 * with a per-row causal bound and a per-row early exit over key tiles).  Same
 * arguments and result as dsa_indexer_logits_paged; pages are read directly
 * through the block table, so no gathered copy of K is needed.  Tuned for
 * q_len_b >> 1 (fp8-MFMA bound); correct for any q_len.
 */
int dsa_indexer_logits_prefill(const dsa_batch_t* batch, const uint8_t* q_fp8, const float* weights,
                               const uint8_t* idx_cache, int64_t idx_page_stride, float* logits,
                               int64_t logits_stride, int clean_logits, void* stream);

/*
 * dsa_topk -- indices of the k largest logits[r, 0:e_r) of every row (PR page
 * review thread: index_topk = 2048 and the exact chunked top-k argument).
 *  Order of selection: larger value first; equal values (IEEE equality, so -0
 *  equals +0) go to the lower index.  indices[r, 0:n) = the chosen
 *  n = min(k, e_r) indices in ascending order, indices[r, n:k) = -1.  Only
 *  columns [0, e_r) are read.  NaN logits give an unspecified (but in-range)
 *  selection: a NaN either ranks at one end of the order or is never taken
 *  (negative NaNs with bits at or above 0xFFE00000); a row with fewer than
 *  min(k, e_r) keys that can be taken returns those, then -1.
 *  logits     [R, logits_stride] fp32, 16-byte aligned, logits_stride % 4 == 0
 *  k          1 <= k <= DSA_MAX_TOPK; rows may hold up to (65536 / k) * 131072
 *             keys (4,194,304 for k = 2048), longer max_seq_len is UNSUPPORTED.
 *             With max_seq_len <= 65536 every row is selected by one
 *             workgroup.  Longer rows are cut into 32768-key chunks whose top k
 *             are candidates; beyond 4 chunks, groups of 4 chunks are first
 *             reduced to their top k (exact: a winner of the row is a winner
 *             of its chunk and of its group -- the pages' chunking argument,
 *             review thread).
 *  indices    [R, k] int32
 *  workspace  device scratch of at least dsa_topk_workspace_bytes(batch, k)
 *             bytes (may be NULL when that is 0); 256-byte aligned.
 */
int dsa_topk(const dsa_batch_t* batch, const float* logits, int64_t logits_stride, int32_t k,
             int32_t* indices, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode -- sparse MLA over the selected tokens (PR page,
 * Changes item 3: split-KV decode with an N-way online-softmax merge, a
 * single-pass fast path, and -1e30 as the masked sentinel so all-masked tiles
 * never form (-inf) - (-inf)).  For every row r and head h, over the valid
 * entries s of indices[r, 0:k) (0 <= s < e_r and on an in-range page; others
 * are masked; duplicates count as listed):
 *     z_s = softmax_scale * q[r, h, 0:576] . c_s[0:576]
 *     out[r, h, :] = sum_s softmax(z)_s * c_s[0:512]      (bf16, round to nearest even)
 *     lse[r, h]    = ln sum_s exp(z_s)                     (fp32; -inf, out = 0 if none valid)
 *  q           [R, H, 576] bf16, 16-byte aligned
 *  num_heads   H: a multiple of 16 from 16 to 1024 (one GPU's share of the
 *              MLA heads: 16 of 128 at TP = 8 ... all 128 at TP = 1)
 *  kv_cache    latent pages, 16-byte aligned; kv_page_stride in elements
 *  indices     [R, k] int32 logical token ids (typically dsa_topk's output)
 *  k           1 <= k <= DSA_MAX_TOPK
 *  num_splits  0 = automatic (dsa_sparse_mla_pick_splits), 1 = single pass
 *              (batch-invariant: a row's results do not depend on the batch),
 *              n > 1 = the k slots cut into n contiguous ranges merged N-way
 *              (clamped to the number of 64-slot tiles)
 *  out         [R, H, 512] bf16;  lse [R, H] fp32 (either may not be NULL)
 *  workspace   at least dsa_sparse_mla_workspace_bytes(batch, H, k, num_splits)
 *              bytes, 256-byte aligned (NULL allowed when that is 0)
 */
int dsa_sparse_mla_decode(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads,
                          const uint16_t* kv_cache, int64_t kv_page_stride, const int32_t* indices,
                          int32_t k, float softmax_scale, int32_t num_splits, uint16_t* out,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode_noalloc -- dsa_sparse_mla_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments, kernels and
 * results without the workspace.  The split partials live in a device array
 * inside the library, DSA_NOALLOC_SCRATCH_BYTES (32 MiB) on every device the
 * call runs on, held until the process ends.  The call allocates nothing; on
 * its first call on a device it looks that array's address up (with the
 * device current).
 *  num_splits  0 = the automatic split count, lowered until the partials
 *              (splits * R * H * 2056 bytes) fit the array; n = forced, and a
 *              forced count whose partials do not fit returns
 *              DSA_ERR_UNSUPPORTED (nothing is launched).
 *  Calls on one device share the array: two calls that overlap in time on one
 *  device (different streams, or different threads) race and give undefined
 *  results; calls ordered on one stream are safe.  Nothing in the array needs
 *  clearing (a call writes every partial it reads).
 */
int dsa_sparse_mla_decode_noalloc(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads,
                                  const uint16_t* kv_cache, int64_t kv_page_stride, const int32_t* indices,
                                  int32_t k, float softmax_scale, int32_t num_splits, uint16_t* out, float* lse,
                                  void* stream);

/*
 * dsa_sparse_mla_decode_fp8 -- dsa_sparse_mla_decode over an fp8 latent cache,
 * which the pages list as missing from their backend (PR page, Limitations:
 * bf16-only latent cache).  fp8 latent page (64 tokens, DSA_KV8_PAGE_BYTES):
 *   bytes [640 t, 640 t + 512)        512 e4m3fn codes of token t's latent
 *   bytes [640 t + 512, 640 t + 640)  its 64 rope values, bf16
 *   bytes [40960 + 16 t, +16)         4 fp32 scales, one per 128 latent values
 * Latent value d of token t = scale[d / 128] * e4m3(code[d]) (written by
 * dsa_latent_cache_write_fp8).  The attention is computed over these
 * dequantised rows exactly as dsa_sparse_mla_decode does over bf16 rows (q
 * stays bf16; products are exact, sums fp32; the probabilities times the group
 * scale are rounded to bf16 for the PV products).  Same arguments, masking,
 * splits, workspace (dsa_sparse_mla_workspace_bytes) and outputs, except:
 *  kv_cache_fp8          fp8 latent pages, 16-byte aligned
 *  kv_page_stride_bytes  >= DSA_KV8_PAGE_BYTES, a multiple of 16 (128 keeps
 *                        every row on whole 128-byte lines)
 *  batch->num_pages      at most 2^25 (UNSUPPORTED above)
 */
int dsa_sparse_mla_decode_fp8(const dsa_batch_t* batch, const uint16_t* q, int32_t num_heads,
                              const uint8_t* kv_cache_fp8, int64_t kv_page_stride_bytes, const int32_t* indices,
                              int32_t k, float softmax_scale, int32_t num_splits, uint16_t* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The steps just before the path: the indexer-q quantiser and the two cache
 * writers (vllm-dsa-mtp-sm80 README, skew fixes 0 and 1, which name the
 * unfused per_token_group_quant_fp8 for the indexer q and the indexer-K cache
 * writer indexer_k_quant_and_cache that addresses pages through their stride).
 * The pages do not print their arithmetic; the reading implemented is:
 *   per group of 128 values x (one (row, head) of q, or one K token), in IEEE
 *   fp32:  amax = max |x|;  scale = amax / 448, or 1 when amax == 0;
 *          code = e4m3fn(x / scale), round to nearest even, saturating at
 *          +-448 (so the largest element always lands on +-448), sign kept.
 *   Results are bit-exact functions of the inputs (no reduction-order freedom).
 * Non-finite inputs give unspecified codes and scales (but no fault).
 *
 * Slots: slot_mapping[t] = page * 64 + slot-in-page of token t (int64).  A
 * negative slot (a padding token) or one >= num_pages * 64 writes nothing.
 * Two tokens with the same slot in one call race: which one lands is
 * unspecified.  Only the token's own bytes in its page are written; other
 * slots and the page padding are never touched.
 */

/*
 * dsa_indexer_q_quant_fp8 -- quantise the indexer q per (row, head) and fold
 * the scale into the head weights, producing dsa_indexer_logits_*'s inputs.
 *  q            [R, 64, 128] bf16, 16-byte aligned
 *  weights      [R, 64] fp32 head weights, 4-byte aligned
 *  q_fp8        [R, 64, 128] e4m3fn codes out, 8-byte aligned
 *  weights_out  [R, 64] fp32 out: weights[r, h] * scale[r, h] (one fp32
 *               multiply); may be the same buffer as `weights` (in place)
 *  0 <= R <= DSA_MAX_WRITE_ITEMS.
 */
int dsa_indexer_q_quant_fp8(int32_t num_rows, const uint16_t* q, const float* weights, uint8_t* q_fp8,
                            float* weights_out, void* stream);

/*
 * dsa_indexer_k_quant_and_cache -- quantise each new token's indexer K and
 * write its 128 codes to page * idx_page_stride + slot * 128 and its fp32
 * scale to page * idx_page_stride + 8192 + slot * 4 of idx_cache.
 *  k             [T, k_stride] bf16 (first 128 used); k_stride >= 128 and a
 *                multiple of 8 elements; 16-byte aligned
 *  slot_mapping  [T] int64, 8-byte aligned (see "Slots" above)
 *  idx_cache     indexer pages (layout above), 16-byte aligned;
 *                idx_page_stride >= 8448 bytes, a multiple of 16
 *  num_pages     pages in idx_cache
 *  0 <= T <= DSA_MAX_WRITE_ITEMS.
 */
int dsa_indexer_k_quant_and_cache(int32_t num_tokens, const uint16_t* k, int64_t k_stride,
                                  const int64_t* slot_mapping, uint8_t* idx_cache, int64_t idx_page_stride,
                                  int32_t num_pages, void* stream);

/*
 * dsa_latent_cache_write -- copy each new token's latent row (512 bf16) and
 * rope part (64 bf16) into its latent-cache slot, latent first, unchanged:
 * kv_cache[page * kv_page_stride + slot * 576 + (0..575)].
 *  latent  [T, latent_stride] bf16 (first 512 used), latent_stride >= 512
 *  rope    [T, rope_stride] bf16 (first 64 used), rope_stride >= 64
 *          (strides in elements, multiples of 8; both 16-byte aligned)
 *  slot_mapping  [T] int64, 8-byte aligned (see "Slots" above)
 *  kv_cache      latent pages, 16-byte aligned; kv_page_stride >= 36864
 *                elements, a multiple of 8
 *  0 <= T <= DSA_MAX_WRITE_ITEMS.
 */
int dsa_latent_cache_write(int32_t num_tokens, const uint16_t* latent, int64_t latent_stride, const uint16_t* rope,
                           int64_t rope_stride, const int64_t* slot_mapping, uint16_t* kv_cache,
                           int64_t kv_page_stride, int32_t num_pages, void* stream);

/*
 * dsa_latent_cache_write_fp8 -- quantise each new token's latent row in 4
 * groups of 128 (the quantiser above) and write codes, scales and the bf16 rope
 * part into its slot of the fp8 latent cache (layout at
 * dsa_sparse_mla_decode_fp8).  Arguments as dsa_latent_cache_write, with
 *  kv_cache_fp8          fp8 latent pages, 16-byte aligned
 *  kv_page_stride_bytes  >= DSA_KV8_PAGE_BYTES, a multiple of 16
 */
int dsa_latent_cache_write_fp8(int32_t num_tokens, const uint16_t* latent, int64_t latent_stride,
                               const uint16_t* rope, int64_t rope_stride, const int64_t* slot_mapping,
                               uint8_t* kv_cache_fp8, int64_t kv_page_stride_bytes, int32_t num_pages,
                               void* stream);

/* Workspace sizes (host fields of `batch` only; 0 when none is needed). */
size_t dsa_topk_workspace_bytes(const dsa_batch_t* batch, int32_t k);
size_t dsa_sparse_mla_workspace_bytes(const dsa_batch_t* batch, int32_t num_heads, int32_t k,
                                      int32_t num_splits);
/* The split count num_splits = 0 resolves to (depends on host fields only). */
int32_t dsa_sparse_mla_pick_splits(const dsa_batch_t* batch, int32_t num_heads, int32_t k);

const char* dsa_status_string(int status);
const char* dsa_last_error_message(void);
/* "libdsa <version> gfx950" */
const char* dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_DSA_H */
