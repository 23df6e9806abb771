// Internal launchers of the libdsa kernels (host side).  Each enqueues on
// `stream` and returns the HIP launch status; arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct BatchArgs;

hipError_t launch_indexer_paged(const BatchArgs& batch, const uint8_t* q, const float* w,
                                const uint8_t* cache, int64_t page_stride, float* logits,
                                int64_t logits_stride, int clean, int num_cus, hipStream_t stream);

hipError_t launch_indexer_prefill(const BatchArgs& batch, const uint8_t* q, const float* w,
                                  const uint8_t* cache, int64_t page_stride, float* logits,
                                  int64_t logits_stride, int clean, int num_cus, hipStream_t stream);

int topk_num_chunks(int max_seq_len);
int64_t topk_max_seq_len(int k);  // longest row one dsa_topk call handles
size_t topk_workspace_bytes(int num_rows, int max_seq_len, int k);
hipError_t launch_topk(const BatchArgs& batch, const float* logits, int64_t logits_stride, int k,
                       int32_t* indices, void* workspace, hipStream_t stream);

struct MlaPlan {
  int splits;       // >= 1
  int split_slots;  // k slots per split, a multiple of 64
  int head_blocks;  // ceil(H / 64)
};
MlaPlan plan_sparse_mla(int num_rows, int max_seq_len, int H, int k, int num_splits, int num_cus);
size_t sparse_mla_workspace_bytes(int num_rows, int H, const MlaPlan& plan);
hipError_t launch_sparse_mla(const BatchArgs& batch, const uint16_t* q, int H, const uint16_t* kv,
                             int64_t kv_stride, const int32_t* indices, int k, float softmax_scale,
                             const MlaPlan& plan, uint16_t* out, float* lse, void* workspace,
                             hipStream_t stream);

// The device scratch behind dsa_sparse_mla_decode_noalloc: its size, and its
// address on the current device (looked up on the first call per device).
size_t static_scratch_bytes();
hipError_t static_scratch(void** ptr);

hipError_t launch_sparse_mla_fp8(const BatchArgs& batch, const uint16_t* q, int H, const uint8_t* kv8,
                                 int64_t kv8_stride, const int32_t* indices, int k, float softmax_scale,
                                 const MlaPlan& plan, uint16_t* out, float* lse, void* workspace,
                                 hipStream_t stream);

hipError_t launch_latent_cache_write_fp8(int num_tokens, const uint16_t* latent, int64_t latent_stride,
                                         const uint16_t* rope, int64_t rope_stride, const int64_t* slots,
                                         uint8_t* cache, int64_t page_stride, int num_pages, hipStream_t stream);

hipError_t launch_indexer_q_quant(int num_rows, const uint16_t* q, const float* w, uint8_t* codes, float* w_out,
                                  hipStream_t stream);
hipError_t launch_indexer_k_quant_cache(int num_tokens, const uint16_t* k, int64_t k_stride, const int64_t* slots,
                                        uint8_t* cache, int64_t page_stride, int num_pages, hipStream_t stream);
hipError_t launch_latent_cache_write(int num_tokens, const uint16_t* latent, int64_t latent_stride,
                                     const uint16_t* rope, int64_t rope_stride, const int64_t* slots,
                                     uint16_t* cache, int64_t page_stride, int num_pages, hipStream_t stream);

}  // namespace dsa
