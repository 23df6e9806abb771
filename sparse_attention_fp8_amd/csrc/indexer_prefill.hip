// Lightning-indexer logits for chunked prefill (many query rows per sequence).
#include "common.h"
#include "kernels.h"

namespace dsa {

hipError_t launch_indexer_prefill(const BatchArgs& batch, const uint8_t* q, const float* w,
                                  const uint8_t* cache, int64_t page_stride, float* logits,
                                  int64_t logits_stride, int clean, int num_cus, hipStream_t stream) {
  return launch_indexer_paged(batch, q, w, cache, page_stride, logits, logits_stride, clean, num_cus, stream);
}

}  // namespace dsa
