// Per-row top-k of the indexer logits (index_topk = 2048).
//
// Selection rule (vLLM PR "[Feature] TRITON_MLA_SPARSE backend ..." review
// thread, chunked exact top-k discussion): the k largest logits of
// row r over its causal range [0, e_r); equal values go to the lower index;
// the chosen indices are written in ascending order, -1 padded.
//
// gfx950 design: exact radix select on order-preserving 32-bit keys.
//  * A row is cut into chunks of kChunk = 16384 keys.  One 1024-thread
//    workgroup per (row, chunk) stages its keys in LDS (64 KB) and finds the
//    chunk's k-th largest key T in three digit passes (11, 11 and 10 bits, so
//    the exponent-heavy top digit spreads over 2048 bins and the LDS atomics
//    rarely collide).  The selected entries (key > T, plus the first
//    k - #(key > T) entries equal to T in index order) are then emitted in
//    index order with wave ballots and a block scan, so the output is sorted
//    for free.
//  * A row that fits one chunk is finished there.  A longer row leaves its
//    chunk winners as (key, index) candidates; every member of the row's
//    top-k is in its own chunk's top-k (fewer than k entries precede it in the
//    row, hence in the chunk), so one more selection over the concatenated
//    candidates -- already in ascending index order -- gives the exact answer
//    (the pages' chunked exact top-k argument).
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 16384;
constexpr int kBins = 2048;

struct TopkArgs {
  BatchArgs batch;
  const float* logits;
  int64_t logits_stride;
  int k;
  int32_t* indices;
  int nchunks;            // ceil(max_seq_len / kChunk)
  uint32_t* cand_keys;    // [R, nchunks, k]
  int32_t* cand_idx;      // [R, nchunks, k]
  int32_t* cand_count;    // [R, nchunks]
};

struct Shared {
  uint32_t keys[kChunk];
  int hist[kBins];
  int wave_a[kWaves];
  int wave_b[kWaves];
  int misc[4];
};

// Inclusive scan over the 1024 threads of the block.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wave_tot, int* total) {
  const int wave = threadIdx.x >> 6;
  int incl = wave_inclusive_scan(v);
  if (lane_id() == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = wave_tot[i];
    before += (i < wave) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl;
}

struct Selection {
  uint32_t threshold;  // the k-th largest key
  int need_eq;         // how many keys equal to threshold are taken (lowest index first)
};

// Exact k-th largest of keys[0, n) (n > k >= 1); `keys` may be LDS or global.
__device__ Selection radix_select(const uint32_t* keys, int n, int k, Shared& sh) {
  uint32_t prefix = 0, mask = 0;
  int rem = k;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1);
    }
    __syncthreads();
    // Thread t owns bins (descending) 2t and 2t+1 -> digits kBins-1-2t, kBins-2-2t.
    const int d0 = kBins - 1 - 2 * (int)threadIdx.x, d1 = d0 - 1;
    const int c0 = sh.hist[d0], c1 = sh.hist[d1];
    int total;
    const int incl = block_inclusive_scan(c0 + c1, sh.wave_a, &total);
    const int excl = incl - c0 - c1;
    if (excl < rem && rem <= incl) {
      if (excl + c0 >= rem) { sh.misc[0] = d0; sh.misc[1] = excl; }
      else { sh.misc[0] = d1; sh.misc[1] = excl + c0; }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sh.misc[0];
    rem -= sh.misc[1];
    prefix |= digit << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  return Selection{prefix, rem};
}

// Emits the selected positions of keys[0, n) in ascending order:
// emit(out_pos, i) for each chosen i.
template <class Emit>
__device__ void emit_selected(const uint32_t* keys, int n, Selection sel, Shared& sh, Emit emit) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, eq_before = 0;
  for (int start = 0; start < n; start += kThreads) {
    const int i = start + (int)threadIdx.x;
    const uint32_t key = i < n ? keys[i] : 0u;
    const bool gt = i < n && key > sel.threshold;
    const bool eq = i < n && key == sel.threshold;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      sh.wave_a[wave] = __popcll(bg);
      sh.wave_b[wave] = __popcll(be);
    }
    __syncthreads();
    int pg = __popcll(bg & lt), pe = __popcll(be & lt), tg = 0, te = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int a = sh.wave_a[w], b = sh.wave_b[w];
      if (w < wave) { pg += a; pe += b; }
      tg += a;
      te += b;
    }
    __syncthreads();
    const int eq_quota = max(0, sel.need_eq - eq_before);  // ties still to take
    if (gt || (eq && pe < eq_quota)) emit(base + pg + min(pe, eq_quota), i);
    base += tg + min(te, eq_quota);
    eq_before += te;
  }
}

__device__ void stage_keys(const float* src, int n, uint32_t* dst) {
  for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * kThreads) {
    if (i + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      dst[i] = float_key(v.x);
      dst[i + 1] = float_key(v.y);
      dst[i + 2] = float_key(v.z);
      dst[i + 3] = float_key(v.w);
    } else {
      for (int t = i; t < n; ++t) dst[t] = float_key(src[t]);
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kThreads) topk_chunk_kernel(TopkArgs a) {
  __shared__ Shared sh;
  const int r = blockIdx.x / a.nchunks;
  const int c = blockIdx.x % a.nchunks;
  const int b = seq_of_row(a.batch.query_start, a.batch.num_seqs, r);
  const int e = b >= 0 ? row_extent(a.batch, b, r) : 0;
  const int k = a.k;
  const float* row = a.logits + (int64_t)r * a.logits_stride;

  if (e <= kChunk) {  // the whole row is this workgroup's (chunk 0)
    if (c != 0) return;
    int32_t* out = a.indices + (int64_t)r * k;
    if (e <= k) {
      for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < e ? i : -1;
      return;
    }
    stage_keys(row, e, sh.keys);
    const Selection sel = radix_select(sh.keys, e, k, sh);
    emit_selected(sh.keys, e, sel, sh, [&](int pos, int i) { out[pos] = i; });
    return;
  }

  // multi-chunk row: emit this chunk's candidates
  const int lo = c * kChunk;
  const int64_t slot = (int64_t)r * a.nchunks + c;
  if (lo >= e) {
    if (threadIdx.x == 0) a.cand_count[slot] = 0;
    return;
  }
  const int n = min(kChunk, e - lo);
  uint32_t* ck = a.cand_keys + slot * k;
  int32_t* ci = a.cand_idx + slot * k;
  stage_keys(row + lo, n, sh.keys);
  if (n <= k) {
    for (int i = threadIdx.x; i < n; i += kThreads) { ck[i] = sh.keys[i]; ci[i] = lo + i; }
    if (threadIdx.x == 0) a.cand_count[slot] = n;
    return;
  }
  const Selection sel = radix_select(sh.keys, n, k, sh);
  emit_selected(sh.keys, n, sel, sh, [&](int pos, int i) { ck[pos] = sh.keys[i]; ci[pos] = lo + i; });
  if (threadIdx.x == 0) a.cand_count[slot] = k;
}

__global__ void __launch_bounds__(kThreads) topk_merge_kernel(TopkArgs a) {
  __shared__ Shared sh;
  const int r = blockIdx.x;
  const int b = seq_of_row(a.batch.query_start, a.batch.num_seqs, r);
  const int e = b >= 0 ? row_extent(a.batch, b, r) : 0;
  if (e <= kChunk) return;
  const int k = a.k;
  const int nch = (e + kChunk - 1) / kChunk;
  // Every chunk but the last is full (kChunk >= k keys -> exactly k winners),
  // so the candidates of row r are contiguous: (nch - 1) * k + count_last.
  const int64_t row_slot = (int64_t)r * a.nchunks;
  const int n = (nch - 1) * k + a.cand_count[row_slot + nch - 1];
  const uint32_t* ck = a.cand_keys + row_slot * k;
  const int32_t* ci = a.cand_idx + row_slot * k;
  int32_t* out = a.indices + (int64_t)r * k;
  const uint32_t* keys = ck;
  if (n <= kChunk) {
    for (int i = threadIdx.x; i < n; i += kThreads) sh.keys[i] = ck[i];
    __syncthreads();
    keys = sh.keys;
  }
  const Selection sel = radix_select(keys, n, k, sh);
  emit_selected(keys, n, sel, sh, [&](int pos, int i) { out[pos] = ci[i]; });
}

}  // namespace

int topk_num_chunks(int max_seq_len) { return max_seq_len <= kChunk ? 1 : (max_seq_len + kChunk - 1) / kChunk; }

size_t topk_workspace_bytes(int num_rows, int max_seq_len, int k) {
  const int nch = topk_num_chunks(max_seq_len);
  if (nch <= 1 || num_rows <= 0) return 0;
  const size_t slots = (size_t)num_rows * nch;
  size_t bytes = slots * (size_t)k * 8;     // keys + indices
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += slots * 4;                       // counts
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_topk(const BatchArgs& batch, const float* logits, int64_t logits_stride, int k,
                       int32_t* indices, void* workspace, hipStream_t stream) {
  if (batch.num_rows <= 0) return hipSuccess;
  TopkArgs a{};
  a.batch = batch;
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.k = k;
  a.indices = indices;
  a.nchunks = topk_num_chunks(batch.max_seq_len);
  if (a.nchunks > 1) {
    const size_t slots = (size_t)batch.num_rows * a.nchunks;
    char* ws = static_cast<char*>(workspace);
    a.cand_keys = reinterpret_cast<uint32_t*>(ws);
    a.cand_idx = reinterpret_cast<int32_t*>(ws + slots * (size_t)k * 4);
    size_t off = (slots * (size_t)k * 8 + 255) & ~(size_t)255;
    a.cand_count = reinterpret_cast<int32_t*>(ws + off);
  }
  const int64_t grid = (int64_t)batch.num_rows * a.nchunks;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nchunks <= 1) return err;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
