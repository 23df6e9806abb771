// Per-row top-k of the indexer logits (index_topk = 2048).
//
// Selection rule (vLLM PR "[Feature] TRITON_MLA_SPARSE backend ..." review
// thread, chunked exact top-k discussion): the k largest logits of row r
// over its causal range [0, e_r); equal values go to the lower index; the
// chosen indices are written in ascending order, -1 padded.
//
// gfx950 design: exact radix select on order-preserving 32-bit keys held in
// registers.
//  * One 1024-thread workgroup takes up to kChunk = 32768 keys of a row;
//    thread t holds the KPT consecutive keys [t*KPT, (t+1)*KPT) in VGPRs
//    (KPT = 8, 16 or 32, picked on the host from the longest row), so the
//    keys are read from memory once and index order is thread order.
//  * Up to three digit passes (11, 11 and 10 bits) build an LDS histogram of
//    the keys that still match the threshold prefix; one wave scans the 2048
//    bins from the top.  A pass stops the search early when the threshold
//    bin is taken whole.  Only a few percent of the keys survive pass one.
//  * Emission: each thread counts its keys above the threshold and equal to
//    it, one block-wide scan gives every thread its output offset and tie
//    budget, and each thread writes its selected indices in order -- ties at
//    the threshold are taken lowest index first, so the output is sorted and
//    deterministic without any sort.
//  * A longer row is cut into chunks whose winners are kept as (key, index)
//    candidates.  Every member of the row's top-k is in its own chunk's top-k
//    (fewer than k entries precede it in the row, hence in the chunk), so one
//    more selection over the concatenated candidates -- already in index
//    order -- is exact (the chunked exact top-k argument of the pages).
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 32768;          // keys per workgroup in the row pass
constexpr int kMergeMax = 65536;       // candidates per row in the merge pass
constexpr int kBins = 2048;

struct TopkArgs {
  BatchArgs batch;
  const float* logits;
  int64_t logits_stride;
  int k;
  int32_t* indices;
  int nchunks;            // ceil(max_seq_len / kChunk) when > 1
  uint32_t* cand_keys;    // [R, nchunks, k]
  int32_t* cand_idx;      // [R, nchunks, k]
  int32_t* cand_count;    // [R, nchunks]
};

// LDS of one workgroup.  hist has two alternating digit histograms (so one is
// cleared while the other is counted) plus one private overflow counter per
// lane: keys that do not match the current prefix are counted there, which
// keeps every atomic unconditional (no per-key branch) and conflict-free.
constexpr int kHist = kBins + 64;
constexpr int kCand = 4096;            // LDS list for the threshold bin's keys
struct Shared {
  int hist[2][kHist];
  uint32_t cand[kCand + 64];           // (+ one dummy slot per lane)
  int out[DSA_MAX_TOPK + 64];  // staged output (+ one dummy slot per lane)
  uint64_t wave_pair[kWaves];
  int wave_tot[kWaves];
  int misc[4];
};

// Keys [t*KPT, (t+1)*KPT) of thread t.  Positions >= n get key 0: every finite
// float and +-inf maps to a key >= 2^21, so with n > k valid keys the k-th
// largest key is never 0 and a key-0 slot is never selected.
template <int KPT>
struct Keys {
  uint32_t v[KPT];
};

// The float4 holding an in-range key is inside the row: logits_stride and
// chunk starts are multiples of 4.
template <int KPT>
__device__ void load_float_keys(Keys<KPT>& keys, const float* src, int n) {
  const int base = (int)threadIdx.x * KPT;
#pragma unroll
  for (int j = 0; j < KPT / 4; ++j) {
    const int p = base + 4 * j;
    if (p < n) {
      const float4 x = *reinterpret_cast<const float4*>(src + p);
      keys.v[4 * j] = float_key(x.x);
      keys.v[4 * j + 1] = p + 1 < n ? float_key(x.y) : 0u;
      keys.v[4 * j + 2] = p + 2 < n ? float_key(x.z) : 0u;
      keys.v[4 * j + 3] = p + 3 < n ? float_key(x.w) : 0u;
    } else {
      keys.v[4 * j] = keys.v[4 * j + 1] = keys.v[4 * j + 2] = keys.v[4 * j + 3] = 0u;
    }
  }
}

// Candidate keys (4-byte aligned only: a row's candidates start at r * k).
template <int KPT>
__device__ void load_raw_keys(Keys<KPT>& keys, const uint32_t* src, int n) {
  const int base = (int)threadIdx.x * KPT;
#pragma unroll
  for (int j = 0; j < KPT; ++j) keys.v[j] = base + j < n ? src[base + j] : 0u;
}

struct Selection {
  uint32_t threshold;  // keys above it are selected
  int need_eq;         // how many keys equal to it are taken, lowest index first
};

// Finds the threshold digit of one pass from sh.hist-like counts `hist`
// (bins in ascending digit order): the digit d whose bin holds the rem-th
// largest matching key, the count of matching keys above its bin, and its bin
// count.  One block scan over the 2048 bins (2 per thread, descending).
__device__ __forceinline__ void find_digit(const int* hist, int rem, Shared& sh) {
  const int w = threadIdx.x >> 6, l = lane_id();
  const int d0 = kBins - 1 - 2 * (int)threadIdx.x, d1 = d0 - 1;
  const int c0 = hist[d0], c1 = hist[d1];
  int incl = wave_inclusive_scan(c0 + c1);
  if (l == 63) sh.wave_tot[w] = incl;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kWaves; ++i) incl += (i < w) ? sh.wave_tot[i] : 0;
  const int excl = incl - c0 - c1;
  if (excl < rem && rem <= incl) {
    const bool first = excl + c0 >= rem;
    sh.misc[0] = first ? d0 : d1;               // threshold digit
    sh.misc[1] = first ? excl : excl + c0;      // keys above its bin
    sh.misc[2] = first ? c0 : c1;               // keys in its bin
  }
  __syncthreads();
}

// Exact selection of the k largest of the n valid keys (n > k >= 1).
//  pass 1: 11-bit top digit of every key (no prefix test needed);
//  then the keys of the threshold bin (usually a few percent) are compacted
//  into an LDS list and passes 2 and 3 (11 and 10 bits) run over that list;
//  if the bin is too large for the list, passes 2 and 3 scan the registers.
template <int KPT>
__device__ Selection radix_select(const Keys<KPT>& keys, int k, Shared& sh) {
  const int l = lane_id();
  for (int i = threadIdx.x; i < kHist; i += kThreads) { sh.hist[0][i] = 0; sh.hist[1][i] = 0; }
  if (threadIdx.x == 0) { sh.misc[0] = 0; sh.misc[1] = 0; sh.misc[2] = 0; sh.misc[3] = 0; }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t key = keys.v[j];
    atomicAdd(&sh.hist[0][key != 0u ? (int)(key >> 21) : kBins + l], 1);
  }
  __syncthreads();
  find_digit(sh.hist[0], k, sh);
  uint32_t prefix = (uint32_t)sh.misc[0] << 21;
  int rem = k - sh.misc[1];
  const int in_bin = sh.misc[2];
  if (rem == in_bin) return Selection{prefix - 1u, 0};  // the whole bin is taken

  constexpr int shifts[2] = {10, 0};
  constexpr int widths[2] = {11, 10};
  uint32_t mask = 0xFFE00000u;
  if (in_bin <= kCand) {
    // compact the bin's keys: one LDS atomic per wave reserves the slots
    int mine = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) mine += (keys.v[j] & mask) == prefix && keys.v[j] != 0u;
    int incl = wave_inclusive_scan(mine);
    int base = 0;
    if (l == 63) base = atomicAdd(&sh.misc[3], incl);
    base = __shfl(base, 63, 64) + incl - mine;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t key = keys.v[j];
      const bool match = (key & mask) == prefix && key != 0u;
      sh.cand[match ? base : kCand + l] = key;
      base += match;
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      int* hist = sh.hist[(pass + 1) & 1];
      for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      const uint32_t dmask = (1u << widths[pass]) - 1u;
      for (int i = threadIdx.x; i < in_bin; i += kThreads) {
        const uint32_t key = sh.cand[i];
        atomicAdd(&hist[(key & mask) == prefix ? (int)((key >> shifts[pass]) & dmask) : kBins + l], 1);
      }
      __syncthreads();
      find_digit(hist, rem, sh);
      rem -= sh.misc[1];
      prefix |= (uint32_t)sh.misc[0] << shifts[pass];
      mask |= dmask << shifts[pass];
      if (rem == sh.misc[2]) return Selection{prefix - 1u, 0};
    }
    return Selection{prefix, rem};
  }
  // large threshold bin: passes 2 and 3 over the registers
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    int* hist = sh.hist[(pass + 1) & 1];
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t dmask = (1u << widths[pass]) - 1u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t key = keys.v[j];
      const bool match = key != 0u && (key & mask) == prefix;
      atomicAdd(&hist[match ? (int)((key >> shifts[pass]) & dmask) : kBins + l], 1);
    }
    __syncthreads();
    find_digit(hist, rem, sh);
    rem -= sh.misc[1];
    prefix |= (uint32_t)sh.misc[0] << shifts[pass];
    mask |= dmask << shifts[pass];
    if (rem == sh.misc[2]) return Selection{prefix - 1u, 0};
  }
  return Selection{prefix, rem};
}

// Stages the selected keys' chunk positions in sh.out[0, k), in chunk order:
// one block scan of the per-thread counts, then unconditional LDS writes
// (unselected keys write to the lane's dummy slot).  Out-of-range slots (key
// 0) are never taken and positions are clamped to k, so whatever the logits
// hold (NaN included) every staged position is -1 or a valid key position.
template <int KPT>
__device__ void stage_selected(const Keys<KPT>& keys, Selection sel, int k, Shared& sh) {
  const int w = threadIdx.x >> 6, l = lane_id();
  for (int i = threadIdx.x; i < k; i += kThreads) sh.out[i] = -1;
  int ng = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t key = keys.v[j];
    ng += key > sel.threshold;
    ne += key == sel.threshold && key != 0u;
  }
  const uint64_t packed = (uint64_t)ng | ((uint64_t)ne << 32);
  uint64_t incl = wave_inclusive_scan_u64(packed);
  if (l == 63) sh.wave_pair[w] = incl;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kWaves; ++i) incl += (i < w) ? sh.wave_pair[i] : 0ull;
  const uint64_t excl = incl - packed;
  int g = (int)(uint32_t)excl;
  int e = (int)(excl >> 32);
  const int base = (int)threadIdx.x * KPT;
  const int dummy = k + l;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t key = keys.v[j];
    const bool gt = key > sel.threshold;
    const bool eq = key == sel.threshold && key != 0u;
    const int pos = g + min(e, sel.need_eq);
    const bool take = (gt || (eq && e < sel.need_eq)) && pos < k;
    sh.out[take ? pos : dummy] = base + j;
    g += gt;
    e += eq;
  }
  __syncthreads();
}

template <int KPT>
__global__ void __launch_bounds__(kThreads) topk_rows_kernel(TopkArgs a) {
  __shared__ Shared sh;
  const int r = blockIdx.x / a.nchunks;
  const int c = blockIdx.x % a.nchunks;
  const int b = seq_of_row_wave(a.batch.query_start, a.batch.num_seqs, r);
  const int e = b >= 0 ? row_extent(a.batch, b, r) : 0;
  const int k = a.k;
  const float* row = a.logits + (int64_t)r * a.logits_stride;
  Keys<KPT> keys;

  if (e <= kChunk) {  // the whole row is this workgroup's (chunk 0)
    if (c != 0) return;
    int32_t* out = a.indices + (int64_t)r * k;
    if (e <= k) {
      for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < e ? i : -1;
      return;
    }
    load_float_keys(keys, row, e);
    const Selection sel = radix_select(keys, k, sh);
    stage_selected(keys, sel, k, sh);
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = sh.out[i];
    return;
  }

  // multi-chunk row: this chunk's winners become candidates
  const int lo = c * kChunk;
  const int64_t slot = (int64_t)r * a.nchunks + c;
  if (lo >= e) {
    if (threadIdx.x == 0) a.cand_count[slot] = 0;
    return;
  }
  const int n = min(kChunk, e - lo);
  uint32_t* ck = a.cand_keys + slot * k;
  int32_t* ci = a.cand_idx + slot * k;
  load_float_keys(keys, row + lo, n);
  if (n <= k) {  // a short last chunk: every key is a candidate, in order
    const int base = (int)threadIdx.x * KPT;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (base + j < n) { ck[base + j] = keys.v[j]; ci[base + j] = lo + base + j; }
    if (threadIdx.x == 0) a.cand_count[slot] = n;
    return;
  }
  const Selection sel = radix_select(keys, k, sh);
  stage_selected(keys, sel, k, sh);
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int pos = sh.out[i];
    ci[i] = pos >= 0 ? lo + pos : -1;
    ck[i] = pos >= 0 ? float_key(row[lo + pos]) : 0u;   // key 0: never selected again
  }
  if (threadIdx.x == 0) a.cand_count[slot] = k;
}

template <int KPT>
__global__ void __launch_bounds__(kThreads) topk_merge_kernel(TopkArgs a) {
  __shared__ Shared sh;
  const int r = blockIdx.x;
  const int b = seq_of_row_wave(a.batch.query_start, a.batch.num_seqs, r);
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
  Keys<KPT> keys;
  load_raw_keys(keys, ck, n);
  const Selection sel = radix_select(keys, k, sh);
  stage_selected(keys, sel, k, sh);
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int p = sh.out[i];
    out[i] = p >= 0 ? ci[p] : -1;
  }
}

}  // namespace

int topk_num_chunks(int max_seq_len) { return max_seq_len <= kChunk ? 1 : (max_seq_len + kChunk - 1) / kChunk; }

int64_t topk_max_seq_len(int k) { return (int64_t)(kMergeMax / k) * kChunk; }

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
  // keys per thread: the smallest of 8 / 16 / 32 that covers a chunk
  const int longest = a.nchunks > 1 ? kChunk : batch.max_seq_len;
  const int64_t grid = (int64_t)batch.num_rows * a.nchunks;
  if (longest <= 8 * kThreads) {
    hipLaunchKernelGGL(topk_rows_kernel<8>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  } else if (longest <= 16 * kThreads) {
    hipLaunchKernelGGL(topk_rows_kernel<16>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(topk_rows_kernel<32>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nchunks <= 1) return err;
  const int64_t cands = (int64_t)a.nchunks * k;
  if (cands <= 8 * kThreads) {
    hipLaunchKernelGGL(topk_merge_kernel<8>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  } else if (cands <= 32 * kThreads) {
    hipLaunchKernelGGL(topk_merge_kernel<32>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(topk_merge_kernel<64>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
