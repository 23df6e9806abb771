// Device-side helpers shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

constexpr int kPage = DSA_PAGE_SIZE;            // tokens per block
constexpr int kIdxHeads = DSA_INDEXER_HEADS;    // 64
constexpr int kIdxDim = DSA_INDEXER_DIM;        // 128
constexpr int kIdxScaleOff = kPage * kIdxDim;   // 8192: scales follow the codes
constexpr int kKvDim = DSA_KV_DIM;              // 576
constexpr int kVDim = DSA_V_DIM;                // 512
constexpr float kMaskSentinel = -1e30f;         // running-max start of masked tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// The host-visible batch fields the kernels need, passed by value.
struct BatchArgs {
  int num_seqs, num_rows, max_seq_len, max_q_len, bt_stride, num_pages;
  const int* seq_lens;
  const int* query_start;
  const int* block_table;
};

__device__ __forceinline__ int clamp_len(int L, int max_len) { return L < 0 ? 0 : (L > max_len ? max_len : L); }

// Row r's sequence: the b with query_start[b] <= r < query_start[b+1] (binary
// search; query_start is non-decreasing).  Returns -1 when r lies outside.
__device__ __forceinline__ int seq_of_row(const int* qs, int num_seqs, int r) {
  int lo = 0, hi = num_seqs;  // answer in [lo, hi)
  if (num_seqs <= 0 || r < qs[0] || r >= qs[num_seqs]) return -1;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (qs[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// Wave-cooperative seq_of_row: every lane of a full wave calls it with the same
// r.  Two rounds of lane-parallel loads (a 64-way fan-out over query_start,
// then 64 entries within the chosen stride) replace the binary search's chain
// of dependent loads; num_seqs <= 4096 keeps the stride <= 64.
__device__ __forceinline__ int seq_of_row_wave(const int* qs, int num_seqs, int r) {
  if (num_seqs <= 0) return -1;
  const int lane = threadIdx.x & 63;
  const int step = (num_seqs + 63) >> 6;
  const int j1 = lane * step;
  const int v1 = j1 < num_seqs ? qs[j1] : 0x7FFFFFFF;
  const int last = qs[num_seqs];
  const int n1 = __popcll(__ballot(v1 <= r));
  if (n1 == 0 || r >= last) return -1;
  if (step == 1) return n1 - 1;
  const int lo = (n1 - 1) * step;
  const int j2 = lo + lane;
  const int v2 = (lane < step && j2 < num_seqs) ? qs[j2] : 0x7FFFFFFF;
  const int n2 = __popcll(__ballot(v2 <= r));
  return lo + n2 - 1;
}

// Causal extent of row r of sequence b: e_r = L_b - q_len_b + i + 1, in [0, L_b].
__device__ __forceinline__ int row_extent(const BatchArgs& a, int b, int r) {
  const int q0 = a.query_start[b], q1 = a.query_start[b + 1];
  const int L = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int e = L - (q1 - q0) + (r - q0) + 1;
  return e < 0 ? 0 : (e > L ? L : e);
}

// Sequence b of row r and its causal extent e_r (b = -1, e = 0 when no
// sequence holds the row), for a full wave calling with the same r.  With at
// most 63 sequences one round of lane-parallel loads gives both: lane j reads
// query_start[j] and seq_lens[j], and b's entries are picked out by shuffles.
// More sequences take the two-round search, then the extent loads.
__device__ __forceinline__ void seq_and_extent_wave(const BatchArgs& a, int r, int& b, int& e) {
  const int B = a.num_seqs;
  if (B > 63) {
    b = seq_of_row_wave(a.query_start, B, r);
    e = b >= 0 ? row_extent(a, b, r) : 0;
    return;
  }
  b = -1;
  e = 0;
  if (B <= 0) return;
  const int lane = threadIdx.x & 63;
  const int qv = lane <= B ? a.query_start[lane] : 0x7FFFFFFF;
  const int lv = lane < B ? a.seq_lens[lane] : 0;
  const int n1 = __popcll(__ballot(lane < B && qv <= r));
  const int last = __shfl(qv, B, 64);
  if (n1 == 0 || r >= last) return;
  b = n1 - 1;
  const int q0 = __shfl(qv, b, 64), q1 = __shfl(qv, b + 1, 64);
  const int L = clamp_len(__shfl(lv, b, 64), a.max_seq_len);
  const int x = L - (q1 - q0) + (r - q0) + 1;
  e = x < 0 ? 0 : (x > L ? L : x);
}

// Order-preserving map float -> uint32 (larger float -> larger key), with -0
// folded onto +0 (x + 0 is +0 for both zeros under round-to-nearest) so the
// two compare equal.  NaN keeps its sign side: above +inf or below -inf.
__device__ __forceinline__ uint32_t float_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ (uint32_t)(((int32_t)u >> 31) | (int32_t)0x80000000);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_inclusive_scan_u64(uint64_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// x from lane l ^ 32 / l ^ 16 through the VALU lane-swap instructions (no LDS
// round trip).  permlane32_swap exchanges the upper half of its first operand
// with the lower half of its second; permlane16_swap the odd 16-lane rows of
// the first with the even rows of the second.
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane_id() & 16) ? r[0] : r[1]);
}

// max(x, 0) in one instruction (v_med3_f32 with 0 and the largest float) for
// finite inputs such as MFMA results; fmaxf() adds a NaN-quieting max first.
__device__ __forceinline__ float relu_finite(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f); }

// bf16 helpers (bit patterns in uint16 / packed pairs in uint32).
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 32-bit LDS address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global->LDS copies: 16 (or 4) bytes per lane into LDS at
// lds + 16 * lane (4 * lane), lds wave-uniform.  Written as inline asm so the
// compiler does not treat a copy as an LDS store that every later LDS read
// must wait for (that would drain the next tile's copy before the current one
// is read).  The kernels wait for their copies themselves (vmcnt).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}

// s_waitcnt that waits until at most N vector-memory operations of this wave
// are outstanding (N < 64), leaving the LDS and export counters alone.
// Followed by a compiler barrier so no LDS read of copied data is hoisted
// above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
  asm volatile("" ::: "memory");
}

}  // namespace dsa
