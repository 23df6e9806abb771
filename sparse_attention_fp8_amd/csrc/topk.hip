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
//    (KPT = 8, 16 or 32, picked on the host from the longest row), so index
//    order is thread order.  The keys reach the registers through LDS: each
//    wave copies its 64*KPT floats with line-coalesced global->LDS loads into
//    an XOR-swizzled layout and reads its own keys back without bank
//    conflicts (a direct per-thread float4 read would touch 64 cache lines
//    per wave instruction).
//  * Up to three digit passes (11, 11 and 10 bits).  Pass one counts every
//    key into 8 copies of a 2048-bin LDS histogram (lane l adds to copy
//    l % 8), which spreads the atomics of the few hot bins; the copies are
//    stored copy-major with a padded stride, so the digit search reads each
//    thread's two bins of a copy as one conflict-free 8-byte load.  A block
//    scan over the bins from the top finds the threshold bin.  A pass stops
//    the search when the threshold bin is taken whole.  Passes two and three
//    rescan the registers, counting only keys that match the prefix so far;
//    when the bin left after pass two holds at most 64 keys (the usual case
//    for real-valued logits), those keys are collected instead and ranked by
//    one wave, which replaces pass three's rescan.
//    Every pass is branch-free: keys that do not count go to a per-lane sink
//    past the bins.  The candidate merges stage their keys through LDS the
//    same way as the row pass.
//  * Emission: each thread forms bit masks of its keys above the threshold
//    and equal to it; one block scan gives every thread its output offset and
//    tie budget; each thread walks the set bits of its mask, so it writes
//    only selected indices, in order -- ties at the threshold are taken
//    lowest index first and the output is sorted without any sort.
//  * A longer row is cut into chunks whose winners are kept as (key, index)
//    candidates.  Every member of the row's top-k is in its own chunk's top-k
//    (fewer than k entries precede it in the row, hence in the chunk), so one
//    more selection over the concatenated candidates -- already in index
//    order -- is exact (the chunked exact top-k argument of the pages).  Past
//    four chunks the candidates of each group of four chunks are first reduced
//    to their top k, in parallel, by the same argument one level up.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 32768;          // keys per workgroup in the row pass
constexpr int kSingleMax = 2 * kChunk; // longest row one workgroup selects from (two segments)
constexpr int kMergeMax = 65536;       // candidates per row in the merge pass
constexpr int kGroupChunks = 4;        // chunks one group merge reduces to k candidates
constexpr int kBins = 2048;
constexpr int kCopies = 8;             // copies of the pass-one histogram
constexpr int kCopyStride = kBins + 8;  // ints between copies: copy c of bin b sits in bank (8 c + b) % 64

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
  int ngroups;            // ceil(nchunks / kGroupChunks) when the merge has two levels, else 0
  uint32_t* grp_keys;     // [R, ngroups, k]
  int32_t* grp_idx;       // [R, ngroups, k]
  int32_t* grp_count;     // [R, ngroups]
};

// Selection state of one workgroup.  hist1 is pass one's histogram, copy-major
// with a padded stride (the copies of a bin, and bins 8 apart in one copy, sit
// in different banks); its first kBins entries are reused by pass three while
// hist2 serves pass two, so no pass clears a histogram it must wait for.
struct Shared {
  // zeroed before a selection (kInitBytes): both histograms and misc
  int hist1[kCopies * kCopyStride + 64];   // + one sink per lane for key 0 (never read)
  // out shares hist2's bytes: it is first written after the selection, when
  // every thread is past the last barrier of the digit searches that read
  // hist2.  Selection state then takes ~73 KB, so the candidate merges (8 or
  // 16 keys per thread: no larger staging area) fit two workgroups per CU.
  union {
    int hist2[kBins + 64];           // pass two (+ one sink per lane, never read)
    int out[DSA_MAX_TOPK];           // staged positions
  };
  int misc[4];
  // the rest is written before it is read
  int wave_tot[kWaves];
  uint32_t cand[64];                 // keys of a small threshold bin after two digits
};
constexpr int kInitBytes = (int)offsetof(Shared, wave_tot);
static_assert(kInitBytes % 16 == 0, "zeroed with 16-byte stores");

// The key staging area overlaps the selection state: it is dead once every
// wave has read its keys back (a barrier separates the two uses).  Wave w
// stages its keys in bytes [w R, (w + 1) R) of it (R = 256 KPT), and nobody
// else touches them, so each wave zeroes the selection state inside its own
// region as soon as it has read its keys back, and the state past all the
// regions is zeroed while the keys are in flight: the barrier that frees the
// staging area also publishes the zeroed state.
template <int KPT>
union TopkLds {
  Shared s;
  float4 stage[kThreads * KPT / 4];
};


// Zeroes the part of the selection state in bytes [lo, hi) of the LDS union,
// with threads tid, tid + nthr, ... of the caller's group.
__device__ __forceinline__ void zero_state(void* lds, int lo, int hi, int tid, int nthr) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > kInitBytes ? kInitBytes : hi;
  int4* p = reinterpret_cast<int4*>(lds);
  for (int i = lo / 16 + tid; i < hi / 16; i += nthr) p[i] = make_int4(0, 0, 0, 0);
}

template <int KPT>
struct Keys {
  uint32_t v[KPT];
};

template <int KPT>
using MaskT = typename std::conditional<(KPT > 32), uint64_t, uint32_t>::type;

__device__ __forceinline__ int popc(uint32_t m) { return __popc(m); }
__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }
__device__ __forceinline__ int ctz(uint32_t m) { return __builtin_ctz(m); }
__device__ __forceinline__ int ctz(uint64_t m) { return __builtin_ctzll(m); }
__device__ __forceinline__ uint32_t drop_highest(uint32_t m) { return m & ~(0x80000000u >> __builtin_clz(m)); }
__device__ __forceinline__ uint64_t drop_highest(uint64_t m) {
  return m & ~(0x8000000000000000ull >> __builtin_clzll(m));
}

// Inclusive prefix sum over the 64 lanes: DPP shifts inside each row of 16
// lanes, then the row totals are read out as scalars and added.
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane_id() >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Block-wide inclusive scan of one int per thread (one barrier).  Two calls
// need a barrier between them: the second overwrites sh.wave_tot.
__device__ __forceinline__ int block_scan(int v, Shared& sh) {
  const int w = threadIdx.x >> 6;
  const int incl = wave_scan_dpp(v);
  if (lane_id() == 63) sh.wave_tot[w] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) before += (i < w) ? sh.wave_tot[i] : 0;
  return incl + before;
}

// Keys [t*KPT, (t+1)*KPT) of thread t from src[0, n).  Positions >= n get key
// 0.  Every finite float and +-inf maps to a key >= 2^21; keys below 2^21 (key
// 0, and the negative NaNs whose bits are at or above 0xFFE00000) are not
// orderable: the selection counts them nowhere and never takes them.
// Wave w copies the V = KPT / 4 float4s of each of its lanes to LDS: owner
// lane L's float4 j goes to slot L V + (j ^ swz(L)) of the wave's area, with
// swz(L) = (L / (16 / V)) % V.  The 16 lanes a 128-bit LDS read serves per
// cycle then hit 16 distinct 16-byte units modulo 256 bytes of banks, and each
// group of 8 lanes of one copy instruction reads one whole 128-byte line.
// Float4s at or past n are not read (their slot gets a copy of the row's first
// float4 and is masked afterwards); src is 16-byte aligned and every float4
// that starts below n lies inside the row.
// A staged value as a key: logits go through float_key, candidate keys (RAW)
// are already keys.
template <bool RAW>
__device__ __forceinline__ uint32_t to_key(float x) { return RAW ? __float_as_uint(x) : float_key(x); }

template <int KPT, bool RAW = false>
__device__ void load_keys(Keys<KPT>& keys, const void* src, int n, float4* stage) {
  constexpr int V = KPT / 4;
  constexpr int F = 16 / V;
  constexpr int kRegion = 64 * V * 16;             // staging bytes per wave
  const int w = threadIdx.x >> 6, l = lane_id();
  const float4* src4 = reinterpret_cast<const float4*>(src);
  float4* wst = stage + w * 64 * V;
  const int f0 = w * 64 * V;                       // first float4 of this wave
  // selection state past every wave's staging region: no one stages there
  if (kWaves * kRegion < kInitBytes) zero_state(stage, kWaves * kRegion, kInitBytes, threadIdx.x, kThreads);
  if (4 * f0 < n) {
    const uint32_t wdst = lds_addr(wst);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int S = 64 * i + l;                    // slot this lane fills
      const int L = S / V;                         // owner lane of the slot
      const int j = (S % V) ^ ((L / F) % V);       // owner's float4 index
      const int f = f0 + L * V + j;
      lds_dma16(4 * f < n ? src4 + f : src4, wdst + i * 1024);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  const int base = (int)threadIdx.x * KPT;
  if (64 * KPT * (w + 1) <= n) {      // the whole wave lies inside the row: no range selects
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float4 x = wst[l * V + (j ^ ((l / F) % V))];
      keys.v[4 * j] = to_key<RAW>(x.x);
      keys.v[4 * j + 1] = to_key<RAW>(x.y);
      keys.v[4 * j + 2] = to_key<RAW>(x.z);
      keys.v[4 * j + 3] = to_key<RAW>(x.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int p = base + 4 * j;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p < n) x = wst[l * V + (j ^ ((l / F) % V))];
      keys.v[4 * j] = p < n ? to_key<RAW>(x.x) : 0u;
      keys.v[4 * j + 1] = p + 1 < n ? to_key<RAW>(x.y) : 0u;
      keys.v[4 * j + 2] = p + 2 < n ? to_key<RAW>(x.z) : 0u;
      keys.v[4 * j + 3] = p + 3 < n ? to_key<RAW>(x.w) : 0u;
    }
  }
  // materialise the keys here: otherwise the compiler sinks the range selects
  // into later loops and keeps one lane mask per key alive in scalar registers
#pragma unroll
  for (int j = 0; j < KPT; ++j) asm volatile("" : "+v"(keys.v[j]));
  // this wave's reads of its region are issued (and the LDS operations of a
  // wave execute in order): zero the selection state that lies in it.  The
  // memory clobber keeps the compiler from moving these int4 stores above the
  // float4 reads of the same bytes.
  asm volatile("" ::: "memory");
  zero_state(stage, w * kRegion, (w + 1) * kRegion, l, 64);
}

// Candidate keys read directly (per-thread strided loads), for candidate
// counts whose staging would not fit in LDS.
template <int KPT>
__device__ void load_raw_keys(Keys<KPT>& keys, const uint32_t* src, int n, void* lds) {
  zero_state(lds, 0, kInitBytes, threadIdx.x, kThreads);
  const int base = (int)threadIdx.x * KPT;
#pragma unroll
  for (int j = 0; j < KPT; ++j) keys.v[j] = base + j < n ? src[base + j] : 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) asm volatile("" : "+v"(keys.v[j]));
}

struct Selection {
  uint32_t threshold;  // keys above it are selected
  int need_eq;         // how many keys equal to it are taken, lowest index first
};

// Finds the threshold digit of one pass from a histogram (bins in ascending
// digit order, NC copies kCopyStride ints apart): the digit d whose bin holds
// the rem-th largest counted key, the count of keys above its bin, and its
// bin count -> sh.misc[0..2].  Thread t takes bins 2047 - 2t and 2046 - 2t,
// one 8-byte read per copy (consecutive lanes read consecutive 8 bytes).
template <int NC>
__device__ __forceinline__ void find_digit(const int* hist, int rem, Shared& sh) {
  const int d0 = kBins - 1 - 2 * (int)threadIdx.x, d1 = d0 - 1;
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int2 v = *reinterpret_cast<const int2*>(hist + c * kCopyStride + d1);
    c1 += v.x;
    c0 += v.y;
  }
  const int incl = block_scan(c0 + c1, sh);
  const int excl = incl - c0 - c1;
  if (excl < rem && rem <= incl) {
    const bool first = excl + c0 >= rem;
    sh.misc[0] = first ? d0 : d1;               // threshold digit
    sh.misc[1] = first ? excl : excl + c0;      // keys above its bin
    sh.misc[2] = first ? c0 : c1;               // keys in its bin
  }
  __syncthreads();
}

// Exact selection of the k largest orderable keys (keys >= 2^21) of the n
// valid keys (n > k >= 1).  Keys below 2^21 (an out-of-range slot is key 0) go
// to pass one's sink, so the threshold digit is never 0 and every prefix and
// threshold below is at least 2^21 - 1: the later comparisons exclude those
// keys by themselves.
//  pass 1: 11-bit top digit of every key;
//  passes 2 and 3 (11 and 10 bits) scan the registers again and count only
//  the keys whose higher digits match the prefix found so far.  (Compacting
//  the threshold bin into an LDS list after pass 1 costs more than it saves:
//  that bin holds thousands of keys.  After pass 2 it usually holds a few,
//  and resolve_small_bin replaces pass 3.)
//
// The threshold bin after two digits holds at most 64 keys: they are
// collected into LDS -- a ballot per key slot, so a wave without a matching
// key in that slot skips it -- and one wave ranks them: the rem-th largest is
// the threshold key, the bin's keys above it are taken whole and rem minus
// their count of the keys equal to it.
template <int KPT>
__device__ Selection resolve_small_bin(const Keys<KPT>& keys, uint32_t prefix, uint32_t mask, int rem, Shared& sh) {
  const int l = lane_id();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool m = (keys.v[j] & mask) == prefix;
    const uint64_t bal = __ballot(m);
    if (bal != 0ull) {   // wave-uniform
      int base = 0;
      if (l == 0) base = __hip_atomic_fetch_add(&sh.misc[3], popc((uint64_t)bal), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      base = __builtin_amdgcn_readfirstlane(base);
      const int pos = base + popc((uint64_t)(bal & ((1ull << l) - 1ull)));
      if (m && pos < 64) sh.cand[pos] = keys.v[j];
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int nb = min(sh.misc[3], 64);
    const uint32_t x = l < nb ? sh.cand[l] : 0u;
    int gt = 0, eq = 0;
    for (int j = 0; j < nb; ++j) {
      const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, j);
      gt += y > x ? 1 : 0;
      eq += y == x ? 1 : 0;
    }
    if (l < nb && gt < rem && rem <= gt + eq) {
      // every key equal to x taken: the same selection as "above x - 1",
      // which spares the staging its tie masks (x >= 2^21, no wrap)
      const bool all = rem == gt + eq;
      sh.misc[0] = (int)(all ? x - 1u : x);
      sh.misc[1] = all ? 0 : rem - gt;
    }
  }
  __syncthreads();
  return Selection{(uint32_t)sh.misc[0], sh.misc[1]};
}

// Precondition: the selection state (first kInitBytes of sh) is zero and
// visible to every thread (load_keys / load_raw_keys, then a barrier).
template <int KPT>
__device__ Selection radix_select(const Keys<KPT>& keys, int k, Shared& sh) {
  const int l = lane_id();
  // Keys below 2^21 count into a per-lane sink past the bins instead of
  // branching around the atomic: a branch per key costs more than the select.
  const int copy = l & (kCopies - 1);
  const int sink = kCopies * kCopyStride + l;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t key = keys.v[j];
    const int addr = key >= (1u << 21) ? copy * kCopyStride + (int)(key >> 21) : sink;
    __hip_atomic_fetch_add(&sh.hist1[addr], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  find_digit<kCopies>(sh.hist1, k, sh);
  uint32_t prefix = (uint32_t)sh.misc[0] << 21;
  int rem = k - sh.misc[1];
  const int in_bin = sh.misc[2];
  // No crossing: fewer than k keys are orderable.  Take all of them.
  if (in_bin == 0) return Selection{(1u << 21) - 1u, 0};
  if (rem == in_bin) return Selection{prefix - 1u, 0};  // the whole bin is taken

  // pass three counts into hist1's first kBins entries
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist1[i] = 0;
  constexpr int shifts[2] = {10, 0};
  constexpr int widths[2] = {11, 10};
  uint32_t mask = 0xFFE00000u;
  int* const hists[2] = {sh.hist2, sh.hist1};
  // keys outside the prefix count into a per-lane sink (never read), as in pass one
  int* const sinks[2] = {sh.hist2 + kBins + l, sh.hist1 + kCopies * kCopyStride + l};
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    int* hist = hists[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t key = keys.v[j];
      int* const dst = (key & mask) == prefix ? hist + ((key >> shifts[pass]) & dmask) : sinks[pass];
      __hip_atomic_fetch_add(dst, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    find_digit<1>(hist, rem, sh);
    rem -= sh.misc[1];
    prefix |= (uint32_t)sh.misc[0] << shifts[pass];
    mask |= dmask << shifts[pass];
    if (rem == sh.misc[2]) return Selection{prefix - 1u, 0};
    if (pass == 0 && sh.misc[2] <= 64) return resolve_small_bin(keys, prefix, mask, rem, sh);
  }
  return Selection{prefix, rem};
}

// Emits the selected keys' chunk positions in chunk order: emit(pos, i) for
// output slot pos of chunk position i.  Per thread: masks of keys above the
// threshold (gt) and equal to it (eq); one block scan of the packed counts (gt
// in the low 12 bits -- a prefix of gt counts never exceeds k <= 2048 -- and
// eq above) gives the thread's output offset and how many ties precede it.
// The thread keeps its first (need_eq - ties before it) eq keys and emits the
// set bits of the combined mask in order.  Out-of-range slots (key 0) are
// never taken and slots are clamped to k.  Returns how many slots were
// emitted: slots [0, that) each exactly once -- k, unless the row holds fewer
// than k orderable keys (some NaNs are not orderable, see load_keys).
template <int KPT, class Emit>
__device__ int emit_selected(const Keys<KPT>& keys, Selection sel, int k, Shared& sh, Emit emit,
                             int* eq_total = nullptr) {
  MaskT<KPT> gtb = 0, eqb = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) gtb |= (MaskT<KPT>)(keys.v[j] > sel.threshold) << j;
  // Ties matter only when some are taken, and then only in waves holding one.
  if (sel.need_eq > 0) {
    bool any = false;
#pragma unroll
    for (int j = 0; j < KPT; ++j) any |= keys.v[j] == sel.threshold;
    if (__ballot(any) != 0ull) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) eqb |= (MaskT<KPT>)(keys.v[j] == sel.threshold) << j;
    }
  }
  const int ng = popc(gtb), ne = popc(eqb);
  const int packed = ng | (ne << 12);
  const int excl = block_scan(packed, sh) - packed;   // barrier inside
  int tot = 0;                                        // block totals (all wave sums are in)
#pragma unroll
  for (int i = 0; i < kWaves; ++i) tot += sh.wave_tot[i];
  const int g = excl & 0xFFF;
  const int e = excl >> 12;
  int take = sel.need_eq - e;                         // ties this thread may take
  take = take < 0 ? 0 : (take > ne ? ne : take);
  MaskT<KPT> eqsel = eqb;
  for (int drop = ne - take; drop > 0; --drop) eqsel = drop_highest(eqsel);   // keep the lowest `take`
  MaskT<KPT> selb = gtb | eqsel;
  int pos = g + min(e, sel.need_eq);
  const int base = (int)threadIdx.x * KPT;
  while (selb != 0) {
    const int j = ctz(selb);
    if (pos < k) emit(pos, base + j);
    ++pos;
    selb &= selb - 1;
  }
  if (eq_total) *eq_total = tot >> 12;               // keys equal to the threshold, taken or not
  return min(k, (tot & 0xFFF) + min(tot >> 12, sel.need_eq));
}

// The selected chunk positions in sh.out[0, k) (-1 past the emitted slots),
// visible to the whole workgroup on return.
template <int KPT>
__device__ void stage_selected(const Keys<KPT>& keys, Selection sel, int k, Shared& sh) {
  for (int i = threadIdx.x; i < k; i += kThreads) sh.out[i] = -1;   // before the scan's barrier
  emit_selected(keys, sel, k, sh, [&](int pos, int i) { sh.out[pos] = i; });
  __syncthreads();
}

template <int KPT>
__global__ void __launch_bounds__(kThreads) topk_rows_kernel(TopkArgs a) {
  __shared__ TopkLds<KPT> lds;
  Shared& sh = lds.s;
  const int r = blockIdx.x / a.nchunks;
  const int c = blockIdx.x % a.nchunks;
  int b, e;
  seq_and_extent_wave(a.batch, r, b, e);
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
    load_keys(keys, row, e, lds.stage);
    __syncthreads();   // every wave has read its keys: the staging area is free
    const Selection sel = radix_select(keys, k, sh);
    // positions are the indices here: straight to the output, no staging
    const int emitted = emit_selected(keys, sel, k, sh, [&](int pos, int i) { out[pos] = i; });
    for (int i = emitted + (int)threadIdx.x; i < k; i += kThreads) out[i] = -1;
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
  load_keys(keys, row + lo, n, lds.stage);
  if (n <= k) {  // a short last chunk: every key is a candidate, in order
    const int base = (int)threadIdx.x * KPT;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (base + j < n) { ck[base + j] = keys.v[j]; ci[base + j] = lo + base + j; }
    if (threadIdx.x == 0) a.cand_count[slot] = n;
    return;
  }
  __syncthreads();   // staging area free
  const Selection sel = radix_select(keys, k, sh);
  stage_selected(keys, sel, k, sh);
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int pos = sh.out[i];
    ci[i] = pos >= 0 ? lo + pos : -1;
    ck[i] = pos >= 0 ? float_key(row[lo + pos]) : 0u;   // key 0: never selected again
  }
  if (threadIdx.x == 0) a.cand_count[slot] = k;
}

// Rows of up to kSingleMax = 2 kChunk keys, one workgroup each, no
// candidates and no merge launch: thread t holds keys [32 t, 32 t + 32) of
// the row (segment 0) and [kChunk + 32 t, kChunk + 32 t + 32) (segment 1) in
// registers, each segment staged through the same LDS area in turn.  The
// radix select counts the 64 keys of every thread whatever their positions;
// the emission then walks segment 0 and segment 1 in turn, so the output
// stays in ascending index order and ties at the threshold go to segment 0's
// (lower) indices first.  Rows of at most kChunk keys take the 32-key path.
__global__ void __launch_bounds__(kThreads) topk_rows64_kernel(TopkArgs a) {
  __shared__ TopkLds<32> lds;
  Shared& sh = lds.s;
  const int r = blockIdx.x;
  int b, e;
  seq_and_extent_wave(a.batch, r, b, e);
  const int k = a.k;
  const float* row = a.logits + (int64_t)r * a.logits_stride;
  int32_t* out = a.indices + (int64_t)r * k;
  if (e <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < e ? i : -1;
    return;
  }
  Keys<32> k0;
  load_keys(k0, row, min(e, kChunk), lds.stage);
  if (e <= kChunk) {
    __syncthreads();   // every wave has read its keys: the staging area is free
    const Selection sel = radix_select(k0, k, sh);
    const int emitted = emit_selected(k0, sel, k, sh, [&](int pos, int i) { out[pos] = i; });
    for (int i = emitted + (int)threadIdx.x; i < k; i += kThreads) out[i] = -1;
    return;
  }
  // Each wave stages both segments in its own region of the staging area, so
  // its copy of segment 1 goes out as soon as it has read back segment 0,
  // with no barrier between the two loads.
  Keys<32> k1;
  load_keys(k1, row + kChunk, e - kChunk, lds.stage);   // 128 KB in: kChunk * 4 bytes is 16-byte aligned
  __syncthreads();   // segment 1 read back; the selection state (zeroed by both loads) is visible
  Keys<64> kk;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    kk.v[j] = k0.v[j];
    kk.v[32 + j] = k1.v[j];
  }
  const Selection sel = radix_select(kk, k, sh);
  int eq0 = 0;
  const int n0 = emit_selected(k0, sel, k, sh, [&](int pos, int i) { out[pos] = i; }, &eq0);
  __syncthreads();   // the second emission's scan reuses sh.wave_tot
  const Selection sel1{sel.threshold, max(0, sel.need_eq - eq0)};
  const int n1 = emit_selected(k1, sel1, k - n0, sh, [&](int pos, int i) { out[n0 + pos] = kChunk + i; });
  for (int i = n0 + n1 + (int)threadIdx.x; i < k; i += kThreads) out[i] = -1;
}

// First level of the merge for rows of more than kGroupChunks chunks: group g
// of row r reduces the candidates of chunks [4 g, 4 g + 4) to its top k, kept
// in ascending candidate order (= ascending key index), so the final level
// sees the same tie order.  Exact by the chunking argument once more: a key of
// the row's top k is in the top k of its group.
template <int KPT>
__global__ void __launch_bounds__(kThreads) topk_group_kernel(TopkArgs a) {
  __shared__ TopkLds<KPT> lds;
  Shared& sh = lds.s;
  const int r = blockIdx.x / a.ngroups;
  const int g = blockIdx.x % a.ngroups;
  int b, e;
  seq_and_extent_wave(a.batch, r, b, e);
  const int k = a.k;
  const int nch = (e + kChunk - 1) / kChunk;
  const int c0 = g * kGroupChunks;
  const int64_t gslot = (int64_t)r * a.ngroups + g;
  if (e <= kChunk * kGroupChunks || c0 >= nch) {
    if (threadIdx.x == 0) a.grp_count[gslot] = 0;
    return;
  }
  const int c1 = min(c0 + kGroupChunks, nch);
  // chunks before the row's last hold exactly k candidates, so the group's
  // candidates are contiguous
  const int64_t row_slot = (int64_t)r * a.nchunks;
  const int n = (c1 - c0 - 1) * k + a.cand_count[row_slot + c1 - 1];
  const uint32_t* ck = a.cand_keys + (row_slot + c0) * k;
  const int32_t* ci = a.cand_idx + (row_slot + c0) * k;
  uint32_t* gk = a.grp_keys + gslot * k;
  int32_t* gi = a.grp_idx + gslot * k;
  if (n <= k) {
    for (int i = threadIdx.x; i < n; i += kThreads) { gk[i] = ck[i]; gi[i] = ci[i]; }
    if (threadIdx.x == 0) a.grp_count[gslot] = n;
    return;
  }
  Keys<KPT> keys;
  load_keys<KPT, true>(keys, ck, n, lds.stage);   // candidate slots are 8 KB aligned
  __syncthreads();   // every wave has read its keys: the staging area is free
  const Selection sel = radix_select(keys, k, sh);
  stage_selected(keys, sel, k, sh);
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int p = sh.out[i];
    gk[i] = p >= 0 ? ck[p] : 0u;
    gi[i] = p >= 0 ? ci[p] : -1;
  }
  if (threadIdx.x == 0) a.grp_count[gslot] = k;
}

// Final selection of a multi-chunk row over the chunk candidates, or over the
// group candidates when the merge has two levels.
template <int KPT>
__global__ void __launch_bounds__(kThreads) topk_merge_kernel(TopkArgs a) {
  constexpr bool kStaged = KPT <= 32;   // 64 keys per thread would need 256 KB of staging
  __shared__ TopkLds<kStaged ? KPT : 4> lds;
  Shared& sh = lds.s;
  const int r = blockIdx.x;
  int b, e;
  seq_and_extent_wave(a.batch, r, b, e);
  if (e <= kChunk) return;
  const int k = a.k;
  const int nch = (e + kChunk - 1) / kChunk;
  // Every chunk (group) but the last is full (exactly k winners), so the
  // candidates of row r are contiguous: (units - 1) * k + count_last.
  const uint32_t* ck;
  const int32_t* ci;
  int n;
  if (a.ngroups > 0 && nch > kGroupChunks) {
    const int ng = (nch + kGroupChunks - 1) / kGroupChunks;
    const int64_t row_slot = (int64_t)r * a.ngroups;
    n = (ng - 1) * k + a.grp_count[row_slot + ng - 1];
    ck = a.grp_keys + row_slot * k;
    ci = a.grp_idx + row_slot * k;
  } else {
    const int64_t row_slot = (int64_t)r * a.nchunks;
    n = (nch - 1) * k + a.cand_count[row_slot + nch - 1];
    ck = a.cand_keys + row_slot * k;
    ci = a.cand_idx + row_slot * k;
  }
  int32_t* out = a.indices + (int64_t)r * k;
  Keys<KPT> keys;
  if constexpr (kStaged) {
    load_keys<KPT, true>(keys, ck, n, lds.stage);   // candidate slots are 8 KB aligned
    __syncthreads();   // every wave has read its keys: the staging area is free
  } else {
    load_raw_keys(keys, ck, n, &sh);
    __syncthreads();   // the zeroed selection state is visible
  }
  const Selection sel = radix_select(keys, k, sh);
  stage_selected(keys, sel, k, sh);
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int p = sh.out[i];
    out[i] = p >= 0 ? ci[p] : -1;
  }
}

}  // namespace

// Rows of up to kSingleMax keys are selected by one workgroup; longer rows in
// kChunk-key chunks and a candidate merge.
int topk_num_chunks(int max_seq_len) {
  return max_seq_len <= kSingleMax ? 1 : (max_seq_len + kChunk - 1) / kChunk;
}

// Rows of up to kGroupChunks chunks merge in one level (candidates <=
// kGroupChunks * k), longer rows in two (final candidates <= groups * k).
int topk_num_groups(int max_seq_len) {
  const int nch = topk_num_chunks(max_seq_len);
  return nch > kGroupChunks ? (nch + kGroupChunks - 1) / kGroupChunks : 0;
}

int64_t topk_max_seq_len(int k) { return (int64_t)(kMergeMax / k) * kGroupChunks * kChunk; }

size_t topk_workspace_bytes(int num_rows, int max_seq_len, int k) {
  const int nch = topk_num_chunks(max_seq_len);
  if (nch <= 1 || num_rows <= 0) return 0;
  const size_t slots = (size_t)num_rows * nch;
  size_t bytes = slots * (size_t)k * 8;     // keys + indices
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += slots * 4;                       // counts
  bytes = (bytes + 255) & ~(size_t)255;
  const int ng = topk_num_groups(max_seq_len);
  if (ng > 0) {
    const size_t gslots = (size_t)num_rows * ng;
    bytes += gslots * (size_t)k * 8;        // group keys + indices
    bytes = (bytes + 255) & ~(size_t)255;
    bytes += gslots * 4;                    // group counts
    bytes = (bytes + 255) & ~(size_t)255;
  }
  return bytes;
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
    off = (off + slots * 4 + 255) & ~(size_t)255;
    a.ngroups = topk_num_groups(batch.max_seq_len);
    if (a.ngroups > 0) {
      const size_t gslots = (size_t)batch.num_rows * a.ngroups;
      a.grp_keys = reinterpret_cast<uint32_t*>(ws + off);
      a.grp_idx = reinterpret_cast<int32_t*>(ws + off + gslots * (size_t)k * 4);
      off = (off + gslots * (size_t)k * 8 + 255) & ~(size_t)255;
      a.grp_count = reinterpret_cast<int32_t*>(ws + off);
    }
  }
  // keys per thread: the smallest of 8 / 16 / 32 that covers a chunk, or two
  // 32-key segments for single rows of up to kSingleMax keys
  const int longest = a.nchunks > 1 ? kChunk : batch.max_seq_len;
  const int64_t grid = (int64_t)batch.num_rows * a.nchunks;
  if (a.nchunks == 1 && longest > kChunk) {
    hipLaunchKernelGGL(topk_rows64_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  } else if (longest <= 8 * kThreads) {
    hipLaunchKernelGGL(topk_rows_kernel<8>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  } else if (longest <= 16 * kThreads) {
    hipLaunchKernelGGL(topk_rows_kernel<16>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(topk_rows_kernel<32>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nchunks <= 1) return err;
  if (a.ngroups > 0) {
    // a group holds kGroupChunks * k <= 8192 candidates (k <= 2048)
    hipLaunchKernelGGL(topk_group_kernel<8>, dim3((unsigned)((int64_t)batch.num_rows * a.ngroups)), dim3(kThreads),
                       0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t cands = (int64_t)(a.ngroups > 0 ? a.ngroups : a.nchunks) * k;
  if (cands <= 8 * kThreads) {
    hipLaunchKernelGGL(topk_merge_kernel<8>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  } else if (cands <= 16 * kThreads) {
    hipLaunchKernelGGL(topk_merge_kernel<16>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  } else if (cands <= 32 * kThreads) {
    hipLaunchKernelGGL(topk_merge_kernel<32>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(topk_merge_kernel<64>, dim3((unsigned)batch.num_rows), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
