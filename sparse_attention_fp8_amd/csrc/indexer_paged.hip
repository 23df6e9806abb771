// Lightning-indexer logits over the paged FP8 indexer-K cache, decode shape.
//
// Computes logits[r, s] = sum_h w[r, h] * relu(q[r, h, :] . k[s, :]) * kscale[s]
// for s < e_r (vLLM PR "[Feature] TRITON_MLA_SPARSE backend for SM8x/11x/12x
// DSA Sparse MLA Support", Changes item 2: paged MQA logits, FP8 decoded in
// the kernel, K-side scale applied to the fp32 dot).
//
// gfx950 design.  One wave owns one 64-token page at a time and computes the
// whole [64 heads x 64 tokens] block of one or two query rows with the fp8
// MFMA v_mfma_f32_32x32x64_f8f6f4 (M = 32 heads, N = 32 tokens, K = 64; the
// e4m3 decode happens inside the MFMA): 2 head tiles x 2 token steps x 2 K
// halves = 8 instructions per row and page, issued in pairs between the VALU
// operations of the previous pair's epilogue (a software pipeline over
// (row, token step, head tile) that holds two accumulators, not a row's
// four: 3 % fewer cycles at two rows per page; the page's next copy then
// waits longer to issue, since the CU's memory queue is what bounds the
// steady state).  (The 16x16x128 shape needs
// about 1.4x the issue time per product here, and that time was not hidden
// behind the loads.)  C layout: lane l holds 16 heads of token l % 32, so the
// weighted ReLU head sum is 32 in-lane FMAs (ReLU as one v_med3_f32) per
// token step, and one v_permlane32_swap leaves token l of the page in lane l
// -- one coalesced 256-byte store per row and page.
//
// Loads: each page (8 KB codes + 256 B scales) is copied whole into a per-wave
// LDS ring with global_load_lds_dwordx4, eight whole 128-byte key rows per
// instruction; key row n's 16-byte chunk c sits in slot c ^ ((n >> 1) & 7),
// so the B-operand reads (16 consecutive keys, one chunk) hit distinct
// banks.  Reading the operands straight from HBM in the MFMA layout touches
// 32 half-used lines per instruction and measured about 30 % slower.  Two
// pages per wave are in flight: the next copy into a slot goes out once the
// page in it has been read into registers and its logits stored.  The ring
// is wave-private, so no barrier follows the prefix build.
//
// Work balance: the pages of all sequences form one list; every workgroup
// (8 waves, one per CU) rebuilds its prefix sum in LDS and each wave takes an
// equal contiguous run of it (so the grid depends only on host hints and no
// wave sits idle on a short sequence).  A wave looks up the physical ids of
// up to 64 pages of its run with one lane-parallel block-table load; the q
// rows of its first sequence are loaded with it.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

struct PagedArgs {
  BatchArgs batch;
  const uint8_t* q;
  const float* w;
  const uint8_t* cache;
  int64_t page_stride;
  float* logits;
  int64_t logits_stride;
  int clean;
};

constexpr int kWavesPg = 8;                              // waves per workgroup, one workgroup per CU
constexpr int kRingPg = 2;                               // pages in flight per wave (LDS ring)
constexpr int kPageLds = kPage * kIdxDim + kPage * 4;    // 8448: codes, then the 64 scales
constexpr int kCopiesPerPage = kPage * kIdxDim / 1024 + 1;   // 8 code copies + 1 scale copy

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int n) { return (n >> 1) & 7; }
__device__ __attribute__((aligned(16))) uint8_t g_zero_page[kPageLds] = {};

struct PagedShared {
  unsigned char ring[kWavesPg][kRingPg][kPageLds];
  union {
    int pref[DSA_MAX_SEQS + 1];             // more than 64 sequences: one prefix per workgroup
    int wave_pref[kWavesPg][64 + 1];        // at most 64: a private prefix per wave
  };
  int wave_tot[kWavesPg];
};

// Pages to compute for sequence b: ceil(L_b / 64) if it has rows, else 0.
__device__ __forceinline__ int seq_pages(const BatchArgs& a, int b) {
  const int q0 = a.query_start[b], q1 = a.query_start[b + 1];
  if (q1 <= q0) return 0;
  return (clamp_len(a.seq_lens[b], a.max_seq_len) + kPage - 1) / kPage;
}

// pref[b] = sum of seq_pages over sequences before b; pref[B] = total.
__device__ void build_page_prefix(const BatchArgs& a, int* pref, int* wave_tot) {
  const int B = a.num_seqs;
  const int per = (B + blockDim.x - 1) / blockDim.x;
  const int start = threadIdx.x * per;
  const int stop = min(start + per, B);
  int local = 0;
  for (int b = start; b < stop; ++b) local += seq_pages(a, b);
  const int incl = wave_inclusive_scan(local);
  const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  if (lane_id() == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < nwaves; ++i) {
    if (i < wave) before += wave_tot[i];
    total += wave_tot[i];
  }
  int run = before + incl - local;
  for (int b = start; b < stop; ++b) {
    pref[b] = run;
    run += seq_pages(a, b);
  }
  if (threadIdx.x == 0) pref[B] = total;
  __syncthreads();
}

// Largest b with pref[b] <= p (p < total).
__device__ __forceinline__ int find_seq(const int* pref, int B, int p) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (pref[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ v8i load_v8i_cached(const uint8_t* p) {
  const uint4* s = reinterpret_cast<const uint4*>(p);
  uint4 x0 = s[0], x1 = s[1];
  v8i r;
  r[0] = x0.x; r[1] = x0.y; r[2] = x0.z; r[3] = x0.w;
  r[4] = x1.x; r[5] = x1.y; r[6] = x1.z; r[7] = x1.w;
  return r;
}

struct QRow {
  v8i q[2][2];       // A operands: head tile mt (32 heads), K half kh
  float w[2][16];    // weights of the 16 heads this lane holds per head tile
};

// A operand: lane l supplies head 32 mt + l % 32, code bytes 64 kh +
// 32 (l / 32) .. +32.  C layout: item i of lane l is head 32 mt + (i % 4) +
// 4 (l / 32) + 8 (i / 4) of token l % 32 (the layout the prefill kernel's
// in-bounds lane probe checked), so the lane's weights are those heads'.
__device__ __forceinline__ void load_qrow(QRow& t, const uint8_t* q, const float* w, int r, int lane) {
  const int hq = lane & 31, hk = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const uint8_t* qp = q + ((size_t)r * kIdxHeads + 32 * mt + hq) * kIdxDim + 32 * hk;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) t.q[mt][kh] = load_v8i_cached(qp + 64 * kh);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 ww = *reinterpret_cast<const float4*>(w + (size_t)r * kIdxHeads + 32 * mt + 8 * g + 4 * hk);
      t.w[mt][4 * g] = ww.x; t.w[mt][4 * g + 1] = ww.y; t.w[mt][4 * g + 2] = ww.z; t.w[mt][4 * g + 3] = ww.w;
    }
  }
}

// A half unit: one query row, one token step (32 tokens), one head tile
// (32 heads): the MFMA pair over both K halves.  b[kh]: B operand of the step.
__device__ __forceinline__ void half_mfma(const QRow& qr, const v8i (&b)[2], int mt, v16f& acc) {
  const v16f z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qr.q[mt][0], b[0], z, 0, 0, 0, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qr.q[mt][1], b[1], acc, 0, 0, 0, 0, 0, 0);
}

// Its weighted ReLU terms added into the four partial sums p (head tile 0
// first, then head tile 1, so the sum's order is fixed).
__device__ __forceinline__ void half_epilogue(const QRow& qr, int mt, const v16f& acc, float (&p)[4]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i & 3] = fmaf(qr.w[mt][i], relu_finite(acc[i]), p[i & 3]);
}

// Lane l holds half the heads of token l % 32 of both steps; one lane swap
// gives lanes 0-31 the other half of step 0 and lanes 32-63 the other half
// of step 1, so afterwards lane l holds page token l.
__device__ __forceinline__ float row_logit(float part0, float part1) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int QL>
__global__ void __launch_bounds__(64 * kWavesPg) indexer_paged_kernel(PagedArgs a) {
  __shared__ PagedShared sh;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int B = a.batch.num_seqs;
  // Page prefix over the sequences.  With at most 64 sequences every wave
  // builds its own with one wave scan (lane b: sequence b) into a private LDS
  // copy -- no workgroup barrier between the kernel's start and its first
  // block-table load; more sequences take the workgroup-wide build.
  const int* s_pref;
  // with at most 64 sequences lane b also keeps sequence b's row range and
  // length, so switching sequences needs no memory round trip
  int sq0 = 0, sq1 = 0, sL = 0;
  if (B <= 64) {
    if (lane < B) {
      sq0 = a.batch.query_start[lane];
      sq1 = a.batch.query_start[lane + 1];
      sL = clamp_len(a.batch.seq_lens[lane], a.batch.max_seq_len);
    }
    const int pages = lane < B && sq1 > sq0 ? (sL + kPage - 1) / kPage : 0;
    const int incl = wave_inclusive_scan(pages);
    int* wp = sh.wave_pref[wave];
    if (lane < B) wp[lane] = incl - pages;
    if (lane == 63) wp[B] = incl;     // lanes past B add nothing: lane 63 holds the total
    s_pref = wp;
  } else {
    build_page_prefix(a.batch, sh.pref, sh.wave_tot);
    s_pref = sh.pref;
  }

  const int total = s_pref[B];
  const int64_t nw = (int64_t)gridDim.x * kWavesPg;
  const int64_t gw = (int64_t)blockIdx.x * kWavesPg + wave;
  const int p_begin = (int)((int64_t)total * gw / nw);
  const int p_end = (int)((int64_t)total * (gw + 1) / nw);
  if (p_begin >= p_end) return;

  // Page table of up to 64 pages of this wave's run, one page per lane: its
  // sequence, its page index inside the sequence and its physical page (-1
  // when out of range).  One lane-parallel block-table load replaces a
  // dependent load per page.
  int pb = -1, lb = 0, lj = 0, lid = -1;
  auto load_batch = [&](int first) {
    pb = first;
    const int p = first + lane;
    lb = 0; lj = 0; lid = -1;
    if (p < p_end) {
      lb = find_seq(s_pref, B, p);
      lj = p - s_pref[lb];
      const int id = a.batch.block_table[(int64_t)lb * a.batch.bt_stride + lj];
      lid = (id >= 0 && id < a.batch.num_pages) ? id : -1;
    }
  };
  // Copy of page p into ring slot (p - p_begin) % kRingPg: 8 copies of eight key
  // rows each (lane l: row 8 i + l / 8, slot l % 8 holding chunk
  // (l % 8) ^ swz(row)), then the 64 scales (lanes 0-15).  A page outside the
  // cache copies a static zero page, so every page costs exactly
  // kCopiesPerPage copies and the waits below count them exactly.
  int m_id[kRingPg], m_b[kRingPg], m_j[kRingPg];
  auto issue = [&](int p) {
    if (p - pb >= 64) load_batch(p);
    const int slot = (p - p_begin) % kRingPg;
    m_id[slot] = __builtin_amdgcn_readlane(lid, p - pb);
    m_b[slot] = __builtin_amdgcn_readlane(lb, p - pb);
    m_j[slot] = __builtin_amdgcn_readlane(lj, p - pb);
    const uint8_t* src = m_id[slot] >= 0 ? a.cache + (int64_t)m_id[slot] * a.page_stride : g_zero_page;
    const uint32_t dst = lds_addr(sh.ring[wave][slot]);
    const int rl = lane >> 3, sl = lane & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + rl;
      lds_dma16(src + row * kIdxDim + 16 * (sl ^ swz(row)), dst + i * 1024);
    }
    if (lane < 16) lds_dma16(src + kIdxScaleOff + 16 * lane, dst + kPage * kIdxDim);
  };

  QRow qr[QL];
  int cur_b = -1, row0 = 0, nrows = 0, L = 0, q_len = 0, q0 = 0;
  // Switch to sequence b; with at most QL rows their q and weights are loaded
  // once here.
  auto set_seq = [&](int b) {
    cur_b = b;
    int q1;
    if (B <= 64) {
      q0 = __builtin_amdgcn_readlane(sq0, b);
      q1 = __builtin_amdgcn_readlane(sq1, b);
      L = __builtin_amdgcn_readlane(sL, b);
    } else {
      q0 = a.batch.query_start[b];
      q1 = a.batch.query_start[b + 1];
      L = clamp_len(a.batch.seq_lens[b], a.batch.max_seq_len);
    }
    q_len = q1 - q0;
    row0 = max(q0, 0);
    nrows = min(q1, a.batch.num_rows) - row0;
    if (nrows <= QL) {
#pragma unroll
      for (int jj = 0; jj < QL; ++jj)
        if (jj < nrows) load_qrow(qr[jj], a.q, a.w, row0 + jj, lane);
    }
  };

  // B-operand offsets inside a page: token 32 ks + l % 32, chunks
  // 4 kh + 2 (l / 32) and the next one.
  const int nb = lane & 31, hb = lane >> 5;
  int boff[2][2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 32 * ks + nb;
        boff[ks][kh][c] = row * kIdxDim + 16 * ((4 * kh + 2 * hb + c) ^ swz(row));
      }

  auto compute = [&](int p) {
    const int slot = (p - p_begin) % kRingPg;
    const int id = m_id[slot], b = m_b[slot], j = m_j[slot];
    const unsigned char* tile = sh.ring[wave][slot];
    v8i bop[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const v4i x0 = *reinterpret_cast<const v4i*>(tile + boff[ks][kh][0]);
        const v4i x1 = *reinterpret_cast<const v4i*>(tile + boff[ks][kh][1]);
        bop[ks][kh] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    const float scale = reinterpret_cast<const float*>(tile + kPage * kIdxDim)[lane];
    wait_lgkmcnt0();
    if (b != cur_b) set_seq(b);

    const int s = j * kPage + lane;  // logical token of this lane
    const bool in_stride = s < a.logits_stride;
    for (int g0 = 0; g0 < nrows; g0 += QL) {
      if (nrows > QL) {
#pragma unroll
        for (int jj = 0; jj < QL; ++jj)
          if (g0 + jj < nrows) load_qrow(qr[jj], a.q, a.w, row0 + g0 + jj, lane);
      }
      // Software pipeline over half units h = (row jj, step ks, head tile
      // mt), in that order: the MFMA pair of half unit h + 1 is issued
      // between the VALU operations of half unit h's epilogue.  A group with
      // fewer than QL rows runs every half unit anyway (the extra rows'
      // results are dropped), so the schedule has no branches.
      constexpr int NH = 4 * QL;
      v16f acc[2];
      float p[QL][2][4];
#pragma unroll
      for (int jj = 0; jj < QL; ++jj)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int c = 0; c < 4; ++c) p[jj][ks][c] = 0.f;
      half_mfma(qr[0], bop[0], 0, acc[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int hn = h + 1;
        if (hn < NH) half_mfma(qr[hn >> 2], bop[(hn >> 1) & 1], hn & 1, acc[hn & 1]);
        half_epilogue(qr[h >> 2], h & 1, acc[h & 1], p[h >> 2][(h >> 1) & 1]);
        if (hn < NH) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float part[QL][2];
#pragma unroll
      for (int jj = 0; jj < QL; ++jj)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          part[jj][ks] = (p[jj][ks][0] + p[jj][ks][1]) + (p[jj][ks][2] + p[jj][ks][3]);
          // computed here, not sunk into the store's branch below
          asm volatile("" : "+v"(part[jj][ks]));
        }
#pragma unroll
      for (int jj = 0; jj < QL; ++jj) {
        if (g0 + jj >= nrows) break;
        const int r = row0 + g0 + jj;
        int e = L - q_len + (r - q0) + 1;
        e = e < 0 ? 0 : e;
        const float v = id >= 0 ? row_logit(part[jj][0], part[jj][1]) * scale : -INFINITY;
        float* dst = a.logits + (int64_t)r * a.logits_stride + s;
        if (s < e) {
          if (in_stride) *dst = v;
        } else if (a.clean && in_stride) {
          *dst = -INFINITY;
        }
      }
    }
    // page p + kRingPg goes into this slot (its data is in registers since
    // the wait above); issued after the page's products and stores rather
    // than before them (GRBM cycles -0.9 % with two query rows per page over
    // 64 sequences, -4.2 % with one row per page over 32 sequences)
    if (p + kRingPg < p_end) issue(p + kRingPg);
  };

  load_batch(p_begin);
  // the first pages' copies go out as soon as the block table is in, then
  // the q rows of the first page's sequence (their latency hides behind the
  // copies')
#pragma unroll
  for (int i = 0; i < kRingPg; ++i)
    if (p_begin + i < p_end) issue(p_begin + i);
  set_seq(find_seq(s_pref, B, p_begin));
  for (int p = p_begin; p < p_end; ++p) {
    // this page's copies; what was issued after them (the next pages' copies,
    // logit stores, any reload) may stay in flight
    const int later = min(p_end - 1 - p, kRingPg - 1);
    static_assert(kRingPg <= 4, "wait cases");
    if (later >= 3) wait_vmcnt<3 * kCopiesPerPage>();
    else if (later == 2) wait_vmcnt<2 * kCopiesPerPage>();
    else if (later == 1) wait_vmcnt<kCopiesPerPage>();
    else wait_vmcnt<0>();
    compute(p);
  }
}

// -inf over the columns past each row's computed pages: [64*pages_b, stride).
__global__ void __launch_bounds__(256) indexer_clean_tail_kernel(PagedArgs a, int segs_per_row) {
  const int64_t nseg = (int64_t)a.batch.num_rows * segs_per_row;
  for (int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); seg < nseg; seg += (int64_t)gridDim.x * 4) {
    const int r = (int)(seg / segs_per_row);
    const int c0 = (int)(seg % segs_per_row) * 256;
    const int b = seq_of_row(a.batch.query_start, a.batch.num_seqs, r);
    int first = 0;
    if (b >= 0) first = ((clamp_len(a.batch.seq_lens[b], a.batch.max_seq_len) + kPage - 1) / kPage) * kPage;
    float* row = a.logits + (int64_t)r * a.logits_stride;
    for (int c = c0 + 4 * lane_id(); c < c0 + 256; c += 256) {
      if (c >= first && c + 3 < a.logits_stride) {
        *reinterpret_cast<float4*>(row + c) = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      } else {
        for (int t = 0; t < 4; ++t)
          if (c + t >= first && c + t < a.logits_stride) row[c + t] = -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_indexer_paged(const BatchArgs& batch, const uint8_t* q, const float* w,
                                const uint8_t* cache, int64_t page_stride, float* logits,
                                int64_t logits_stride, int clean, int num_cus, hipStream_t stream) {
  PagedArgs a{batch, q, w, cache, page_stride, logits, logits_stride, clean};
  const int64_t max_pages = (int64_t)batch.num_seqs * ((batch.max_seq_len + kPage - 1) / kPage);
  // One 8-wave workgroup per CU (its LDS ring takes most of the CU); fewer
  // when there is less than a page per wave.
  int64_t grid = (max_pages + kWavesPg - 1) / kWavesPg;
  grid = grid < 1 ? 1 : grid;
  if (grid > (int64_t)num_cus) grid = num_cus;
  if (batch.num_rows > 0 && batch.num_seqs > 0 && max_pages > 0) {
    if (batch.max_q_len <= 1) {
      hipLaunchKernelGGL(indexer_paged_kernel<1>, dim3((unsigned)grid), dim3(64 * kWavesPg), 0, stream, a);
    } else {
      hipLaunchKernelGGL(indexer_paged_kernel<2>, dim3((unsigned)grid), dim3(64 * kWavesPg), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (clean && batch.num_rows > 0) {
    const int segs = (int)((logits_stride + 255) / 256);
    int64_t total = (int64_t)batch.num_rows * segs;
    int64_t g2 = (total + 3) / 4;
    if (g2 > 4 * (int64_t)num_cus) g2 = 4 * (int64_t)num_cus;
    hipLaunchKernelGGL(indexer_clean_tail_kernel, dim3((unsigned)g2), dim3(256), 0, stream, a, segs);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace dsa
