// Lightning-indexer logits over the paged FP8 indexer-K cache, decode shape.
//
// Computes logits[r, s] = sum_h w[r, h] * relu(q[r, h, :] . k[s, :]) * kscale[s]
// for s < e_r (vLLM PR "[Feature] TRITON_MLA_SPARSE backend for SM8x/11x/12x
// DSA Sparse MLA Support", Changes item 2: paged MQA logits, FP8 decoded in
// the kernel, K-side scale applied to the fp32 dot).
//
// gfx950 design.  One wave owns one 64-token page at a time and computes the
// whole [64 heads x 64 tokens] block of one or two query rows with the fp8
// MFMA v_mfma_f32_16x16x128_f8f6f4 (M = 16 heads, N = 16 tokens, K = 128, the
// full head dim in one instruction): 4 head tiles x 4 token tiles = 16
// instructions per row and page.  The e4m3 decode happens inside the MFMA.
// Accumulator layout: lane l holds token 16*nt + (l & 15) and heads
// 16*mt + 4*(l >> 4) + i, so the weighted ReLU head sum is 16 in-lane FMAs
// (ReLU as one v_med3_f32) followed by a reduce-scatter of two VALU lane
// swaps (v_permlane32_swap, v_permlane16_swap) that leaves token l of the page
// in lane l -- one coalesced 256-byte store per row and page.
//
// Work balance: the pages of all sequences form one list; every workgroup
// rebuilds its prefix sum in LDS and each wave takes an equal contiguous run
// of it (so the grid depends only on host hints and no wave sits idle on
// a short sequence).  A wave looks up the physical ids of up to 64 pages of
// its run with one lane-parallel block-table load, and keeps the K tiles of
// its next pages in flight in a register ring while it multiplies the current
// one (two pages for one query row per sequence, one for two rows, which keeps
// two waves per SIMD).  HBM traffic per page: 8 KB codes + 256 B scales, read
// once, coalesced 16-byte loads.
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

// Pages to compute for sequence b: ceil(L_b / 64) if it has rows, else 0.
__device__ __forceinline__ int seq_pages(const BatchArgs& a, int b) {
  const int q0 = a.query_start[b], q1 = a.query_start[b + 1];
  if (q1 <= q0) return 0;
  return (clamp_len(a.seq_lens[b], a.max_seq_len) + kPage - 1) / kPage;
}

// s_pref[b] = sum of seq_pages over sequences before b; s_pref[B] = total.
__device__ void build_page_prefix(const BatchArgs& a, int* s_pref, int* s_wave) {
  const int B = a.num_seqs;
  const int per = (B + blockDim.x - 1) / blockDim.x;
  const int start = threadIdx.x * per;
  const int stop = min(start + per, B);
  int local = 0;
  for (int b = start; b < stop; ++b) local += seq_pages(a, b);
  int incl = wave_inclusive_scan(local);
  const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  if (lane_id() == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < nwaves; ++i) {
    if (i < wave) before += s_wave[i];
    total += s_wave[i];
  }
  int run = before + incl - local;
  for (int b = start; b < stop; ++b) {
    s_pref[b] = run;
    run += seq_pages(a, b);
  }
  if (threadIdx.x == 0) s_pref[B] = total;
  __syncthreads();
}

// Largest b with s_pref[b] <= p (p < total).
__device__ __forceinline__ int find_seq(const int* s_pref, int B, int p) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

struct KTile {
  v8i k[4];     // B operands of the 4 token tiles
  float scale;  // kscale of token `lane` of the page
};

typedef int v4i __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) load of 32 bytes: K pages are read exactly once.
__device__ __forceinline__ v8i load_v8i(const uint8_t* p) {
  const v4i* s = reinterpret_cast<const v4i*>(p);
  const v4i x0 = __builtin_nontemporal_load(s);
  const v4i x1 = __builtin_nontemporal_load(s + 1);
  v8i r;
  r[0] = x0[0]; r[1] = x0[1]; r[2] = x0[2]; r[3] = x0[3];
  r[4] = x1[0]; r[5] = x1[1]; r[6] = x1[2]; r[7] = x1[3];
  return r;
}

__device__ __forceinline__ v8i load_v8i_cached(const uint8_t* p) {
  const uint4* s = reinterpret_cast<const uint4*>(p);
  uint4 x0 = s[0], x1 = s[1];
  v8i r;
  r[0] = x0.x; r[1] = x0.y; r[2] = x0.z; r[3] = x0.w;
  r[4] = x1.x; r[5] = x1.y; r[6] = x1.z; r[7] = x1.w;
  return r;
}

__device__ __forceinline__ void load_ktile(KTile& t, const uint8_t* page, int lane) {
  const int n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) t.k[nt] = load_v8i(page + (16 * nt + n) * kIdxDim + kg * 32);
  t.scale = __builtin_nontemporal_load(reinterpret_cast<const float*>(page + kIdxScaleOff) + lane);
}

struct QRow {
  v8i q[4];      // A operands of the 4 head tiles
  v4f w[4];      // weights of this lane's 16 heads (4 per head tile)
};

__device__ __forceinline__ void load_qrow(QRow& t, const uint8_t* q, const float* w, int r, int lane) {
  const int n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    t.q[mt] = load_v8i_cached(q + ((size_t)r * kIdxHeads + 16 * mt + n) * kIdxDim + kg * 32);
    const float4 ww = *reinterpret_cast<const float4*>(w + (size_t)r * kIdxHeads + 16 * mt + 4 * kg);
    t.w[mt][0] = ww.x; t.w[mt][1] = ww.y; t.w[mt][2] = ww.z; t.w[mt][3] = ww.w;
  }
}

// sum_h w_h * relu(q_h . k_s) for token `lane` of the page (before the K scale).
__device__ __forceinline__ float page_row_logit(const QRow& qr, const KTile& kt, int lane) {
  // The four products of a token tile are issued before any is consumed (and
  // the next tile's before this tile's epilogue), so no product waits alone
  // for the MFMA latency.
  float part[4];
  v4f acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    acc[0][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qr.q[mt], kt.k[0], v4f{0.f, 0.f, 0.f, 0.f},
                                                                  0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (nt + 1 < 4) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[(nt + 1) & 1][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            qr.q[mt], kt.k[nt + 1], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(qr.w[mt][i], relu_finite(acc[nt & 1][mt][i]), s);
    part[nt] = s;
  }
  // Reduce-scatter over the 4 lane groups g = lane >> 4 (each holds 16 of the
  // 64 heads of every token tile): afterwards lane l holds token tile g,
  // column l & 15, i.e. page token l.
  const int g = lane >> 4;
  const bool hi = g >= 2;
  float send0 = hi ? part[0] : part[2];
  float send1 = hi ? part[1] : part[3];
  float a0 = (hi ? part[2] : part[0]) + lane_xor32(send0);
  float a1 = (hi ? part[3] : part[1]) + lane_xor32(send1);
  const bool odd = g & 1;
  float send = odd ? a0 : a1;
  return (odd ? a1 : a0) + lane_xor16(send);
}

template <int QL>
__global__ void __launch_bounds__(256) indexer_paged_kernel(PagedArgs a) {
  __shared__ int s_pref[DSA_MAX_SEQS + 1];
  __shared__ int s_wave[4];
  build_page_prefix(a.batch, s_pref, s_wave);

  const int lane = lane_id();
  const int B = a.batch.num_seqs;
  const int total = s_pref[B];
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
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
  // K tiles of the next kRing pages stay in flight (a register ring); each
  // slot keeps its page's id, sequence and page index, so reloading the page
  // table for later pages never disturbs a pending slot.
  constexpr int kRing = QL == 1 ? 2 : 1;
  KTile kt[kRing];
  int m_id[kRing], m_b[kRing], m_j[kRing];
  auto issue = [&](int slot, int p) {
    if (p < p_end) {
      if (p - pb >= 64) load_batch(p);
      m_id[slot] = __builtin_amdgcn_readlane(lid, p - pb);
      m_b[slot] = __builtin_amdgcn_readlane(lb, p - pb);
      m_j[slot] = __builtin_amdgcn_readlane(lj, p - pb);
      if (m_id[slot] >= 0) load_ktile(kt[slot], a.cache + (int64_t)m_id[slot] * a.page_stride, lane);
    }
  };

  QRow qr[QL];
  int cur_b = -1, row0 = 0, nrows = 0, L = 0, q_len = 0, q0 = 0;

  auto compute = [&](int slot) {
    const KTile& t = kt[slot];
    const int id = m_id[slot], b = m_b[slot], j = m_j[slot];
    if (b != cur_b) {
      cur_b = b;
      q0 = a.batch.query_start[b];
      const int q1 = a.batch.query_start[b + 1];
      q_len = q1 - q0;
      row0 = max(q0, 0);
      nrows = min(q1, a.batch.num_rows) - row0;
      L = clamp_len(a.batch.seq_lens[b], a.batch.max_seq_len);
      if (nrows <= QL) {
#pragma unroll
        for (int jj = 0; jj < QL; ++jj)
          if (jj < nrows) load_qrow(qr[jj], a.q, a.w, row0 + jj, lane);
      }
    }
    const int s = j * kPage + lane;  // logical token of this lane
    const bool in_stride = s < a.logits_stride;
    for (int g0 = 0; g0 < nrows; g0 += QL) {
      if (nrows > QL) {
#pragma unroll
        for (int jj = 0; jj < QL; ++jj)
          if (g0 + jj < nrows) load_qrow(qr[jj], a.q, a.w, row0 + g0 + jj, lane);
      }
#pragma unroll
      for (int jj = 0; jj < QL; ++jj) {
        if (g0 + jj >= nrows) break;
        const int r = row0 + g0 + jj;
        int e = L - q_len + (r - q0) + 1;
        e = e < 0 ? 0 : e;
        const float v = id >= 0 ? page_row_logit(qr[jj], t, lane) * t.scale : -INFINITY;
        float* dst = a.logits + (int64_t)r * a.logits_stride + s;
        if (s < e) {
          if (in_stride) *dst = v;
        } else if (a.clean && in_stride) {
          *dst = -INFINITY;
        }
      }
    }
  };

  load_batch(p_begin);
#pragma unroll
  for (int i = 0; i < kRing; ++i) issue(i, p_begin + i);
  for (int p = p_begin; p < p_end; p += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      if (p + i < p_end) {
        compute(i);
        issue(i, p + i + kRing);
      }
    }
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
  // Two 4-wave workgroups per CU keep every SIMD busy; fewer when there is
  // less than a page per wave.
  int64_t grid = (max_pages + 3) / 4;
  grid = grid < 1 ? 1 : grid;
  if (grid > 2 * (int64_t)num_cus) grid = 2 * (int64_t)num_cus;
  if (batch.num_rows > 0 && batch.num_seqs > 0 && max_pages > 0) {
    if (batch.max_q_len <= 1) {
      hipLaunchKernelGGL(indexer_paged_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL(indexer_paged_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
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
