// Sparse MLA decode over the top-k selected latent rows.
//
// For every row r and head h, over the valid entries s of indices[r, :]
// (vLLM PR "[Feature] TRITON_MLA_SPARSE backend ...", Changes item 3):
//   z_s = softmax_scale * q[r,h,:576] . c_s[:576]
//   out[r,h,:] = sum_s softmax(z)_s c_s[:512],  lse[r,h] = ln sum_s exp(z_s)
// with split-KV partials merged N-way by online softmax, a single-pass fast
// path when there is one split, and -1e30 as the running-max sentinel so an
// all-masked tile never computes (-inf) - (-inf).
//
// gfx950 design.
//  * Workgroup = 4 waves = one (row, split, block of 16 or 32 heads).  Its
//    k-slot range is walked in tiles of 64 selected tokens.
//  * Gather: the 64 selected latent rows (64 x 1152 B) are copied from HBM
//    straight into LDS with global_load_lds_dwordx4 (no VGPR round trip).  Each
//    lane supplies its own source address, so the gather through the block
//    table costs nothing extra; masked slots read a static zero row.  Rows are
//    padded to 73 sixteen-byte chunks (1168 B): an odd chunk count puts the 16
//    token rows one MFMA operand read touches on distinct LDS banks, and every
//    operand address stays "lane base + immediate".
//  * QK: S^T[token, head] = C . Q^T with v_mfma_f32_16x16x32_bf16 (M = 16
//    tokens, N = 16 heads, K = 32 dims, 18 steps over 576 dims); Q stays in
//    registers for the whole workgroup.
//  * Softmax: the S^T accumulator layout gives each lane one head and 4
//    tokens of each token tile, so the running max / sum need only two
//    cross-lane steps per tile, and the probabilities are already in the B
//    operand layout of the PV product.
//  * PV: O^T[dim, head] += V^T . P^T (M = 16 dims, N = 16 heads, K = 32
//    tokens) with V^T read from the token-major LDS tile.
//  * Each wave owns 16 heads x 128 dims (16-head rows) or 16 heads x 256 dims
//    (the rest, in 32-head workgroups), so the output accumulator stays at
//    <= 64 VGPRs; the head blocks of one (row, split) are placed on one XCD so
//    their identical gathers meet in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kTile = 64;                      // selected tokens per LDS tile
constexpr int kChunks = kKvDim * 2 / 16;       // 72 sixteen-byte chunks per latent row
constexpr int kRowChunks = kChunks + 1;        // 73: one pad chunk per LDS row
constexpr int kRowStride = kRowChunks * 16;    // 1168 bytes
constexpr int kTileBytes = kTile * kRowStride; // 74752
constexpr int kTileLoads = kTile * kRowChunks / 64;     // 73 wave-wide 1 KB loads per tile
constexpr int kLoadsPerWave = (kTileLoads + 3) / 4;    // 19 (the last wave issues 16)

__device__ __attribute__((aligned(16))) uint4 g_zero_row[kChunks] = {};

struct MlaArgs {
  BatchArgs batch;
  const uint16_t* q;
  int H;
  const uint16_t* kv;
  int64_t kv_stride;       // elements between pages
  const int32_t* indices;
  int k;
  float scale_log2;        // softmax_scale * log2(e)
  int splits;
  int split_slots;         // k slots per split (multiple of 64)
  int head_blocks;         // H / 16 for H == 16 (1), else H / 32
  uint16_t* out;
  float* lse;
  float* part_acc;         // [splits, R, H, 512]
  float* part_ml;          // [splits, R, H, 2]: running max (log2 domain), sum
};

__device__ __forceinline__ v8bf as_v8bf(uint4 x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

template <int DQ>
__global__ void __launch_bounds__(256, 2) sparse_mla_kernel(MlaArgs a) {
  constexpr int HT = 4 / DQ;          // head tiles of 16 per workgroup
  constexpr int DW = kVDim / DQ;      // output dims per wave
  constexpr int NDT = DW / 16;        // dim tiles per wave
  __shared__ __attribute__((aligned(16))) unsigned char s_tile[kTileBytes];
  __shared__ const unsigned char* s_rowptr[kTile];
  __shared__ uint64_t s_mask;

  const int R = a.batch.num_rows;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;            // k-group of the MFMA operands
  const int n16 = lane & 15;

  // Workgroup -> (row, split, head block); the head blocks of one (row, split)
  // land on the same XCD (workgroup ids 8 apart) so their identical gathers
  // meet in that XCD's L2.
  const int bid = blockIdx.x;
  const int q8 = bid >> 3;
  const int hb = q8 % a.head_blocks;
  const int rest = (q8 / a.head_blocks) * 8 + (bid & 7);
  if (rest >= R * a.splits) return;
  const int r = rest / a.splits;
  const int sp = rest % a.splits;

  const int ht = wave % HT, dq = wave / HT;
  const int h = hb * (16 * HT) + ht * 16 + n16;
  const int d_base = dq * DW;

  const int b = seq_of_row(a.batch.query_start, a.batch.num_seqs, r);
  const int e = b >= 0 ? row_extent(a.batch, b, r) : 0;
  const int slot0 = sp * a.split_slots;
  const int slot1 = min(slot0 + a.split_slots, a.k);

  // Q^T operand: lane supplies head h, dims 32*ks + 8*g .. +8.
  uint4 qreg[18];
  {
    const uint16_t* qp = a.q + ((int64_t)r * a.H + h) * kKvDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);
  }
  // LDS operand bases: QK reads token n16 (+16*tt), dims 8*g (+32*ks);
  // PV reads tokens 4*g (+16*tt + i), dim d_base + n16 (+16*dt).
  const unsigned char* qk_base = s_tile + n16 * kRowStride + 16 * g;
  const unsigned char* pv_base = s_tile + 4 * g * kRowStride + 2 * (d_base + n16);

  v4f acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = kMaskSentinel;   // running max of the log2-domain scores of head h
  float l_part = 0.f;            // this lane's share of the running sum

  for (int t0 = slot0; t0 < slot1; t0 += kTile) {
    __syncthreads();  // the previous tile is no longer being read
    if (threadIdx.x < kTile) {
      const int j = t0 + (int)threadIdx.x;
      const int idx = j < slot1 ? a.indices[(int64_t)r * a.k + j] : -1;
      bool valid = idx >= 0 && idx < e;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(g_zero_row);
      if (valid) {
        const int page = a.batch.block_table[(int64_t)b * a.batch.bt_stride + (idx >> 6)];
        valid = page >= 0 && page < a.batch.num_pages;
        if (valid) src = reinterpret_cast<const unsigned char*>(a.kv + (int64_t)page * a.kv_stride + (idx & 63) * kKvDim);
      }
      s_rowptr[threadIdx.x] = src;
      const uint64_t m = __ballot(valid);
      if (threadIdx.x == 0) s_mask = m;
    }
    __syncthreads();
    const uint64_t mask = s_mask;
    if (mask == 0) continue;

    // Gather: LDS chunk p = 64 * load + lane holds (row p / 73, chunk p % 73);
    // chunk 72 of each row is padding and re-reads chunk 0 of the row.
    {
      int p = (wave * kLoadsPerWave) * 64 + lane;
      // Recompute the cursor per tile instead of keeping 19 hoisted copies of it
      // live across the loop (they would not fit in registers).
      asm volatile("" : "+v"(p));
      int t = p / kRowChunks;
      int c = p - t * kRowChunks;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int blk = wave * kLoadsPerWave + i;
        if (blk < kTileLoads) {
          const unsigned char* src = s_rowptr[t] + (c < kChunks ? (c << 4) : 0);
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                           reinterpret_cast<void*>(s_tile + blk * 1024), 16, 0, 0);
        }
        c += 64;
        if (c >= kRowChunks) { c -= kRowChunks; ++t; }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // S^T = C . Q^T for the 4 token tiles of 16
    v4f s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const uint4 cv = *reinterpret_cast<const uint4*>(qk_base + tt * 16 * kRowStride + 64 * ks);
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(cv), as_v8bf(qreg[ks]), s[tt], 0, 0, 0);
      }
    }
    // online softmax (log2 domain); lane holds tokens 16*tt + 4*g + i of head h
    float tmax = kMaskSentinel;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (mask >> (tt * 16 + 4 * g + i)) & 1ull;
        const float z = v ? s[tt][i] * a.scale_log2 : kMaskSentinel;
        s[tt][i] = z;
        tmax = fmaxf(tmax, z);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (mask >> (tt * 16 + 4 * g + i)) & 1ull;
        const float pv = v ? exp2f(s[tt][i] - m_new) : 0.f;
        s[tt][i] = pv;
        psum += pv;
      }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;

    // O^T += V^T . P^T, 32 tokens (two token tiles) per MFMA; k slot i of lane
    // group g is token 16*(2tp) + 4g + i, slot 4 + i is token 16*(2tp+1) + 4g + i.
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      v8bf pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)s[2 * tp][i];
        pb[4 + i] = (__bf16)s[2 * tp + 1][i];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const unsigned char* vb = pv_base + (2 * tp) * 16 * kRowStride + 32 * dt;
        v8s vv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vv[i] = *reinterpret_cast<const short*>(vb + i * kRowStride);
          vv[4 + i] = *reinterpret_cast<const short*>(vb + (16 + i) * kRowStride);
        }
        v8bf va;
        __builtin_memcpy(&va, &vv, 16);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[dt], 0, 0, 0);
      }
    }
  }

  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  if (a.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = a.out + ((int64_t)r * a.H + h) * kVDim + d_base + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16_rne(acc[dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[dt][1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16_rne(acc[dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + dt * 16) = pk;
    }
    if (dq == 0 && g == 0)
      a.lse[(int64_t)r * a.H + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t base = ((int64_t)sp * R + r) * a.H + h;
    float* pa = a.part_acc + base * kVDim + d_base + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4*>(pa + dt * 16) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (dq == 0 && g == 0) {
      a.part_ml[base * 2] = l_tot > 0.f ? m_run : kMaskSentinel;
      a.part_ml[base * 2 + 1] = l_tot;
    }
  }
}

// N-way merge of the split partials: one wave per (row, head), 8 dims per lane.
__global__ void __launch_bounds__(256) sparse_mla_merge_kernel(MlaArgs a) {
  const int R = a.batch.num_rows;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)R * a.H) return;
  const int lane = lane_id();
  const int64_t RH = (int64_t)R * a.H;
  float M = kMaskSentinel;
  for (int i = 0; i < a.splits; ++i) M = fmaxf(M, a.part_ml[(i * RH + pair) * 2]);
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < a.splits; ++i) {
    const float mi = a.part_ml[(i * RH + pair) * 2];
    const float li = a.part_ml[(i * RH + pair) * 2 + 1];
    const float wgt = li > 0.f ? exp2f(mi - M) : 0.f;
    L += li * wgt;
    const float4* src = reinterpret_cast<const float4*>(a.part_acc + (i * RH + pair) * kVDim + 8 * lane);
    const float4 x0 = src[0], x1 = src[1];
    o[0] += wgt * x0.x; o[1] += wgt * x0.y; o[2] += wgt * x0.z; o[3] += wgt * x0.w;
    o[4] += wgt * x1.x; o[5] += wgt * x1.y; o[6] += wgt * x1.z; o[7] += wgt * x1.w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint4 pk;
  pk.x = (uint32_t)f32_to_bf16_rne(o[0] * inv) | ((uint32_t)f32_to_bf16_rne(o[1] * inv) << 16);
  pk.y = (uint32_t)f32_to_bf16_rne(o[2] * inv) | ((uint32_t)f32_to_bf16_rne(o[3] * inv) << 16);
  pk.z = (uint32_t)f32_to_bf16_rne(o[4] * inv) | ((uint32_t)f32_to_bf16_rne(o[5] * inv) << 16);
  pk.w = (uint32_t)f32_to_bf16_rne(o[6] * inv) | ((uint32_t)f32_to_bf16_rne(o[7] * inv) << 16);
  *reinterpret_cast<uint4*>(a.out + pair * kVDim + 8 * lane) = pk;
  if (lane == 0) a.lse[pair] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

MlaPlan plan_sparse_mla(int num_rows, int max_seq_len, int H, int k, int num_splits, int num_cus) {
  MlaPlan p{};
  const int head_blocks = H == 16 ? 1 : H / 32;   // 16- or 32-head workgroups
  const int live = max(1, min(k, max(max_seq_len, 1)));
  const int tiles = (live + kTile - 1) / kTile;      // tiles that can hold valid entries
  const int all_tiles = (k + kTile - 1) / kTile;
  int s = num_splits;
  if (s <= 0) {
    // about one 4-wave workgroup per CU, never more splits than useful tiles
    const int64_t groups = (int64_t)max(num_rows, 1) * head_blocks;
    s = (int)((num_cus + groups - 1) / groups);
    s = max(1, min(s, tiles));
  }
  s = max(1, min(s, all_tiles));
  p.split_slots = ((k + s - 1) / s + kTile - 1) / kTile * kTile;
  p.splits = (k + p.split_slots - 1) / p.split_slots;
  p.head_blocks = head_blocks;
  return p;
}

size_t sparse_mla_workspace_bytes(int num_rows, int H, const MlaPlan& p) {
  if (p.splits <= 1 || num_rows <= 0) return 0;
  const size_t n = (size_t)p.splits * num_rows * H;
  size_t bytes = n * kVDim * 4;
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += n * 8;
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_sparse_mla(const BatchArgs& batch, const uint16_t* q, int H, const uint16_t* kv,
                             int64_t kv_stride, const int32_t* indices, int k, float softmax_scale,
                             const MlaPlan& p, uint16_t* out, float* lse, void* workspace,
                             hipStream_t stream) {
  if (batch.num_rows <= 0) return hipSuccess;
  MlaArgs a{};
  a.batch = batch;
  a.q = q;
  a.H = H;
  a.kv = kv;
  a.kv_stride = kv_stride;
  a.indices = indices;
  a.k = k;
  a.scale_log2 = softmax_scale * kLog2e;
  a.splits = p.splits;
  a.split_slots = p.split_slots;
  a.head_blocks = p.head_blocks;
  a.out = out;
  a.lse = lse;
  if (p.splits > 1) {
    const size_t n = (size_t)p.splits * batch.num_rows * H;
    char* ws = static_cast<char*>(workspace);
    a.part_acc = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws + (((size_t)n * kVDim * 4 + 255) & ~(size_t)255));
  }
  const int64_t units = (int64_t)batch.num_rows * p.splits;
  const int64_t grid = (units + 7) / 8 * 8 * p.head_blocks;
  if (H == 16) {
    hipLaunchKernelGGL(sparse_mla_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sparse_mla_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1) return err;
  const int64_t pairs = (int64_t)batch.num_rows * H;
  hipLaunchKernelGGL(sparse_mla_merge_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
