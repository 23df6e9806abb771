// Lightning-indexer logits for chunked prefill (many query rows per sequence).
//
// Same operation as the paged decode kernel (vLLM PR "[Feature] TRITON_MLA_SPARSE
// backend ...", Changes item 2: paged MQA logits, FP8 decoded in the kernel,
// K-side scale applied to the fp32 dot):
//   logits[r, s] = sum_h w[r, h] * relu(q[r, h, :] . k[s, :]) * kscale[s],  s < e_r,
// organised for many rows per sequence, where the work is a dense fp8
// contraction (16384 flop per (row, key)) and the MFMA rate is the bound.
//
// gfx950 design.
//  * Workgroup = 8 query rows of one sequence x a chunk of 4096 keys; one wave
//    per row.  The wave keeps its row's q (64 heads x 128 e4m3) in registers
//    as the A operand of v_mfma_f32_32x32x64_f8f6f4 (M = 32 heads, N = 32
//    keys, K = 64; 4 instructions per 32 keys), the fastest fp8 shape on this
//    chip.  The C layout gives each lane 16 heads of one key, so the weighted
//    ReLU head sum is 32 in-lane FMAs plus one cross-lane add.
//  * K arrives in stages of 128 keys (two 64-token pages, located through the
//    block table): every wave loads 2 KB of a stage into registers two stages
//    ahead and writes it to a double-buffered LDS tile, where key n's 16-byte
//    chunk c sits in slot c ^ (n & 7) of its 128-byte row: the B-operand reads
//    of 8 consecutive keys then hit distinct bank groups.  All 8 rows share
//    each K tile, so a stage costs one 17 KB global read per 8 MB of flops.
//  * Workgroup ids run over the key chunks fastest, so the 8 XCDs each serve
//    two key chunks from their own L2 to every row block.
//  * Keys s >= e_r are masked (written -inf when clean_logits); chunks cover
//    the whole logits stride, so no separate tail pass is needed.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kRowsPerBlock = 8;                 // one row per wave
constexpr int kThreadsPf = 64 * kRowsPerBlock;
constexpr int kChunkKeys = 4096;                 // keys per workgroup
constexpr int kStageKeys = 128;                  // keys per LDS stage (two pages)
constexpr int kStagesPerChunk = kChunkKeys / kStageKeys;
constexpr int kPagesPerChunk = kChunkKeys / kPage;
constexpr int kStageCodeBytes = kStageKeys * kIdxDim;   // 16 KB

typedef int v4i __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  BatchArgs batch;
  const uint8_t* q;
  const float* w;
  const uint8_t* cache;
  int64_t page_stride;
  float* logits;
  int64_t logits_stride;
  int clean;
  int row_blocks;   // ceil(max_q_len / 8)
  int key_chunks;   // ceil(logits_stride / 4096)
};

struct PrefillShared {
  unsigned char codes[2][kStageCodeBytes];   // swizzled key rows
  float scales[2][kStageKeys];
  int page[kPagesPerChunk];                  // physical page of each page of the chunk (-1: none)
};

// Stage data a wave carries from global memory to LDS: the codes of keys
// 16 w .. 16 w + 15 and, for waves 0 and 1, the 64 scales of one page.
struct StageRegs {
  v4i c[2];
  float s;
};

__device__ __forceinline__ v4i load16_or_zero(const uint8_t* p, bool ok) {
  v4i z = {0, 0, 0, 0};
  return ok ? __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p)) : z;
}

__global__ void __launch_bounds__(kThreadsPf) indexer_prefill_kernel(PrefillArgs a) {
  __shared__ PrefillShared sh;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int kc = blockIdx.x % a.key_chunks;
  const int t = blockIdx.x / a.key_chunks;
  const int rb = t % a.row_blocks;
  const int b = t / a.row_blocks;
  if (b >= a.batch.num_seqs) return;
  const int q0 = a.batch.query_start[b], q1 = min(a.batch.query_start[b + 1], a.batch.num_rows);
  const int row0 = q0 + kRowsPerBlock * rb;
  const int nrows = min(kRowsPerBlock, q1 - row0);
  if (nrows <= 0 || row0 < 0) return;
  const int q_len = a.batch.query_start[b + 1] - q0;
  const int L = clamp_len(a.batch.seq_lens[b], a.batch.max_seq_len);
  auto extent = [&](int r) {
    const int e = L - q_len + (r - q0) + 1;
    return e < 0 ? 0 : (e > L ? L : e);
  };
  const int e_max = extent(row0 + nrows - 1);     // extents grow with the row
  const int key0 = kc * kChunkKeys;
  const int key_end = (int)min((int64_t)key0 + kChunkKeys, a.logits_stride);
  if (key0 >= key_end) return;
  // stages that hold a key some row of the block can see
  const int live = e_max > key0 ? (min(e_max, key_end) - key0 + kStageKeys - 1) / kStageKeys : 0;
  const int nstages = a.clean ? (key_end - key0 + kStageKeys - 1) / kStageKeys : live;
  if (nstages <= 0) return;

  // physical pages of the chunk
  const int pages_b = (L + kPage - 1) / kPage;
  if (wave == 0) {
    const int j = kc * kPagesPerChunk + lane;
    int id = -1;
    if (j < pages_b && lane < kPagesPerChunk) {
      id = a.batch.block_table[(int64_t)b * a.batch.bt_stride + j];
      if (id < 0 || id >= a.batch.num_pages) id = -1;
    }
    if (lane < kPagesPerChunk) sh.page[lane] = id;
  }
  __syncthreads();

  // Loads of stage st: wave w copies keys 16 w .. 16 w + 15 (2 KB) in two
  // loads; in load j lane l takes chunk l % 8 of key 16 w + 8 j + l / 8, so
  // every 8 lanes read one whole 128-byte key row.  Waves 0 and 1 also take
  // the 64 scales of page 2 st + w.
  auto load_stage = [&](StageRegs& R, int st) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int key = st * kStageKeys + 16 * wave + 8 * j + (lane >> 3);   // key within the chunk
      const int id = sh.page[key >> 6];
      const bool ok = id >= 0;
      const uint8_t* row = a.cache + (int64_t)(ok ? id : 0) * a.page_stride + (key & 63) * kIdxDim;
      R.c[j] = load16_or_zero(row + 16 * (lane & 7), ok);
    }
    R.s = 0.f;
    if (wave < 2) {
      const int pid = sh.page[2 * st + wave];
      if (pid >= 0)
        R.s = __builtin_nontemporal_load(reinterpret_cast<const float*>(a.cache + (int64_t)pid * a.page_stride +
                                                                          kIdxScaleOff) + lane);
    }
  };
  auto write_stage = [&](const StageRegs& R, int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = 16 * wave + 8 * j + (lane >> 3);
      *reinterpret_cast<v4i*>(sh.codes[buf] + n * kIdxDim + 16 * ((lane & 7) ^ (n & 7))) = R.c[j];
    }
    if (wave < 2) sh.scales[buf][64 * wave + lane] = R.s;
  };

  // This wave's row: q as A operands (head 32 mt + l % 32, bytes
  // 64 j + 32 (l / 32) .. +32) and the weights of the 16 heads each lane
  // holds per head tile in the C layout (head 32 mt + (i % 4) + 4 (l / 32) +
  // 8 (i / 4) for item i).
  const bool has_row = wave < nrows;
  const int r = row0 + (has_row ? wave : 0);
  const int e_r = has_row ? extent(r) : 0;
  v8i qa[2][2];
  float wr[2][16];
  {
    const int hq = lane & 31, hk = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint8_t* qp = a.q + ((int64_t)r * kIdxHeads + 32 * mt + hq) * kIdxDim + 32 * hk;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(qp + 64 * j);
        const uint4 x1 = *reinterpret_cast<const uint4*>(qp + 64 * j + 16);
        qa[mt][j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 ww = *reinterpret_cast<const float4*>(a.w + (int64_t)r * kIdxHeads + 32 * mt + 8 * g + 4 * hk);
        wr[mt][4 * g] = ww.x; wr[mt][4 * g + 1] = ww.y; wr[mt][4 * g + 2] = ww.z; wr[mt][4 * g + 3] = ww.w;
      }
    }
  }

  // B-operand slots of this lane: key n = l % 32 of a 32-key step, chunks
  // {2 h, 2 h + 1} (K half 0) and {4 + 2 h, 5 + 2 h} (K half 1), h = l / 32.
  const int nb = lane & 31, hb = lane >> 5;
  int boff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int chunk = (c < 2 ? 2 * hb + c : 4 + 2 * hb + (c - 2));
    boff[c] = nb * kIdxDim + 16 * (chunk ^ (nb & 7));
  }

  auto compute_stage = [&](int st, int buf) {
    const int skey0 = key0 + st * kStageKeys;
#pragma unroll
    for (int step = 0; step < kStageKeys / 32; ++step) {
      const unsigned char* tb = sh.codes[buf] + step * 32 * kIdxDim;
      v8i bop[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const v4i x0 = *reinterpret_cast<const v4i*>(tb + boff[2 * j]);
        const v4i x1 = *reinterpret_cast<const v4i*>(tb + boff[2 * j + 1]);
        bop[j] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
      v16f acc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        v16f z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt][0], bop[0], z, 0, 0, 0, 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt][1], bop[1], acc[mt], 0, 0, 0, 0, 0, 0);
      }
      float s = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) s = fmaf(wr[mt][i], fmaxf(acc[mt][i], 0.f), s);
      s += __shfl_xor(s, 32, 64);
      const int key = skey0 + step * 32 + nb;
      const float v = s * sh.scales[buf][step * 32 + nb];
      if (has_row && hb == 0 && key < key_end) {
        float* dst = a.logits + (int64_t)r * a.logits_stride + key;
        if (key < e_r) *dst = v;
        else if (a.clean) *dst = -INFINITY;
      }
    }
  };

  // Two register sets carry stages two ahead of the LDS buffers.
  StageRegs R0, R1;
  load_stage(R0, 0);
  if (nstages > 1) load_stage(R1, 1);
  write_stage(R0, 0);
  __syncthreads();
  for (int st = 0; st < nstages; st += 2) {
    if (st + 2 < nstages) load_stage(R0, st + 2);
    compute_stage(st, 0);
    if (st + 1 < nstages) write_stage(R1, 1);
    __syncthreads();
    if (st + 1 >= nstages) break;
    if (st + 3 < nstages) load_stage(R1, st + 3);
    compute_stage(st + 1, 1);
    if (st + 2 < nstages) write_stage(R0, 0);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_indexer_prefill(const BatchArgs& batch, const uint8_t* q, const float* w,
                                  const uint8_t* cache, int64_t page_stride, float* logits,
                                  int64_t logits_stride, int clean, int num_cus, hipStream_t stream) {
  (void)num_cus;
  if (batch.num_rows <= 0 || batch.num_seqs <= 0) return hipSuccess;
  PrefillArgs a{batch, q, w, cache, page_stride, logits, logits_stride, clean, 0, 0};
  a.row_blocks = (max(batch.max_q_len, 1) + kRowsPerBlock - 1) / kRowsPerBlock;
  a.key_chunks = (int)((logits_stride + kChunkKeys - 1) / kChunkKeys);
  const int64_t grid = (int64_t)batch.num_seqs * a.row_blocks * a.key_chunks;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_prefill_kernel, dim3((unsigned)grid), dim3(kThreadsPf), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
