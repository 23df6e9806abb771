// Lightning-indexer logits for chunked prefill (many query rows per sequence).
//
// Same operation as the paged decode kernel (vLLM PR "[Feature] TRITON_MLA_SPARSE
// backend ...", Changes item 2: paged MQA logits, FP8 decoded in the kernel,
// K-side scale applied to the fp32 dot):
//   logits[r, s] = sum_h w[r, h] * relu(q[r, h, :] . k[s, :]) * kscale[s],  s < e_r,
// organised for many rows per sequence, where the work is a dense fp8
// contraction (16384 flop per (row, key)).
//
// gfx950 design.
//  * Workgroup = 16 query rows of one sequence x a chunk of 8192 keys; each of
//    the 8 waves owns two rows and keeps their q (64 heads x 128 e4m3 each) in
//    registers as A operands of v_mfma_f32_32x32x64_f8f6f4 (M = 32 heads,
//    N = 32 keys, K = 64; 4 instructions per row and 32 keys), the fastest
//    fp8 shape on this chip.  One B-operand read of 32 keys feeds both rows.
//  * The C layout gives each lane 16 heads of one key, so the weighted ReLU
//    head sum is 32 in-lane FMAs (ReLU as one v_med3_f32) plus one lane swap
//    (v_permlane32_swap): about 70 VALU operations per row and 32 keys, whose
//    issue time (4 cycles each) exceeds the 4 MFMAs' 256 cycles.  The kernel
//    is bound by VALU issue, and the schedule is built to overlap the two:
//    the MFMAs of one row are interleaved (sched_group_barrier) with the
//    epilogue of the other row's previous product.
//  * K arrives in stages of 256 keys (four 64-token pages, located through the
//    block table), copied global->LDS (global_load_lds_dwordx4, one whole
//    128-byte key row per 8 lanes) into a double-buffered tile where key n's
//    16-byte chunk c sits in slot c ^ ((n >> 1) & 7) of its row: the B-operand
//    reads of 16 consecutive keys then hit distinct banks.  The copy of stage
//    s + 1 is in flight while stage s is multiplied.
//  * Workgroup ids run over the key chunks fastest, so for a 65,536-key
//    sequence each of the 8 XCDs serves one key chunk from its own L2 to every
//    row block.
//  * Per-row causal bound with an early exit: only the stages holding a key
//    some row of the block can see are copied and multiplied; stores past a
//    row's extent e_r fall outside its buffer range and are dropped.  With
//    clean_logits each row's keys from e_r to the chunk end get -inf stores
//    only, so a block whose rows see a short prefix pays for its causal
//    extent, not the whole rectangle.  Chunks cover the whole logits stride,
//    so no separate tail pass is needed.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kWavesPf = 8;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerBlock = kWavesPf * kRowsPerWave;   // 16 query rows per workgroup
constexpr int kThreadsPf = 64 * kWavesPf;
constexpr int kChunkKeys = 8192;                 // keys per workgroup
constexpr int kStageKeys = 256;                  // keys per LDS stage (four pages)
constexpr int kPagesPerChunk = kChunkKeys / kPage;
constexpr int kStageCodeBytes = kStageKeys * kIdxDim;    // 32 KB
constexpr int kDmaPerWave = kStageCodeBytes / 1024 / kWavesPf;   // 1 KB copies per wave and stage
constexpr int kPagesPerStage = kStageKeys / kPage;       // also the waves that copy one page's scales
static_assert(kDmaPerWave * 8 <= kPage && kPage % (kDmaPerWave * 8) == 0, "a wave's copy blocks lie in one page");
static_assert(kPagesPerStage <= kWavesPf, "one wave per page's scales");

typedef int v4i __attribute__((ext_vector_type(4)));

// Slot swizzle of key row n (128 bytes): 16 lanes of a 128-bit LDS access are
// served per cycle from 256 bytes of banks, so the 16 key rows one B-operand
// read touches must land on 16 distinct 16-byte units modulo 256 -- row parity
// times the slot XORed with (n >> 1) & 7 does that.
__device__ __forceinline__ int swz(int n) { return (n >> 1) & 7; }

// Source of rows and scales of pages the chunk does not have.
__device__ __attribute__((aligned(16))) uint32_t g_zero_kv[64] = {};

struct PrefillArgs {
  BatchArgs batch;
  const uint8_t* q;
  const float* w;
  const uint8_t* cache;
  int64_t page_stride;
  float* logits;
  int64_t logits_stride;
  int clean;
  int row_blocks;   // ceil(max_q_len / 16)
  int key_chunks;   // ceil(logits_stride / 4096)
};

struct PrefillShared {
  unsigned char codes[2][kStageCodeBytes];   // swizzled key rows
  float scales[2][kStageKeys];
};

// One query row of a wave: q as MFMA A operands and the head weights of the
// lane's C-layout heads.
struct RowOperands {
  v8i qa[2][2];      // [head tile][K half]
  float wr[2][16];   // [head tile][C item]
};

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
  // Clean logits: -inf over keys [max(e_r, key0), key_end) of every row of the
  // block, stored here (the product stores of those keys are dropped by the
  // row's buffer range below); aligned float4 stores, scalar at the ends.
  if (a.clean) {
    for (int ri = wave; ri < nrows; ri += kWavesPf) {
      float* rowp = a.logits + (int64_t)(row0 + ri) * a.logits_stride;
      const int c0 = max(extent(row0 + ri), key0);
      const int c4 = min((c0 + 3) & ~3, key_end);
      if (lane < c4 - c0) rowp[c0 + lane] = -INFINITY;
      for (int c = c4 + 4 * lane; c < key_end; c += 256) {
        if (c + 3 < key_end) *reinterpret_cast<float4*>(rowp + c) = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        else
          for (int x = c; x < key_end; ++x) rowp[x] = -INFINITY;
      }
    }
  }
  const int nstages = live;
  if (nstages <= 0) return;

  // Physical pages of the chunk, lane p of every wave holding page p (-1:
  // none); a copy picks its page with readlane (a scalar, no LDS round trip).
  const int pages_b = (L + kPage - 1) / kPage;
  static_assert(kPagesPerChunk == 128, "two page registers");
  int pg[2] = {-1, -1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = kc * kPagesPerChunk + 64 * h + lane;
    if (j < pages_b) {
      const int id = a.batch.block_table[(int64_t)b * a.batch.bt_stride + j];
      pg[h] = (id >= 0 && id < a.batch.num_pages) ? id : -1;
    }
  }
  auto page_id = [&](int p) __attribute__((always_inline)) {   // p wave-uniform
    return p < 64 ? __builtin_amdgcn_readlane(pg[0], p) : __builtin_amdgcn_readlane(pg[1], p - 64);
  };
  const unsigned char* const zero_src = reinterpret_cast<const unsigned char*>(g_zero_kv);

  // Copy of stage st into buffer buf: wave w fills 1 KB blocks w * kDmaPerWave
  // + i (8 key rows each, all in page st * kPagesPerStage + w * kDmaPerWave /
  // 8); lane l fills slot l % 8 of row l / 8 of the block with chunk (l % 8) ^
  // swz(row), so every 8 lanes read one whole 128-byte key row.  The first
  // kPagesPerStage waves also copy one page's 256 scale bytes (lanes 0-15).
  auto copy_stage = [&](int st, int buf) __attribute__((always_inline)) {
    const uint32_t dst = lds_addr(sh.codes[buf]);
    const int id = page_id(st * kPagesPerStage + (wave * kDmaPerWave * 8) / kPage);
    const unsigned char* base = id >= 0 ? a.cache + (int64_t)id * a.page_stride : zero_src;
    // Key row n = 8 blk + l / 8 of the stage: swz(n) = (4 blk + l / 16) & 7 =
    // l / 16 + 4 (blk & 1), so the slot offsets take two per-lane values.
    const uint32_t slot = 16u * (uint32_t)((lane & 7) ^ (lane >> 4));
    const uint32_t row = id >= 0 ? (uint32_t)(lane >> 3) * kIdxDim : 0u;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int blk = wave * kDmaPerWave + i;
      const uint32_t off = (id >= 0 ? (uint32_t)(((8 * blk) & 63) * kIdxDim) : 0u) + row + (slot ^ ((blk & 1) ? 64u : 0u));
      lds_dma16(base + off, dst + blk * 1024);
    }
    if (wave < kPagesPerStage) {
      const int ids = page_id(st * kPagesPerStage + wave);
      const unsigned char* src = ids >= 0 ? a.cache + (int64_t)ids * a.page_stride + kIdxScaleOff : zero_src;
      if (lane < 16) lds_dma16(src + 16 * lane, lds_addr(&sh.scales[buf][kPage * wave]));
    }
  };

  // This wave's rows row0 + wave and row0 + wave + 8: q as A operands (head
  // 32 mt + l % 32, bytes 64 j + 32 (l / 32) .. +32) and the weights of the
  // 16 heads each lane holds per head tile in the C layout (head 32 mt +
  // (i % 4) + 4 (l / 32) + 8 (i / 4) for item i).
  const int hq = lane & 31, hk = lane >> 5;
  RowOperands ro[kRowsPerWave];
  bool has_row[kRowsPerWave];
  int rr[kRowsPerWave], e_r[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int ri = wave + kWavesPf * j;   // rows of the block, wave-major
    has_row[j] = ri < nrows;
    rr[j] = row0 + (has_row[j] ? ri : 0);
    e_r[j] = has_row[j] ? extent(rr[j]) : 0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint8_t* qp = a.q + ((int64_t)rr[j] * kIdxHeads + 32 * mt + hq) * kIdxDim + 32 * hk;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(qp + 64 * kh);
        const uint4 x1 = *reinterpret_cast<const uint4*>(qp + 64 * kh + 16);
        ro[j].qa[mt][kh] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 ww = *reinterpret_cast<const float4*>(a.w + (int64_t)rr[j] * kIdxHeads + 32 * mt + 8 * g + 4 * hk);
        ro[j].wr[mt][4 * g] = ww.x; ro[j].wr[mt][4 * g + 1] = ww.y;
        ro[j].wr[mt][4 * g + 2] = ww.z; ro[j].wr[mt][4 * g + 3] = ww.w;
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
    boff[c] = nb * kIdxDim + 16 * (chunk ^ swz(nb));
  }

  // Logits stores of this wave's rows go through buffer resources based at
  // the chunk start of the row with the row's causal part of the chunk,
  // [key0, min(e_r, key_end)), as their range: stores of keys past e_r (and
  // of lanes 32-63, which hold copies of lanes 0-31's sums) fall outside it
  // and the hardware drops them, so the step body has no compares or
  // branches and its MFMAs and VALU work can be interleaved freely.
  constexpr uint32_t kDrop = 0x7FFF0000u;
  __amdgpu_buffer_rsrc_t out_rsrc[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int span = has_row[j] ? max(0, min(e_r[j], key_end) - key0) : 0;
    out_rsrc[j] = __builtin_amdgcn_make_buffer_rsrc(a.logits + (int64_t)rr[j] * a.logits_stride + key0, (short)0,
                                                    span * 4, 0x00020000);
  }
  const uint32_t lane_off = hb == 0 ? 4u * (uint32_t)nb : kDrop;

  // Epilogue of row j and the 32 keys at chunk offset kb + nb: weighted ReLU
  // head sum (in-lane over the lane's 32 heads in one chain, head tile 0
  // first, then lanes 0-31 add lanes 32-63 with one lane swap of the sum held
  // twice) times the K scale.  Split in two parts so a half step can be cut
  // into two scheduling regions.
  auto epi_part = [&](int j, const v16f& acc_t, int mt, float p) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) p = fmaf(ro[j].wr[mt][i], relu_finite(acc_t[i]), p);
    return p;
  };
  auto epi_finish = [&](float p, float scale) __attribute__((always_inline)) {
    float x = p, y = p;
    asm volatile("" : "+v"(y));      // two registers, so the swap needs no copies
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * scale;
  };
  auto epi_value = [&](int j, const v16f* acc, float scale) __attribute__((always_inline)) {
    return epi_finish(epi_part(j, acc[1], 1, epi_part(j, acc[0], 0, 0.f)), scale);
  };
  auto epi_store = [&](int j, float v, int kb) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out_rsrc[j], lane_off + 4u * (uint32_t)kb, 0, 0);
  };

  // B operand (32 keys x 128 dims, this lane's slots, K half kh) and K scale
  // of one step.
  v8i bop[2];
  auto load_b_half = [&](int buf, int step, int kh) __attribute__((always_inline)) {
    const unsigned char* tb = sh.codes[buf] + step * 32 * kIdxDim;
    const v4i x0 = *reinterpret_cast<const v4i*>(tb + boff[2 * kh]);
    const v4i x1 = *reinterpret_cast<const v4i*>(tb + boff[2 * kh + 1]);
    bop[kh] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto load_scale = [&](int buf, int step) __attribute__((always_inline)) { return sh.scales[buf][step * 32 + nb]; };
  // Both head tiles of row j over K half kh.
  auto mfma_half = [&](int j, int kh, v16f* acc) __attribute__((always_inline)) {
    v16f z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ro[j].qa[mt][kh], bop[kh], kh == 0 ? z : acc[mt],
                                                                0, 0, 0, 0, 0, 0);
  };
  // Issue orders.  A half step without operand reads: one MFMA per ~18 VALU
  // operations of the epilogue (70 in all).  A half step that reads the next
  // step's operand: two regions, each an MFMA pair (both head tiles of one
  // K half), then the LDS reads of that K half (into the registers the pair
  // has just consumed), then half the epilogue.
  auto order_plain = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 18, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto order_reload = [&](int nds) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (nds == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    else __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Software pipeline over steps of 32 keys, two rows per wave: the MFMAs of
  // one row run while the VALU epilogue of the other row's previous product
  // is issued (row 0 of step t + 1 beside row 1 of step t, row 1 of step t
  // beside row 0 of step t).  Stages of 256 keys are double-buffered: the
  // copy of stage st + 1 is in flight while stage st is multiplied; each wave
  // waits for its own copies before the barrier that opens a stage.
  v16f acc0[2], acc1[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc1[mt][i] = 0.f;
  float sc = 0.f, sc_prev = 0.f;
  int kb_prev = key_end - key0;        // the first stage has no previous step: its store is dropped
  // The last two logits of a stage are stored after the next stage's barrier:
  // the wait before that barrier (for this wave's copies) then does not also
  // wait for stores issued just before it.
  float held0 = 0.f, held1 = 0.f;
  int kb_held = key_end - key0 + 32;  // nothing held before the first stage: both stores dropped
  copy_stage(0, 0);
  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();            // stage st landed; buffer (st + 1) & 1 is free
    if (st + 1 < nstages) copy_stage(st + 1, buf ^ 1);
    load_b_half(buf, 0, 0);
    load_b_half(buf, 0, 1);
    sc = load_scale(buf, 0);
    mfma_half(0, 0, acc0);
    mfma_half(0, 1, acc0);
    epi_store(1, epi_value(1, acc1, sc_prev), kb_prev);
    epi_store(1, held1, kb_held - 32);
    epi_store(0, held0, kb_held);
    order_plain();
#pragma unroll
    for (int step = 0; step < kStageKeys / 32; ++step) {
      const int kb = st * kStageKeys + step * 32;
      const bool last = step + 1 == kStageKeys / 32;
      const float sc_cur = sc;
      if (!last) {
        // row 1's product beside row 0's epilogue, reading the next operand
        mfma_half(1, 0, acc1);
        load_b_half(buf, step + 1, 0);
        const float p = epi_part(0, acc0[0], 0, 0.f);
        order_reload(2);
        mfma_half(1, 1, acc1);
        load_b_half(buf, step + 1, 1);
        sc = load_scale(buf, step + 1);
        epi_store(0, epi_finish(epi_part(0, acc0[1], 1, p), sc_cur), kb);
        order_reload(3);
        // row 0's next product beside row 1's epilogue
        mfma_half(0, 0, acc0);
        mfma_half(0, 1, acc0);
        const float v1 = epi_value(1, acc1, sc_cur);
        if (step + 2 < kStageKeys / 32) epi_store(1, v1, kb);
        else held1 = v1;
        order_plain();
      } else {
        mfma_half(1, 0, acc1);
        mfma_half(1, 1, acc1);
        held0 = epi_value(0, acc0, sc_cur);
        order_plain();
        sc_prev = sc_cur;
        kb_prev = kb;
        kb_held = kb;
      }
    }
  }
  epi_store(1, held1, kb_held - 32);
  epi_store(0, held0, kb_held);
  epi_store(1, epi_value(1, acc1, sc_prev), kb_prev);
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
