// Sparse MLA decode over an fp8 latent cache.
//
// Same result contract as the bf16 path (vLLM PR "[Feature] TRITON_MLA_SPARSE
// backend ...", Changes item 3: split-KV partials with an N-way online-softmax
// merge, single-pass fast path, -1e30 running-max sentinel), over a cache the
// pages list as missing (section Limitations: bf16-only latent cache).  The
// fp8 page layout (64 tokens): row t at byte 640 t = 512 e4m3 latent codes
// then 64 bf16 rope values; the 4 fp32 scales of token t (one per 128 latent
// values) at byte 40960 + 16 t.  A latent value is scale[d / 128] * code[d].
//
// gfx950 design, differences from the bf16 kernel only:
//  * Gather: 656 bytes per token instead of 1152 -- five 128-byte column
//    groups (4 of codes, 1 of rope) plus one 16-byte scale record, all copied
//    global -> LDS with global_load_lds_dwordx4.  LDS tile = 1 KB blocks
//    (column group, group of 8 rows); the 16-byte slot s of row r8 in row
//    group rg holds chunk s ^ r8 ^ (rg & 1).  The extra (rg & 1) term puts the
//    16 rows of an MFMA operand read on all 64 banks of the 256-byte window
//    (conflict-free 128-bit and transposing 64-bit reads).
//  * QK: the fp8 codes are converted to bf16 exactly
//    (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and multiplied on
//    v_mfma_f32_16x16x32_bf16 with q in registers; each of the 4 scale groups
//    accumulates separately, so z = sum_g scale_g * acc_g + acc_rope in fp32
//    keeps every product exact.  One 128-bit read feeds two MFMAs (the k
//    order inside a 64-dim pair is permuted identically for C and q).
//  * 64-head blocks use the wave-specialised kernel at the end of this file
//    (codes converted once per tile into a bf16 tile, scorers and PV waves
//    on each SIMD); the notes below are the 16- and 32-head forms'.
//  * PV: the V^T operand is read with the 8-bit transposing LDS read
//    (ds_read_b64_tr_b8: lane n gets byte n % 8 of the vectors of lanes
//    n / 8 + 2 j) and converted to bf16 exactly; the group scale is folded
//    into the probabilities, P'_g = bf16(p * scale_g), written by the scoring
//    wave for each of the 4 groups.
#include "common.h"
#include "kernels.h"
#include "mla_common.h"

namespace dsa {

namespace {

constexpr int kTile8 = 64;                           // selected tokens per tile
constexpr int kRow8 = 640;                           // codes + rope bytes per token
constexpr int kScaleOff8 = kPage * kRow8;            // 40960: scale records in a page
constexpr int kCg8 = 5;                              // 128-byte column groups per row
constexpr int kRg8 = kTile8 / 8;                     // row groups per tile
constexpr int kTileScaleOff = kCg8 * kRg8 * 1024;    // 40960: scale records in a tile
constexpr int kTileBytes8 = kTileScaleOff + kTile8 * 16;   // 41984
constexpr int kPStride = kTile8 + 8;                 // bf16 per (group, head) row of P'

__device__ __attribute__((aligned(16))) uint4 g_zero_row8[kRow8 / 16] = {};

typedef int v2i __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b8: within each group of 16 lanes, lane n receives byte n % 8
// of the 8-byte vectors addressed by lanes n / 8 + 2 j, j = 0..7 (checked by
// an in-bounds lane probe).
__device__ __forceinline__ v2i lds_read_tr8(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i*)(const __attribute__((address_space(3))) void*)p);
}

// Two e4m3 codes (bytes 0,1 or 2,3 of w) -> two bf16, exactly (every finite
// e4m3 value is a bf16 value; scale 1 leaves it unchanged).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  const v2bf16 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 codes (two words) -> 8 bf16 as an MFMA operand.
__device__ __forceinline__ v8bf fp8x8_to_v8bf(uint32_t w0, uint32_t w1) {
  const uint4 u = make_uint4(fp8x2_to_bf16x2(w0, false), fp8x2_to_bf16x2(w0, true),
                             fp8x2_to_bf16x2(w1, false), fp8x2_to_bf16x2(w1, true));
  return as_v8bf(u);
}

constexpr int kMaxTiles8 = DSA_MAX_TOPK / kTile8;   // 32 tiles per split at most
constexpr int kDeepTiles = 8;                        // tiles per split from which two stay in flight

// Tile buffers: three (two 41 KB tiles in flight while one is multiplied) when
// the head block's P' fits beside them, else two.
template <int HT>
struct MlaBuffers8 {
  static constexpr int value = HT <= 2 ? 3 : 2;
};

template <int HT, int TP>
struct MlaShared8 {
  unsigned char tile[MlaBuffers8<HT>::value][kTileBytes8];   // gathered rows, ring of buffers
  int slot[kMaxTiles8 * kTile8];                             // cache slot (page * 64 + s) or -1
  uint64_t mask[kMaxTiles8];                                  // valid slots of each tile
  alignas(16) uint16_t p[HT][4][16][kPStride];                // bf16 p * scale_g [tile][group][head][token]
  float tmax[HT][TP][16];                                     // per-part tile maxima
};

// Byte offset inside a tile of the 16-byte slot `slot` of token `tok`, column
// group `cg`.
__device__ __forceinline__ int tile_off(int cg, int tok, int slot) {
  const int rg = tok >> 3, r8 = tok & 7;
  return (cg * kRg8 + rg) * 1024 + r8 * 128 + ((slot ^ r8 ^ (rg & 1)) << 4);
}

template <int HT, int TP>
__global__ void __launch_bounds__(64 * HT * TP) sparse_mla_fp8_kernel(MlaArgs a) {
  constexpr int NW = HT * TP;          // waves
  constexpr int TPT = 4 / TP;          // token tiles of 16 scored per wave
  constexpr int DW = kVDim / TP;       // output dims per wave
  constexpr int NDT = DW / 16;         // dim tiles per wave
  constexpr int NG = DW / 128;         // scale groups per wave's dims
  constexpr int RGW = kRg8 / NW;       // row groups each wave gathers
  static_assert(RGW * NW == kRg8, "waves must split the row groups evenly");
  constexpr int NBUF = MlaBuffers8<HT>::value;
  constexpr int DEPTH = NBUF - 1;      // tiles in flight while one is multiplied
  constexpr int SCALE_WAVE = NW - 1;   // the wave that also copies the scale records
  constexpr int NDR = RGW * kCg8;      // row loads per wave and tile
  constexpr int ND = NDR + 1;          // + the scale load (scale wave only)
  __shared__ MlaShared8<HT, TP> sh;

  const int R = a.batch.num_rows;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n16 = lane & 15;

  const int bid = blockIdx.x;
  const int q8 = bid >> 3;
  const int hb = q8 % a.head_blocks;
  const int rest = (q8 / a.head_blocks) * 8 + (bid & 7);
  if (rest >= R * a.splits) return;
  const int r = rest / a.splits;
  const int sp = rest % a.splits;

  const int ht = wave % HT, part = wave / HT;
  const int h = hb * (16 * HT) + ht * 16 + n16;
  const int d_base = part * DW;
  // Whether this wave's head tile exists (a last block of H % 64 heads has
  // fewer; its tile 0 always does).  A missing tile is scored with the q of
  // the block's first tile and its results are not stored: the same
  // instruction stream as a full block (a branch inside the tile loop costs
  // registers and speed at every head count).  Wave-uniform.
  const bool on = hb * (16 * HT) + ht * 16 < a.H;
  const int hq = on ? h : hb * (16 * HT) + n16;
  const int slot0 = sp * a.split_slots;
  const int slot1 = min(slot0 + a.split_slots, a.k);
  const int ntiles = (slot1 - slot0 + kTile8 - 1) / kTile8;

  uint4 qreg[18];
  // q operands.  Latent pair j (dims 64 j .. 64 j + 63): MFMA 2 j takes dims
  // 64 j + 16 g + 0..7, MFMA 2 j + 1 dims 64 j + 16 g + 8..15 (the k order the
  // 128-bit code reads deliver).  Rope step s: dims 512 + 32 s + 8 g + 0..7.
  {
    const uint16_t* qp = a.q + ((int64_t)r * a.H + hq) * kKvDim;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qreg[2 * j] = *reinterpret_cast<const uint4*>(qp + 64 * j + 16 * g);
      qreg[2 * j + 1] = *reinterpret_cast<const uint4*>(qp + 64 * j + 16 * g + 8);
    }
    qreg[16] = *reinterpret_cast<const uint4*>(qp + kVDim + 8 * g);
    qreg[17] = *reinterpret_cast<const uint4*>(qp + kVDim + 32 + 8 * g);
  }
  asm volatile("" ::: "memory");   // q stays ahead of the prologue's loads, whose waits cover it
  // Prologue.  Every wave turns its tiles' indices into cache slots: tile t
  // belongs to wave t % NW, its entry lane to this lane.  All index loads go
  // out with the sequence search, then all block-table loads, so the chain is
  // two round trips whatever the number of tiles.  A slot is -1 when the index
  // is padding, outside [0, e_r) or on a page outside the cache.
  {
    constexpr int MT = kMaxTiles8 / NW;
    const int32_t* idx_row = a.indices + (int64_t)r * a.k;
    int idx[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = wave + NW * m;
      const int j = slot0 + t * kTile8 + lane;
      idx[m] = (t < ntiles && j < slot1) ? idx_row[j] : -1;
    }
    const int b = seq_of_row_wave(a.batch.query_start, a.batch.num_seqs, r);
    // The table needs only idx < max_seq_len to stay inside the row; e and the
    // page range are checked below.
    int page[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      page[m] = (b >= 0 && idx[m] >= 0 && idx[m] < a.batch.max_seq_len)
                    ? a.batch.block_table[(int64_t)b * a.batch.bt_stride + (idx[m] >> 6)] : -1;
    const int e = b >= 0 ? row_extent(a.batch, b, r) : 0;   // rides with the block-table loads
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = wave + NW * m;
      if (t < ntiles) {
        const bool valid = idx[m] < e && page[m] >= 0 && page[m] < a.batch.num_pages;
        sh.slot[t * kTile8 + lane] = valid ? page[m] * kPage + (idx[m] & 63) : -1;
        const uint64_t msk = __ballot(valid);
        if (lane == 0) sh.mask[t] = msk;
      }
    }
  }
  __syncthreads();                                   // slots and masks of every tile published

  // Gather of tile t into buffer t % NBUF: one wave-wide load fills one 1 KB
  // block; lane l copies slot l & 7 of row l >> 3 (chunk (l & 7) ^ r8 ^ (rg & 1)
  // of that row's 128-byte column group).  The scale wave adds one load of the
  // 64 scale records (lane l: token l).  Every tile is gathered (masked slots
  // read a static zero row), so each wave issues the same number of loads per
  // tile and the in-flight count below is exact.
  auto gather_src = [&](int t, int j) -> const unsigned char* {
    const int rg = wave * RGW + j;
    const int sl = sh.slot[t * kTile8 + rg * 8 + (lane >> 3)];
    const unsigned char* row = sl >= 0 ? a.kv8 + (int64_t)(sl >> 6) * a.kv8_stride + (sl & 63) * kRow8
                                       : reinterpret_cast<const unsigned char*>(g_zero_row8);
    return row + (((lane & 7) ^ (lane >> 3) ^ (rg & 1)) << 4);
  };
  auto scale_src = [&](int t) -> const unsigned char* {
    const int sl = sh.slot[t * kTile8 + lane];
    return sl >= 0 ? a.kv8 + (int64_t)(sl >> 6) * a.kv8_stride + kScaleOff8 + (sl & 63) * 16
                   : reinterpret_cast<const unsigned char*>(g_zero_row8);
  };
  auto gather_one = [&](const unsigned char* const* src, const unsigned char* ssrc, uint32_t dst, int i) {
    if (i < NDR) {
      const int j = i / kCg8, cg = i % kCg8;
      lds_dma16(src[j] + cg * 128, dst + (cg * kRg8 + wave * RGW + j) * 1024);
    } else if (wave == SCALE_WAVE) {
      lds_dma16(ssrc, dst + kTileScaleOff);
    }
  };
  auto gather_all = [&](int t) __attribute__((always_inline)) {
    const unsigned char* src[RGW];
#pragma unroll
    for (int j = 0; j < RGW; ++j) src[j] = gather_src(t, j);
    const unsigned char* ssrc = scale_src(t);
    const uint32_t dst = lds_addr(sh.tile[t % NBUF]);
#pragma unroll
    for (int i = 0; i < ND; ++i) gather_one(src, ssrc, dst, i);
  };
  // Two tiles in flight pay off only once the pipeline runs for a while: with
  // 4 tiles per split (32 decode rows of 16 heads, 8 splits) asking for two
  // at once delays the first (24.9 us against 24.0 us).
  const int depth = (DEPTH > 1 && ntiles >= kDeepTiles) ? DEPTH : 1;
  // q went out before the prologue's loads and the prologue waited for those,
  // so inside the loop no load but the copies is ever outstanding and the
  // waits there count copies only.
#pragma unroll
  for (int t = 0; t < DEPTH; ++t)
    if (t < depth && t < ntiles) gather_all(t);

  // PV read address parts: lane i of group g addresses token 8 g + i / 2 of
  // the 32-token step, bytes 16 (dim tile % 8) + 8 (i % 2) of its column group.
  const int pv_r8 = n16 >> 1;
  const int pv_half = (n16 & 1) * 8;

  v4f acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = kMaskSentinel;
  float l_part = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    // Wait for this wave's copies of tile t: the copies of the DEPTH - 1 later
    // tiles already issued may stay in flight.
    if (DEPTH > 1 && depth > 1 && t + 1 < ntiles) {
      if (wave == SCALE_WAVE) wait_vmcnt<(DEPTH - 1) * (NDR + 1)>();
      else wait_vmcnt<(DEPTH - 1) * NDR>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();                                   // tile t landed in every wave; buffer (t + depth) % NBUF is free
    const uint64_t mask = sh.mask[t];
    const int tn = t + depth;                          // the tile whose copy starts now
    const bool pre = tn < ntiles;
    const unsigned char* gsrc[RGW];
    const unsigned char* gssrc = nullptr;
    const uint32_t gdst = lds_addr(sh.tile[tn % NBUF]);
    if (pre) {
#pragma unroll
      for (int j = 0; j < RGW; ++j) gsrc[j] = gather_src(tn, j);
      gssrc = scale_src(tn);
    }
    if (pre && mask == 0ull) {
#pragma unroll
      for (int i = 0; i < ND; ++i) gather_one(gsrc, gssrc, gdst, i);
    }

    if (mask != 0ull) {
      const unsigned char* tile = sh.tile[t % NBUF];
      float z[TPT][4];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int tt = part * TPT + u;
        const int tok = tt * 16 + n16;             // the C row this lane supplies
        v4f sg[4], sr = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) sg[c] = v4f{0.f, 0.f, 0.f, 0.f};
        constexpr int NQ = TPT * 10;
#pragma unroll
        for (int st = 0; st < 10; ++st) {
          const int q = u * 10 + st;
          if constexpr (HT < 4) {
#pragma unroll
            for (int i = 0; i < ND; ++i)
              if (i * NQ / ND == q && pre) gather_one(gsrc, gssrc, gdst, i);
          }
          if (st < 8) {
            const int cg = st >> 1;
            const uint4 raw = *reinterpret_cast<const uint4*>(tile + tile_off(cg, tok, 4 * (st & 1) + g));
            sg[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_v8bf(raw.x, raw.y), as_v8bf(qreg[2 * st]),
                                                             sg[cg], 0, 0, 0);
            sg[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_v8bf(raw.z, raw.w),
                                                             as_v8bf(qreg[2 * st + 1]), sg[cg], 0, 0, 0);
          } else {
            const int ks = st - 8;
            const uint4 cv = *reinterpret_cast<const uint4*>(tile + tile_off(4, tok, 4 * ks + g));
            sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(cv), as_v8bf(qreg[16 + ks]), sr, 0, 0, 0);
          }
        }
        // z of tokens tt*16 + 4g + i (head h) = sum_c scale_c acc_c + acc_rope
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = tt * 16 + 4 * g + i;
          const float4 s4 = *reinterpret_cast<const float4*>(tile + kTileScaleOff + tk * 16);
          float v = sr[i];
          v = fmaf(s4.x, sg[0][i], v);
          v = fmaf(s4.y, sg[1][i], v);
          v = fmaf(s4.z, sg[2][i], v);
          v = fmaf(s4.w, sg[3][i], v);
          z[u][i] = v;
        }
      }
      float tmax = kMaskSentinel;
#pragma unroll
      for (int u = 0; u < TPT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = (part * TPT + u) * 16 + 4 * g + i;
          const bool v = (mask >> tok) & 1ull;
          const float zz = v ? z[u][i] * a.scale_log2 : kMaskSentinel;
          z[u][i] = zz;
          tmax = fmaxf(tmax, zz);
        }
      tmax = fmaxf(tmax, lane_xor16(tmax));
      tmax = fmaxf(tmax, lane_xor32(tmax));
      if (TP > 1) {
        if (g == 0) {
          // The address is formed here rather than held across the loop: near
          // the VGPR limit the compiler otherwise spills it, and the reload's
          // vmcnt(0) would wait for the copies in flight.
          int n = n16;
          asm volatile("" : "+v"(n));
          sh.tmax[ht][part][n] = tmax;
        }
        __syncthreads();
#pragma unroll
        for (int pp = 0; pp < TP; ++pp) tmax = fmaxf(tmax, sh.tmax[ht][pp][n16]);
      }
      // Lazy rescaling, as the bf16 kernel: the reference max moves only when
      // the tile max passes it by more than kRescaleLog2 (or on the first
      // tile with a valid key), so the accumulators are rescaled only then.
      float alpha;
      const bool rescale = lazy_max_advance(m_run, tmax, alpha);
      const float m_new = m_run;
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int tk0 = (part * TPT + u) * 16 + 4 * g;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = (mask >> (tk0 + i)) & 1ull;
          pv[i] = v ? __builtin_amdgcn_exp2f(z[u][i] - m_new) : 0.f;
          psum += pv[i];
        }
        // P'_c = p * scale_c for the 4 scale groups
        float s4[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 s = *reinterpret_cast<const float4*>(tile + kTileScaleOff + (tk0 + i) * 16);
          s4[i][0] = s.x; s4[i][1] = s.y; s4[i][2] = s.z; s4[i][3] = s.w;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint2 pk;
          pk.x = pack_bf16x2(pv[0] * s4[0][c], pv[1] * s4[1][c]);
          pk.y = pack_bf16x2(pv[2] * s4[2][c], pv[3] * s4[3][c]);
          *reinterpret_cast<uint2*>(&sh.p[ht][c][n16][tk0]) = pk;
        }
      }
      l_part = l_part * alpha + psum;
      if (__ballot(rescale) != 0ull) {                 // rare: a head's maximum moved up
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      }
      // At 64-head blocks the next copy goes out after the softmax instead of
      // between the QK steps (GRBM cycles at 64 heads over 128 rows -3.2 %; at
      // 16 heads it costs 6 %, so smaller blocks keep the spread copies).
      if constexpr (HT >= 4) {
        if (pre) {
#pragma unroll
          for (int i = 0; i < ND; ++i) gather_one(gsrc, gssrc, gdst, i);
        }
      }
      __syncthreads();                                 // P' of all token tiles

      // O^T += V^T . P'^T over the 64 tokens, 32 per MFMA: k slot j of lane
      // group g is token 32 tp + 8 g + j.
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        v8bf pb[NG];
#pragma unroll
        for (int c = 0; c < NG; ++c)
          pb[c] = as_v8bf(*reinterpret_cast<const uint4*>(&sh.p[ht][d_base / 128 + c][n16][32 * tp + 8 * g]));
        const int tok = 32 * tp + 8 * g + pv_r8;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int dta = d_base / 16 + dt;                // dim tile over the 512 latent dims
          const v2i raw = lds_read_tr8(tile + tile_off(dta >> 3, tok, dta & 7) + pv_half);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_v8bf((uint32_t)raw[0], (uint32_t)raw[1]),
                                                            pb[dt / 8], acc[dt], 0, 0, 0);
        }
      }
    }
  }

  float l_tot = l_part + lane_xor16(l_part);
  l_tot += lane_xor32(l_tot);
  if (TP > 1) {
    __syncthreads();
    if (g == 0) sh.tmax[ht][part][n16] = l_tot;
    __syncthreads();
    l_tot = 0.f;
#pragma unroll
    for (int pp = 0; pp < TP; ++pp) l_tot += sh.tmax[ht][pp][n16];
  }

  // Output addresses from a lane index the compiler cannot see through, so
  // they are formed here and not held (or spilled) across the tile loop.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int ho = hb * (16 * HT) + ht * 16 + (ln & 15);   // = h
  const int go = ln >> 4;                                  // = g
  if (!on) return;
  if (a.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = a.out + ((int64_t)r * a.H + ho) * kVDim + d_base + 4 * go;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      pk.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + dt * 16) = pk;
    }
    if (part == 0 && go == 0)
      a.lse[(int64_t)r * a.H + ho] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t base = ((int64_t)sp * R + r) * a.H + ho;
    float* pa = a.part_acc + base * kVDim + d_base + 4 * go;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4*>(pa + dt * 16) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (part == 0 && go == 0) {
      a.part_ml[base * 2] = l_tot > 0.f ? m_run : kMaskSentinel;
      a.part_ml[base * 2 + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// 64-head blocks over the fp8 cache, wave-specialised like the bf16 kernel's
// 64-head form: waves 0-3 score (wave w: head tile w over all 32 tokens of a
// tile), waves 4-7 multiply (wave 4 + w: dims 128 w .. 128 w + 127, which is
// exactly scale group w, of all four head tiles).  PV wave 4 + w copies row
// group w (8 tokens: 640 bytes of codes and rope, 16 bytes of scales) of each
// tile into a ring of three fp8 buffers three tiles ahead, and one iteration
// before a tile is scored it converts those rows (e4m3 -> bf16, exact, scale
// 1) into one of two bf16 tiles laid out as the bf16 kernel's, rope copied.
// The scorers then run the bf16 kernel's QK with one accumulator per scale
// group (and one for the rope): z = rope + sum_g scale_g * acc_g in fp32
// keeps every product exact.  The scorers store fp32 probabilities; PV wave
// 4 + w folds its own group's scale in, P'_w = bf16(p * scale_w), and
// multiplies the converted V^T.  The index ring is kept by scorer wave 0, so
// the PV waves' memory counters hold only their copies.  At 64 heads over
// 128 rows (k = 2048) it takes 7.7 % fewer cycles than the four-head-tile
// form of the kernel above; the PV waves bound it (probability scaling,
// conversion and copies on top of the products: ~3,800 cycles an iteration
// against the scorers' ~2,100).
constexpr int kTileF = 32;                               // tokens per tile
constexpr int kRgF = kTileF / 8;                         // row groups per tile
constexpr int kCvBytes = kTileF * kKvDim * 2;            // 36864: converted tile (bf16 layout)
constexpr int kF8Scale = 5 * kRgF * 1024;                // 20480: scale records in an fp8 ring tile
constexpr int kF8Bytes = kF8Scale + kTileF * 16;         // 20992
constexpr int kF8Buf = 3;                                // fp8 ring tiles
constexpr int kPairSlotsF = 8;
constexpr int kQkAheadF = 4;
constexpr int kCopiesF = 6;                              // copies per PV wave and tile (5 column groups + scales)

struct WsShared8 {
  float4 pf[2][4][2][4][16];        // fp32 probabilities [tile & 1][head tile][token tile][g][head]
  float alpha[2][64];               // rescale factor of each head for tile & 1
  int resc[2][4];                   // scorer w moved the reference max of some head in tile & 1
  float m[64];                      // final reference max of each head (log2 domain)
  float l[64];                      // final row sum of each head
  int idx[kPairSlotsF][64];         // indices of tiles 2P, 2P + 1 in slot P % 8
  int page[kPairSlotsF][64];        // their block-table entries
  float4 scl[3][kTileF];            // the 4 group scales of each token of tile t in slot t % 3
  unsigned char cv[2][kCvBytes];    // converted tiles (bf16, the bf16 kernel's tile layout)
  unsigned char f8[kF8Buf][kF8Bytes];   // copied fp8 rows: 1 KB blocks (column group, row group), unswizzled
};

__global__ void __launch_bounds__(512) sparse_mla_fp8_ws_kernel(MlaArgs a) {
  constexpr int NDT = 8;                  // 16-dim tiles per PV wave
  __shared__ WsShared8 sh;

  const int R = a.batch.num_rows;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n16 = lane & 15;
  const int bid = blockIdx.x;
  const int q8 = bid >> 3;
  const int hb = q8 % a.head_blocks;
  const int rest = (q8 / a.head_blocks) * 8 + (bid & 7);
  if (rest >= R * a.splits) return;
  const int r = rest / a.splits;
  const int sp = rest % a.splits;
  const int hbase = hb * 64;
  const bool scorer = wave < 4;
  const int w4 = wave & 3;

  const int slot0 = sp * a.split_slots;
  const int slot1 = min(slot0 + a.split_slots, a.k);
  const int ntiles = (slot1 - slot0 + kTileF - 1) / kTileF;

  // Index ring: the indices of tile pair P go to slot P % 8 of sh.idx, then
  // their block-table entries to sh.page (wave 0: pairs 0-4 and 0-3 before
  // the loop, pair (i + 9) / 2 and (i + 7) / 2 after odd iterations i).
  const int32_t* idx_row = a.indices + (int64_t)r * a.k;
  int bc = 0, e = 0;
  auto issue_idx = [&](int P) {
    const int j = min(slot0 + P * 64 + lane, slot1 - 1);
    lds_dma4(idx_row + j, lds_addr(sh.idx[P & 7]));
  };
  auto issue_page_from = [&](int P, int idx) {
    const int ic = (idx >= 0 && idx < a.batch.max_seq_len) ? idx : 0;
    lds_dma4(a.batch.block_table + (int64_t)bc * a.batch.bt_stride + (ic >> 6), lds_addr(sh.page[P & 7]));
  };
  auto entry = [&](int t, int tok, int& ix, int& pg) __attribute__((always_inline)) {
    const int o = (t & 1) * kTileF + tok;
    ix = sh.idx[(t >> 1) & 7][o];
    pg = sh.page[(t >> 1) & 7][o];
  };
  auto valid_tok = [&](int t, int tok, int ix, int pg) __attribute__((always_inline)) {
    return slot0 + t * kTileF + tok < slot1 && ix >= 0 && ix < e && pg >= 0 && pg < a.batch.num_pages;
  };

  if (wave == 0 && ntiles > 0) {
#pragma unroll
    for (int P = 0; P < 5; ++P) issue_idx(P);
  }
  {
    int b;
    seq_and_extent_wave(a.batch, r, b, e);
    bc = b >= 0 ? b : 0;
  }

  if (scorer) {
    // ------------------------------------------------------------ scorers
    const int ht = w4;
    const int hq = hbase + ht * 16 < a.H ? hbase + ht * 16 + n16 : hbase + n16;
    uint4 qreg[18];
    {
      const uint16_t* qp = a.q + ((int64_t)r * a.H + hq) * kKvDim + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);
    }
    wait_vmcnt<0>();
    if (wave == 0 && ntiles > 0) {
#pragma unroll
      for (int P = 0; P < 4; ++P) issue_page_from(P, sh.idx[P & 7][lane]);
      wait_vmcnt<0>();
    }
    __syncthreads();                                     // B_pre0: table entries of pairs 0-3 visible
    __syncthreads();                                     // B_pre1: tile 0 converted

    const int r8 = n16 & 7;
    const int qk0 = (n16 >> 3) * 1024 + r8 * 128 + ((g ^ r8) << 4);
    float m_run = kMaskSentinel;
    float l_part = 0.f;
    uint32_t mask_n = 0u;
    if (ntiles > 0) {
      int ix, pg;
      entry(0, lane & 31, ix, pg);
      mask_n = (uint32_t)__ballot(valid_tok(0, lane & 31, ix, pg));
    }
    for (int i = 0; i <= ntiles; ++i) {
      const bool ring = wave == 0 && (i & 1) && ((i + 7) >> 1) * 2 < ntiles;
      if (i < ntiles) {
        const uint32_t mask = mask_n;
        // ring entries for the next mask, the tile's scales, wave 0's index for its table lookups
        int idx_m, page_m;
        entry(i + 1, lane & 31, idx_m, page_m);
        const int idx_r = sh.idx[((i + 7) >> 1) & 7][lane];
        float4 sc[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) sc[tt][j] = sh.scl[i % 3][16 * tt + 4 * g + j];
        asm volatile("" ::: "memory");   // issue those reads here, ahead of the QK operand reads
        const int sl = i & 1;
        // accumulators: scale groups 0-3 of the latent dims, then the rope
        v4f s[5][2];
#pragma unroll
        for (int gg = 0; gg < 5; ++gg)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) s[gg][tt] = v4f{0.f, 0.f, 0.f, 0.f};
        if (mask != 0u) {
          const unsigned char* tile = sh.cv[i & 1];
          // step q: token tile q & 1, k-step q >> 1 (scale group (q >> 1) / 4, rope from k-step 16)
          auto c_operand = [&](int q) __attribute__((always_inline)) {
            const int tt = q & 1, ks = q >> 1;
            return *reinterpret_cast<const uint4*>(tile + (qk0 ^ ((ks & 1) << 6)) + (ks >> 1) * (kRgF * 1024) +
                                                   tt * 2048);
          };
          uint4 cr[kQkAheadF + 1];
#pragma unroll
          for (int q = 0; q < kQkAheadF; ++q) cr[q] = c_operand(q);
#pragma unroll
          for (int q = 0; q < 36; ++q) {
            if (q + kQkAheadF < 36) cr[(q + kQkAheadF) % (kQkAheadF + 1)] = c_operand(q + kQkAheadF);
            const int gg = (q >> 1) < 16 ? (q >> 3) : 4;
            s[gg][q & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(cr[q % (kQkAheadF + 1)]),
                                                                  as_v8bf(qreg[q >> 1]), s[gg][q & 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // softmax of head tile ht over the tile's 32 tokens (token 16 tt + 4 g + j in s[.][tt][j])
        float z[2][4];
        float tmax = kMaskSentinel;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float d = s[4][tt][j];
            d = fmaf(sc[tt][j].x, s[0][tt][j], d);
            d = fmaf(sc[tt][j].y, s[1][tt][j], d);
            d = fmaf(sc[tt][j].z, s[2][tt][j], d);
            d = fmaf(sc[tt][j].w, s[3][tt][j], d);
            const bool v = (mask >> (16 * tt + 4 * g + j)) & 1u;
            z[tt][j] = v ? d * a.scale_log2 : kMaskSentinel;
            tmax = fmaxf(tmax, z[tt][j]);
          }
        tmax = fmaxf(tmax, lane_xor16(tmax));
        tmax = fmaxf(tmax, lane_xor32(tmax));
        float alpha;
        const bool rescale = lazy_max_advance(m_run, tmax, alpha);
        {
          const int t = i + 1;
          const bool v = t < ntiles && valid_tok(t, lane & 31, idx_m, page_m);
          mask_n = (uint32_t)__ballot(v);
        }
        __builtin_amdgcn_sched_barrier(0);
        float psum = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float pv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool v = (mask >> (16 * tt + 4 * g + j)) & 1u;
            pv[j] = v ? __builtin_amdgcn_exp2f(z[tt][j] - m_run) : 0.f;
            psum += pv[j];
          }
          sh.pf[sl][ht][tt][g][n16] = make_float4(pv[0], pv[1], pv[2], pv[3]);
        }
        l_part = l_part * alpha + psum;
        if (g == 0) sh.alpha[sl][ht * 16 + n16] = alpha;
        const bool any = __ballot(rescale) != 0ull;
        if (lane == 0) sh.resc[sl][ht] = any ? 1 : 0;
        // wave 0, odd iterations: the index ring -- table entries of pair
        // (i + 7) / 2, indices of pair (i + 9) / 2; they land before the next barrier
        if (ring) {
          issue_page_from((i + 7) >> 1, idx_r);
          issue_idx((i + 9) >> 1);
        }
      }
      if (ring) wait_vmcnt<2>();
      else wait_vmcnt<0>();
      __syncthreads();                                   // B_i
    }
    const float l_own = l_part + lane_xor16(l_part);
    const float l_sum = l_own + lane_xor32(l_own);
    if (g == 0) {
      sh.m[ht * 16 + n16] = m_run;
      sh.l[ht * 16 + n16] = l_sum;
    }
    __syncthreads();                                     // B_end
  } else {
    // ------------------------------------------------------------ PV waves
    // Copy of tile t (row group w4 into fp8 buffer t % 3): lane l copies slot
    // l & 7 of row l / 8 of each 128-byte column group (4 of codes, 1 of
    // rope); lanes 0-7 copy the scale records of the group's 8 tokens.
    auto copy_fp8 = [&](int t, int ix, int pg, int ixs, int pgs) __attribute__((always_inline)) {
      const int tok = 8 * w4 + (lane >> 3);
      const unsigned char* row =
          valid_tok(t, tok, ix, pg) ? a.kv8 + (int64_t)pg * a.kv8_stride + (ix & 63) * kRow8
                                    : reinterpret_cast<const unsigned char*>(g_zero_row8);
      const uint32_t dst = lds_addr(sh.f8[t % kF8Buf]);
#pragma unroll
      for (int cg = 0; cg < 5; ++cg) lds_dma16(row + cg * 128 + ((lane & 7) << 4), dst + (cg * kRgF + w4) * 1024);
      const int toks = 8 * w4 + (lane & 7);
      const unsigned char* srec =
          valid_tok(t, toks, ixs, pgs) ? a.kv8 + (int64_t)pgs * a.kv8_stride + kScaleOff8 + (ixs & 63) * 16
                                       : reinterpret_cast<const unsigned char*>(g_zero_row8);
      if (lane < 8) lds_dma16(srec, dst + kF8Scale + w4 * 128);
    };
    // Conversion of tile t's row group w4: lane l takes row l / 8, 16-byte
    // slot l & 7 of each column group; codes go to the bf16 tile (slot s of
    // row r8 holds chunk s ^ r8, as the bf16 kernel's copies leave it), rope
    // is copied, lanes 0-7 move the scale records.
    auto convert = [&](int t) __attribute__((always_inline)) {
      const unsigned char* src = sh.f8[t % kF8Buf];
      unsigned char* dst = sh.cv[t & 1];
      const int r8 = lane >> 3, c = lane & 7;
      uint4 raw[5];
#pragma unroll
      for (int cg = 0; cg < 5; ++cg)
        raw[cg] = *reinterpret_cast<const uint4*>(src + (cg * kRgF + w4) * 1024 + lane * 16);
      float4 srec = make_float4(0.f, 0.f, 0.f, 0.f);
      if (lane < 8) srec = *reinterpret_cast<const float4*>(src + kF8Scale + (8 * w4 + lane) * 16);
#pragma unroll
      for (int cg8 = 0; cg8 < 4; ++cg8) {
        // 16 codes: dims 128 cg8 + 16 c .. + 15 -> bf16 column group 2 cg8 + c / 4, chunks 2 (c % 4) and + 1
        const uint4 w = raw[cg8];
        const uint4 lo = make_uint4(fp8x2_to_bf16x2(w.x, false), fp8x2_to_bf16x2(w.x, true),
                                    fp8x2_to_bf16x2(w.y, false), fp8x2_to_bf16x2(w.y, true));
        const uint4 hi = make_uint4(fp8x2_to_bf16x2(w.z, false), fp8x2_to_bf16x2(w.z, true),
                                    fp8x2_to_bf16x2(w.w, false), fp8x2_to_bf16x2(w.w, true));
        const int cg = 2 * cg8 + (c >> 2), ch = 2 * (c & 3);
        unsigned char* blk = dst + (cg * kRgF + w4) * 1024 + r8 * 128;
        *reinterpret_cast<uint4*>(blk + ((ch ^ r8) << 4)) = lo;
        *reinterpret_cast<uint4*>(blk + (((ch + 1) ^ r8) << 4)) = hi;
      }
      *reinterpret_cast<uint4*>(dst + (8 * kRgF + w4) * 1024 + r8 * 128 + ((c ^ r8) << 4)) = raw[4];
      if (lane < 8) sh.scl[t % 3][8 * w4 + lane] = srec;
    };
    __syncthreads();                                     // B_pre0: table entries of pairs 0-3 visible
    int ixg = 0, pgg = 0, ixs = 0, pgs = 0;              // entries of this lane's rows of the next tile to copy
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t < ntiles) {
        entry(t, 8 * w4 + (lane >> 3), ixg, pgg);
        entry(t, 8 * w4 + (lane & 7), ixs, pgs);
        copy_fp8(t, ixg, pgg, ixs, pgs);
      }
    }
    entry(3, 8 * w4 + (lane >> 3), ixg, pgg);
    entry(3, 8 * w4 + (lane & 7), ixs, pgs);
    if (ntiles > 0) {
      if (ntiles > 2) wait_vmcnt<2 * kCopiesF>();
      else if (ntiles > 1) wait_vmcnt<kCopiesF>();
      else wait_vmcnt<0>();
      convert(0);
    }
    __syncthreads();                                     // B_pre1: tile 0 converted
    const int d_base = w4 * 128;
    const int pv_Lt = ((n16 >> 1) & 1) ^ (((g & 1) << 2) | (n16 >> 2));
    const int pv_lane = (g >> 1) * 1024 + (((g & 1) << 2) + (n16 >> 2)) * 128 + 8 * (n16 & 1);
    const int pv_part = (d_base >> 6) * (kRgF * 1024);
    v4f acc[4][NDT];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[ht][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    int idx_p = 0, page_p = -1;          // ring entries of tile i - 1, read one iteration ahead
    // V^T operands (dims 16 dt .. 16 dt + 15 of this wave's 128, all 32 tokens) of converted tile t
    auto v_operand = [&](int t, int dt) __attribute__((always_inline)) {
      const unsigned char* vb = sh.cv[t & 1] + pv_part + pv_lane + (dt >> 2) * (kRgF * 1024) +
                                ((pv_Lt ^ (2 * (dt & 3))) << 4);
      const v4s lo = lds_read_tr16(vb);
      const v4s hi = lds_read_tr16(vb + 2048);
      const v8s vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      v8bf va;
      __builtin_memcpy(&va, &vv, 16);
      return va;
    };
    v8bf vpre[NDT];                      // V^T operands of tile i - 1, read before the last barrier
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vpre[dt] = v8bf{};
    for (int i = 0; i <= ntiles; ++i) {
      int idx_c, page_c;
      entry(i, lane & 31, idx_c, page_c);
      // this wave's row group of tile i + 3 into the fp8 buffer tile i left
      // (converted last iteration); entries read one iteration ago
      const bool more3 = i + 3 < ntiles;
      if (more3) copy_fp8(i + 3, ixg, pgg, ixs, pgs);
      entry(i + 4, 8 * w4 + (lane >> 3), ixg, pgg);
      entry(i + 4, 8 * w4 + (lane & 7), ixs, pgs);
      asm volatile("" ::: "memory");
      if (i >= 1) {
        const int j = i - 1;
        const bool v = valid_tok(j, lane & 31, idx_p, page_p);
        const uint32_t mask = (uint32_t)__ballot(v);
        if (mask != 0u) {
          const int sl = j & 1;
          // one batch of reads: the rescale flags, the probabilities, this group's scales
          const int4 rs = *reinterpret_cast<const int4*>(sh.resc[sl]);
          float4 pp[4][2];
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) pp[ht][tt] = sh.pf[sl][ht][tt][g][n16];
          float sw[2][4];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              sw[tt][jj] = reinterpret_cast<const float*>(&sh.scl[j % 3][16 * tt + 4 * g + jj])[w4];
          v8bf pb[4];
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            uint4 u;
            u.x = pack_bf16x2(pp[ht][0].x * sw[0][0], pp[ht][0].y * sw[0][1]);
            u.y = pack_bf16x2(pp[ht][0].z * sw[0][2], pp[ht][0].w * sw[0][3]);
            u.z = pack_bf16x2(pp[ht][1].x * sw[1][0], pp[ht][1].y * sw[1][1]);
            u.w = pack_bf16x2(pp[ht][1].z * sw[1][2], pp[ht][1].w * sw[1][3]);
            pb[ht] = as_v8bf(u);
          }
          if ((rs.x | rs.y | rs.z | rs.w) != 0) {
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
              const float al = sh.alpha[sl][ht * 16 + n16];
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) acc[ht][dt] *= al;
            }
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
              acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vpre[dt], pb[ht], acc[ht][dt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      idx_p = idx_c;
      page_p = page_c;
      // tile i + 1: its copies (issued two iterations ago) have landed once at
      // most the later tiles' copies are in flight; converted for the next iteration
      if (i + 1 < ntiles) {
        const bool more2 = i + 2 < ntiles;
        if (more2 && more3) wait_vmcnt<2 * kCopiesF>();
        else if (more2 | more3) wait_vmcnt<kCopiesF>();
        else wait_vmcnt<0>();
        convert(i + 1);
      }
      // V^T operands of tile i for the next iteration
      if (i < ntiles) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vpre[dt] = v_operand(i, dt);
      }
      __syncthreads();                                   // B_i
    }
    __syncthreads();                                     // B_end: m and l of every head
    if (a.splits == 1) {
      // This wave's output (64 heads x its 128 dims) is staged as bf16 rows of
      // 256 B in half a converted-tile buffer (free: no copy, conversion or
      // operand read is outstanding past B_end; 16-byte chunks XOR-swizzled by
      // the head's low bits), then stored as whole lines, four heads per
      // instruction, as in the bf16-cache kernel.  Only this wave touches its
      // half, and the LDS operations of a wave execute in order.
      static_assert(2 * 64 * 256 <= kCvBytes, "two waves' output staging fit one converted tile");
      unsigned char* st = sh.cv[w4 >> 1] + (w4 & 1) * 16384;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const int h = ht * 16 + n16;
        const float l_tot = sh.l[h];
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const v4f o = acc[ht][dt];
          uint2 pk;
          pk.x = pack_bf16x2(o[0] * inv, o[1] * inv);
          pk.y = pack_bf16x2(o[2] * inv, o[3] * inv);
          *reinterpret_cast<uint2*>(st + h * 256 + (((2 * dt + (g >> 1)) ^ n16) << 4) + 8 * (g & 1)) = pk;
        }
        if (w4 == 0 && g == 0 && hbase + ht * 16 < a.H)
          a.lse[(int64_t)r * a.H + hbase + h] = l_tot > 0.f ? (sh.m[h] + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
      asm volatile("" ::: "memory");
      const int c = lane & 15;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (hbase + 16 * (q >> 2) >= a.H) break;          // missing head tiles (the last ones)
        const int h = 4 * q + (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(st + h * 256 + ((c ^ (h & 15)) << 4));
        *reinterpret_cast<uint4*>(a.out + ((int64_t)r * a.H + hbase + h) * kVDim + d_base + 8 * c) = v;
      }
    } else {
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        if (hbase + ht * 16 >= a.H) continue;            // a missing head tile
        const int hp = hbase + ht * 16 + n16;
        const float l_tot = sh.l[ht * 16 + n16];
        const float m_fin = sh.m[ht * 16 + n16];
        const int64_t base = ((int64_t)sp * R + r) * a.H + hp;
        float* pa = a.part_acc + base * kVDim + d_base + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const v4f o = acc[ht][dt];
          *reinterpret_cast<float4*>(pa + dt * 16) = make_float4(o[0], o[1], o[2], o[3]);
        }
        if (w4 == 0 && g == 0) {
          a.part_ml[base * 2] = l_tot > 0.f ? m_fin : kMaskSentinel;
          a.part_ml[base * 2 + 1] = l_tot;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_sparse_mla_fp8(const BatchArgs& batch, const uint16_t* q, int H, const uint8_t* kv8,
                                 int64_t kv8_stride, const int32_t* indices, int k, float softmax_scale,
                                 const MlaPlan& p, uint16_t* out, float* lse, void* workspace,
                                 hipStream_t stream) {
  if (batch.num_rows <= 0) return hipSuccess;
  MlaArgs a{};
  a.batch = batch;
  a.q = q;
  a.H = H;
  a.kv8 = kv8;
  a.kv8_stride = kv8_stride;
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
    hipLaunchKernelGGL((sparse_mla_fp8_kernel<1, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  } else if (H == 32) {
    hipLaunchKernelGGL((sparse_mla_fp8_kernel<2, 2>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sparse_mla_fp8_ws_kernel, dim3((unsigned)grid), dim3(512), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1) return err;
  return launch_sparse_mla_merge(a, p.splits, stream);
}

}  // namespace dsa
