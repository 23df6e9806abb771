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
  // 4 tiles per split (c2) asking for two at once delays the first (24.9 us
  // against 24.0 us).
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
    hipLaunchKernelGGL((sparse_mla_fp8_kernel<4, 2>), dim3((unsigned)grid), dim3(512), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1) return err;
  return launch_sparse_mla_merge(a, p.splits, stream);
}

}  // namespace dsa
