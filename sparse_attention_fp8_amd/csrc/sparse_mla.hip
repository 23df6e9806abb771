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
//  * Workgroup = one (row, split, head block).  Head block and wave roles:
//      16 heads:  4 waves, each scores 16 of the tile's 64 tokens and
//                 accumulates 128 of the 512 output dims;
//      32 heads:  4 waves = 2 head tiles x 2 parts (32 tokens / 256 dims each);
//      >=48 heads: 8 waves = 4 head tiles x 2 parts, 64-head blocks; in PV
//      each wave instead takes two head tiles over 128 dims.  When H is not a
//      multiple of 64 the last block holds H % 64 heads: its missing head
//      tiles score the block's first head tile and store nothing (the same
//      instruction stream as a full block: a branch inside the tile loop
//      costs every head count a fifth of its speed).
//    Scores of a head tile are computed once; the tile maxima and the bf16
//    probabilities are exchanged through LDS between the waves, and every
//    wave accumulates its own (heads, dims) block over all 64 tokens.
//  * Gather: the 64 selected latent rows of a tile (64 x 1152 B) are copied
//    from HBM straight into LDS with global_load_lds_dwordx4 into two buffers.
//    With 16 heads the copy of tile i+2 is issued as soon as tile i's buffer
//    is released, so two tiles are in flight whenever a wave waits (a wait
//    with one tile in flight leaves the HBM queue half empty: the gather of
//    32 decode rows of 16 heads over k = 2048 takes about 1.6x as long).  Larger head blocks keep one tile
//    ahead and spread its copy over the QK steps of the tile being
//    multiplied, which hides the copy issue behind their MFMAs.  Each lane
//    supplies its own source address, so the gather through the block table
//    costs nothing extra; masked slots read a static
//    zero row.  The LDS tile is made of 1 KB blocks (128-byte column group of
//    the row, group of 8 rows) whose 16-byte slot s of row r8 holds the row's
//    chunk s ^ r8: one wave-wide copy fills one block from eight whole
//    128-byte lines, and the operand reads spread over the banks.  The V^T
//    operand of PV comes from transposing 16-bit LDS reads
//    (ds_read_b64_tr_b16).
//  * Row pointers: wave 0 copies each tile's indices and then their
//    block-table entries into a 4-slot LDS ring with direct global->LDS
//    copies, three and two tiles ahead of use.  No register is ever written
//    by a pending load, so every wait is an exact count of outstanding copies
//    and none waits for a gather issued after the copy it needs.
//  * QK: S^T[token, head] = C . Q^T with v_mfma_f32_16x16x32_bf16 (M = 16
//    tokens, N = 16 heads, K = 32 dims, 18 steps over 576 dims); Q stays in
//    registers.  The S^T accumulator gives each lane one head and 4 tokens of
//    a token tile -- exactly the B-operand layout of PV.
//  * PV: O^T[dim, head] += V^T . P^T (M = 16 dims, N = 16 heads, K = 32
//    tokens) with V^T read from the token-major LDS tile.
//  * The head blocks of one (row, split) are placed on one XCD (workgroup ids
//    8 apart) so their identical gathers meet in that XCD's L2.
#include "common.h"
#include "kernels.h"
#include "mla_common.h"

namespace dsa {

namespace {

constexpr int kTile = 64;                      // selected tokens per LDS tile
constexpr int kChunks = kKvDim * 2 / 16;       // 72 sixteen-byte chunks per latent row
constexpr int kChunkGroups = kChunks / 8;      // 9 groups of 128 B per row
constexpr int kRowGroups = kTile / 8;          // 8 groups of 8 rows per tile
constexpr int kTileBytes = kTile * kChunks * 16;   // 73728

__device__ __attribute__((aligned(16))) uint4 g_zero_row[kChunks] = {};

// LDS of one workgroup with HT head tiles and TP parts per head tile.  The
// small arrays come first: one per-lane base register plus the instructions'
// 16-bit offsets then reaches all of them (behind the 147 KB of tiles every
// distinct access would hold an address register across the tile loop).
template <int HT, int TP>
struct MlaShared {
  uint2 p[HT][4][4][16];                             // bf16 probabilities [tile][g][head]
  float tmax[HT][TP][16];                             // per-part tile maxima
  int idx[4][kTile];                                  // indices of tile t (ring slot t % 4)
  int page[4][kTile];                                 // their block-table entries
  unsigned char tile[2][kTileBytes];                 // double-buffered gathered rows
};

// DEEP: two tiles in flight while a wave waits (tile t + 2's copy goes out in
// one burst when tile t's buffer is released).  Otherwise one tile ahead, its
// copy spread over the QK steps of the tile being multiplied: with 64 heads a
// tile carries enough MFMA work that a burst of copies stalls the waves longer
// than the second tile in flight saves (measured: 64 heads over 128 rows,
// 87.6 us one ahead against 96.8 us two ahead; 32 heads over 32 rows, 31.8
// against 33.6 us; 16 heads over the same rows, 27.0 against 25.8 us).
//
// PVH: head tiles per wave in PV.  QK keeps one 16-head tile per wave (its q
// operand takes 72 VGPRs), but a PV wave can take PVH head tiles over fewer
// dims, so that each transposed V^T read feeds PVH MFMAs.  With four head
// tiles the QK and PV phases both run at the LDS bandwidth (operand reads
// plus the next tile's copy).  The 16- and 32-head blocks launched below use
// PVH = 1; 64-head blocks go to the wave-specialised kernel further down
// (with this kernel, PVH = 4 -- V^T read once per tile by eight waves of 64
// dims -- was its best form).
template <int HT, int TP, bool DEEP, int PVH>
__global__ void __launch_bounds__(64 * HT * TP) sparse_mla_kernel(MlaArgs a) {
  constexpr int NW = HT * TP;          // waves
  constexpr int TPT = 4 / TP;          // token tiles of 16 scored per wave
  constexpr int HGP = HT / PVH;        // head groups in PV
  constexpr int TPV = NW / HGP;        // dim parts in PV
  constexpr int DW = kVDim / TPV;      // output dims per wave
  constexpr int NDT = DW / 16;         // dim tiles per wave
  constexpr int RGW = kRowGroups / NW; // row groups each wave gathers
  constexpr int ND = RGW * kChunkGroups;   // gather loads per wave and tile
  static_assert(RGW * NW == kRowGroups, "waves must split the row groups evenly");
  static_assert(DW % 64 == 0, "PV parts are whole 64-dim column groups");
  static_assert(ND + 2 < 64, "vmcnt range");
  static_assert(HGP * PVH == HT && TPV * HGP == NW, "PV roles must cover heads and dims");
  static_assert(TP > 1, "the tile maxima and sums are exchanged through LDS");
  __shared__ MlaShared<HT, TP> sh;

  const int R = a.batch.num_rows;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;            // k-group of the MFMA operands
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
  const int hgp = wave % HGP, dpart = wave / HGP;
  const int hp0 = hb * (16 * HT) + hgp * (16 * PVH) + n16;
  // Head tiles of this block that exist (a last block of H % 64 heads has
  // fewer; its tile 0 always does).  A missing tile is scored with the q of
  // the block's first tile and its results are not stored.  Wave-uniform.
  const int hq = hb * (16 * HT) + ht * 16 < a.H ? h : hb * (16 * HT) + n16;
  const int d_base = dpart * DW;

  const int slot0 = sp * a.split_slots;
  const int slot1 = min(slot0 + a.split_slots, a.k);
  const int ntiles = (slot1 - slot0 + kTile - 1) / kTile;

  // Row pointers.  Wave 0 copies the indices of tile t (lane = token) into
  // ring slot t % 4 of sh.idx, and later their block-table entries into
  // sh.page, both with direct global->LDS copies: the chain then needs no
  // register that a pending load writes, and every wait below is an exact
  // count of this wave's outstanding copies.  Positions past the split are
  // clamped to its last entry (and masked by position); an index outside
  // [0, max_seq_len) reads table entry 0 of the row (and is masked by value).
  const int32_t* idx_row = a.indices + (int64_t)r * a.k;
  int bc = 0, e = 0;
  auto issue_idx = [&](int t) {
    const int j = min(slot0 + t * kTile + lane, slot1 - 1);
    lds_dma4(idx_row + j, lds_addr(sh.idx[t & 3]));
  };
  auto issue_page = [&](int t) {
    const int idx = sh.idx[t & 3][lane];
    const int ic = (idx >= 0 && idx < a.batch.max_seq_len) ? idx : 0;
    lds_dma4(a.batch.block_table + (int64_t)bc * a.batch.bt_stride + (ic >> 6), lds_addr(sh.page[t & 3]));
  };
  // Source row of token tok of tile t; the static zero row when the token is
  // padding, past the split, outside [0, e_r) or on a page outside the cache.
  auto row_src = [&](int t, int tok, bool& valid) -> const unsigned char* {
    const int idx = sh.idx[t & 3][tok];
    const int page = sh.page[t & 3][tok];
    valid = slot0 + t * kTile + tok < slot1 && idx >= 0 && idx < e && page >= 0 && page < a.batch.num_pages;
    return valid ? reinterpret_cast<const unsigned char*>(a.kv + (int64_t)page * a.kv_stride + (idx & 63) * kKvDim)
                 : reinterpret_cast<const unsigned char*>(g_zero_row);
  };
  // Gather of tile t into buffer t & 1.  LDS layout of a tile: 1 KB block
  // (cg, rg) = (128-B column group of the row, group of 8 rows) at
  // (8 cg + rg) KB; inside it row r8 takes 128 B whose 16-B slot s holds the
  // row's chunk s ^ r8.  One wave-wide load fills one block: lane l copies
  // slot l & 7 of row l >> 3, so each load reads eight whole 128-B lines and
  // each lane needs one row pointer per row group.  Masked rows read the zero
  // row, so every wave issues exactly ND loads per tile.
  auto gather = [&](int t) __attribute__((always_inline)) {
    const unsigned char* src[RGW];
#pragma unroll
    for (int j = 0; j < RGW; ++j) {
      bool v;
      src[j] = row_src(t, (wave * RGW + j) * 8 + (lane >> 3), v) + (((lane & 7) ^ (lane >> 3)) << 4);
    }
    const uint32_t dst = lds_addr(sh.tile[t & 1]);
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int j = i / kChunkGroups, cg = i % kChunkGroups;
      lds_dma16(src[j] + cg * 128, dst + (cg * kRowGroups + wave * RGW + j) * 1024);
    }
  };

  // Prologue: wave 0's index copies of tiles 0..3 go out first, then Q (all
  // waves), then the sequence search; the block-table copies of tiles 0..2
  // follow once the indices are in.  Everything is waited for before the
  // first gather, so inside the loop only copies are ever outstanding.
  if (wave == 0 && ntiles > 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) issue_idx(t);
  }
  // Q^T operand: lane supplies head h, dims 32*ks + 8*g .. +8.
  uint4 qreg[18];
  {
    const uint16_t* qp = a.q + ((int64_t)r * a.H + hq) * kKvDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);
  }
  {
    int b;
    seq_and_extent_wave(a.batch, r, b, e);
    bc = b >= 0 ? b : 0;
  }
  wait_vmcnt<0>();
  if (wave == 0 && ntiles > 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t) issue_page(t);
    wait_vmcnt<0>();
  }
  __syncthreads();
  if (ntiles > 0) gather(0);
  if (DEEP && ntiles > 1) gather(1);

  // Operand addresses (bytes into a tile).  QK: lane reads row tt*16 + n16,
  // chunk 4 ks + g; the swizzle term is x0 for even ks and x0 ^ 64 for odd.
  const int r8 = n16 & 7;
  const int qk0 = (n16 >> 3) * 1024 + r8 * 128 + (((g ^ r8) << 4));
  // PV: the V^T operand comes from two transposed reads per MFMA.  Lane n16
  // of group g addresses token 32 tp + 4 g + n16 / 4 (+16 for the second
  // read), dims d_base + 16 dt + 4 (n16 % 4) .. +3, so after the transpose it
  // holds dim d_base + 16 dt + n16 of tokens 32 tp + 4 g + j.  The swizzle
  // slot is Lt ^ 2 (dt & 3) with the lane part Lt.
  const int pv_Lt = ((n16 >> 1) & 1) ^ (((g & 1) << 2) | (n16 >> 2));
  const int pv_lane = (g >> 1) * 1024 + (((g & 1) << 2) + (n16 >> 2)) * 128 + 8 * (n16 & 1);
  const int pv_part = (d_base >> 6) * (kRowGroups * 1024);

  v4f acc[PVH][NDT];
  float m_pv[PVH];
#pragma unroll
  for (int hh = 0; hh < PVH; ++hh) {
#pragma unroll
    for (int i = 0; i < NDT; ++i) acc[hh][i] = v4f{0.f, 0.f, 0.f, 0.f};
    m_pv[hh] = kMaskSentinel;
  }
  float m_run = kMaskSentinel;   // reference max of the log2-domain scores of head h (see below)
  float l_part = 0.f;            // this lane's share of the running sum

  // DEEP pipeline: the copy of tile t + 2 goes out as soon as every wave is
  // done with tile t's buffer, and wave 0 issues the table copy of tile t + 3
  // and the index copy of tile t + 4 just before it (copies retire in issue
  // order, so waiting for those never waits for a gather issued after them).
  // Otherwise: everything issued is waited for at the top of tile t, then wave
  // 0 issues the table copy of tile t + 2 and the index copy of tile t + 3, and
  // tile t + 1's copy is spread over tile t's QK steps.
  for (int t = 0; t < ntiles; ++t) {
    // this wave's copies of tile t: what was issued after them may stay out
    if (!DEEP || t + 1 >= ntiles) wait_vmcnt<0>();
    else if (wave == 0 && t >= 1 && t + 2 < ntiles) wait_vmcnt<ND + 2>();
    else wait_vmcnt<ND>();
    __syncthreads();                                   // tile t landed in every wave
    uint64_t mask;
    {
      bool v;
      row_src(t, lane, v);
      mask = __ballot(v);
    }
    // one-ahead schedule: sources of tile t + 1 (its table copy landed above)
    const bool pre = !DEEP && t + 1 < ntiles;
    const unsigned char* gsrc[RGW];
    const uint32_t gdst = lds_addr(sh.tile[(t + 1) & 1]);
    if (pre) {
#pragma unroll
      for (int j = 0; j < RGW; ++j) {
        bool v;
        gsrc[j] = row_src(t + 1, (wave * RGW + j) * 8 + (lane >> 3), v) + (((lane & 7) ^ (lane >> 3)) << 4);
      }
    }
    if (!DEEP && wave == 0 && t >= 1 && t + 2 < ntiles) {
      issue_page(t + 2);
      issue_idx(t + 3);
    }
    auto gather_one = [&](int i) {
      const int j = i / kChunkGroups, cg = i % kChunkGroups;
      lds_dma16(gsrc[j] + cg * 128, gdst + (cg * kRowGroups + wave * RGW + j) * 1024);
    };
    if (pre && mask == 0ull) {
#pragma unroll
      for (int i = 0; i < ND; ++i) gather_one(i);
    }

    if (mask != 0ull) {
      const unsigned char* tile = sh.tile[t & 1];
      // scores of this wave's token tiles
      v4f s[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int tt = part * TPT + u;
        s[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          constexpr int NQ = TPT * 18;
          const int q = u * 18 + ks;
#pragma unroll
          for (int i = 0; i < ND; ++i)
            if (i * NQ / ND == q && pre) gather_one(i);
          const unsigned char* cb = tile + (qk0 ^ ((ks & 1) << 6)) + (ks >> 1) * (kRowGroups * 1024) + tt * 2048;
          const uint4 cv = *reinterpret_cast<const uint4*>(cb);
          s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(cv), as_v8bf(qreg[ks]), s[u], 0, 0, 0);
        }
      }
      float tmax = kMaskSentinel;
#pragma unroll
      for (int u = 0; u < TPT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = (part * TPT + u) * 16 + 4 * g + i;
          const bool v = (mask >> tok) & 1ull;
          const float z = v ? s[u][i] * a.scale_log2 : kMaskSentinel;
          s[u][i] = z;
          tmax = fmaxf(tmax, z);
        }
      tmax = fmaxf(tmax, lane_xor16(tmax));
      tmax = fmaxf(tmax, lane_xor32(tmax));
      if (g == 0) {
        // The address is formed here rather than held across the loop: at
        // 256 VGPRs the compiler otherwise spills it, and the reload's
        // vmcnt(0) would wait for the next tile's copy.
        int n = n16;
        asm volatile("" : "+v"(n));
        sh.tmax[ht][part][n] = tmax;
      }
      __syncthreads();
#pragma unroll
      for (int pp = 0; pp < TP; ++pp) tmax = fmaxf(tmax, sh.tmax[ht][pp][n16]);
      // Lazy rescaling: a head's reference max moves only when the tile max
      // passes it by more than kRescaleLog2 (or on its first tile with a valid
      // key, when there is nothing to rescale).  The probabilities exp2(z - m)
      // then stay below 2^kRescaleLog2 -- in range for bf16 and fp32 -- and the
      // accumulators are rescaled only on those rare tiles (for these scores,
      // about never after the first), not with a VALU pass on every tile;
      // out = acc / l and lse = m + log2 l do not depend on which m was used.
      // The scoring wave and every PV wave holding a head take the same
      // decision from the same maxima.  v_exp_f32 directly: exp2f's extra
      // scaling only matters below 2^-126.
      float alpha;
      bool rescale = lazy_max_advance(m_run, tmax, alpha);
      const float m_new = m_run;
      float alpha_pv[PVH];
      if constexpr (PVH == 1) {
        alpha_pv[0] = alpha;
        m_pv[0] = m_new;
      } else {
        rescale = false;
#pragma unroll
        for (int hh = 0; hh < PVH; ++hh) {
          float tm = kMaskSentinel;
#pragma unroll
          for (int pp = 0; pp < TP; ++pp) tm = fmaxf(tm, sh.tmax[hgp * PVH + hh][pp][n16]);
          rescale |= lazy_max_advance(m_pv[hh], tm, alpha_pv[hh]);
        }
      }
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        uint2 pk;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = (part * TPT + u) * 16 + 4 * g + i;
          const bool v = (mask >> tok) & 1ull;
          pv[i] = v ? __builtin_amdgcn_exp2f(s[u][i] - m_new) : 0.f;
          psum += pv[i];
        }
        v4bf16 b4;
        b4[0] = (__bf16)pv[0]; b4[1] = (__bf16)pv[1]; b4[2] = (__bf16)pv[2]; b4[3] = (__bf16)pv[3];
        __builtin_memcpy(&pk, &b4, 8);
        sh.p[ht][part * TPT + u][g][n16] = pk;
      }
      l_part = l_part * alpha + psum;
      if (__ballot(rescale) != 0ull) {                 // rare: a head's maximum moved up
#pragma unroll
        for (int hh = 0; hh < PVH; ++hh)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[hh][dt] *= alpha_pv[hh];
      }
      __syncthreads();                                 // probabilities of all token tiles

      // O^T += V^T . P^T over the 64 tokens, 32 per MFMA: k slot i of lane group
      // g is token 32tp + 4g + i, slot 4 + i is token 32tp + 16 + 4g + i.
      const unsigned char* pv_base = tile + pv_part + pv_lane;
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        v8bf pb[PVH];
#pragma unroll
        for (int hh = 0; hh < PVH; ++hh) {
          const uint2 pa = sh.p[hgp * PVH + hh][2 * tp][g][n16];
          const uint2 pb2 = sh.p[hgp * PVH + hh][2 * tp + 1][g][n16];
          uint4 pcat = make_uint4(pa.x, pa.y, pb2.x, pb2.y);
          pb[hh] = as_v8bf(pcat);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const unsigned char* vb = pv_base + (dt >> 2) * (kRowGroups * 1024) + tp * 4096 +
                                    ((pv_Lt ^ (2 * (dt & 3))) << 4);
          const v4s lo = lds_read_tr16(vb);
          const v4s hi = lds_read_tr16(vb + 2048);
          const v8s vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          v8bf va;
          __builtin_memcpy(&va, &vv, 16);
#pragma unroll
          for (int hh = 0; hh < PVH; ++hh)
            acc[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hh], acc[hh][dt], 0, 0, 0);
        }
        asm volatile("" ::: "memory");   // the second step's reads stay behind the first's MFMAs (no spill at 64 heads)
      }
    }

    if (DEEP && t + 2 < ntiles) {
      if (wave == 0) wait_vmcnt<ND>();                 // table copy of tile t + 2, index copy of t + 3
      __syncthreads();                                 // buffer t & 1 is free; tile t + 2's table visible
      if (wave == 0 && t + 3 < ntiles) {
        issue_page(t + 3);
        issue_idx(t + 4);
      }
      gather(t + 2);
    }
  }

  // l of each PV head over all tokens: lane groups, then the parts of its head tile
  {
    const float l_own = l_part + lane_xor16(l_part);
    const float l_sum = l_own + lane_xor32(l_own);
    __syncthreads();
    if (g == 0) sh.tmax[ht][part][n16] = l_sum;
    __syncthreads();
  }
#pragma unroll
  for (int hh = 0; hh < PVH; ++hh) {
    float l_tot = 0.f;
#pragma unroll
    for (int pp = 0; pp < TP; ++pp) l_tot += sh.tmax[hgp * PVH + hh][pp][n16];
    const int hp = hp0 + 16 * hh;
    if (hp - n16 >= a.H) continue;                    // a missing head tile
    if (a.splits == 1) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* op = a.out + ((int64_t)r * a.H + hp) * kVDim + d_base + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const v4f o = acc[hh][dt];
        uint2 pk;
        pk.x = pack_bf16x2(o[0] * inv, o[1] * inv);
        pk.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        *reinterpret_cast<uint2*>(op + dt * 16) = pk;
      }
      if (dpart == 0 && g == 0)
        a.lse[(int64_t)r * a.H + hp] = l_tot > 0.f ? (m_pv[hh] + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else if constexpr (PVH == 1) {
      // The wave's partial (16 heads x DW dims, fp32) is staged in tile
      // buffer 0 (free: every wave is past two barriers since its last read,
      // and no copy is outstanding), 16-byte chunks XOR-swizzled by the head,
      // and stored as whole rows of DW dims: stored straight from the
      // accumulators every instruction writes 64 bytes to each of 16 rows.
      // Only this wave touches its part of the buffer, and the LDS operations
      // of a wave execute in order.
      constexpr int CH = DW / 4;                       // 16-byte chunks per head row
      static_assert(NW * 16 * DW * 4 <= kTileBytes, "partial staging fits one tile buffer");
      float* st = reinterpret_cast<float*>(sh.tile[0] + wave * (16 * DW * 4));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const v4f o = acc[0][dt];
        *reinterpret_cast<float4*>(st + n16 * DW + (((4 * dt + g) ^ n16) << 2)) = make_float4(o[0], o[1], o[2], o[3]);
      }
      asm volatile("" ::: "memory");
      const int64_t base0 = ((int64_t)sp * R + r) * a.H + (hp0 - n16);
#pragma unroll
      for (int q = 0; q < 16 * CH / 64; ++q) {
        const int hrow = (q * 64 + lane) / CH, c = (q * 64 + lane) % CH;
        const float4 v = *reinterpret_cast<const float4*>(st + hrow * DW + ((c ^ hrow) << 2));
        *reinterpret_cast<float4*>(a.part_acc + (base0 + hrow) * kVDim + d_base + 4 * c) = v;
      }
      if (dpart == 0 && g == 0) {
        const int64_t base = base0 + n16;
        a.part_ml[base * 2] = l_tot > 0.f ? m_pv[0] : kMaskSentinel;
        a.part_ml[base * 2 + 1] = l_tot;
      }
    } else {
      const int64_t base = ((int64_t)sp * R + r) * a.H + hp;
      float* pa = a.part_acc + base * kVDim + d_base + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const v4f o = acc[hh][dt];
        *reinterpret_cast<float4*>(pa + dt * 16) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (dpart == 0 && g == 0) {
        a.part_ml[base * 2] = l_tot > 0.f ? m_pv[hh] : kMaskSentinel;
        a.part_ml[base * 2 + 1] = l_tot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 64-head blocks, wave-specialised.  Waves 0-3 score (wave w: head tile w
// over all tokens of a tile), waves 4-7 multiply (wave 4 + d: dims
// 128 d .. 128 d + 127 of all four head tiles).  Tiles are 32 tokens in a
// ring of four LDS buffers: in iteration i the scorers run QK and the softmax
// of tile i while the PV waves copy tile i + 2 and accumulate tile i - 1,
// and one barrier ends the iteration.  Each SIMD holds one scoring and one PV
// wave, so the softmax's VALU work overlaps the other wave's MFMAs; a
// scorer holds all tokens of its head tile, so the tile maximum needs no
// exchange; and each V^T read feeds four MFMAs.  Measured against the
// eight-wave kernel above at 64 heads over 128 rows (k = 2048): 15 % fewer
// cycles.  The copies decide much of it: issued by the PV waves at the top of
// the iteration, from table entries read an iteration ahead, they have almost
// two iterations to land; issued after the PV products the kernel takes 4 %
// more cycles, issued by the scorers 8-12 % more.  Every LDS read a wave
// waits on after the barrier is issued in one batch (ring entries, rescale
// flags, probabilities), and the PV waves read their V^T operands for the
// next iteration before it (2 % fewer cycles): each round trip after the
// barrier costs several hundred cycles behind the scorers' operand reads.  What bounds it: the
// scorers' QK (each head tile reads the whole tile; the PV products share the
// matrix cores), then the softmax and its stores before the barrier, and on
// the PV side the round trip of the probabilities and the products.
constexpr int kTileW = 32;                            // tokens per tile
constexpr int kRgW = kTileW / 8;                      // row groups per tile
constexpr int kTileBytesW = kTileW * kChunks * 16;    // 36864
constexpr int kBufW = 4;                              // tile buffers
constexpr int kPairSlots = 8;                         // ring of 64-entry index / table slots
constexpr int kQkAheadW = 4;                          // C-operand reads in flight in QK

// Small arrays first: one per-lane base register plus 16-bit offsets reaches them.
struct WsShared {
  uint2 p[2][4][2][4][16];          // bf16 probabilities [tile & 1][head tile][token tile][g][head]
  float alpha[2][64];               // rescale factor of each head for tile & 1
  int resc[2][4];                   // scorer w moved the reference max of some head in tile & 1
  float m[64];                      // final reference max of each head (log2 domain)
  float l[64];                      // final row sum of each head
  int idx[kPairSlots][64];          // indices of tiles 2P, 2P + 1 in slot P % 8
  int page[kPairSlots][64];         // their block-table entries
  unsigned char tile[kBufW][kTileBytesW];   // gathered rows (1 KB blocks as above, 4 row groups)
};

__global__ void __launch_bounds__(512) sparse_mla_ws_kernel(MlaArgs a) {
  constexpr int ND = kChunkGroups;        // copies per scorer and tile (its row group, 9 column groups)
  constexpr int NDT = 8;                  // 16-dim tiles per PV wave
  __shared__ WsShared sh;

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
  const int ntiles = (slot1 - slot0 + kTileW - 1) / kTileW;

  // Row pointers: the indices of tile pair P (64 slots) are copied into ring
  // slot P % 8 of sh.idx, then their block-table entries into sh.page (wave 0
  // for pairs 0-3 before the loop, PV wave 4 inside it, so no scorer waits
  // for those round trips).
  const int32_t* idx_row = a.indices + (int64_t)r * a.k;
  int bc = 0, e = 0;
  auto issue_idx = [&](int P) {
    const int j = min(slot0 + P * 64 + lane, slot1 - 1);
    lds_dma4(idx_row + j, lds_addr(sh.idx[P & 7]));
  };
  auto issue_page = [&](int P) {
    const int idx = sh.idx[P & 7][lane];
    const int ic = (idx >= 0 && idx < a.batch.max_seq_len) ? idx : 0;
    lds_dma4(a.batch.block_table + (int64_t)bc * a.batch.bt_stride + (ic >> 6), lds_addr(sh.page[P & 7]));
  };
  auto row_src = [&](int t, int tok, bool& valid) -> const unsigned char* {
    const int o = (t & 1) * kTileW + tok;
    const int idx = sh.idx[(t >> 1) & 7][o];
    const int page = sh.page[(t >> 1) & 7][o];
    valid = slot0 + t * kTileW + tok < slot1 && idx >= 0 && idx < e && page >= 0 && page < a.batch.num_pages;
    return valid ? reinterpret_cast<const unsigned char*>(a.kv + (int64_t)page * a.kv_stride + (idx & 63) * kKvDim)
                 : reinterpret_cast<const unsigned char*>(g_zero_row);
  };
  auto tile_mask = [&](int t) -> uint32_t {
    bool v;
    row_src(t, lane & 31, v);
    return (uint32_t)__ballot(v);
  };
  // Copies of tile t: wave 4 + w takes row group w (lane l: slot l & 7 of row 8 w + l / 8).
  auto gather_src = [&](int t) -> const unsigned char* {
    bool v;
    return row_src(t, 8 * w4 + (lane >> 3), v) + (((lane & 7) ^ (lane >> 3)) << 4);
  };
  auto gather_dst = [&](int t) -> uint32_t { return lds_addr(sh.tile[t & 3]) + w4 * 1024; };
  // the same from ring entries read ahead (idx, page of this lane's row of tile t)
  auto gather_src_pre = [&](int t, int idx, int page) -> const unsigned char* {
    const int tok = 8 * w4 + (lane >> 3);
    const bool valid = slot0 + t * kTileW + tok < slot1 && idx >= 0 && idx < e && page >= 0 &&
                       page < a.batch.num_pages;
    const unsigned char* row = valid ? reinterpret_cast<const unsigned char*>(a.kv + (int64_t)page * a.kv_stride +
                                                                              (idx & 63) * kKvDim)
                                     : reinterpret_cast<const unsigned char*>(g_zero_row);
    return row + (((lane & 7) ^ (lane >> 3)) << 4);
  };

  if (wave == 0 && ntiles > 0) {
#pragma unroll
    for (int P = 0; P < 4; ++P) issue_idx(P);
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
      for (int P = 0; P < 3; ++P) issue_page(P);
      wait_vmcnt<0>();
    }
    __syncthreads();                                     // B_pre0: pairs 0-2 visible
    __syncthreads();                                     // B_pre1: tile 0 landed

    const int r8 = n16 & 7;
    const int qk0 = (n16 >> 3) * 1024 + r8 * 128 + ((g ^ r8) << 4);
    float m_run = kMaskSentinel;
    float l_part = 0.f;
    // The index-ring entries of the next iteration's mask (tile i + 1) are
    // read at the top of iteration i and used at its end: an LDS read right
    // after the barrier waits behind every wave's operand traffic (~800
    // cycles).  Table entries of tile t are visible from iteration t - 3 on.
    uint32_t mask_n = ntiles > 0 ? tile_mask(0) : 0u;
    for (int i = 0; i <= ntiles; ++i) {
      if (i < ntiles) {
        const uint32_t mask = mask_n;
        // raw ring entries for the next iteration
        const int om = ((i + 1) & 1) * kTileW + (lane & 31);
        const int idx_m = sh.idx[((i + 1) >> 1) & 7][om];
        const int page_m = sh.page[((i + 1) >> 1) & 7][om];
        asm volatile("" ::: "memory");   // issue those reads here, ahead of the QK operand reads
        const int sl = i & 1;
        v4f s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
        if (mask != 0u) {
          const unsigned char* tile = sh.tile[i & 3];
          // step q: token tile q & 1, k-step q >> 1; copies on every fourth step
          auto c_operand = [&](int q) __attribute__((always_inline)) {
            const int tt = q & 1, ks = q >> 1;
            return *reinterpret_cast<const uint4*>(tile + (qk0 ^ ((ks & 1) << 6)) + (ks >> 1) * (kRgW * 1024) +
                                                   tt * 2048);
          };
          uint4 cr[kQkAheadW + 1];
#pragma unroll
          for (int q = 0; q < kQkAheadW; ++q) cr[q] = c_operand(q);
#pragma unroll
          for (int q = 0; q < 36; ++q) {
            if (q + kQkAheadW < 36) cr[(q + kQkAheadW) % (kQkAheadW + 1)] = c_operand(q + kQkAheadW);
            s[q & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(cr[q % (kQkAheadW + 1)]),
                                                              as_v8bf(qreg[q >> 1]), s[q & 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // softmax of head tile ht over the tile's 32 tokens (token 16 tt + 4 g + j in s[tt][j])
        float tmax = kMaskSentinel;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool v = (mask >> (16 * tt + 4 * g + j)) & 1u;
            const float z = v ? s[tt][j] * a.scale_log2 : kMaskSentinel;
            s[tt][j] = z;
            tmax = fmaxf(tmax, z);
          }
        tmax = fmaxf(tmax, lane_xor16(tmax));
        tmax = fmaxf(tmax, lane_xor32(tmax));
        float alpha;
        const bool rescale = lazy_max_advance(m_run, tmax, alpha);
        {
          // the next tile's mask before this tile's stores, so its wait on the
          // ring reads (long landed) does not also wait for the stores
          const int t = i + 1;
          const bool v = t < ntiles && slot0 + t * kTileW + (lane & 31) < slot1 && idx_m >= 0 && idx_m < e &&
                         page_m >= 0 && page_m < a.batch.num_pages;
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
            pv[j] = v ? __builtin_amdgcn_exp2f(s[tt][j] - m_run) : 0.f;
            psum += pv[j];
          }
          v4bf16 b4;
          b4[0] = (__bf16)pv[0]; b4[1] = (__bf16)pv[1]; b4[2] = (__bf16)pv[2]; b4[3] = (__bf16)pv[3];
          uint2 pk;
          __builtin_memcpy(&pk, &b4, 8);
          sh.p[sl][ht][tt][g][n16] = pk;
        }
        l_part = l_part * alpha + psum;
        if (g == 0) sh.alpha[sl][ht * 16 + n16] = alpha;
        const bool any = __ballot(rescale) != 0ull;
        if (lane == 0) sh.resc[sl][ht] = any ? 1 : 0;
      }
      // this wave's copies of tile i + 1 (issued one iteration ago) have landed
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
    // PV wave 4 + w copies row group w of every tile (lane l: slot l % 8 of
    // row 8 w + l / 8); the scorers issue no copies.
    __syncthreads();                                     // B_pre0: pairs 0-2 visible
    auto gather_all = [&](int t) __attribute__((always_inline)) {
      const unsigned char* src = gather_src(t);
      const uint32_t dst = gather_dst(t);
#pragma unroll
      for (int cg = 0; cg < ND; ++cg) lds_dma16(src + cg * 128, dst + cg * (kRgW * 1024));
    };
    if (ntiles > 0) gather_all(0);
    if (ntiles > 1) {
      gather_all(1);
      wait_vmcnt<ND>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();                                     // B_pre1: tile 0 landed
    // this lane's copy source entries of tile 2 (pair 1, visible since B_pre0)
    int idx_g = sh.idx[1][8 * w4 + (lane >> 3)];
    int page_g = sh.page[1][8 * w4 + (lane >> 3)];
    const int d_base = w4 * 128;
    const int pv_Lt = ((n16 >> 1) & 1) ^ (((g & 1) << 2) | (n16 >> 2));
    const int pv_lane = (g >> 1) * 1024 + (((g & 1) << 2) + (n16 >> 2)) * 128 + 8 * (n16 & 1);
    const int pv_part = (d_base >> 6) * (kRgW * 1024);
    v4f acc[4][NDT];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[ht][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    int idx_p = 0, page_p = -1;          // ring entries of tile i - 1, read one iteration ahead
    // V^T operands (dims 16 dt .. 16 dt + 15 of this wave's 128, all 32 tokens) of tile t
    auto v_operand = [&](int t, int dt) __attribute__((always_inline)) {
      const unsigned char* vb = sh.tile[t & 3] + pv_part + pv_lane + (dt >> 2) * (kRgW * 1024) +
                                ((pv_Lt ^ (2 * (dt & 3))) << 4);
      const v4s lo = lds_read_tr16(vb);
      const v4s hi = lds_read_tr16(vb + 2048);
      const v8s vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      v8bf va;
      __builtin_memcpy(&va, &vv, 16);
      return va;
    };
    // V^T operands of tile i - 1, read before the last barrier: after it the
    // scorers' operand reads fill the LDS queue, and a wave reading its
    // operands there waits behind them
    v8bf vpre[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vpre[dt] = v8bf{};
    for (int i = 0; i <= ntiles; ++i) {
      const int om = (i & 1) * kTileW + (lane & 31);
      const int idx_c = sh.idx[(i >> 1) & 7][om];
      const int page_c = sh.page[(i >> 1) & 7][om];
      // this lane's copy source of tile i + 3 (entries visible since iteration i)
      const int og = ((i + 3) & 1) * kTileW + 8 * w4 + (lane >> 3);
      const int idx_gn = sh.idx[((i + 3) >> 1) & 7][og];
      const int page_gn = sh.page[((i + 3) >> 1) & 7][og];
      asm volatile("" ::: "memory");
      // the copy of tile i + 2, into the buffer tile i - 2 left (its PV ended
      // before the last barrier), from the entries read one iteration ago
      const bool more = i + 2 < ntiles;
      if (more) {
        const unsigned char* src = gather_src_pre(i + 2, idx_g, page_g);
        const uint32_t dst = gather_dst(i + 2);
#pragma unroll
        for (int cg = 0; cg < ND; ++cg) lds_dma16(src + cg * 128, dst + cg * (kRgW * 1024));
      }
      if (i >= 1) {
        const int j = i - 1;
        const bool v = slot0 + j * kTileW + (lane & 31) < slot1 && idx_p >= 0 && idx_p < e && page_p >= 0 &&
                       page_p < a.batch.num_pages;
        const uint32_t mask = (uint32_t)__ballot(v);
        if (mask != 0u) {
          const int sl = j & 1;
          // one batch of reads: the rescale flags and the probabilities
          const int4 rs = *reinterpret_cast<const int4*>(sh.resc[sl]);
          v8bf pb[4];
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            const uint2 p0 = sh.p[sl][ht][0][g][n16];
            const uint2 p1 = sh.p[sl][ht][1][g][n16];
            pb[ht] = as_v8bf(make_uint4(p0.x, p0.y, p1.x, p1.y));
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
      idx_g = idx_gn;
      page_g = page_gn;
      // V^T operands of tile i (landed since the last barrier) for the next iteration
      if (i < ntiles) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vpre[dt] = v_operand(i, dt);
      }
      // wave 4, odd iterations: the index ring -- the table entries of pair
      // (i + 5) / 2 and the indices of pair (i + 7) / 2
      const bool ring = wave == 4 && (i & 1) && ((i + 5) >> 1) * 2 < ntiles;
      if (ring) {
        issue_page((i + 5) >> 1);
        issue_idx((i + 7) >> 1);
      }
      // landed before the barrier: tile i + 1 (issued one iteration ago) and
      // the ring copies issued then; this iteration's may stay in flight
      if (more && ring) wait_vmcnt<ND + 2>();
      else if (more) wait_vmcnt<ND>();
      else if (ring) wait_vmcnt<2>();
      else wait_vmcnt<0>();
      __syncthreads();                                   // B_i
    }
    __syncthreads();                                     // B_end: m and l of every head
    if (a.splits == 1) {
      // This wave's output (64 heads x its 128 dims) is staged as bf16 rows of
      // 256 B in tile buffer w4 (free: no copy or operand read is outstanding
      // past B_end; 16-byte chunks XOR-swizzled by the head's low bits), then
      // stored as whole lines, four heads per instruction: stored straight
      // from the accumulators every instruction writes 32 bytes to each of 16
      // rows.  Only this wave touches the buffer, and the LDS operations of a
      // wave execute in order.
      static_assert(64 * 256 <= kTileBytesW, "output staging fits one tile buffer");
      unsigned char* st = sh.tile[w4];
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

MlaPlan plan_sparse_mla(int num_rows, int max_seq_len, int H, int k, int num_splits, int num_cus) {
  MlaPlan p{};
  const int head_blocks = H <= 32 ? 1 : (H + 63) / 64;   // 16-, 32- or 64-head workgroups
  const int live = max(1, min(k, max(max_seq_len, 1)));
  const int tiles = (live + kTile - 1) / kTile;      // tiles that can hold valid entries
  const int all_tiles = (k + kTile - 1) / kTile;
  int s = num_splits;
  if (s <= 0) {
    // one workgroup per CU (a workgroup holds two 73 KB tiles of LDS), never
    // more splits than tiles that can hold valid entries
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
    hipLaunchKernelGGL((sparse_mla_kernel<1, 4, true, 1>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  } else if (H == 32) {
    hipLaunchKernelGGL((sparse_mla_kernel<2, 2, false, 1>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sparse_mla_ws_kernel, dim3((unsigned)grid), dim3(512), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1) return err;
  return launch_sparse_mla_merge(a, p.splits, stream);
}

}  // namespace dsa
