// Pieces shared by the sparse MLA kernels over the bf16 and the fp8 latent
// caches: the argument block, the LDS helpers (direct global->LDS copies,
// transposing LDS reads) and the N-way merge of split partials, whose layout
// both kernels write identically.
#pragma once

#include "common.h"

namespace dsa {
namespace {

struct MlaArgs {
  BatchArgs batch;
  const uint16_t* q;
  int H;
  const uint16_t* kv;      // bf16 latent cache
  int64_t kv_stride;       // elements between pages
  const uint8_t* kv8;      // fp8 latent cache (the fp8 kernel)
  int64_t kv8_stride;      // bytes between pages
  const int32_t* indices;
  int k;
  float scale_log2;        // softmax_scale * log2(e)
  int splits;
  int split_slots;         // k slots per split (multiple of 64)
  int head_blocks;         // workgroups per (row, split)
  uint16_t* out;
  float* lse;
  float* part_acc;         // [splits, R, H, 512]
  float* part_ml;          // [splits, R, H, 2]: running max (log2 domain), sum
};

typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane n receives element
// n % 4 of the 8-byte vectors addressed by lanes n / 4 + 4 j, j = 0..3.
__device__ __forceinline__ v4s lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(const __attribute__((address_space(3))) void*)p);
}

typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
// The packed pair is read back whole: element-wise reads of a bf16 vector
// have given wrong lanes with this compiler.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const v2bf16 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Lazy rescaling of the online softmax: a head's reference max m (log2
// domain) moves only when a tile's max tm passes it by more than
// kRescaleLog2, or on its first tile with a valid key (m still the -1e30
// sentinel, nothing accumulated yet).  The probabilities exp2(z - m) then stay
// below 2^kRescaleLog2, in range for bf16 and fp32, and out = acc / l and
// lse = m + log2 l do not depend on which m was used, so the accumulators need
// rescaling (by alpha) only on the tiles where this returns true.
constexpr float kRescaleLog2 = 8.f;
__device__ __forceinline__ bool lazy_max_advance(float& m, float tm, float& alpha) {
  const bool first = m == kMaskSentinel;
  const bool move = first || tm > m + kRescaleLog2;
  alpha = (move && !first) ? __builtin_amdgcn_exp2f(m - tm) : 1.f;   // v_exp_f32 directly
  m = move ? tm : m;
  return move && !first;
}

__device__ __forceinline__ v8bf as_v8bf(uint4 x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// N-way merge of the split partials.  A (row, head) pair is spread over
// 8 / DPL waves, each lane merging DPL consecutive dims, and a wave keeps
// U = 64 / DPL splits in flight (64 accumulator values per lane): every load
// of a round goes out before any is used -- the split maxima and sums
// (lane-parallel, lane i <-> split i) and the accumulators of U splits -- so
// up to U splits cost one memory round trip.  The launcher picks the smallest
// DPL that still holds every split in one round (8 splits: one wave per pair
// with 8 dims per lane; 32 splits: four waves per pair with 2 dims per lane).
template <int DPL>
__global__ void __launch_bounds__(256) sparse_mla_merge_kernel(MlaArgs a) {
  static_assert(DPL == 2 || DPL == 4 || DPL == 8, "dims per lane");
  constexpr int WPP = 8 / DPL;        // waves per (row, head) pair
  constexpr int U = 64 / DPL;         // splits per load round
  const int R = a.batch.num_rows;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t pair = gw / WPP;
  if (pair >= (int64_t)R * a.H) return;
  const int lane = lane_id();
  const int d0 = (int)(gw % WPP) * (64 * DPL) + DPL * lane;
  const int64_t RH = (int64_t)R * a.H;
  float x[U][DPL];
  auto load = [&](int u, int split) __attribute__((always_inline)) {
    const float* src = a.part_acc + (split * RH + pair) * kVDim + d0;
    if constexpr (DPL == 8) {
      const float4 v0 = reinterpret_cast<const float4*>(src)[0], v1 = reinterpret_cast<const float4*>(src)[1];
      x[u][0] = v0.x; x[u][1] = v0.y; x[u][2] = v0.z; x[u][3] = v0.w;
      x[u][4] = v1.x; x[u][5] = v1.y; x[u][6] = v1.z; x[u][7] = v1.w;
    } else if constexpr (DPL == 4) {
      const float4 v = *reinterpret_cast<const float4*>(src);
      x[u][0] = v.x; x[u][1] = v.y; x[u][2] = v.z; x[u][3] = v.w;
    } else {
      const float2 v = *reinterpret_cast<const float2*>(src);
      x[u][0] = v.x; x[u][1] = v.y;
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < a.splits) load(u, u);
  float mi = kMaskSentinel, li = 0.f;
  if (lane < a.splits) {
    mi = a.part_ml[(lane * RH + pair) * 2];
    li = a.part_ml[(lane * RH + pair) * 2 + 1];
  }
  const float M = wave_max(mi);
  const float wi = li > 0.f ? exp2f(mi - M) : 0.f;
  const float L = wave_sum(li * wi);
  float o[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) o[d] = 0.f;
  for (int i0 = 0; i0 < a.splits; i0 += U) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u < a.splits) load(u, i0 + u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < a.splits) {
        const float wgt = __shfl(wi, i0 + u, 64);
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[d] += wgt * x[u][d];
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t pk[DPL / 2];
#pragma unroll
  for (int d = 0; d < DPL / 2; ++d)
    pk[d] = pack_bf16x2(o[2 * d] * inv, o[2 * d + 1] * inv);
  uint16_t* dst = a.out + pair * kVDim + d0;
  if constexpr (DPL == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  else if constexpr (DPL == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
  else *reinterpret_cast<uint32_t*>(dst) = pk[0];
  if (lane == 0 && gw % WPP == 0) a.lse[pair] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// Launch of the merge for R rows of H heads over `splits` partials.
__host__ inline hipError_t launch_sparse_mla_merge(const MlaArgs& a, int splits, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.batch.num_rows * a.H;
  if (splits <= 8) {
    hipLaunchKernelGGL(sparse_mla_merge_kernel<8>, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream, a);
  } else if (splits <= 16) {
    hipLaunchKernelGGL(sparse_mla_merge_kernel<4>, dim3((unsigned)((pairs + 1) / 2)), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sparse_mla_merge_kernel<2>, dim3((unsigned)pairs), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace dsa
