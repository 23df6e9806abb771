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

__device__ __forceinline__ v8bf as_v8bf(uint4 x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// N-way merge of the split partials: one wave per (row, head), 8 dims per lane.
// Every load goes out before any is used -- the split maxima and sums
// (lane-parallel, lane i <-> split i) and the accumulators of the first U
// splits -- so the merge costs one memory round trip, not two.
__global__ void __launch_bounds__(256) sparse_mla_merge_kernel(MlaArgs a) {
  const int R = a.batch.num_rows;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)R * a.H) return;
  const int lane = lane_id();
  const int64_t RH = (int64_t)R * a.H;
  constexpr int U = 8;
  float4 x[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < a.splits) {
      const float4* src = reinterpret_cast<const float4*>(a.part_acc + (u * RH + pair) * kVDim + 8 * lane);
      x[u][0] = src[0];
      x[u][1] = src[1];
    }
  }
  float mi = kMaskSentinel, li = 0.f;
  if (lane < a.splits) {
    mi = a.part_ml[(lane * RH + pair) * 2];
    li = a.part_ml[(lane * RH + pair) * 2 + 1];
  }
  const float M = wave_max(mi);
  const float wi = li > 0.f ? exp2f(mi - M) : 0.f;
  const float L = wave_sum(li * wi);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < a.splits; i0 += U) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u < a.splits) {
          const float4* src =
              reinterpret_cast<const float4*>(a.part_acc + ((i0 + u) * RH + pair) * kVDim + 8 * lane);
          x[u][0] = src[0];
          x[u][1] = src[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < a.splits) {
        const float wgt = __shfl(wi, i0 + u, 64);
        o[0] += wgt * x[u][0].x; o[1] += wgt * x[u][0].y; o[2] += wgt * x[u][0].z; o[3] += wgt * x[u][0].w;
        o[4] += wgt * x[u][1].x; o[5] += wgt * x[u][1].y; o[6] += wgt * x[u][1].z; o[7] += wgt * x[u][1].w;
      }
    }
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
}  // namespace dsa
