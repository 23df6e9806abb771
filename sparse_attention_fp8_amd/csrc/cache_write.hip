// The steps just before the path: per-group fp8 quantisation of the indexer q
// (with the scale folded into the head weights), the paged indexer-K cache
// writer, and the bf16 latent-cache writer.
//
// The vllm-dsa-mtp-sm80 README names the first two (skew fix 1: the unfused
// per_token_group_quant_fp8 for the indexer q; skew fix 0: the indexer-K cache
// writer addressing pages through their stride) without printing them.  The
// arithmetic follows the plain reading: one fp32 scale per 128 values,
// scale = amax / 448 (1 for an all-zero group), codes = e4m3fn(x / scale)
// rounded to nearest even and saturated at +-448, every step in IEEE fp32.
//
// All three are HBM-streaming kernels.  A 128-value group (256 bytes of bf16)
// is owned by 16 lanes, 16 bytes each, so a wave moves 4 groups with 1 KB of
// fully coalesced loads; the group amax is a 4-step DPP max inside each row of
// 16 lanes (no LDS, no barrier), and each lane converts its 8 values with the
// hardware e4m3 converter and stores 8 code bytes.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kGroup = 128;            // values per quantisation group
constexpr int kGroupsPerBlock = 16;    // 16 lanes per group, 256 threads
constexpr float kE4m3Max = 448.f;

// DPP controls of the max tree inside a row of 16 lanes.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i inside each 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i inside each 16

template <int Ctrl>
__device__ __forceinline__ float dpp_max(float x) {
  const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
  return fmaxf(x, y);
}

// amax over the 16 lanes of a group (every lane gets it).  Inputs are >= 0.
__device__ __forceinline__ float group_amax(float v) {
  v = dpp_max<kDppXor1>(v);
  v = dpp_max<kDppXor2>(v);
  v = dpp_max<kDppHalfMirror>(v);
  return dpp_max<kDppMirror>(v);
}

struct GroupValues {
  float x[8];
};

__device__ __forceinline__ GroupValues load_group_part(const uint16_t* src) {
  const uint4 p = *reinterpret_cast<const uint4*>(src);
  GroupValues g;
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    g.x[2 * i] = bf16_lo(w[i]);
    g.x[2 * i + 1] = bf16_hi(w[i]);
  }
  return g;
}

// Quantises this lane's 8 values against the group scale: returns the 8 code
// bytes packed little-endian and the scale.
__device__ __forceinline__ uint2 quantise_part(const GroupValues& g, float& scale_out) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(g.x[i]));
  const float amax = group_amax(a);
  const float scale = amax > 0.f ? amax / kE4m3Max : 1.f;   // IEEE division
  uint32_t packed[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = __builtin_amdgcn_fmed3f(g.x[4 * h + i] / scale, -kE4m3Max, kE4m3Max);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);
    packed[h] = static_cast<uint32_t>(v);
  }
  scale_out = scale;
  return make_uint2(packed[0], packed[1]);
}

__global__ __launch_bounds__(256) void indexer_q_quant_kernel(const uint16_t* __restrict__ q,
                                                              const float* w, uint8_t* __restrict__ codes,
                                                              float* w_out, int64_t num_groups) {
  const int64_t g = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  // Whole 16-lane rows are in or out together, so the DPP tree never reads a
  // lane of another group.
  if (g >= num_groups) return;
  const GroupValues vals = load_group_part(q + g * kGroup + part * 8);
  float scale;
  const uint2 c = quantise_part(vals, scale);
  *reinterpret_cast<uint2*>(codes + g * kGroup + part * 8) = c;
  if (part == 0) w_out[g] = w[g] * scale;
}

__global__ __launch_bounds__(256) void indexer_k_quant_cache_kernel(const uint16_t* __restrict__ k, int64_t k_stride,
                                                                    const int64_t* __restrict__ slots,
                                                                    uint8_t* __restrict__ cache, int64_t page_stride,
                                                                    int num_pages, int num_tokens) {
  const int t = blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  if (t >= num_tokens) return;
  const int64_t slot = slots[t];
  // Padding tokens (slot < 0) and slots past the cache write nothing.  The
  // test is uniform over the 16 lanes of the token.
  if (slot < 0 || slot >= (int64_t)num_pages * kPage) return;
  const GroupValues vals = load_group_part(k + (int64_t)t * k_stride + part * 8);
  float scale;
  const uint2 c = quantise_part(vals, scale);
  uint8_t* page = cache + (slot / kPage) * page_stride;
  const int s = (int)(slot % kPage);
  *reinterpret_cast<uint2*>(page + s * kGroup + part * 8) = c;
  if (part == 0) *reinterpret_cast<float*>(page + kIdxScaleOff + 4 * s) = scale;
}

constexpr int kLatentChunks = kVDim * 2 / 16;   // 64 x 16 B of latent per token
constexpr int kRopeChunks = (kKvDim - kVDim) * 2 / 16;   // 8 x 16 B of rope
constexpr int kRowChunks = kLatentChunks + kRopeChunks;   // 72

__global__ __launch_bounds__(256) void latent_cache_write_kernel(const uint16_t* __restrict__ latent,
                                                                 int64_t latent_stride,
                                                                 const uint16_t* __restrict__ rope,
                                                                 int64_t rope_stride,
                                                                 const int64_t* __restrict__ slots,
                                                                 uint16_t* __restrict__ cache,
                                                                 int64_t page_stride, int num_pages,
                                                                 int64_t num_chunks) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_chunks) return;
  const int64_t t = i / kRowChunks;
  const int c = (int)(i - t * kRowChunks);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (int64_t)num_pages * kPage) return;
  const uint16_t* src = c < kLatentChunks ? latent + t * latent_stride + c * 8
                                          : rope + t * rope_stride + (c - kLatentChunks) * 8;
  uint16_t* dst = cache + (slot / kPage) * page_stride + (slot % kPage) * kKvDim + c * 8;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// fp8 latent cache page: row t at 640 t = 512 e4m3 codes + 64 bf16 rope;
// scale record (4 fp32) of token t at 40960 + 16 t.
constexpr int kRow8 = 640;
constexpr int kScaleOff8 = kPage * kRow8;

// One wave per token: lanes 16 c .. 16 c + 15 quantise latent group c (dims
// 128 c .. 128 c + 127), lanes 0..7 also copy 16 bytes of rope each.
__global__ __launch_bounds__(256) void latent_cache_write_fp8_kernel(const uint16_t* __restrict__ latent,
                                                                     int64_t latent_stride,
                                                                     const uint16_t* __restrict__ rope,
                                                                     int64_t rope_stride,
                                                                     const int64_t* __restrict__ slots,
                                                                     uint8_t* __restrict__ cache,
                                                                     int64_t page_stride, int num_pages,
                                                                     int num_tokens) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= num_tokens) return;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (int64_t)num_pages * kPage) return;
  const int c = lane >> 4, part = lane & 15;
  const GroupValues vals = load_group_part(latent + (int64_t)t * latent_stride + c * kGroup + part * 8);
  float scale;
  const uint2 codes = quantise_part(vals, scale);
  uint8_t* page = cache + (slot / kPage) * page_stride;
  const int s = (int)(slot % kPage);
  *reinterpret_cast<uint2*>(page + s * kRow8 + c * kGroup + part * 8) = codes;
  if (part == 0) *reinterpret_cast<float*>(page + kScaleOff8 + 16 * s + 4 * c) = scale;
  if (lane < 8)
    *reinterpret_cast<uint4*>(page + s * kRow8 + kVDim + 16 * lane) =
        *reinterpret_cast<const uint4*>(rope + (int64_t)t * rope_stride + 8 * lane);
}

}  // namespace

hipError_t launch_latent_cache_write_fp8(int num_tokens, const uint16_t* latent, int64_t latent_stride,
                                         const uint16_t* rope, int64_t rope_stride, const int64_t* slots,
                                         uint8_t* cache, int64_t page_stride, int num_pages, hipStream_t stream) {
  const int blocks = (num_tokens + 3) / 4;
  hipLaunchKernelGGL(latent_cache_write_fp8_kernel, dim3(blocks), dim3(256), 0, stream, latent, latent_stride, rope,
                     rope_stride, slots, cache, page_stride, num_pages, num_tokens);
  return hipGetLastError();
}

hipError_t launch_indexer_q_quant(int num_rows, const uint16_t* q, const float* w, uint8_t* codes, float* w_out,
                                  hipStream_t stream) {
  const int64_t groups = (int64_t)num_rows * kIdxHeads;
  const int64_t blocks = (groups + kGroupsPerBlock - 1) / kGroupsPerBlock;
  hipLaunchKernelGGL(indexer_q_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, q, w, codes, w_out,
                     groups);
  return hipGetLastError();
}

hipError_t launch_indexer_k_quant_cache(int num_tokens, const uint16_t* k, int64_t k_stride, const int64_t* slots,
                                        uint8_t* cache, int64_t page_stride, int num_pages, hipStream_t stream) {
  const int blocks = (num_tokens + kGroupsPerBlock - 1) / kGroupsPerBlock;
  hipLaunchKernelGGL(indexer_k_quant_cache_kernel, dim3(blocks), dim3(256), 0, stream, k, k_stride, slots, cache,
                     page_stride, num_pages, num_tokens);
  return hipGetLastError();
}

hipError_t launch_latent_cache_write(int num_tokens, const uint16_t* latent, int64_t latent_stride,
                                     const uint16_t* rope, int64_t rope_stride, const int64_t* slots,
                                     uint16_t* cache, int64_t page_stride, int num_pages, hipStream_t stream) {
  const int64_t chunks = (int64_t)num_tokens * kRowChunks;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(latent_cache_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, latent,
                     latent_stride, rope, rope_stride, slots, cache, page_stride, num_pages, chunks);
  return hipGetLastError();
}

}  // namespace dsa
