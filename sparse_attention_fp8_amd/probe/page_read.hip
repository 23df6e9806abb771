// Read-only ceiling probe for the paged indexer's memory traffic.
//
// Reads a list of whole indexer-cache pages (64 tokens x 132 bytes = 8,448
// bytes each) with the same copy pattern, ring depth and launch shape as the
// paged indexer -- eight 8-wave workgroups' worth of waves per CU, each wave an
// equal contiguous run of the list, every page copied global -> LDS with
// global_load_lds_dwordx4 into a two-page wave-private ring (eight 1 KB copies
// of eight 128-byte key rows, then the 256-byte scale block) -- but computes
// nothing: one dword per lane of each landed page is folded into a checksum
// so the copies cannot be dropped.  Its rate is what the indexer's bytes
// cost with this copy scheme and no arithmetic; bench.py reports it next to
// the device copy rate.  Built into its own library (libdsa_probe.so), not
// into libdsa.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 8;
constexpr int kRing = 2;
constexpr int kPageBytes = 64 * 132;     // 8448
constexpr int kCodeBytes = 64 * 128;     // 8192

__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
// 32-bit LDS address of a pointer into a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__global__ void __launch_bounds__(64 * kWaves) page_read_kernel(const uint8_t* cache, int64_t page_stride,
                                                                const int* ids, int total, uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kRing][kPageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
  const int p0 = (int)((int64_t)total * gw / nw);
  const int p1 = (int)((int64_t)total * (gw + 1) / nw);
  uint32_t sum = 0;
  // page ids of up to 64 pages of the run, one per lane (as the indexer's
  // block-table batch), so an issue needs no dependent load
  int pb = p0, lid = 0;
  auto load_ids = [&](int first) {
    pb = first;
    lid = 0;
    if (first + lane < p1) {
      const int id = ids[first + lane];
      lid = id >= 0 ? id : 0;       // used here, so the wait for it stays on this (rare) path
    }
  };
  if (p0 < p1) load_ids(p0);
  auto issue = [&](int p) {
    if (p - pb >= 64) load_ids(p);
    const int id = __builtin_amdgcn_readlane(lid, p - pb);
    const uint8_t* src = cache + (int64_t)id * page_stride;
    const uint32_t dst = lds_addr(ring[wave][(p - p0) % kRing]);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(src + i * 1024 + lane * 16, dst + i * 1024);
    if (lane < 16) dma16(src + kCodeBytes + lane * 16, dst + kCodeBytes);
  };
  for (int p = p0; p < p0 + kRing && p < p1; ++p) issue(p);
  for (int p = p0; p < p1; ++p) {
    // this page's nine copies; the next page's may stay in flight
    if (p + 1 < p1) wait_vm<9>(); else wait_vm<0>();
    sum ^= *reinterpret_cast<const uint32_t*>(&ring[wave][(p - p0) % kRing][lane * 16]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (p + kRing < p1) issue(p + kRing);
  }
  out[gw * 64 + lane] = sum;
}

}  // namespace

// cache: device pointer to the page pool; page_stride: bytes between pages
// (at least 8,448); ids: device array of `total` page ids, each in
// [0, pool pages); out: device array of grid * 512 uint32 (checksums);
// grid: workgroups (the indexer's grid, at most one per CU).  Returns the
// launch's hipError_t as an int (0 on success); the caller synchronises.
extern "C" int dsa_probe_page_read(const void* cache, int64_t page_stride, const int* ids, int total, void* out,
                                   int grid, hipStream_t stream) {
  if (!cache || !ids || !out || total < 0 || grid < 1 || page_stride < kPageBytes) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(page_read_kernel, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream,
                     static_cast<const uint8_t*>(cache), page_stride, ids, total, static_cast<uint32_t*>(out));
  return (int)hipGetLastError();
}
