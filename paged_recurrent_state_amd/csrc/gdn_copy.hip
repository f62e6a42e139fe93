// Streaming device copy: the reference rate of an HBM-bound kernel on this
// GPU, moving bytes the way the decode kernel moves state rows (16-byte
// non-temporal loads and stores, a fixed grid that walks the buffer, the
// next unit's loads issued before the current unit's stores).  It computes
// nothing of the method; the benchmark prints its rate beside the decode's.
#include <algorithm>

#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyVec = 8;                                // 16-byte vectors a thread moves per unit
constexpr int64_t kCopyUnit = kCopyThreads * kCopyVec;     // 16-byte vectors per unit (32 KiB)

__device__ __forceinline__ void unit_load(const u32x4* __restrict__ src, int64_t n16, int64_t u,
                                          u32x4 (&v)[kCopyVec]) {
  const int64_t base = u * kCopyUnit + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kCopyVec; ++i) {
    const int64_t e = base + (int64_t)kCopyThreads * i;
    if (e < n16) v[i] = __builtin_nontemporal_load(src + e);
  }
}

__device__ __forceinline__ void unit_store(u32x4* __restrict__ dst, int64_t n16, int64_t u,
                                           const u32x4 (&v)[kCopyVec]) {
  const int64_t base = u * kCopyUnit + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kCopyVec; ++i) {
    const int64_t e = base + (int64_t)kCopyThreads * i;
    if (e < n16) __builtin_nontemporal_store(v[i], dst + e);
  }
}

// Workgroup b copies units b, b + grid, b + 2 grid, ...: every wave leaves
// the loop once its unit index passes the last unit.
__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t n16, int64_t units) {
  int64_t u = blockIdx.x;
  if (u >= units) return;
  u32x4 cur[kCopyVec], nxt[kCopyVec];
  unit_load(src, n16, u, cur);
  for (; u < units; u += gridDim.x) {
    const int64_t un = u + gridDim.x;
    if (un < units) unit_load(src, n16, un, nxt);
    unit_store(dst, n16, u, cur);
#pragma unroll
    for (int i = 0; i < kCopyVec; ++i) cur[i] = nxt[i];
  }
}

}  // namespace

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t units = (n16 + kCopyUnit - 1) / kCopyUnit;
  if (units == 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(units, (int64_t)device_cus() * 8);
  stream_copy_kernel<<<(unsigned)grid, kCopyThreads, 0, s>>>((const u32x4*)src, (u32x4*)dst, n16, units);
  return hipGetLastError();
}

}  // namespace gdn
