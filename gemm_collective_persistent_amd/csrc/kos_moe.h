// Shared pieces of the expert-layer kernels (dispatch and combine).
#pragma once

#include "kos_device.h"

namespace kos {

constexpr int kMoeTokBlock = 64;    // tokens per router entry (one bit each in a 64-bit mask)
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxLocal = 64;
constexpr int kMoeMaxTopk = 16;

// Copies one row of `bytes` (multiple of 16) with one wave.
__device__ __forceinline__ void wave_copy_row(void* __restrict__ dst, const void* __restrict__ src, int bytes) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int lane = threadIdx.x & 63;
  const int n = bytes >> 4;
  int i = lane;
  for (; i + 3 * 64 < n; i += 4 * 64) {
    u32x4 v0 = s[i], v1 = s[i + 64], v2 = s[i + 128], v3 = s[i + 192];
    d[i] = v0;
    d[i + 64] = v1;
    d[i + 128] = v2;
    d[i + 192] = v3;
  }
  for (; i < n; i += 64) d[i] = s[i];
}

// Same, reading the source with device-scope loads (rows written by other
// workgroups of the same launch): src_off is the row's byte offset in `src`
// (wave-uniform; offsets below 2 GiB).
__device__ __forceinline__ void wave_copy_row_dev_src(void* __restrict__ dst, const DevBuf& src, uint32_t src_off,
                                                      int bytes) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int lane = threadIdx.x & 63;
  const int n = bytes >> 4;
  int i = lane;
  for (; i + 3 * 64 < n; i += 4 * 64) {
    const u32x4 v0 = src.ld128(src_off + i * 16u), v1 = src.ld128(src_off + (i + 64) * 16u);
    const u32x4 v2 = src.ld128(src_off + (i + 128) * 16u), v3 = src.ld128(src_off + (i + 192) * 16u);
    d[i] = v0;
    d[i + 64] = v1;
    d[i + 128] = v2;
    d[i + 192] = v3;
  }
  for (; i < n; i += 64) d[i] = src.ld128(src_off + i * 16u);
}

}  // namespace kos
