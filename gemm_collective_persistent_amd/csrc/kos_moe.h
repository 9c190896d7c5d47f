// Shared pieces of the expert-layer kernels (dispatch and combine).
#pragma once

#include "kos_device.h"

namespace kos {

constexpr int kMoeTokBlock = 64;    // tokens per router entry (one bit each in a 64-bit mask)
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxLocal = 64;
constexpr int kMoeMaxTopk = 16;

// Copies one row of `bytes` (multiple of 16) with one wave, up to 16 loads
// per lane in flight.
__device__ __forceinline__ void wave_copy_row(void* __restrict__ dst, const void* __restrict__ src, int bytes) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int lane = threadIdx.x & 63;
  const int n = bytes >> 4;
  constexpr int U = 16;
  for (int b = lane; b < n; b += U * 64) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u * 64 < n) v[u] = __builtin_nontemporal_load(&s[b + u * 64]);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u * 64 < n) d[b + u * 64] = v[u];
  }
}

// Same, storing with device-scope stores (rows read later in the same
// launch by other workgroups): dst is wave-uniform, below 2 GiB of rows.
__device__ __forceinline__ void wave_copy_row_dev_dst(void* __restrict__ dst, const void* __restrict__ src, int bytes) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  const DevBuf d(dst);
  const int lane = threadIdx.x & 63;
  const int n = bytes >> 4;
  constexpr int U = 16;
  for (int b = lane; b < n; b += U * 64) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u * 64 < n) v[u] = __builtin_nontemporal_load(&s[b + u * 64]);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u * 64 < n) d.st128((uint32_t)(b + u * 64) * 16u, v[u]);
  }
}

// Same, reading the source with device-scope loads (rows written by other
// workgroups of the same launch): src_off is the row's byte offset in `src`
// (wave-uniform; offsets below 2 GiB).  Up to 16 loads per lane in flight.
__device__ __forceinline__ void wave_copy_row_dev_src(void* __restrict__ dst, const DevBuf& src, uint32_t src_off,
                                                      int bytes) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int lane = threadIdx.x & 63;
  const int n = bytes >> 4;
  constexpr int U = 16;
  for (int b = lane; b < n; b += U * 64) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u * 64 < n) v[u] = src.ld128(src_off + (uint32_t)(b + u * 64) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u * 64 < n) d[b + u * 64] = v[u];
  }
}

// Exclusive prefix sums of in[0, n) into out[0, n], out[n] = total; n <=
// 4 * blockDim.x; wave_tot holds one int per wave.  All threads call it; it
// synchronizes the workgroup before and after writing out.
__device__ inline void block_exclusive_scan(const int32_t* in, int32_t* out, int n, int32_t* wave_tot) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
  int v[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = 4 * t + i < n ? in[4 * t + i] : 0;
    sum += v[i];
  }
  int inc = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int ex = inc - sum;
  for (int w = 0; w < wave; ++w) ex += wave_tot[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * t + i < n) out[4 * t + i] = ex;
    ex += v[i];
  }
  if (t == 0) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += wave_tot[w];
    out[n] = tot;
  }
  __syncthreads();
}

}  // namespace kos
