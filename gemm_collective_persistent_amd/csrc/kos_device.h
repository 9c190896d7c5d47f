// Device runtime of the persistent self-scheduling kernels (gfx950).
//
// One workgroup (4 or 8 wave64s) per compute unit.  Workgroups
// take entries from atomic queue heads ("ticket rail"), publish finished
// pieces through ready counters, and wait on them with a bounded poll
// [KOSMOS explainer, "KOSMOS removes the manager" and "Role switching only
// works if ..." paragraphs].
//
// Memory ordering: the MI355X's eight XCDs each have their own L2, which is
// not coherent with the others for ordinary accesses.  Data that another
// workgroup of the same launch reads is stored with device-scope (sc1)
// stores; the producer waits for its stores to complete (vmcnt(0)) in every
// thread, then one thread bumps the ready counter (wg_publish); the consumer
// polls the counter and reads the data with device-scope (sc1) loads
// (wg_observe).  No kernel uses agent-scope fences: on this part a release
// fence writes back the whole L2 of the XCD it runs on and an acquire fence
// invalidates it, which stalls every workgroup on that XCD.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kos_common.h"

namespace kos {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// atomics (agent scope = the whole GPU)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Records the first device-side error and tells every workgroup to drain.
__device__ inline void raise_error(WsHeader* h, uint32_t code, uint32_t info) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(&h->status, &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_relaxed(&h->err_info, info);
  }
  st_relaxed(&h->abort, 1u);
}

__device__ __forceinline__ bool aborted(WsHeader* h) { return ld_relaxed(&h->abort) != 0; }

// Per-workgroup LDS slots used by the helpers below.
struct WgSlots {
  uint32_t claim;
  int32_t ok;
  uint32_t aux[6];
};

constexpr uint32_t kNoEntry = 0xFFFFFFFFu;

// Thread 0 takes the next entry of a queue; every thread gets it.  Returns
// kNoEntry once an error has been recorded, so that the decision to stop is
// the same in every wave.
__device__ __forceinline__ uint32_t wg_claim(uint32_t* head, WsHeader* h, WgSlots* s) {
  __syncthreads();
  if (threadIdx.x == 0) s->claim = aborted(h) ? kNoEntry : add_relaxed(head, 1u);
  __syncthreads();
  return s->claim;
}

// Coherent exchange, producer side: this workgroup's device-scope stores
// have completed (every thread waits), then `v` is added to the counter.
__device__ __forceinline__ void wg_publish(uint32_t* counter, uint32_t v) {
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) add_relaxed(counter, v);
}

// Coherent exchange, consumer side: waits until *counter >= target, then the
// caller reads the data with device-scope loads.  Bounded: after `limit`
// polls it records KOS_ERR_TIMEOUT (with `info`) and returns false; it also
// returns false as soon as another workgroup has recorded an error.
__device__ inline bool wg_observe(const uint32_t* counter, uint32_t target, WsHeader* h, uint32_t limit,
                                  uint32_t info, WgSlots* s) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    uint32_t it = 0;
    while (ld_relaxed(counter) < target) {
      if (aborted(h)) { ok = 0; break; }
      if (++it >= limit) { raise_error(h, KOS_ERR_TIMEOUT, info); ok = 0; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    s->ok = ok;
  }
  __syncthreads();
  return s->ok != 0;
}

// Device-scope (sc1) stores and loads for the coherent exchange.  All are
// compiler-visible (atomics or buffer builtins), so the compiler accounts
// for their waits and for the register hazards of wide stores.
__device__ __forceinline__ void st_dev_b32(void* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-scope (sc1) loads of data written by other workgroups of the same
// launch (compiler-visible atomics; no cache invalidation needed).
__device__ __forceinline__ uint32_t ld_dev_b32(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_b64(const void* p) {   // p 8-byte aligned
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A pointer that is the same in every lane of the wave, moved to scalar
// registers (the caller guarantees the uniformity).
template <class T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Lane j's value of a 64-bit quantity, as a scalar.  The readlane builtin
// returns a signed int: each half goes through uint32_t before it is
// widened, or a low word with bit 31 set would be sign-extended into the
// high word.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int j) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)v, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(v >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int kCpolSc1 = 16;                 // cache-policy operand: sc1 (device scope)
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw buffer descriptor word 3 (32-bit data format)

// 16-byte device-scope accesses at byte offsets (below 2 GiB) from a
// wave-uniform base, through a raw buffer descriptor.
struct DevBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ DevBuf() : r(__builtin_amdgcn_make_buffer_rsrc(nullptr, (short)0, 0, kRawBufferWord3)) {}
  __device__ __forceinline__ explicit DevBuf(const void* base)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wave_uniform(base)), (short)0, 0x7fffffff,
                                            kRawBufferWord3)) {}
  __device__ __forceinline__ void st128(uint32_t off, u32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolSc1);
  }
  __device__ __forceinline__ u32x4 ld128(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
  }
  __device__ __forceinline__ void st16(uint32_t off, uint16_t v) const {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kCpolSc1);
  }
};

// Role assignment ticket: arrival order of the workgroups.
__device__ __forceinline__ uint32_t wg_ticket(WsHeader* h, WgSlots* s) {
  __syncthreads();
  if (threadIdx.x == 0) s->claim = add_relaxed(&h->ticket, 1u);
  __syncthreads();
  return s->claim;
}

// Departure: the last workgroup out returns the workspace to all-zero (queue
// heads, tickets, the first `n_counters` ready counters), keeping only the
// sticky error word, so the next call needs no clearing launch.  Those words
// are only touched by device-scope atomics and device-coherent stores, which
// complete at the device's coherence point: waiting for this workgroup's own
// memory operations before it counts itself out orders them before the
// reset, with no fence.  (An agent-scope fence writes back and invalidates
// the XCD's whole L2, stalling every workgroup still running there; the
// launch's outputs become visible to later work when it ends.)
//
// hand_over: the call keeps no sticky error word (the library's own scratch,
// shared by every call on the device); the last one out hands the status to
// `status_out` (if non-null) and clears it.  Every workgroup's error, if any,
// was recorded before it counted itself out, so the last one sees them all.
__device__ inline void wg_exit(WsHeader* h, uint32_t* counters, uint32_t n_counters, WgSlots* s,
                               bool hand_over = false, int32_t* status_out = nullptr) {
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt, expcnt, lgkmcnt = 0
  __syncthreads();
  if (threadIdx.x == 0)
    s->claim = __hip_atomic_fetch_add(&h->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s->claim != gridDim.x - 1) return;
  for (uint32_t i = threadIdx.x; i < n_counters; i += blockDim.x) st_relaxed(&counters[i], 0u);
  if (threadIdx.x < kNumHeads) st_relaxed(&h->head[threadIdx.x], 0u);
  if (threadIdx.x == 0) {
    if (hand_over) {
      const uint32_t st = ld_relaxed(&h->status);
      if (status_out)
        __hip_atomic_store(status_out, (int32_t)st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      st_relaxed(&h->status, 0u);
      st_relaxed(&h->err_info, 0u);
    }
    st_relaxed(&h->ticket, 0u);
    st_relaxed(&h->abort, 0u);
    st_relaxed(&h->exit_count, 0u);
  }
}

// ---------------------------------------------------------------------------
// optional timeline (kos_opts.trace): one row of KOS_TRACE_RECORDS records
// per workgroup, written by thread 0
// ---------------------------------------------------------------------------

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ uint32_t xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u; }

struct Tracer {
  kos_trace_rec* row;   // this workgroup's row; null when tracing is off
  uint32_t n;           // records used, header and clock record included
  uint64_t t_begin;     // constant-rate counter at the start
  uint64_t c_begin;     // shader-clock counter at the start

  __device__ __forceinline__ explicit Tracer(kos_trace_rec* base)
      : row(base ? base + (size_t)blockIdx.x * KOS_TRACE_RECORDS : nullptr), n(2), t_begin(now()),
        c_begin(row ? __builtin_amdgcn_s_memtime() : 0) {}
  __device__ __forceinline__ bool on() const { return row != nullptr; }
  // The constant-rate counter when tracing, else 0.
  __device__ __forceinline__ uint64_t now() const { return row ? __builtin_amdgcn_s_memrealtime() : 0; }
  // One piece of work of `kind` on `entry`, begun at t0 (from now()).
  __device__ __forceinline__ void put(uint32_t kind, uint32_t entry, uint64_t t0) {
    if (!row) return;
    if (threadIdx.x == 0 && n < KOS_TRACE_RECORDS) {
      kos_trace_rec r;
      r.t0 = t0;
      r.dt = (uint32_t)(__builtin_amdgcn_s_memrealtime() - t0);
      r.tag = (kind << 24) | (entry & 0xFFFFFFu);
      row[n] = r;
    }
    ++n;
  }
  // Same, for a piece of work the whole workgroup shares whose waves may end
  // at different times: the record ends when the last wave is done (a
  // barrier, taken only when tracing).
  __device__ __forceinline__ void put_wg(uint32_t kind, uint32_t entry, uint64_t t0) {
    if (!row) return;
    __syncthreads();
    put(kind, entry, t0);
  }
  // The header (start, lifetime, arrival ticket, the accelerator complex die
  // (XCD) the workgroup runs on, the record count) and the clock record
  // (shader-clock cycles over the same lifetime).
  __device__ __forceinline__ void finish(uint32_t ticket) {
    if (!row || threadIdx.x != 0) return;
    const uint64_t cycles = __builtin_amdgcn_s_memtime() - c_begin;
    kos_trace_rec r;
    r.t0 = t_begin;
    r.dt = (uint32_t)(__builtin_amdgcn_s_memrealtime() - t_begin);
    r.tag = (ticket << 16) | (xcd_id() << 12) | (n < KOS_TRACE_RECORDS ? n : KOS_TRACE_RECORDS);
    row[0] = r;
    kos_trace_rec c;
    c.t0 = cycles;
    c.dt = r.dt;
    c.tag = (uint32_t)KOS_TR_CLOCK << 24;
    row[1] = c;
  }
};

// ---------------------------------------------------------------------------
// movers: coalesced 128-bit copies
// ---------------------------------------------------------------------------

// Copies `bytes` (a multiple of 16, below 2 GiB) from src to dst with the
// whole workgroup, stores device-coherent (see wg_publish); consecutive
// threads touch consecutive 16-byte chunks and each thread keeps 8 loads in
// flight.  dst and src are the same in every thread.
__device__ inline void wg_copy_dev(void* __restrict__ dst, const void* __restrict__ src, size_t bytes) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  const DevBuf d(dst);
  const uint32_t n = (uint32_t)(bytes >> 4);
  const uint32_t nt = blockDim.x;
  uint32_t i = threadIdx.x;
  constexpr int U = 8;
  for (; i + (U - 1) * nt < n; i += U * nt) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&s[i + u * nt]);
#pragma unroll
    for (int u = 0; u < U; ++u) d.st128((i + u * nt) * 16u, v[u]);
  }
  for (; i < n; i += nt) d.st128(i * 16u, __builtin_nontemporal_load(&s[i]));
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);   // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, b);
}
// Four floats to four packed bf16 (round to nearest even), lowest first.
__device__ __forceinline__ u32x2 pack4_bf16(f32x4 v) {
  u32x2 r;
  r.x = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
  r.y = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
  return r;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

}  // namespace kos
