// The builders' MXFP8 tile (gfx950): C[BM x BN] = A[BM x K] . W[BN x K]^T,
// both operands FP8 E4M3 with one E8M0 scale per 32 consecutive k (OCP
// Microscaling v1.0), fp32 accumulate, on v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Same machinery as the bf16 tile (kos_tile.h): a workgroup of WGM x WGN
// wave64s, accumulators in registers for the whole K loop, operands loaded
// straight into a four-stage LDS ring (buffer_load ... lds), each stage one
// 64-k step of the scaled MFMA.  The weight is stored N x K, so both operands
// are rows of 64 bytes per stage and share one LDS layout.
//
// Scaled MFMA operand layout (32x32x64, E4M3; checked on the hardware with
// random codes and scales): lane l, h = l/32, holds 32 bytes of row l%32 of
// its operand.  Bytes 0-15 belong to the first 32-k scale block of the step
// and bytes 16-31 to the second; the order of k inside a block is free as
// long as both operands use the same one.  The 32-bit scale operand of lane
// l (byte 0 selected) is the scale of row l%32, block h, and applies to that
// block's bytes in every lane.  Here lane h takes k [16h, 16h+16) and
// [32+16h, 32+16h+16): 16-byte chunks h and 2+h of the row.
//
// LDS layout per stage:
//   A:  BM rows x 4 chunks of 16 bytes, chunk c of row m at position
//       c ^ ((m >> 2) & 3) (the bf16 A layout: a row is 64 bytes either way).
//   B:  BN rows (output columns) x 4 chunks, the same layout.
//   SA: BM x 4 bytes, SB: BN x 4 bytes: each row's two scales of the step
//       in bytes 0 and 1 of its word (a direct LDS load of 2 bytes per lane
//       fills one 4-byte word per lane, upper half zero; checked on the
//       hardware).
//
// Scale layout in memory (the MX operands' contract): K/64 slabs, slab s
// holding, for every row r of the operand, the scales of blocks 2s and 2s+1
// (bytes 2r and 2r+1 of the slab).  A stage's scales for 64 rows are then
// one 128-byte line, where row-major scales (row stride K/32 bytes) would
// cost one cache line per row.
//
// Accumulator layout: the B fragment is the first MFMA operand, as in the
// bf16 tile, so tile_foreach4 visits the results unchanged.
//
// Pipeline: one workgroup barrier per stage; each A fragment of the next
// step is read right after its row block's last MFMA of this step (in
// place), the B fragments into a second set, so LDS reads overlap the
// matrix cores instead of waiting in front of them.
#pragma once

#include "kos_tile.h"

namespace kos {

template <int BM_, int BN_, int WGM_ = 2, int WGN_ = 4>
struct TileShapeMX {
  static constexpr bool MX = true;
  static constexpr int BM = BM_, BN = BN_, BK = 64, STAGES = 4;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN;
  static constexpr int NT = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;          // one byte per element
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SB_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE_BYTES = SB_OFF + BN * 4;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NW;                // 1 KiB loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / NW;
  // scales: 64-row groups, 2 bytes per lane, SC_LOADS groups per wave
  static constexpr int SC_GROUPS = (BM + BN) / 64;
  static constexpr int SC_LOADS = SC_GROUPS / NW;
  static constexpr int LOADS = A_LOADS + B_LOADS + SC_LOADS;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
  static_assert(A_LOADS >= 1 && A_BYTES == A_LOADS * 1024 * NW, "whole A loads per wave");
  static_assert(B_LOADS >= 1 && B_BYTES == B_LOADS * 1024 * NW, "whole B loads per wave");
  static_assert(SC_LOADS >= 1 && SC_GROUPS == SC_LOADS * NW, "whole scale loads per wave");
  static_assert((BM / 64) % SC_LOADS == 0, "a wave's scale groups lie on one operand");
  static_assert(TM >= 1 && TN >= 1, "at least one 32x32 block per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(3 * LOADS <= 63, "vmcnt range");
};

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// One MX operand from the tile's first row: rows of K E4M3 codes (row
// stride ld bytes), and that row's two scales in slab 0 (slab stride
// slab bytes = 2 x the operand's row count).
struct MxSrc {
  const uint8_t* p;
  const uint8_t* s;
  int64_t ld, slab;
};

// This wave's direct loads for a tile: descriptors and per-lane byte offsets
// (rows clamped to the valid ones: rows past them feed only results that are
// never stored); a stage adds k0 (data) or its aligned scale-word offset.
template <class S, bool COH_A>
struct MxPlan {
  __amdgpu_buffer_rsrc_t ra, rb, rsc;
  uint32_t a_off[S::A_LOADS];
  uint32_t b_off[S::B_LOADS];
  uint32_t sc_off[S::SC_LOADS];
  int a_lds, b_lds, sc_lds;   // this wave's bytes into a stage (uniform)
  int sc_slab;                // slab stride of the wave's scale operand (uniform)
};

template <class S, bool COH_A>
__device__ __forceinline__ void mx_plan(MxPlan<S, COH_A>& P, const MxSrc& a, int m_valid, const MxSrc& b, int n_valid,
                                        const WaveCtx& w) {
  const int lane = w.lane, wave = w.wave;
  P.a_lds = wave * S::A_LOADS * 1024;
  P.b_lds = S::A_BYTES + wave * S::B_LOADS * 1024;
  P.ra = raw_rsrc(a.p);
  P.rb = raw_rsrc(b.p);
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i) {
    const int slot = (wave * S::A_LOADS + i) * 64 + lane;   // 16-byte slot in the A stage
    const int m = slot >> 2, c = (slot & 3) ^ a_swz(slot >> 2);
    const int mr = m < m_valid ? m : m_valid - 1;
    P.a_off[i] = (uint32_t)(mr * a.ld + c * 16);
  }
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i) {
    const int slot = (wave * S::B_LOADS + i) * 64 + lane;
    const int n = slot >> 2, c = (slot & 3) ^ a_swz(slot >> 2);
    const int nr = n < n_valid ? n : n_valid - 1;
    P.b_off[i] = (uint32_t)(nr * b.ld + c * 16);
  }
  // Scales: 64-row groups of the stage's slab, A rows first; a wave's
  // groups all lie on one operand.  Rows past the valid ones re-read the
  // last valid row.
  const int g0 = wave * S::SC_LOADS;
  const bool on_a = g0 < S::BM / 64;
  const int gl = on_a ? g0 : g0 - S::BM / 64;
  const int valid = on_a ? m_valid : n_valid;
  P.rsc = raw_rsrc(on_a ? a.s : b.s);
  P.sc_lds = (on_a ? S::SA_OFF : S::SB_OFF) + gl * 256;
  P.sc_slab = (int)(on_a ? a.slab : b.slab);
#pragma unroll
  for (int i = 0; i < S::SC_LOADS; ++i) {
    const int r = (gl + i) * 64 + lane;
    P.sc_off[i] = (uint32_t)((r < valid ? r : valid - 1) * 2);
  }
}

// Issues this wave's loads of the stage at k0 (a multiple of 64).
template <class S, bool COH_A>
__device__ __forceinline__ void mx_stage_load(char* lds_stage, const MxPlan<S, COH_A>& P, int k0) {
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(P.ra, (lds_void*)(lds_stage + P.a_lds + i * 1024), 16, P.a_off[i], k0, 0,
                                             COH_A ? kCpolDevice : 0);
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(P.rb, (lds_void*)(lds_stage + P.b_lds + i * 1024), 16, P.b_off[i], k0, 0,
                                             0);
  // the scales of A rows written by this launch follow the A policy
#pragma unroll
  for (int i = 0; i < S::SC_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(P.rsc, (lds_void*)(lds_stage + P.sc_lds + i * 256), 2, P.sc_off[i],
                                             (k0 >> 6) * P.sc_slab, 0, COH_A ? kCpolDevice : 0);
}

// Operand fragments: the A row blocks (reloaded in place, each right after
// its last MFMA of the step) and the B column blocks (two sets, current and
// next step).  Scale words are kept as read (two bytes per row word) and
// shifted to this lane's byte at the MFMA: a shift right after the read would
// wait for it there.
template <class S>
struct MxA {
  i32x8 a[S::TM];
  int32_t sa[S::TM];
};
template <class S>
struct MxB {
  i32x8 b[S::TN];
  int32_t sb[S::TN];
};

// This lane's LDS offsets within a stage.  Row m = (32-row block base) + r
// has swizzle (m >> 2) & 3 = that of r (block bases are multiples of 32), so
// every block's chunks sit at one lane offset plus a constant.
struct MxAddr {
  int lo, hi;        // chunk h and chunk 2+h of row r: (2+h) ^ s = (h ^ s) ^ 2
  int sh;            // this lane's byte (block h) of a scale word
  int a, b, sa, sb;  // A, B and scale rows of this wave's sub-tile (+ lane row)
};

template <class S>
__device__ __forceinline__ MxAddr mx_addr(const WaveCtx& w) {
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int h = lane >> 5, r = lane & 31;
  MxAddr d;
  d.lo = r * 64 + ((h ^ a_swz(r)) << 4);
  d.hi = d.lo ^ 32;
  d.sh = 8 * h;
  d.a = wm * S::WM * 64;
  d.b = S::A_BYTES + wn * S::WN * 64;
  d.sa = S::SA_OFF + wm * S::WM * 4 + r * 4;
  d.sb = S::SB_OFF + wn * S::WN * 4 + r * 4;
  return d;
}

template <class S, int I>
__device__ __forceinline__ void mx_load_a(MxA<S>& f, const char* stage, const MxAddr& d) {
  const char* p = stage + d.a + I * 2048;
  const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + d.lo);
  const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + d.hi);
  f.a[I] = __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  f.sa[I] = (int32_t)*reinterpret_cast<const uint32_t*>(stage + d.sa + I * 128);
}

template <class S>
__device__ __forceinline__ void mx_load_b(MxB<S>& f, const char* stage, const MxAddr& d) {
#pragma unroll
  for (int j = 0; j < S::TN; ++j) {
    const char* p = stage + d.b + j * 2048;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + d.lo);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + d.hi);
    f.b[j] = __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    f.sb[j] = (int32_t)*reinterpret_cast<const uint32_t*>(stage + d.sb + j * 128);
  }
}

// The MFMAs of row block I (formats 0, 0: E4M3 x E4M3; byte 0 of each
// scale operand after the shift).
template <class S, int I>
__device__ __forceinline__ void mx_mfma_row(f32x16 (&acc)[S::TM][S::TN], const MxA<S>& fa, const MxB<S>& fb,
                                            const MxAddr& d) {
  const int32_t sa = (int32_t)((uint32_t)fa.sa[I] >> d.sh);
#pragma unroll
  for (int j = 0; j < S::TN; ++j)
    acc[I][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb.b[j], fa.a[I], acc[I][j], 0, 0, 0,
                                                                (int32_t)((uint32_t)fb.sb[j] >> d.sh), 0, sa);
}

// Row blocks I.. of the step: each block's MFMAs, then its A fragment of the
// next step (scheduling barriers keep that order).
template <class S, int I>
__device__ __forceinline__ void mx_rows_from(f32x16 (&acc)[S::TM][S::TN], MxA<S>& fa, const MxB<S>& fb,
                                             const char* nxt, const MxAddr& d) {
  if constexpr (I < S::TM) {
    mx_mfma_row<S, I>(acc, fa, fb, d);
    __builtin_amdgcn_sched_barrier(0);
    mx_load_a<S, I>(fa, nxt, d);
    __builtin_amdgcn_sched_barrier(0);
    mx_rows_from<S, I + 1>(acc, fa, fb, nxt, d);
  }
}

// One K-loop iteration on stage kt (ring buffer `cur`, stage kt+1 in `nxt`).
// On entry fa + fb hold stage kt's fragments; on exit fa + fn hold stage
// kt+1's.  Row block 0's MFMAs run first; then the wait for stage kt+1 and
// the workgroup barrier (every wave has read stage kt: `cur` takes stage
// kt+4), the look-ahead load, stage kt+1's block-0 A and B fragments, and
// the remaining row blocks, each followed by its next A fragment.  The
// look-ahead load is always issued (past the end it re-reads the last
// stage, never used) so the counts in flight stay uniform and the loop has
// no branches.
template <class S, bool COH_A>
__device__ __forceinline__ void mx_k_iter(f32x16 (&acc)[S::TM][S::TN], MxA<S>& fa, const MxB<S>& fb, MxB<S>& fn,
                                          int kt, int nk, const MxPlan<S, COH_A>& P, char* cur, char* nxt,
                                          const MxAddr& d) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int ST = S::STAGES;
  mx_mfma_row<S, 0>(acc, fa, fb, d);
  __builtin_amdgcn_sched_barrier(0);
  KOS_WAITCNT(2 * S::LOADS, 0);   // stage kt+1 landed (kt+2, kt+3 may fly); reads of stage kt done
  lds_barrier();
  mx_stage_load<S, COH_A>(cur, P, (kt + ST < nk ? kt + ST : nk - 1) * S::BK);
  mx_load_a<S, 0>(fa, nxt, d);
  mx_load_b<S>(fn, nxt, d);
  __builtin_amdgcn_sched_barrier(0);
  mx_rows_from<S, 1>(acc, fa, fb, nxt, d);
#endif
}

// Full K loop: acc = A[0:m_valid) . B[0:n_valid)^T over k in [0, K), K a
// positive multiple of 256 (whole trips of four stages).  Begins and ends
// with the LDS ring free.  COH_A: device-coherent loads of A and its scales
// (rows written by other workgroups of this launch).
template <class S, bool COH_A = false, int RING = S::STAGE_BYTES>
__device__ __forceinline__ void tile_mainloop_mx(f32x16 (&acc)[S::TM][S::TN], const MxSrc& a, int m_valid,
                                                 const MxSrc& b, int n_valid, int K) {
  constexpr int ST = S::STAGES;
  static_assert(S::TM <= 4, "row blocks unrolled below");
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = K / S::BK;
  const WaveCtx w = wave_ctx();
  MxPlan<S, COH_A> P;
  mx_plan<S, COH_A>(P, a, m_valid, b, n_valid, w);
  const MxAddr d = mx_addr<S>(w);
  static_assert(S::STAGE_BYTES <= RING, "tile stage larger than the ring");
  char* r0 = ring<RING, 0>();
  char* r1 = ring<RING, 1>();
  char* r2 = ring<RING, 2>();
  char* r3 = ring<RING, 3>();
  KOS_WAITCNT(0, 0);
  lds_barrier();   // the ring is free (previous user done)
  mx_stage_load<S, COH_A>(r0, P, 0);
  mx_stage_load<S, COH_A>(r1, P, 1 * S::BK);
  mx_stage_load<S, COH_A>(r2, P, 2 * S::BK);
  mx_stage_load<S, COH_A>(r3, P, 3 * S::BK);
  KOS_WAITCNT(3 * S::LOADS, 0);
  lds_barrier();
  MxA<S> fa;
  MxB<S> f0, f1;
  mx_load_a<S, 0>(fa, r0, d);
  if constexpr (S::TM > 1) mx_load_a<S, 1>(fa, r0, d);
  if constexpr (S::TM > 2) mx_load_a<S, 2>(fa, r0, d);
  if constexpr (S::TM > 3) mx_load_a<S, 3>(fa, r0, d);
  mx_load_b<S>(f0, r0, d);
  // four stages per trip: the ring buffers come back to where they started,
  // and the two B sets alternate
  for (int kt = 0; kt < nk; kt += ST) {
    mx_k_iter<S, COH_A>(acc, fa, f0, f1, kt + 0, nk, P, r0, r1, d);
    mx_k_iter<S, COH_A>(acc, fa, f1, f0, kt + 1, nk, P, r1, r2, d);
    mx_k_iter<S, COH_A>(acc, fa, f0, f1, kt + 2, nk, P, r2, r3, d);
    mx_k_iter<S, COH_A>(acc, fa, f1, f0, kt + 3, nk, P, r3, r0, d);
  }
  KOS_WAITCNT(0, 0);
  lds_barrier();
}

}  // namespace kos
