// The builders' MXFP8 tile (gfx950): C[BM x BN] = A[BM x K] . W[BN x K]^T,
// both operands FP8 E4M3 with one E8M0 scale per 32 consecutive k (OCP
// Microscaling v1.0), fp32 accumulate, on v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Same machinery as the bf16 tile (kos_tile.h): a workgroup of WGM x WGN
// wave64s, accumulators in registers for the whole K loop, operands loaded
// straight into LDS (buffer_load ... lds).  One step of the scaled MFMA
// covers 64 k; the LDS holds two buffers of two steps each ("pairs", 128 k):
// a pair's row of either operand is one whole 128-byte line of memory, so
// every direct load covers whole lines (one step per buffer would fetch
// half lines: 10-15 % slower).  The weight is stored N x K, so both
// operands are rows and share one LDS layout.
//
// Scaled MFMA operand layout (32x32x64, E4M3; checked on the hardware with
// random codes and scales): lane l, h = l/32, holds 32 bytes of row l%32 of
// its operand.  Bytes 0-15 belong to the first 32-k scale block of the step
// and bytes 16-31 to the second; the order of k inside a block is free as
// long as both operands use the same one.  The 32-bit scale operand of lane
// l (byte 0 selected) is the scale of row l%32, block h, and applies to that
// block's bytes in every lane.  Here lane h takes k [16h, 16h+16) and
// [32+16h, 32+16h+16) of the step: 16-byte chunks h and 2+h of the step's
// 64 bytes.
//
// LDS layout per pair buffer:
//   A:  BM rows x 8 chunks of 16 bytes (step 0: chunks 0-3, step 1: 4-7),
//       chunk c of row r at position c ^ ((r >> 1) & 7): the rows read by
//       eight consecutive lanes land on distinct banks.
//   B:  BN rows (output columns) x 8 chunks, the same layout.
//   SA: [2][BM] x 4 bytes, SB: [2][BN] x 4 bytes: per step, each row's two
//       scales in bytes 0 and 1 of its word (a direct LDS load of 2 bytes per
//       lane fills one 4-byte word per lane, upper half zero; checked on the
//       hardware).  Tiles whose 64-row scale groups do not divide among the
//       waves (256 x 192 on eight waves: seven groups) end with a padding
//       slot that the spare waves' loads fill and nothing reads.
//
// Scale layout in memory (the MX operands' contract): K/64 slabs, slab s
// holding, for every row r of the operand, the scales of blocks 2s and 2s+1
// (bytes 2r and 2r+1 of the slab).  A step's scales for 64 rows are then
// one 128-byte line, where row-major scales (row stride K/32 bytes) would
// cost one cache line per row.
//
// Accumulator layout: the B fragment is the first MFMA operand, as in the
// bf16 tile, so tile_foreach4 visits the results unchanged.
//
// Pipeline: one workgroup barrier per pair.  Each A fragment of the next
// step is read right after its row block's MFMAs of this step (in place),
// the B fragments into a second set, so LDS reads overlap the matrix cores
// instead of waiting in front of them; the next pair loads while the
// current one is consumed.
#pragma once

#include "kos_tile.h"

namespace kos {

template <int BM_, int BN_, int WGM_ = 2, int WGN_ = 4>
struct TileShapeMX {
  static constexpr bool MX = true;
  static constexpr int BM = BM_, BN = BN_, BK = 64, PAIR_K = 128;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN;
  static constexpr int NT = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = BM * PAIR_K, B_BYTES = BN * PAIR_K;   // one byte per element
  // scales: 64-row groups, 2 bytes per lane, SC_LOADS groups per wave and
  // step; when the groups do not divide among the waves, the waves left over
  // (SC_PAD of them) load A's first group into a slot nobody reads, so that
  // every wave issues the same number of loads (the waits count them)
  static constexpr int SC_GROUPS = (BM + BN) / 64;
  static constexpr int SC_LOADS = (SC_GROUPS + NW - 1) / NW;
  static constexpr int SC_PAD = SC_LOADS * NW - SC_GROUPS;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;                     // [2][BM] words
  static constexpr int SB_OFF = SA_OFF + 2 * BM * 4;                   // [2][BN] words
  static constexpr int PAD_OFF = SB_OFF + 2 * BN * 4;                  // [2][64] words, padding loads
  static constexpr int PAIR_BYTES = PAD_OFF + (SC_PAD ? 2 * 256 : 0);
  static constexpr int LDS_BYTES = 2 * PAIR_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NW;                  // 1 KiB loads per wave per pair
  static constexpr int B_LOADS = B_BYTES / 1024 / NW;
  static constexpr int LOADS = A_LOADS + B_LOADS + 2 * SC_LOADS;     // per wave and pair
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
  static_assert(A_LOADS >= 1 && A_BYTES == A_LOADS * 1024 * NW, "whole A loads per wave");
  static_assert(B_LOADS >= 1 && B_BYTES == B_LOADS * 1024 * NW, "whole B loads per wave");
  static_assert(SC_PAD == 0 || SC_LOADS == 1, "padding waves load one group");
  static_assert((BM / 64) % SC_LOADS == 0, "a wave's scale groups lie on one operand");
  static_assert(TM >= 1 && TM <= 4 && TN >= 1, "one to four row blocks per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LOADS <= 63, "vmcnt range");
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

__device__ __forceinline__ int mx_swz(int r) { return (r >> 1) & 7; }

// This wave's direct loads for a tile: descriptors and per-lane byte offsets
// (rows clamped to the valid ones: rows past them feed only results that are
// never stored); a pair adds k0 (data) or its slab offsets (scales).
template <class S, bool COH_A>
struct MxPlan {
  __amdgpu_buffer_rsrc_t ra, rb, rsc;
  uint32_t a_off[S::A_LOADS];
  uint32_t b_off[S::B_LOADS];
  uint32_t sc_off[S::SC_LOADS];
  int a_lds, b_lds, sc_lds;   // this wave's bytes into a pair buffer (uniform)
  int sc_rows4;               // bytes of one step's scale words of the wave's operand
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
  // 16-byte slot s of a buffer's A (B) part: row s/8, position s%8, which
  // holds chunk (s%8) ^ swizzle of the row's 128 bytes
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i) {
    const int slot = (wave * S::A_LOADS + i) * 64 + lane;
    const int m = slot >> 3, c = (slot & 7) ^ mx_swz(slot >> 3);
    const int mr = m < m_valid ? m : m_valid - 1;
    P.a_off[i] = (uint32_t)(mr * a.ld + c * 16);
  }
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i) {
    const int slot = (wave * S::B_LOADS + i) * 64 + lane;
    const int n = slot >> 3, c = (slot & 7) ^ mx_swz(slot >> 3);
    const int nr = n < n_valid ? n : n_valid - 1;
    P.b_off[i] = (uint32_t)(nr * b.ld + c * 16);
  }
  // Scales: 64-row groups, A rows first; a wave's groups all lie on one
  // operand.  Rows past the valid ones re-read the last valid row.  A
  // padding wave re-reads A's first group into the padding slot.
  const int g0 = wave * S::SC_LOADS;
  const bool pad = g0 >= S::SC_GROUPS;
  const bool on_a = pad || g0 < S::BM / 64;
  const int gl = pad ? 0 : on_a ? g0 : g0 - S::BM / 64;
  const int valid = on_a ? m_valid : n_valid;
  P.rsc = raw_rsrc(on_a ? a.s : b.s);
  P.sc_lds = pad ? S::PAD_OFF : (on_a ? S::SA_OFF : S::SB_OFF) + gl * 256;
  P.sc_rows4 = pad ? 256 : (on_a ? S::BM : S::BN) * 4;
  P.sc_slab = (int)(on_a ? a.slab : b.slab);
#pragma unroll
  for (int i = 0; i < S::SC_LOADS; ++i) {
    const int r = (gl + i) * 64 + lane;
    P.sc_off[i] = (uint32_t)((r < valid ? r : valid - 1) * 2);
  }
}

// Issues this wave's loads of the pair at k0 (a multiple of 128) into `buf`.
template <class S, bool COH_A>
__device__ __forceinline__ void mx_pair_load(char* buf, const MxPlan<S, COH_A>& P, int k0) {
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(P.ra, (lds_void*)(buf + P.a_lds + i * 1024), 16, P.a_off[i], k0, 0,
                                             COH_A ? kCpolDevice : 0);
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(P.rb, (lds_void*)(buf + P.b_lds + i * 1024), 16, P.b_off[i], k0, 0, 0);
  // both steps' scale words, all with A's policy (one instruction form for
  // every wave; W's scales do not need it and do not mind it)
  const int s0 = (k0 >> 6) * P.sc_slab;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < S::SC_LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(P.rsc, (lds_void*)(buf + P.sc_lds + h * P.sc_rows4 + i * 256), 2,
                                               P.sc_off[i], s0 + h * P.sc_slab, 0, COH_A ? kCpolDevice : 0);
}

// Operand fragments of one step: the A row blocks (reloaded in place, each
// right after its last MFMA of the step) and the B column blocks (two sets,
// current and next step).  Scale words are kept as read (two bytes per row
// word) and shifted to this lane's byte at the MFMA: a shift right after the
// read would wait for it there.
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

// This lane's LDS offsets within a pair buffer.  Row m = (32-row block base)
// + r has the swizzle of r (block bases are multiples of 32), so every
// block's chunks sit at one lane offset plus a constant; step 1's chunks are
// step 0's XOR 4 (byte offset XOR 64), chunk 2+h is chunk h XOR 2 (XOR 32).
struct MxAddr {
  int lo, hi;        // step 0 chunks h and 2+h of row r
  int sh;            // this lane's byte (block h) of a scale word
  int a, b, sa, sb;  // A, B and scale rows of this wave's sub-tile (+ lane row)
};

template <class S>
__device__ __forceinline__ MxAddr mx_addr(const WaveCtx& w) {
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int h = lane >> 5, r = lane & 31;
  MxAddr d;
  d.lo = r * 128 + ((h ^ mx_swz(r)) << 4);
  d.hi = d.lo ^ 32;
  d.sh = 8 * h;
  d.a = wm * S::WM * 128;
  d.b = S::A_BYTES + wn * S::WN * 128;
  d.sa = S::SA_OFF + wm * S::WM * 4 + r * 4;
  d.sb = S::SB_OFF + wn * S::WN * 4 + r * 4;
  return d;
}

// A fragment of row block I, step PAR of the pair in `buf`.
template <class S, int I, int PAR>
__device__ __forceinline__ void mx_load_a(MxA<S>& f, const char* buf, const MxAddr& d) {
  const char* p = buf + d.a + I * 32 * 128;
  const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + (d.lo ^ (PAR * 64)));
  const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + (d.hi ^ (PAR * 64)));
  f.a[I] = __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  f.sa[I] = (int32_t)*reinterpret_cast<const uint32_t*>(buf + d.sa + PAR * S::BM * 4 + I * 128);
}

template <class S, int PAR>
__device__ __forceinline__ void mx_load_b(MxB<S>& f, const char* buf, const MxAddr& d) {
#pragma unroll
  for (int j = 0; j < S::TN; ++j) {
    const char* p = buf + d.b + j * 32 * 128;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + (d.lo ^ (PAR * 64)));
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + (d.hi ^ (PAR * 64)));
    f.b[j] = __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    f.sb[j] = (int32_t)*reinterpret_cast<const uint32_t*>(buf + d.sb + PAR * S::BN * 4 + j * 128);
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

// Row blocks I.. of a step: each block's MFMAs, then its A fragment of the
// next step (step PAR of `nxt`); scheduling barriers keep that order.
template <class S, int I, int PAR>
__device__ __forceinline__ void mx_rows_from(f32x16 (&acc)[S::TM][S::TN], MxA<S>& fa, const MxB<S>& fb,
                                             const char* nxt, const MxAddr& d) {
  if constexpr (I < S::TM) {
    mx_mfma_row<S, I>(acc, fa, fb, d);
    __builtin_amdgcn_sched_barrier(0);
    mx_load_a<S, I, PAR>(fa, nxt, d);
    __builtin_amdgcn_sched_barrier(0);
    mx_rows_from<S, I + 1, PAR>(acc, fa, fb, nxt, d);
  }
}

// One pair: p in buffer X (steps 2p, 2p+1), pair p+1 in Y.  On entry fa + fb
// hold step 2p's fragments; on exit step 2p+2's.  Step 2p reads step 2p+1's
// fragments from X (landed); step 2p+1, after its first row block, waits
// for pair p+1 and the workgroup barrier (every wave has read X: it takes
// pair p+2), then reads step 2p+2's fragments from Y.  The look-ahead load
// is always issued (past the end it re-reads the last pair, never used) so
// the loop has no branches.
template <class S, bool COH_A>
__device__ __forceinline__ void mx_pair_iter(f32x16 (&acc)[S::TM][S::TN], MxA<S>& fa, MxB<S>& fb, MxB<S>& fn, int p,
                                             int np, const MxPlan<S, COH_A>& P, char* X, char* Y, const MxAddr& d) {
#if defined(__HIP_DEVICE_COMPILE__)
  mx_mfma_row<S, 0>(acc, fa, fb, d);
  __builtin_amdgcn_sched_barrier(0);
  mx_load_a<S, 0, 1>(fa, X, d);
  mx_load_b<S, 1>(fn, X, d);
  __builtin_amdgcn_sched_barrier(0);
  mx_rows_from<S, 1, 1>(acc, fa, fb, X, d);
  mx_mfma_row<S, 0>(acc, fa, fn, d);
  __builtin_amdgcn_sched_barrier(0);
  KOS_WAITCNT(0, 0);   // pair p+1 landed; this wave's reads of X done
  lds_barrier();
  mx_pair_load<S, COH_A>(X, P, (p + 2 < np ? p + 2 : np - 1) * S::PAIR_K);
  mx_load_a<S, 0, 0>(fa, Y, d);
  mx_load_b<S, 0>(fb, Y, d);
  __builtin_amdgcn_sched_barrier(0);
  mx_rows_from<S, 1, 0>(acc, fa, fn, Y, d);
#endif
}

// Full K loop: acc = A[0:m_valid) . B[0:n_valid)^T over k in [0, K), K a
// positive multiple of 256 (whole trips of two pairs).  Begins and ends with
// the LDS free.  COH_A: device-coherent loads of A and its scales (rows
// written by other workgroups of this launch).
template <class S, bool COH_A = false>
__device__ __forceinline__ void tile_mainloop_mx(f32x16 (&acc)[S::TM][S::TN], const MxSrc& a, int m_valid,
                                                 const MxSrc& b, int n_valid, int K) {
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int np = K / S::PAIR_K;
  const WaveCtx w = wave_ctx();
  MxPlan<S, COH_A> P;
  mx_plan<S, COH_A>(P, a, m_valid, b, n_valid, w);
  const MxAddr d = mx_addr<S>(w);
  char* b0 = ring<S::PAIR_BYTES, 0>();
  char* b1 = ring<S::PAIR_BYTES, 1>();
  KOS_WAITCNT(0, 0);
  lds_barrier();   // the buffers are free (previous user done)
  mx_pair_load<S, COH_A>(b0, P, 0);
  mx_pair_load<S, COH_A>(b1, P, S::PAIR_K);
  KOS_WAITCNT(S::LOADS, 0);   // pair 0 landed
  lds_barrier();
  MxA<S> fa;
  MxB<S> fb, fn;
  mx_load_a<S, 0, 0>(fa, b0, d);
  if constexpr (S::TM > 1) mx_load_a<S, 1, 0>(fa, b0, d);
  if constexpr (S::TM > 2) mx_load_a<S, 2, 0>(fa, b0, d);
  if constexpr (S::TM > 3) mx_load_a<S, 3, 0>(fa, b0, d);
  mx_load_b<S, 0>(fb, b0, d);
  for (int p = 0; p < np; p += 2) {
    mx_pair_iter<S, COH_A>(acc, fa, fb, fn, p, np, P, b0, b1, d);
    mx_pair_iter<S, COH_A>(acc, fa, fb, fn, p + 1, np, P, b1, b0, d);
  }
  KOS_WAITCNT(0, 0);
  lds_barrier();
}

// The LDS ring of a tile shape's K loop (bf16 or MX): buffer size and
// count, for the staged tile stores that reuse it.
template <class S>
constexpr int ring_bytes() {
  if constexpr (S::MX)
    return S::PAIR_BYTES;
  else
    return S::STAGE_BYTES;
}
template <class S>
constexpr int ring_bufs() {
  return S::MX ? 2 : 4;
}

}  // namespace kos
