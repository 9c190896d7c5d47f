// The builders' bf16 MFMA tile (gfx950): C[BM x BN] = A[BM x K] . B[K x BN],
// fp32 accumulate.
//
// Workgroup of WGM x WGN wave64s (2 x 2, or 2 x 4 with two waves per SIMD);
// each wave owns a (BM/WGM) x (BN/WGN) sub-tile of 32 x 32 blocks computed
// with v_mfma_f32_32x32x16_bf16, the accumulators held in registers for the
// whole K loop.
//
// Operands go straight from HBM/L2 into LDS (buffer_load_dwordx4 ... lds
// through raw buffer descriptors: each lane's 16 bytes land at lds_base +
// 16*lane, so the lanes' source offsets are chosen to realise the swizzled
// layouts below; a stage adds one scalar offset), through a ring of STAGES
// buffers of BK = 32 k-columns, loads issued STAGES-1 stages ahead.
//
// LDS layouts per stage:
//   A: BM rows x 4 chunks of 16 bytes (8 k values), chunk c of row m stored
//      at position c ^ ((m >> 2) & 3).  The A operand of lane l (row l%32,
//      8 k values from 8*(l/32)) is one ds_read_b128.
//   B: BK rows (k) x BN/8 chunks, K x N as in HBM, chunk c of row k stored at
//      position b_pos(c, k) (XOR or rotation by 4*(k%4) inside the row); the
//      SwiGLU tile stores a gate half and an up half, each BK rows of BN/16
//      chunks laid out the same way.  The B operand
//      (8 consecutive k of one column) is two ds_read_b64_tr_b16: in each
//      16-lane group, lane j receives element j%4 of source lanes j/4 + 4v,
//      v = 0..3, so source lane i = 4v + q points at row k0+v, columns
//      n0 + 4q .. +4, and lane 4q + c receives column n0 + 4q + c, rows
//      k0 .. k0+3.
//
// MFMA operand layout (32x32x16): lane l holds A[row l%32][k 8*(l/32) .. +8]
// and B[k 8*(l/32) .. +8][col l%32]; accumulator register r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma once

#include "kos_device.h"

namespace kos {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// WGM x WGN waves: 2 x 2 (one wave per SIMD) or 2 x 4 (two waves per SIMD:
// while one waits on LDS or memory the other issues MFMAs; each holds half
// the accumulators).  BNT: B stored N x K (row n holds output column n's K
// values, the transposed weight of a backward pass); its stage is then BN
// rows of 64 bytes laid out and read like A's.
template <int BM_, int BN_, int STAGES_ = 4, int WGM_ = 2, int WGN_ = 2, bool BNT_ = false>
struct TileShape {
  static constexpr bool MX = false;                     // bf16 operands
  static constexpr bool BNT = BNT_;
  static constexpr int BM = BM_, BN = BN_, BK = 32, STAGES = STAGES_;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN;                  // waves
  static constexpr int NT = 64 * NW;                    // threads
  static constexpr int WM = BM / WGM, WN = BN / WGN;    // wave sub-tile
  static constexpr int TM = WM / 32, TN = WN / 32;      // 32x32 blocks per wave
  static constexpr int A_BYTES = BM * BK * 2;           // per stage
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // An A stage of half a KiB per wave (64 rows on eight waves) is loaded by
  // the lower 32 lanes of every wave, so every wave still issues the same
  // number of loads per stage (the waits count instructions).
  static constexpr bool A_HALF = A_BYTES == 512 * NW;
  static constexpr int A_WAVE_BYTES = A_HALF ? 512 : 1024;   // bytes per A load instruction
  static constexpr int A_LOADS = A_HALF ? 1 : A_BYTES / 1024 / NW;   // A loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / NW;                // 1 KiB B loads per wave per stage
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int BROW_CHUNKS = BN / 8;            // 16-byte chunks per B row
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
  static_assert(B_BYTES % (1024 * NW) == 0 && (A_HALF || A_BYTES % (1024 * NW) == 0),
                "whole loads per wave");
  static_assert(TM >= 1 && TN >= 1, "at least one 32x32 block per wave");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "each wave loads at least 1 KiB of A and of B");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(3 * LOADS <= 63, "vmcnt range");
};

// Where the B tile's columns come from: BN consecutive columns of one
// K x N matrix (plain), or, for the SwiGLU tile (dual), BN/2 columns of the
// gate matrix and the same BN/2 columns of the up matrix.  BNT tiles: p0 is
// row n0 of the N x K matrix and ld its row stride.  In the dual
// tile each wave's 32x32 blocks j < TN/2 hold gate values and blocks
// j + TN/2 the up values of the same output columns.
struct BSrc {
  const uint16_t* p0;   // B[0][n0] of the (gate) matrix
  const uint16_t* p1;   // B[0][n0] of the up matrix (dual only)
  int64_t ld;           // row stride of B, in elements
};

__device__ __forceinline__ int a_swz(int m) { return (m >> 2) & 3; }

// B rows of W chunks (16 bytes each): chunk c of row k sits at position
// b_pos<W>(c, k).  Power-of-two widths XOR the chunk index with 4*(k%4);
// other widths rotate it by 4*(k%4).  Both keep aligned 4-chunk groups
// together and send the four rows read by one transpose read to different
// banks.
template <int W>
__device__ __forceinline__ int b_pos(int c, int k) {
  if constexpr ((W & (W - 1)) == 0) {
    return c ^ ((4 * (k & 3)) & (W - 1));
  } else {
    const int p = c + 4 * (k & 3);
    return p >= W ? p - W : p;
  }
}
template <int W>
__device__ __forceinline__ int b_chunk(int p, int k) {
  if constexpr ((W & (W - 1)) == 0) {
    return p ^ ((4 * (k & 3)) & (W - 1));
  } else {
    const int c = p - 4 * (k & 3);
    return c < 0 ? c + W : c;
  }
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// This thread's lane and its wave's index, computed afresh where a tile
// starts or ends.  The empty asm makes them opaque to the optimizer, so the
// addresses derived from them are computed per tile rather than hoisted to
// the start of the persistent kernel and kept live (register pressure)
// through every role.
struct WaveCtx {
  int lane;   // 0..63
  int wave;   // 0..3, uniform (scalar register)
};
__device__ __forceinline__ WaveCtx wave_ctx() {
  int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  int wave = wave_id();
  asm volatile("" : "+v"(lane), "+s"(wave));
  return {lane, wave};
}

// LDS layout of a stage's B part: plain, BK rows of BN/8 chunks; dual, the
// gate half (BK rows of BN/16 chunks) then the up half, same layout.
template <class S, bool DUAL>
struct BLayout {
  static constexpr int W = DUAL ? S::BROW_CHUNKS / 2 : S::BROW_CHUNKS;   // chunks per LDS row
  static constexpr int ROW_BYTES = W * 16;
  static constexpr int HALF_BYTES = S::B_BYTES / 2;
  static_assert(!DUAL || (S::B_LOADS * (S::NW / 2) * 1024 == HALF_BYTES),
                "dual: the first half of the waves load the gate half, the rest the up half");
  static_assert(!DUAL || S::TN % 2 == 0, "dual: gate and up blocks pair up in each wave");
};

// This wave's direct loads, fixed for a tile: raw buffer descriptors of the
// A rows and of its B matrix, and per-lane byte offsets; every stage adds
// k0*2 (A) or k0*ldb*2 (B) as a scalar offset.  Offsets stay below 2^31
// (the entry points check the operand extents).
template <class S, bool DUAL, bool COH_A = false, bool SPLIT = false>
struct LoadPlan {
  __amdgpu_buffer_rsrc_t ra, rb;
  __amdgpu_buffer_rsrc_t ra2, rb2;             // SPLIT: the second A and B matrices, for k >= k1
  int k1;
  uint32_t a_off[S::A_LOADS];
  uint32_t b_off[S::B_LOADS];
  int b_stride;                                // bytes per k row of B
  int a_lds, b_lds;                            // this wave's bytes into a stage (uniform)
  bool a_on;                                   // this lane loads A (A_HALF: lanes 0..31)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wave_uniform(base)), (short)0, 0x7fffffff,
                                           kRawBufferWord3);
}

// A rows are clamped to m_valid-1: rows past the valid ones only feed
// accumulator rows that are never stored.
template <class S, bool DUAL, bool COH_A, bool SPLIT>
__device__ __forceinline__ void plan_loads(LoadPlan<S, DUAL, COH_A, SPLIT>& P, const uint16_t* __restrict__ A, int64_t lda,
                                           int m_valid, const BSrc& b, const WaveCtx& w) {
  using L = BLayout<S, DUAL>;
  const int lane = w.lane, wave = w.wave;
  P.a_lds = wave * S::A_LOADS * S::A_WAVE_BYTES;
  P.b_lds = S::A_BYTES + wave * S::B_LOADS * 1024;
  P.a_on = !S::A_HALF || lane < 32;
  P.ra = raw_rsrc(A);
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i) {
    // 16-byte slot in the A stage
    const int slot = S::A_HALF ? wave * 32 + (lane & 31) : (wave * S::A_LOADS + i) * 64 + lane;
    const int m = slot >> 2, p = slot & 3;
    const int c = p ^ a_swz(m);
    const int mr = m < m_valid ? m : m_valid - 1;
    P.a_off[i] = (uint32_t)(mr * lda * 2 + c * 16);
  }
  P.b_stride = (int)(b.ld * 2);
  if constexpr (S::BNT) {
    static_assert(!DUAL, "the SwiGLU tile reads K x N weights");
    // rows n of 64 bytes, A's layout
    P.rb = raw_rsrc(b.p0);
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i) {
      const int slot = (wave * S::B_LOADS + i) * 64 + lane;
      const int n = slot >> 2, c = (slot & 3) ^ a_swz(slot >> 2);
      P.b_off[i] = (uint32_t)(n * P.b_stride + c * 16);
    }
    return;
  }
  // dual: the first half of the waves fill the gate half, the rest the up half
  const bool up = DUAL && wave >= S::NW / 2;
  P.rb = raw_rsrc(up ? b.p1 : b.p0);
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i) {
    int slot = (wave * S::B_LOADS + i) * 64 + lane;
    if (up) slot -= L::HALF_BYTES / 16;
    const int k = slot / L::W, p = slot % L::W;
    const int c = b_chunk<L::W>(p, k);
    P.b_off[i] = (uint32_t)(k * P.b_stride + c * 16);
  }
}

// Cache policy of loads: device-coherent (sc1) for A rows written by other
// workgroups of the same launch.
constexpr int kCpolDevice = 16;

// Issues this wave's direct loads (buffer -> LDS) of the stage at k0.
// SPLIT: stages at k0 >= k1 come from the second matrices, at k0 - k1.
template <class S, bool DUAL, bool COH_A, bool SPLIT>
__device__ __forceinline__ void stage_load(char* lds_stage, const LoadPlan<S, DUAL, COH_A, SPLIT>& P, int k0) {
  const bool second = SPLIT && k0 >= P.k1;
  const int ka = second ? k0 - P.k1 : k0;
  const __amdgpu_buffer_rsrc_t ra = second ? P.ra2 : P.ra;
  const __amdgpu_buffer_rsrc_t rb = second ? P.rb2 : P.rb;
  const int soa = ka * 2;
  const int sob = S::BNT ? ka * 2 : ka * P.b_stride;
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i)
    if (!S::A_HALF || P.a_on)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(lds_stage + P.a_lds + i * S::A_WAVE_BYTES), 16,
                                               P.a_off[i], soa, 0, COH_A ? kCpolDevice : 0);
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(lds_stage + P.b_lds + i * 1024), 16, P.b_off[i], sob,
                                             0, 0);
}

// Operand fragments of one k16 step.
template <class S>
struct Frags {
  bf16x8 a[S::TM];
  bf16x8 b[S::TN];
};

// LDS -> registers for k16 step s (0 or 1) of a stage.
template <class S, bool DUAL>
__device__ __forceinline__ void frag_load(Frags<S>& f, const char* lds_stage, int s, const WaveCtx& w) {
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const char* ast = lds_stage;
  const char* bst = lds_stage + S::A_BYTES;
  const int g = lane >> 4, jj = lane & 15, v = jj >> 2, q = jj & 3;
  const int kc = 2 * s + (lane >> 5);
#pragma unroll
  for (int i = 0; i < S::TM; ++i) {
    const int m = wm * S::WM + i * 32 + (lane & 31);
    f.a[i] = *reinterpret_cast<const bf16x8*>(ast + m * 64 + ((kc ^ a_swz(m)) << 4));
  }
  if constexpr (S::BNT) {
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      const int n = wn * S::WN + j * 32 + (lane & 31);
      f.b[j] = *reinterpret_cast<const bf16x8*>(bst + n * 64 + ((kc ^ a_swz(n)) << 4));
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < S::TN; ++j) {
    using L = BLayout<S, DUAL>;
    // plain: tile column n; dual: column n of the gate (j < TN/2) or up half
    const bool up = DUAL && j >= S::TN / 2;
    const int jb = up ? j - S::TN / 2 : j;
    const int n = wn * (DUAL ? S::WN / 2 : S::WN) + jb * 32 + 16 * (g & 1) + 4 * q;
    const char* bh = bst + (up ? L::HALF_BYTES : 0);
    s16x4 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = s * 16 + 8 * (g >> 1) + 4 * r + v;
      const int c = b_pos<L::W>(n >> 3, k);
      h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(bh + k * L::ROW_BYTES + (c << 4) + ((n & 7) << 1)));
    }
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 both = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
    f.b[j] = __builtin_bit_cast(bf16x8, both);
  }
}

template <class S>
__device__ __forceinline__ void frag_mfma(f32x16 (&acc)[S::TM][S::TN], const Frags<S>& f) {
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
      // B fragment as the first operand: the product comes out transposed, so
      // each lane holds four consecutive output columns of one row (vector
      // stores in the epilogue)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// s_waitcnt immediate: vmcnt <= v, lgkmcnt <= l (expcnt untouched).
#define KOS_WAITCNT(v, l) __builtin_amdgcn_s_waitcnt(((v) & 15) | (((v) >> 4) << 14) | (0x7 << 4) | ((l) << 8))

// Waits until at most `n` stages of this wave's loads are in flight and all
// its LDS reads have completed.
template <class S>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 2) {
    KOS_WAITCNT(2 * S::LOADS, 0);
  } else if (n == 1) {
    KOS_WAITCNT(S::LOADS, 0);
  } else {
    KOS_WAITCNT(0, 0);
  }
}

// Workgroup barrier without a memory fence (the waits above are explicit);
// the asm memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The LDS ring: one __shared__ array per stage, so the compiler can tell a
// stage being read from the stages being filled and does not wait for them.
// Keyed by the stage size: tile shapes of one kernel share a ring sized for
// the largest.
template <int STAGE_BYTES, int I>
__device__ __forceinline__ char* ring() {
  __shared__ __attribute__((aligned(1024))) char buf[STAGE_BYTES];
  return buf;
}

// Scheduling hints for one basic block: interleave the block's MFMAs with
// its LDS reads (and direct loads), so that operand reads for the next step
// travel while the matrix cores work on this one.
template <int N_MFMA, int N_DS, int N_VMEM>
__device__ __forceinline__ void sched_interleave() {
  constexpr int MFMA = 0x008, DS_READ = 0x100, VMEM = 0x020;
#pragma unroll
  for (int i = 0; i < N_MFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    if (i < N_VMEM) __builtin_amdgcn_sched_group_barrier(VMEM, 1, 0);
    if (i < N_DS) __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
  }
}

// One iteration of the K loop on stage kt, which sits in ring buffer `cur`
// (`nxt` holds stage kt+1).  On entry f0 holds (kt, step 0); leaves f0 =
// (kt+1, step 0).  `steady`: the look-ahead load is always issued (past the
// end it re-reads the last stage: cache hits, never used), so the counts in
// flight stay uniform and the loop body has no branches.
template <class S, bool DUAL, bool COH_A, bool steady, bool SPLIT>
__device__ __forceinline__ void k_iter(f32x16 (&acc)[S::TM][S::TN], Frags<S>& f0, Frags<S>& f1, int kt, int nk,
                                       const LoadPlan<S, DUAL, COH_A, SPLIT>& P, char* cur, char* nxt,
                                       const WaveCtx& w) {
#if defined(__HIP_DEVICE_COMPILE__)   // device code only (the host pass never emits it)
  constexpr int ST = S::STAGES;
  constexpr int NM = S::TM * S::TN, ND = S::TM + (S::BNT ? 1 : 2) * S::TN;
  frag_load<S, DUAL>(f1, cur, 1, w);
  frag_mfma<S>(acc, f0);
  if (steady) sched_interleave<NM, ND, 0>();
  // stage kt+1 must have landed (all waves) and stage kt must be read by all
  // waves before its buffer takes stage kt+ST
  if (steady) {
    KOS_WAITCNT(2 * S::LOADS, 0);
  } else {
    wait_stages<S>(nk - 2 - kt < ST - 2 ? nk - 2 - kt : ST - 2);
  }
  lds_barrier();
  if (steady) {
    stage_load<S, DUAL, COH_A, SPLIT>(cur, P, (kt + ST < nk ? kt + ST : nk - 1) * S::BK);
    frag_load<S, DUAL>(f0, nxt, 0, w);
    frag_mfma<S>(acc, f1);
    sched_interleave<NM, ND, S::LOADS>();
  } else {
    if (kt + ST < nk) stage_load<S, DUAL, COH_A, SPLIT>(cur, P, (kt + ST) * S::BK);
    if (kt + 1 < nk) frag_load<S, DUAL>(f0, nxt, 0, w);
    frag_mfma<S>(acc, f1);
  }
#endif
}

// Full K loop: acc = A[0:m_valid rows] . B over k in [0, K) (K a multiple of
// 32).  Begins and ends with the LDS ring free.  RING: stage size of the
// ring (at least the tile's; a kernel with two tile shapes passes the larger).
// SPLIT: the sum of two products over one K loop, acc = A[:, 0:K1] . B +
// A2[:, 0:K-K1] . B2 (same strides; K1 a multiple of 32; B2 the second
// matrix's first element as b.p0 is the first's).
template <class S, bool DUAL = false, bool COH_A = false, int RING = S::STAGE_BYTES, bool SPLIT = false>
__device__ __forceinline__ void tile_mainloop(f32x16 (&acc)[S::TM][S::TN], const uint16_t* __restrict__ A,
                                              int64_t lda, int m_valid, const BSrc& b, int K,
                                              const uint16_t* A2 = nullptr, const uint16_t* B2 = nullptr, int K1 = 0) {
  constexpr int ST = S::STAGES;
  static_assert(ST == 4, "the ring is unrolled for four stages");
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = K / S::BK;
  const WaveCtx w = wave_ctx();
  LoadPlan<S, DUAL, COH_A, SPLIT> P;
  plan_loads<S, DUAL, COH_A, SPLIT>(P, A, lda, m_valid, b, w);
  if (SPLIT) {
    P.ra2 = raw_rsrc(A2);
    P.rb2 = raw_rsrc(B2);
    P.k1 = K1;
  }
  static_assert(S::STAGE_BYTES <= RING, "tile stage larger than the ring");
  char* r0 = ring<RING, 0>();
  char* r1 = ring<RING, 1>();
  char* r2 = ring<RING, 2>();
  char* r3 = ring<RING, 3>();
  KOS_WAITCNT(0, 0);
  lds_barrier();   // the ring is free (previous user done)
  if (nk >= ST && nk % ST == 0) {
    stage_load<S, DUAL, COH_A, SPLIT>(r0, P, 0);
    stage_load<S, DUAL, COH_A, SPLIT>(r1, P, 1 * S::BK);
    stage_load<S, DUAL, COH_A, SPLIT>(r2, P, 2 * S::BK);
    stage_load<S, DUAL, COH_A, SPLIT>(r3, P, 3 * S::BK);
    KOS_WAITCNT(3 * S::LOADS, 0);
    lds_barrier();
    Frags<S> f0, f1;
    frag_load<S, DUAL>(f0, r0, 0, w);
    for (int kt = 0; kt < nk; kt += ST) {
      k_iter<S, DUAL, COH_A, true, SPLIT>(acc, f0, f1, kt, nk, P, r0, r1, w);
      k_iter<S, DUAL, COH_A, true, SPLIT>(acc, f0, f1, kt + 1, nk, P, r1, r2, w);
      k_iter<S, DUAL, COH_A, true, SPLIT>(acc, f0, f1, kt + 2, nk, P, r2, r3, w);
      k_iter<S, DUAL, COH_A, true, SPLIT>(acc, f0, f1, kt + 3, nk, P, r3, r0, w);
    }
    KOS_WAITCNT(0, 0);
    lds_barrier();
    return;
  }
  stage_load<S, DUAL, COH_A, SPLIT>(r0, P, 0);
  if (1 < nk) stage_load<S, DUAL, COH_A, SPLIT>(r1, P, 1 * S::BK);
  if (2 < nk) stage_load<S, DUAL, COH_A, SPLIT>(r2, P, 2 * S::BK);
  if (3 < nk) stage_load<S, DUAL, COH_A, SPLIT>(r3, P, 3 * S::BK);
  // stage 0 landed; up to three later stages may still fly
  if (nk >= 4) {
    KOS_WAITCNT(3 * S::LOADS, 0);
  } else {
    wait_stages<S>(nk - 1);
  }
  lds_barrier();
  Frags<S> f0, f1;
  frag_load<S, DUAL>(f0, r0, 0, w);
  for (int kt = 0; kt < nk; kt += ST) {
    k_iter<S, DUAL, COH_A, false, SPLIT>(acc, f0, f1, kt, nk, P, r0, r1, w);
    if (kt + 1 < nk) k_iter<S, DUAL, COH_A, false, SPLIT>(acc, f0, f1, kt + 1, nk, P, r1, r2, w);
    if (kt + 2 < nk) k_iter<S, DUAL, COH_A, false, SPLIT>(acc, f0, f1, kt + 2, nk, P, r2, r3, w);
    if (kt + 3 < nk) k_iter<S, DUAL, COH_A, false, SPLIT>(acc, f0, f1, kt + 3, nk, P, r3, r0, w);
  }
  KOS_WAITCNT(0, 0);
  lds_barrier();
}

// Accumulator layout (operands of the 32x32x16 MFMA swapped): in column
// block j of row block i, lane l and register r hold tile element
//   row = wm*WM + i*32 + l%32,  col = wn*WN + j*32 + 8*(r/4) + 4*(l/32) + r%4.
// Visits the accumulators four consecutive columns at a time:
// f(tile row, first tile column, the four values).
template <class S, class F>
__device__ __forceinline__ void tile_foreach4(const f32x16 (&acc)[S::TM][S::TN], F&& f) {
  const WaveCtx w = wave_ctx();
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = wm * S::WM + i * 32 + (lane & 31);
        const int col = wn * S::WN + j * 32 + g * 8 + (lane >> 5) * 4;
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        f(row, col, v);
      }
}

// SwiGLU of a gate and an up value: silu(g) * u = g / (1 + e^-g) * u, fp32,
// with the hardware exponential and reciprocal (about 1 ulp each; the result
// is rounded to bf16 next).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

typedef __attribute__((address_space(3))) char lds_char;

// Ring buffer i (0..3) as an LDS pointer; i is uniform (scalar selects).
template <int RING>
__device__ __forceinline__ lds_char* ring_lds(int i) {
  lds_char* b0 = (lds_char*)ring<RING, 0>();
  lds_char* b1 = (lds_char*)ring<RING, 1>();
  lds_char* b2 = (lds_char*)ring<RING, 2>();
  lds_char* b3 = (lds_char*)ring<RING, 3>();
  return i == 0 ? b0 : i == 1 ? b1 : i == 2 ? b2 : b3;
}

// Stores BM x OW bf16 values as rows [0, m_valid) of dst (row stride ld
// elements) through the LDS ring.  fn(i, j, q) gives the calling lane's four
// fp32 values of row wm*WM + i*32 + lane%32, columns wn*(OW/WGN) + j*32 +
// 8q + 4*(lane/32) + [0, 4), for i < TM, j < OW/(32 WGN), q < 4 (the
// accumulator layout of a 32x32 block; fn may update the accumulators it
// reads).  Every lane writes its four-column pieces into LDS, then each
// group of lanes stores whole rows with 16-byte stores, so the global writes
// are whole cache lines (what device-coherent write-through stores need to
// be cheap).  COH: device-scope (sc1) stores.  Call right after
// tile_mainloop (the ring is free); the next tile_mainloop waits for the
// ring.  dst is the same in every thread.
template <class S, int RING, bool COH, int OW, class Fn>
__device__ __forceinline__ void tile_store_rows_fn(uint16_t* dst, int64_t ld, int m_valid, Fn&& fn) {
  constexpr int OJ = OW / 32 / S::WGN;             // 32-column output blocks per wave
  constexpr int ROW_BYTES = OW * 2;
  constexpr int CPR = ROW_BYTES / 16;              // 16-byte chunks per row
  constexpr int ROWS_PER_RING = RING / ROW_BYTES;
  constexpr int ROWS_PER_PASS = S::NT / CPR;
  static_assert(OW % (32 * S::WGN) == 0, "whole 32-column blocks per wave");
  static_assert(RING % ROW_BYTES == 0 && 4 * ROWS_PER_RING >= S::BM, "the tile must fit the ring");
  static_assert((CPR & (CPR - 1)) == 0 && S::NT % CPR == 0, "power-of-two chunks per row");
  static_assert(ROWS_PER_RING % 32 == 0 && ROWS_PER_RING % ROWS_PER_PASS == 0,
                "32-row groups and store passes stay inside one ring buffer");
  const WaveCtx w = wave_ctx();
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  // chunk c of row r sits at chunk position c ^ (r % CPR) (spreads the 32
  // rows one write instruction touches over the banks)
#pragma unroll
  for (int i = 0; i < S::TM; ++i) {
    const int row0 = wm * S::WM + i * 32;          // uniform: the 32 rows share a ring buffer
    const int row = row0 + (lane & 31);
    lds_char* base = ring_lds<RING>(row0 / ROWS_PER_RING) + (row % ROWS_PER_RING) * ROW_BYTES;
#pragma unroll
    for (int j = 0; j < OJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * (OW / S::WGN) + j * 32 + g * 8 + (lane >> 5) * 4;
        const int chunk = (col >> 3) ^ (row & (CPR - 1));
        const f32x4 v = fn(i, j, g);
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(base + chunk * 16 + (col & 7) * 2) =
            pack4_bf16(v);
        // one 32x32 block at a time: keeps the accumulator reads from being
        // hoisted together (they would need a VGPR each)
        if (g == 3) __builtin_amdgcn_sched_barrier(0);
      }
  }
  KOS_WAITCNT(0, 0);
  lds_barrier();
  const DevBuf d(dst);
  const int t = wave * 64 + lane;
  const int c = t % CPR;
  // passes in batches of 8: the batch's LDS reads, then its stores (rows
  // past m_valid predicated off); the scheduling barrier keeps a batch's
  // registers from being hoisted into the previous one
  constexpr int PASSES = S::BM / ROWS_PER_PASS, BATCH = PASSES < 8 ? PASSES : 8;
  static_assert(PASSES % BATCH == 0, "whole batches");
#pragma unroll
  for (int b0 = 0; b0 < PASSES; b0 += BATCH) {
    u32x4 v[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int r0 = (b0 + q) * ROWS_PER_PASS;
      const int row = r0 + t / CPR;
      v[q] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          ring_lds<RING>(r0 / ROWS_PER_RING) + (row % ROWS_PER_RING) * ROW_BYTES + ((c ^ (row & (CPR - 1))) * 16));
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int row = (b0 + q) * ROWS_PER_PASS + t / CPR;
      const int64_t off = ((int64_t)row * ld + c * 8) * 2;
      if (row < m_valid) {
        if constexpr (COH)
          d.st128((uint32_t)off, v[q]);
        else
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + off) = v[q];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Stores the tile as bf16 rows [0, m_valid) of dst (tile_store_rows_fn).
// SWIGLU: the tile holds gate and up columns (BSrc dual layout) and the BN/2
// output columns are swiglu(gate, up).
template <class S, int RING, bool COH, bool SWIGLU = false>
__device__ __forceinline__ void tile_store_rows(const f32x16 (&acc)[S::TM][S::TN], uint16_t* dst, int64_t ld,
                                                int m_valid) {
  tile_store_rows_fn<S, RING, COH, SWIGLU ? S::BN / 2 : S::BN>(dst, ld, m_valid, [&](int i, int j, int g) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = SWIGLU ? swiglu(acc[i][j][4 * g + e], acc[i][j + S::TN / 2][4 * g + e]) : acc[i][j][4 * g + e];
    return v;
  });
}

// Ring buffer i (i < NBUF, uniform) of a kernel whose ring has NBUF buffers
// of RING bytes; buffers past NBUF are never instantiated.
template <int RING, int NBUF>
__device__ __forceinline__ lds_char* ring_buf(int i) {
  static_assert(NBUF == 2 || NBUF == 4, "rings of two or four buffers");
  if constexpr (NBUF == 2) {
    lds_char* b0 = (lds_char*)ring<RING, 0>();
    lds_char* b1 = (lds_char*)ring<RING, 1>();
    return i == 0 ? b0 : b1;
  } else {
    return ring_lds<RING>(i);
  }
}

// Rounds a tile store takes: the fewest (1, 2 or 4) whose rows fill NBUF
// ring buffers, or fewer, with whole 32-row groups (0: none fits).
template <int BM, int ROW_BYTES, int RING, int NBUF>
constexpr int store_rounds() {
  for (int r = 1; r <= 4; r *= 2) {
    const int rr = BM / r, nb = rr / 32 < NBUF ? rr / 32 : NBUF;
    if (BM % r == 0 && rr % 32 == 0 && nb > 0 && rr % nb == 0 && (rr / nb) % 32 == 0 && (rr / nb) * ROW_BYTES <= RING)
      return r;
  }
  return 0;
}

// Stores the whole BM x BN tile as rows [0, m_valid) of dst (row stride ld
// elements of T: bf16 as uint16_t, or float), through the LDS ring, so that
// the global writes are whole 16-byte chunks of rows, consecutive lanes on
// consecutive chunks (whole cache lines), for any BN with a multiple of 8
// chunks per row.  When the tile is larger than the ring it goes out in
// rounds: round r takes every wave's 32-row blocks [r*TM/R, (r+1)*TM/R), so
// each round frees part of every wave's accumulators.  A round's rows are
// spread evenly over the ring buffers (RPB each), and a store pass never
// leaves its buffer, so every LDS address has a uniform base.  Chunk c of a
// ring row x sits at c ^ (x & SW), SW+1 the largest power of two (up to 32)
// dividing the chunks per row: the 32 rows a write instruction touches fall
// on different banks, and the chunk stays inside its row.  COH:
// device-scope (sc1) stores.  BM rows of ld elements stay below 2 GiB.  Call
// right after the K loop (the ring is free); the next K loop waits for the
// ring.
template <class S, int RING, bool COH, class T, int NBUF = 4>
__device__ __forceinline__ void tile_store_out(const f32x16 (&acc)[S::TM][S::TN], T* dst, int64_t ld, int m_valid) {
  constexpr int ESZ = sizeof(T);
  static_assert(ESZ == 2 || ESZ == 4, "bf16 or fp32 output");
  constexpr int EPC = 16 / ESZ;                       // elements per 16-byte chunk
  constexpr int ROW_BYTES = S::BN * ESZ;
  constexpr int CPR = ROW_BYTES / 16;                 // chunks per row
  constexpr int LOWBIT = CPR & -CPR;
  constexpr int SW = (LOWBIT < 32 ? LOWBIT : 32) - 1;
  constexpr int ROUNDS = store_rounds<S::BM, ROW_BYTES, RING, NBUF>();
  static_assert(ROUNDS > 0, "the tile's rows do not fit the ring in whole 32-row groups");
  constexpr int RR = S::BM / ROUNDS;                  // rows per round
  constexpr int NB = RR / 32 < NBUF ? RR / 32 : NBUF; // ring buffers used
  constexpr int RPB = RR / NB;                        // rows per buffer
  constexpr int TMR = S::TM / ROUNDS;                 // 32-row blocks per wave and round
  constexpr int RWM = S::WM / ROUNDS;                 // rows per wave and round
  constexpr int PPB = RPB * CPR / S::NT;              // store passes per buffer
  constexpr int PASSES = NB * PPB;
  constexpr int BATCH = PASSES % 8 == 0 ? 8 : PASSES % 6 == 0 ? 6 : PASSES % 4 == 0 ? 4 : PASSES % 3 == 0 ? 3
                        : PASSES % 2 == 0 ? 2 : 1;    // passes per batch
  static_assert(CPR % 8 == 0, "whole groups of eight chunks per row");
  static_assert(S::TM % ROUNDS == 0 && RWM % 32 == 0, "whole 32-row blocks per wave and round");
  static_assert(RPB * CPR % S::NT == 0, "whole store passes per buffer");
  static_assert(S::TN * 32 * S::WGN == S::BN, "whole 32-column blocks per wave");
  const WaveCtx w = wave_ctx();
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int t = wave * 64 + lane;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wave_uniform((const void*)dst)), (short)0, 0x7fffffff,
                                        kRawBufferWord3);
  const uint32_t ldb = (uint32_t)(ld * ESZ);
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0) {
      KOS_WAITCNT(0, 0);   // the previous round's ring reads are done
      lds_barrier();
    }
#pragma unroll
    for (int ii = 0; ii < TMR; ++ii) {
      const int i = rd * TMR + ii;
      const int x0 = wm * RWM + ii * 32;             // ring row of the 32-row block (uniform)
      const int x = x0 + (lane & 31);
      lds_char* base = ring_buf<RING, NBUF>(x0 / RPB) + (x % RPB) * ROW_BYTES;
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wn * S::WN + j * 32 + g * 8 + (lane >> 5) * 4;
          const int chunk = (col / EPC) ^ (x & SW);
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
          if constexpr (ESZ == 2)
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(base + chunk * 16 + (col % EPC) * 2) =
                pack4_bf16(v);
          else
            *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(base + chunk * 16) = v;
          if (g == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
    KOS_WAITCNT(0, 0);
    lds_barrier();
#pragma unroll
    for (int b0 = 0; b0 < PASSES; b0 += BATCH) {
      u32x4 v[BATCH];
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        const int ps = b0 + q, bf = ps / PPB;        // buffer bf: compile-time
        const int y = (ps % PPB) * S::NT + t;
        const int xb = y / CPR, c = y % CPR, x = bf * RPB + xb;
        v[q] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            ring_buf<RING, NBUF>(bf) + xb * ROW_BYTES + ((c ^ (x & SW)) * 16));
      }
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        const int ps = b0 + q, bf = ps / PPB;
        const int y = (ps % PPB) * S::NT + t;
        const int x = bf * RPB + y / CPR, c = y % CPR;
        const int row = (x / RWM) * S::WM + rd * RWM + x % RWM;
        if (row < m_valid)
          __builtin_amdgcn_raw_buffer_store_b128(v[q], rs, (uint32_t)row * ldb + (uint32_t)c * 16u, 0,
                                                 COH ? kCpolSc1 : 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Both halves of a dual-layout tile (gate blocks and up blocks, BN/2
// columns each) as bf16 rows [0, m_valid) of dst0 and dst1, in one pass
// through the LDS ring: the gate half takes ring rows [0, BM), the up half
// rows [BM, 2 BM), laid out as in tile_store_rows; then every 16-byte chunk
// of a row goes out with one store.  COH: device-scope (sc1) stores.  Call
// right after tile_mainloop (the ring is free).
template <class S, int RING, bool COH>
__device__ __forceinline__ void tile_store_rows_pair(const f32x16 (&acc)[S::TM][S::TN], uint16_t* dst0,
                                                     uint16_t* dst1, int64_t ld, int m_valid) {
  constexpr int OW = S::BN / 2, OJ = S::TN / 2;
  constexpr int ROW_BYTES = OW * 2;
  constexpr int CPR = ROW_BYTES / 16;
  constexpr int ROWS_PER_RING = RING / ROW_BYTES;
  constexpr int ROWS_PER_PASS = S::NT / CPR;
  static_assert(RING % ROW_BYTES == 0 && 4 * ROWS_PER_RING >= 2 * S::BM, "both halves must fit the ring");
  static_assert((CPR & (CPR - 1)) == 0 && S::NT % CPR == 0, "power-of-two chunks per row");
  static_assert(ROWS_PER_RING % 32 == 0 && ROWS_PER_RING % ROWS_PER_PASS == 0 && S::BM % ROWS_PER_PASS == 0,
                "32-row groups and store passes stay inside one ring buffer and one half");
  const WaveCtx w = wave_ctx();
  const int lane = w.lane, wave = w.wave;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int row0 = hf * S::BM + wm * S::WM + i * 32;   // ring row of the 32-row group (uniform)
      const int row = row0 + (lane & 31);
      lds_char* base = ring_lds<RING>(row0 / ROWS_PER_RING) + (row % ROWS_PER_RING) * ROW_BYTES;
#pragma unroll
      for (int j = 0; j < OJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wn * (OW / S::WGN) + j * 32 + g * 8 + (lane >> 5) * 4;
          const int chunk = (col >> 3) ^ (row & (CPR - 1));
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j + hf * OJ][4 * g + e];
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(base + chunk * 16 + (col & 7) * 2) =
              pack4_bf16(v);
          if (g == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
  KOS_WAITCNT(0, 0);
  lds_barrier();
  const int t = wave * 64 + lane;
  const int c = t % CPR;
  constexpr int HALF_PASSES = S::BM / ROWS_PER_PASS, PASSES = 2 * HALF_PASSES;
  constexpr int BATCH = HALF_PASSES < 8 ? HALF_PASSES : 8;
  static_assert(HALF_PASSES % BATCH == 0, "whole batches, one half each");
#pragma unroll
  for (int b0 = 0; b0 < PASSES; b0 += BATCH) {
    const bool up = b0 * ROWS_PER_PASS >= S::BM;   // uniform: a batch lies in one half
    const DevBuf d(up ? dst1 : dst0);
    uint16_t* dst = up ? dst1 : dst0;
    u32x4 v[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int r0 = (b0 + q) * ROWS_PER_PASS;
      const int row = r0 + t / CPR;
      v[q] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          ring_lds<RING>(r0 / ROWS_PER_RING) + (row % ROWS_PER_RING) * ROW_BYTES + ((c ^ (row & (CPR - 1))) * 16));
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int row = (b0 + q) * ROWS_PER_PASS + t / CPR - (up ? S::BM : 0);
      const int64_t off = ((int64_t)row * ld + c * 8) * 2;
      if (row < m_valid) {
        if constexpr (COH)
          d.st128((uint32_t)off, v[q]);
        else
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + off) = v[q];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace kos
