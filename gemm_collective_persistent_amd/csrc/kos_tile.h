// The builders' bf16 MFMA tile (gfx950): C[BM x BN] += A[BM x K] . B[K x BN],
// fp32 accumulate, operands staged through LDS with double buffering.
//
// Workgroup of WGM x WGN wave64s; each wave owns a (BM/WGM) x (BN/WGN)
// sub-tile made of 32 x 32 blocks computed with v_mfma_f32_32x32x16_bf16.
//
// LDS layout (per stage): A as BM rows x 8 chunks of 16 bytes (k contiguous),
// B transposed as BN rows x 8 chunks (k contiguous, one row per output
// column), both with the 16-byte chunk index XOR-swizzled by the row so that
// the MFMA operand reads (32 consecutive rows, one chunk) and the stores hit
// distinct banks.  B arrives K x N row-major from HBM and is transposed in
// registers: each thread loads an 8 x 8 block (8 rows of 16 bytes) and
// repacks it into 8 k-contiguous columns with byte permutes.
//
// MFMA operand layout (32x32x16): lane l holds A[row l%32][k 8*(l/32) .. +8]
// and B[k 8*(l/32) .. +8][col l%32]; accumulator register r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma once

#include "kos_device.h"

namespace kos {

template <int BM_, int BN_, int WGM_ = 2, int WGN_ = 2>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int NT = 64 * WGM * WGN;             // threads
  static constexpr int WM = BM / WGM, WN = BN / WGN;    // wave sub-tile
  static constexpr int TM = WM / 32, TN = WN / 32;      // 32x32 blocks per wave
  static constexpr int A_PER_T = BM * 8 / NT;           // A chunks per thread per stage
  static constexpr int B_PER_T = (BN + NT - 1) / NT;    // 8x8 B blocks per thread
  static constexpr int STAGE_CHUNKS = (BM + BN) * 8;    // 16-byte chunks per stage
  static constexpr int LDS_BYTES = 2 * STAGE_CHUNKS * 16;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave sub-tile sides are multiples of 32");
  static_assert(A_PER_T >= 1 && (BM * 8) % NT == 0, "A stage must spread evenly");
};

// Where the B tile's columns come from.  Plain: BN consecutive columns of
// one K x N matrix.  Dual (SwiGLU): tile columns in four segments of BN/4,
// [gate s0 | up s0 | gate s1 | up s1], so each wave's 32x32 blocks j and
// j + TN/2 hold the gate and up values of the same output column.
struct BSrc {
  const uint16_t* p0;   // B[0][n0] of the (gate) matrix
  const uint16_t* p1;   // B[0][n0] of the up matrix (dual only)
  int64_t ld;           // row stride of B, in elements
  int seg;              // BN/4 when dual, 0 when plain
  __device__ __forceinline__ const uint16_t* col8(int nb) const {
    const int c = nb * 8;
    if (seg == 0) return p0 + c;
    const int s = c / seg, w = c - s * seg;
    return ((s & 1) ? p1 : p0) + (s >> 1) * seg + w;
  }
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Packs 16-bit lanes: low halves (sel 0x05040100) or high halves (0x07060302)
// of lo_src and hi_src into one dword (lo_src's half in bits 0..15).
__device__ __forceinline__ uint32_t pack_lo(uint32_t lo_src, uint32_t hi_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_src, uint32_t hi_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}

template <class S>
struct TileRegs {
  uint4 a[S::A_PER_T];
  uint4 b[S::B_PER_T][8];
};

// Global -> registers for the stage starting at k0.
template <class S>
__device__ __forceinline__ void tile_gload(TileRegs<S>& r, const uint16_t* __restrict__ A, int64_t lda,
                                           int m_valid, const BSrc& b, int k0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < S::A_PER_T; ++i) {
    const int c = tid + i * S::NT;
    const int row = c >> 3, kc = c & 7;
    if (row < m_valid)
      r.a[i] = *reinterpret_cast<const uint4*>(A + row * lda + k0 + kc * 8);
    else
      r.a[i] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < S::B_PER_T; ++i) {
    const int blk = tid + i * S::NT;
    if (S::BN % S::NT == 0 || blk < S::BN) {
      const int kb = blk & 7, nb = blk >> 3;
      const uint16_t* src = b.col8(nb) + (int64_t)(k0 + kb * 8) * b.ld;
#pragma unroll
      for (int q = 0; q < 8; ++q) r.b[i][q] = *reinterpret_cast<const uint4*>(src + q * b.ld);
    }
  }
}

// Registers -> LDS stage (A as is, B transposed).
template <class S>
__device__ __forceinline__ void tile_lstore(const TileRegs<S>& r, uint4* __restrict__ stage) {
  const int tid = threadIdx.x;
  uint4* As = stage;
  uint4* Bs = stage + S::BM * 8;
#pragma unroll
  for (int i = 0; i < S::A_PER_T; ++i) {
    const int c = tid + i * S::NT;
    const int row = c >> 3, kc = c & 7;
    As[row * 8 + (kc ^ swz(row))] = r.a[i];
  }
#pragma unroll
  for (int i = 0; i < S::B_PER_T; ++i) {
    const int blk = tid + i * S::NT;
    if (S::BN % S::NT == 0 || blk < S::BN) {
      const int kb = blk & 7, nb = blk >> 3;
      const uint32_t* in = reinterpret_cast<const uint32_t*>(&r.b[i][0]);  // in[q*4 + d]
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        uint4 o;
        if ((j & 1) == 0) {
          o.x = pack_lo(in[0 * 4 + d], in[1 * 4 + d]);
          o.y = pack_lo(in[2 * 4 + d], in[3 * 4 + d]);
          o.z = pack_lo(in[4 * 4 + d], in[5 * 4 + d]);
          o.w = pack_lo(in[6 * 4 + d], in[7 * 4 + d]);
        } else {
          o.x = pack_hi(in[0 * 4 + d], in[1 * 4 + d]);
          o.y = pack_hi(in[2 * 4 + d], in[3 * 4 + d]);
          o.z = pack_hi(in[4 * 4 + d], in[5 * 4 + d]);
          o.w = pack_hi(in[6 * 4 + d], in[7 * 4 + d]);
        }
        const int n = nb * 8 + j;
        Bs[n * 8 + (kb ^ swz(n))] = o;
      }
    }
  }
}

// MFMAs over one LDS stage (BK = 64: four k16 steps).
template <class S>
__device__ __forceinline__ void tile_compute(f32x16 (&acc)[S::TM][S::TN], const uint4* __restrict__ stage) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const uint4* As = stage;
  const uint4* Bs = stage + S::BM * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kc = 2 * s + (lane >> 5);
    bf16x8 af[S::TM], bfr[S::TN];
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int row = wm * S::WM + i * 32 + (lane & 31);
      af[i] = __builtin_bit_cast(bf16x8, As[row * 8 + (kc ^ swz(row))]);
    }
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      const int n = wn * S::WN + j * 32 + (lane & 31);
      bfr[j] = __builtin_bit_cast(bf16x8, Bs[n * 8 + (kc ^ swz(n))]);
    }
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

// Full K loop: acc = A[0:m_valid rows] . B over k in [0, K).  Rows >= m_valid
// read as zero.  `lds` holds two stages.  Begins and ends with the LDS free.
template <class S>
__device__ __forceinline__ void tile_mainloop(f32x16 (&acc)[S::TM][S::TN], const uint16_t* __restrict__ A,
                                              int64_t lda, int m_valid, const BSrc& b, int K,
                                              uint4* __restrict__ lds) {
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / S::BK;
  TileRegs<S> regs;
  tile_gload<S>(regs, A, lda, m_valid, b, 0);
  __syncthreads();  // LDS free from the previous user
  tile_lstore<S>(regs, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint4* cur = lds + (kt & 1) * S::STAGE_CHUNKS;
    uint4* nxt = lds + ((kt + 1) & 1) * S::STAGE_CHUNKS;
    const bool more = kt + 1 < nk;
    if (more) tile_gload<S>(regs, A, lda, m_valid, b, (kt + 1) * S::BK);
    tile_compute<S>(acc, cur);
    if (more) tile_lstore<S>(regs, nxt);
    __syncthreads();
  }
}

// Visits every accumulator element with its tile-relative (row, col).
template <class S, class F>
__device__ __forceinline__ void tile_foreach(const f32x16 (&acc)[S::TM][S::TN], F&& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * S::WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * S::WN + j * 32 + (lane & 31);
        f(row, col, acc[i][j][r]);
      }
}

}  // namespace kos
