// Expert layer, combine-direction pieces shared by the combine kernel and
// the single-launch expert layer: work units, the grouped SwiGLU tiles, the
// pushes and the fold (see kos_moe_combine.hip for the queues they run
// under).
#pragma once

#include "kos_moe.h"
#include "kos_order.h"
#include "kos_tile.h"

namespace kos {

constexpr int kFoldTokens = 8;
constexpr int kPushRows = 64;

struct CombineParams {
  int32_t world, rank, T, H, E, k, F, E_loc;
  const uint16_t* xg;
  const int32_t* go_in;
  const int32_t* row_src;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* wd;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* counts;
  const int32_t* perm;
  const int32_t* peer_counts;
  const uint16_t* peer_return[8];
  uint16_t* h;
  uint16_t* g_save;       // optional [cap, F] bf16: X.Wg and X.Wu as computed (for a backward pass)
  uint16_t* u_save;
  uint16_t* yg;
  uint16_t* out_return[8];
  int64_t return_cap[8];  // rows out_return[p] holds
  uint16_t* y;
  int32_t G, D, L;        // gate/up tiles per unit, down tiles per unit, lag (units)
  int32_t u_max;          // bound on units: size of each counter array
  int32_t grouped_cap;    // rows x_grouped, h and y_grouped hold
  int32_t do_gu, do_dn, do_push, do_fold;
  int32_t two_way;        // builders take ready pushes between tiles
  int32_t n_crew;         // > 0: tickets below it only push and fold
  int32_t wait_flags;
  uint32_t spin_limit;
  WsHeader* ws;
  uint32_t* ctr;          // gu_done[u_max], then dn_done[u_max]
  kos_trace_rec* trace;   // null: tracing off
};

struct CombineMeta {
  int32_t go[kMoeMaxLocal + 1];     // grouped offsets
  int32_t ub[kMoeMaxLocal + 1];     // first unit of each local expert
  int32_t before[kMoeMaxLocal];     // grouped rows of sources < rank, per local expert
  int32_t off[kMoeMaxExperts + 1];  // our packed offsets
  int32_t recv[8];                  // rows each rank sent us
  int32_t wave_tot[16];             // scan scratch
};

// Every workgroup's copy of the layer's bookkeeping, in LDS: grouped offsets,
// units per expert, our packed offsets (a block scan of the counts) and the
// rows of lower ranks per expert.  Also checks that every peer buffer that
// would be read or written is non-NULL: returns false (every thread) and
// records KOS_ERR_ARG otherwise.
template <int BM>
__device__ __forceinline__ bool load_combine_meta(const CombineParams& p, CombineMeta& M, WgSlots* s) {
  for (int el = threadIdx.x; el <= p.E_loc; el += blockDim.x) M.go[el] = p.go_in[el];
  for (int el = threadIdx.x; el < p.E_loc; el += blockDim.x) {
    int run = 0;
    for (int q = 0; q < p.rank; ++q) run += p.peer_counts[q * p.E_loc + el];
    M.before[el] = run;
  }
  if (threadIdx.x < 8) M.recv[threadIdx.x] = 0;
  if (threadIdx.x == 0) s->ok = 1;
  block_exclusive_scan(p.counts, M.off, p.E, M.wave_tot);
  for (int i = threadIdx.x; i < p.world * p.E_loc; i += blockDim.x)
    if (p.peer_counts[i] != 0) atomicAdd(&M.recv[i / p.E_loc], p.peer_counts[i]);   // rows each rank sent us
  if (threadIdx.x == 0) {
    // offsets that decrease or run past the caller's capacity would make
    // units overlap the counters and tiles write past h / y_grouped
    bool bad = M.go[0] < 0 || M.go[p.E_loc] > p.grouped_cap;
    M.ub[0] = 0;
    for (int el = 0; el < p.E_loc; ++el) {
      const int n = M.go[el + 1] - M.go[el];
      bad |= n < 0;
      M.ub[el + 1] = M.ub[el] + (n > 0 ? (n + BM - 1) / BM : 0);
    }
    if (bad) {
      raise_error(p.ws, KOS_ERR_CAPACITY, (uint32_t)M.go[p.E_loc]);
      s->ok = 0;
    }
  }
  __syncthreads();
  const int q = threadIdx.x;
  if (q < p.world && q != p.rank) {
    const int sent = M.off[(q + 1) * p.E_loc] - M.off[q * p.E_loc];   // results q returns
    if ((sent > 0 && p.peer_return[q] == nullptr) || (M.recv[q] > 0 && p.out_return[q] == nullptr)) s->ok = 0;
    if (M.recv[q] > p.return_cap[q]) {   // the results p sent us do not fit its return buffer
      raise_error(p.ws, KOS_ERR_CAPACITY, 0x00F00000u | (uint32_t)q);
      s->ok = 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && !s->ok) raise_error(p.ws, KOS_ERR_ARG, 0x00C00000u);   // no-op after a capacity error
  return s->ok != 0;
}

struct Unit {
  int el, rb, row0, m_valid;
};

template <int BM>
__device__ __forceinline__ Unit unit_of(const CombineMeta& M, int E_loc, int u) {
  int el = 0;
  while (el + 1 < E_loc && M.ub[el + 1] <= u) ++el;
  Unit x;
  x.el = el;
  x.rb = u - M.ub[el];
  x.row0 = M.go[el] + x.rb * BM;
  const int n = M.go[el + 1] - M.go[el];
  x.m_valid = min(BM, n - x.rb * BM);
  return x;
}

// Tile entry j of the queue -> (is_down, unit, column tile): the lagged
// consumer order of combine_tile_of.
__device__ __forceinline__ void decode_tile(const CombineParams& p, int U, int j, bool& down, int& u, int& nt) {
  const CombineTile t = combine_tile_of(j, U, p.G, p.D, p.L, p.do_gu != 0, p.do_dn != 0);
  down = t.down;
  u = t.u;
  nt = t.nt;
}

// COH_X: the grouped input rows were written by this launch (the
// single-launch layer's movers): read device-coherent.  SAVE: g and u are
// also stored when p.g_save is set (false: never; the code is left out).
template <class S, int RING, bool COH_X = false, bool SAVE = true>
__device__ __forceinline__ void gate_up_tile(const CombineParams& p, const Unit& x, int nt, f32x16 (&acc)[S::TM][S::TN]) {
  constexpr int HN = S::BN / 2;    // h columns per tile
  const int64_t H = p.H, F = p.F;
  BSrc b{p.wg + (int64_t)x.el * H * F + (int64_t)nt * HN, p.wu + (int64_t)x.el * H * F + (int64_t)nt * HN, F};
  tile_mainloop<S, true, COH_X, RING>(acc, p.xg + (int64_t)x.row0 * H, H, x.m_valid, b, p.H);
  // read by this launch's down tiles: device-coherent stores
  tile_store_rows<S, RING, true, true>(acc, p.h + (int64_t)x.row0 * F + (int64_t)nt * HN, F, x.m_valid);
  if (SAVE && p.g_save) {   // the activations a backward pass reads instead of recomputing them
    KOS_WAITCNT(0, 0);
    lds_barrier();   // every wave has read the h tile out of the ring
    const int64_t off = (int64_t)x.row0 * F + (int64_t)nt * HN;
    tile_store_rows_pair<S, RING, false>(acc, p.g_save + off, p.u_save + off, F, x.m_valid);
  }
}

// COH: h was written by this launch's gate/up tiles (read device-coherent).
template <class S, bool COH, int RING>
__device__ __forceinline__ void down_tile(const CombineParams& p, const Unit& x, int nt, f32x16 (&acc)[S::TM][S::TN]) {
  const int64_t H = p.H, F = p.F;
  BSrc b{p.wd + (int64_t)x.el * F * H + (int64_t)nt * S::BN, nullptr, H};
  tile_mainloop<S, false, COH, RING>(acc, p.h + (int64_t)x.row0 * F, F, x.m_valid, b, p.F);
  // read by pushes and folds of this launch: device-coherent stores
  tile_store_rows<S, RING, true>(acc, p.yg + (int64_t)x.row0 * H + (int64_t)nt * S::BN, H, x.m_valid);
}

// Push entry: rows [slab * kPushRows, +kPushRows) of unit x, one row per
// wave at a time.  COH: the provenance was written by this launch.
template <bool COH = false>
__device__ __forceinline__ void push_slab(const CombineParams& p, const CombineMeta& M, const Unit& x, int slab) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const DevBuf yb(p.yg);
  const int r1 = min(x.m_valid, (slab + 1) * kPushRows);
  for (int r = slab * kPushRows + wave; r < r1; r += nw) {
    const int64_t grow = (int64_t)x.row0 + r;
    const int src = COH ? (int)ld_dev_b32(&p.row_src[grow * 2]) : p.row_src[grow * 2];
    if (src == p.rank) continue;
    const int64_t i = COH ? (int)ld_dev_b32(&p.row_src[grow * 2 + 1]) : p.row_src[grow * 2 + 1];
    // a row must go back to a rank that sent rows, inside what it sent
    if (src < 0 || src >= p.world || i < 0 || i >= M.recv[src]) {
      if ((threadIdx.x & 63) == 0) raise_error(p.ws, KOS_ERR_ARG, 0x00D00000u | (uint32_t)(grow & 0xFFFFF));
      continue;
    }
    wave_copy_row_dev_src(wave_uniform(p.out_return[src] + i * p.H), yb, (uint32_t)(grow * p.H * 2), p.H * 2);
  }
}

// y row of one token = bf16(sum_j w[j] * res_j), fp32, j ascending.  row[j]
// is a scalar descriptor of result j's row (device-coherent loads: local
// rows come from this launch).  KN results (KN == k, or KMAX with the
// weights of j >= k zero and their rows repeating row 0); CB column chunks
// per lane per pass, all CB x KN loads issued unconditionally (tail lanes
// re-read the last chunk) before any use.
template <int KN, int CB>
__device__ __forceinline__ void fold_token(int H, const DevBuf (&row)[KN], const float (&w)[KN], uint16_t* yrow,
                                           int lane) {
  const int nc = H / 8;
  for (int c0 = lane; c0 < nc; c0 += 64 * CB) {
    u32x4 v[CB][KN];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = min(c0 + 64 * u, nc - 1);
#pragma unroll
      for (int j = 0; j < KN; ++j) v[u][j] = row[j].ld128((uint32_t)c * 16u);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = c0 + 64 * u;
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KN; ++j) {
        const uint32_t q[4] = {v[u][j].x, v[u][j].y, v[u][j].z, v[u][j].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          a[2 * m] += w[j] * __builtin_bit_cast(float, q[m] << 16);
          a[2 * m + 1] += w[j] * __builtin_bit_cast(float, q[m] & 0xFFFF0000u);
        }
      }
      u32x4 o;
      o.x = (uint32_t)f32_to_bf16_bits(a[0]) | ((uint32_t)f32_to_bf16_bits(a[1]) << 16);
      o.y = (uint32_t)f32_to_bf16_bits(a[2]) | ((uint32_t)f32_to_bf16_bits(a[3]) << 16);
      o.z = (uint32_t)f32_to_bf16_bits(a[4]) | ((uint32_t)f32_to_bf16_bits(a[5]) << 16);
      o.w = (uint32_t)f32_to_bf16_bits(a[6]) | ((uint32_t)f32_to_bf16_bits(a[7]) << 16);
      if (c < nc) reinterpret_cast<u32x4*>(yrow)[c] = o;
    }
  }
}

// Broadcasts lane j's result row and weight as scalars, then folds.
template <int KN, int CB>
__device__ __forceinline__ void fold_token_rows(int H, int k, uint64_t rowp, float wj, uint16_t* yrow, int lane) {
  const uint64_t row0 = readlane_u64(rowp, 0);
  DevBuf row[KN] = {};
  float w[KN];
#pragma unroll
  for (int j = 0; j < KN; ++j) {
    const uint64_t rj = readlane_u64(rowp, j);
    const float wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, wj), j));
    row[j] = DevBuf(reinterpret_cast<const void*>(j < k ? rj : row0));
    w[j] = j < k ? wv : 0.f;
  }
  fold_token<KN, CB>(H, row, w, yrow, lane);
}

// Folds token t with one wave.  Lane j < k resolves result j (local: a
// row of yg, gated on its unit's down tiles when flagged; remote: the row
// its rank returned); the choices are then broadcast as scalars.  Returns
// false (wave-uniform) on abort or time-out.  COH: the routing was written
// by this launch (read device-coherent).
template <int BM, bool COH = false>
__device__ __forceinline__ bool fold_token_wave(const CombineParams& p, const CombineMeta& M, int t, uint32_t info) {
  const int lane = threadIdx.x & 63;
  const int E_loc = p.E_loc;
  bool local = false;
  int u = 0;
  uint64_t rowp = 0;   // result row of lane j < k
  float wj = 0.f;
  const int k = p.k;
  bool bad = false;   // routing that points outside the rows it may name
  if (lane < k) {
    const int64_t o = (int64_t)t * k + lane;
    const int e = COH ? (int)ld_dev_b32(&p.topk_idx[o]) : p.topk_idx[o];
    const int pos = COH ? (int)ld_dev_b32(&p.perm[o]) : p.perm[o];
    wj = COH ? __builtin_bit_cast(float, ld_dev_b32(&p.topk_w[o])) : p.topk_w[o];
    bad = e < 0 || e >= p.E || pos < M.off[e] || pos >= M.off[e + 1];
    const int d = bad ? p.rank : e / E_loc;
    if (bad) {
    } else if (d == p.rank) {
      const int el = e - p.rank * E_loc;
      const int grow = M.go[el] + M.before[el] + (pos - M.off[e]);
      bad = grow >= M.go[el + 1];
      local = true;
      u = M.ub[el] + (grow - M.go[el]) / BM;
      rowp = reinterpret_cast<uint64_t>(p.yg + (int64_t)grow * p.H);
    } else {
      rowp = reinterpret_cast<uint64_t>(p.peer_return[d] + (int64_t)(pos - M.off[d * E_loc]) * p.H);
    }
  }
  if (__any(bad)) {
    if (lane == 0) raise_error(p.ws, KOS_ERR_ARG, 0x00E00000u | (uint32_t)(t & 0xFFFFF));
    return false;
  }
  if (p.wait_flags) {
    const uint32_t* dn_done = p.ctr + p.u_max;
    uint32_t it = 0;
    for (;;) {
      const bool ready = !local || ld_relaxed(&dn_done[u]) >= (uint32_t)p.D;
      if (__all(ready)) break;
      if (aborted(p.ws)) return false;
      if (++it >= p.spin_limit) {
        if (lane == 0) raise_error(p.ws, KOS_ERR_TIMEOUT, info);
        return false;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  uint16_t* yrow = p.y + (int64_t)t * p.H;
  const int ks = __builtin_amdgcn_readfirstlane(k);
  if (ks == 8)
    fold_token_rows<8, 4>(p.H, ks, rowp, wj, yrow, lane);
  else if (ks < 8)
    fold_token_rows<8, 2>(p.H, ks, rowp, wj, yrow, lane);
  else
    fold_token_rows<kMoeMaxTopk, 1>(p.H, ks, rowp, wj, yrow, lane);
  return true;
}

template <int BM, bool COH = false>
__device__ __forceinline__ bool fold_block(const CombineParams& p, const CombineMeta& M, int fb, WgSlots* s) {
  const int t0 = fb * kFoldTokens;
  const int t1 = min(p.T, t0 + kFoldTokens);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (threadIdx.x == 0) s->ok = 1;
  __syncthreads();
  for (int t = t0 + wave; t < t1; t += nw)
    if (!fold_token_wave<BM, COH>(p, M, t, 0x40000000u | (uint32_t)fb)) {
      if ((threadIdx.x & 63) == 0) s->ok = 0;
      break;
    }
  __syncthreads();
  return s->ok != 0;
}

// Big tile when the widths allow it (hidden % 256, ffn % 128), else 128 x 128.
// The big tiles run eight waves (two per SIMD), which hides more of the LDS
// and memory latency on these long (gate/up) and short (down) K loops.
using CombineTileBig = TileShape<256, 256, 4, 2, 4>;
using CombineTailBig = TileShape<128, 256, 4, 2, 4>;
using CombineTail2Big = TileShape<64, 256, 4, 2, 4>;
using CombineTileSmall = TileShape<128, 128>;
using CombineTailSmall = TileShape<64, 128>;

}  // namespace kos
