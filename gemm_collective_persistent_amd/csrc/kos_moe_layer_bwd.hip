// The whole expert layer, backward direction, as ONE persistent kernel: the
// pairs' output gradients dispatched like the tokens, the experts' data
// gradient (recomputing the SwiGLU activations), the results pushed back,
// and the per-token sum with the router gradient [KOSMOS arXiv abstract:
// the expert layer runs in one launch per direction; KOSMOS explainer,
// "KOSMOS removes the manager": workgroups take the next entry of queues
// laid out in the order consumers need it, and switch both ways between
// sending results back and building tiles].
//
// The pages give no backward formulas: this is the chain rule of the
// forward, y[t] = sum_j w[t,j] * res[t,j], res = bf16(h . Wd),
// h = bf16(silu(X.Wg) * (X.Wu)).
//
// Work units: (local expert, block of 256 grouped rows), expert-major, as
// in the forward's combine.  Queues, taken in this order by every
// workgroup:
//   head[0]  movers: blocks of 8 of our tokens (one per wave) -- each
//            pair's gradient bf16(w * dy) goes to the grouped gradient
//            rows (our experts) or to the send buffer of the expert's rank;
//            then 16-row chunks of the gradients each peer sent us, pulled
//            into the grouped gradient rows.  Each grouped row stored bumps
//            rows_in[its unit].
//   head[1]  tiles in the lagged consumer order of the combine: a unit's
//            first-stage entries (FB = 256, or 128, columns of F each:
//            dH = dres . Wd^T, kept in fp32 in the caller's dH buffer and
//            read back by the same workgroup; then per 128 of those columns
//            g and u recomputed in the SwiGLU tile, whose epilogue forms
//            dG and dU) wait for rows_in, its second-stage tiles (256
//            columns of H: dX = dG . Wg^T + dU . Wu^T, one split-K loop)
//            for the unit's first-stage entries.  Between tiles a
//            workgroup takes the push queue's head if it is ready.  When
//            the forward kept g and u (bf16), a first-stage entry is the dH
//            tile alone, its epilogue reading them (no recomputation).
//   head[2]  pushes: dX rows of rows a peer sent us, back to it.
//   head[3]  fold: per token, dx = bf16(sum of its pairs' dX) and the
//            router gradient through the softmax over the selected logits.
// Every wait is on work earlier in the queue order, already claimed by a
// running workgroup (all are resident, one per compute unit), so none is
// circular.
#include "kos_host.h"
#include "kos_moe_combine.h"

namespace kos {

constexpr int kBwdUnit = 256;      // grouped rows per unit
constexpr int kBwdFCols = 128;     // F columns of a SwiGLU recompute tile
constexpr int kBwdHCols = 256;     // H columns of a second-stage tile
constexpr int kBwdMoveTokens = 8;  // our tokens per mover entry (one per wave)
constexpr int kBwdMoveRows = 16;   // peer rows per mover entry

struct BwdParams {
  // Shared fields as in the combine: world .. E_loc, xg (the forward's
  // grouped input), go_in, row_src, wg, wu, wd, topk_idx, topk_w, counts,
  // perm, peer_counts; peer_return = the dX rows peers return for our
  // pairs, out_return / return_cap = the dX rows we return; yg = the
  // grouped dX; y = dx; G, D, L, u_max, grouped_cap; ctr = t1_done[u_max],
  // t2_done[u_max].
  CombineParams c;
  const uint16_t* dy;
  const uint16_t* y_fwd;                // the forward's grouped results
  const uint16_t* peer_return_fwd[8];   // the forward's results from the peers
  const uint16_t* peer_send_grad[8];
  uint16_t* out_send_grad[8];
  int64_t send_cap[8];
  uint16_t* dres;                       // grouped pair gradients [cap, H]
  uint16_t* dg;                         // [cap, F]
  uint16_t* du;                         // [cap, F]
  float* dh;                            // [cap, F] fp32 (optional with g_in)
  const uint16_t* g_in;                 // optional [cap, F] bf16: the forward's X.Wg and X.Wu
  const uint16_t* u_in;
  float* dlogits;                       // [T, E]
  uint32_t* rows_in;                    // [u_max]; the counters start here
  uint32_t n_counters;                  // 3 * u_max
};

struct BwdLds {
  int32_t cum[8][kMoeMaxLocal + 1];     // rows source q sent us, prefix over local experts
  int32_t before[8][kMoeMaxLocal];      // grouped rows of sources < q, per local expert
  int32_t chunk_base[9];                // first mover entry of each source's rows
};

// The layer's bookkeeping in LDS (the combine's, plus each source's row
// ranges) and the argument checks every workgroup makes alike.  Returns
// false (every thread) after recording an error.
__device__ inline bool bwd_meta(const BwdParams& b, CombineMeta& M, BwdLds& B, WgSlots* s) {
  const CombineParams& p = b.c;
  if (!load_combine_meta<kBwdUnit>(p, M, s)) return false;
  for (int el = threadIdx.x; el < p.E_loc; el += blockDim.x) {
    int run = 0;
    for (int q = 0; q < p.world; ++q) {
      B.before[q][el] = run;
      run += q == p.rank ? p.counts[p.rank * p.E_loc + el] : p.peer_counts[q * p.E_loc + el];
    }
    if (run != M.go[el + 1] - M.go[el]) {   // grouped offsets that do not match the rows that arrive
      raise_error(p.ws, KOS_ERR_ARG, 0x00B00000u | (uint32_t)el);
      s->ok = 0;
    }
  }
  if (threadIdx.x < (unsigned)p.world) {
    const int q = threadIdx.x;
    B.cum[q][0] = 0;
    for (int el = 0; el < p.E_loc; ++el)
      B.cum[q][el + 1] = B.cum[q][el] + (q == p.rank ? 0 : p.peer_counts[q * p.E_loc + el]);
    if (q != p.rank) {
      const int sent = M.off[(q + 1) * p.E_loc] - M.off[q * p.E_loc];
      if (sent > 0 && (b.peer_return_fwd[q] == nullptr || b.out_send_grad[q] == nullptr)) {
        raise_error(p.ws, KOS_ERR_ARG, 0x00B10000u | (uint32_t)q);
        s->ok = 0;
      }
      if (sent > b.send_cap[q]) {
        raise_error(p.ws, KOS_ERR_CAPACITY, 0x00B20000u | (uint32_t)q);
        s->ok = 0;
      }
      if (M.recv[q] > 0 && b.peer_send_grad[q] == nullptr) {
        raise_error(p.ws, KOS_ERR_ARG, 0x00B30000u | (uint32_t)q);
        s->ok = 0;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    B.chunk_base[0] = (p.T + kBwdMoveTokens - 1) / kBwdMoveTokens;
    for (int q = 0; q < p.world; ++q)
      B.chunk_base[q + 1] = B.chunk_base[q] + (B.cum[q][p.E_loc] + kBwdMoveRows - 1) / kBwdMoveRows;
  }
  __syncthreads();
  return s->ok != 0;
}

// Eight bf16 values times w, rounded back to bf16 (fp32 product).
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float w) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
  uint32_t r[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float lo = __builtin_bit_cast(float, q[m] << 16) * w;
    const float hi = __builtin_bit_cast(float, q[m] & 0xFFFF0000u) * w;
    r[m] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

// One of our tokens, one wave: lane j < k resolves pair j's destination,
// then the wave scales dy's row by each pair's weight and stores it there.
// Returns false (wave-uniform) on routing that names rows outside the
// forward's.
__device__ __forceinline__ bool bwd_move_token(const BwdParams& b, const CombineMeta& M, int t) {
  const CombineParams& p = b.c;
  const int lane = threadIdx.x & 63;
  const int k = p.k;
  uint64_t dstp = 0;
  float wj = 0.f;
  int unit = -1;
  bool bad = false;
  if (lane < k) {
    const int64_t o = (int64_t)t * k + lane;
    const int e = p.topk_idx[o];
    const int pos = p.perm[o];
    wj = p.topk_w[o];
    bad = e < 0 || e >= p.E || pos < M.off[e] || pos >= M.off[e + 1];
    if (!bad) {
      const int d = e / p.E_loc;
      if (d == p.rank) {
        const int el = e - p.rank * p.E_loc;
        const int grow = M.go[el] + M.before[el] + (pos - M.off[e]);
        bad = grow >= M.go[el + 1];
        unit = M.ub[el] + (grow - M.go[el]) / kBwdUnit;
        dstp = reinterpret_cast<uint64_t>(b.dres + (int64_t)grow * p.H);
      } else {
        const int64_t r = pos - M.off[d * p.E_loc];   // below the rows sent to d, which fit send_cap[d]
        dstp = reinterpret_cast<uint64_t>(b.out_send_grad[d] + r * p.H);
      }
    }
  }
  if (__any(bad)) {
    if (lane == 0) raise_error(p.ws, KOS_ERR_ARG, 0x00B40000u | (uint32_t)(t & 0xFFFF));
    return false;
  }
  const int nc = p.H / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(b.dy + (int64_t)t * p.H);
  constexpr int U = 16;
  for (int c0 = lane; c0 < nc; c0 += U * 64) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * 64 < nc) v[u] = src[c0 + u * 64];
    for (int j = 0; j < k; ++j) {
      const DevBuf db(reinterpret_cast<const void*>(readlane_u64(dstp, j)));
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, wj), j));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u * 64 < nc) db.st128((uint32_t)(c0 + u * 64) * 16u, scale_bf16x8(v[u], w));
    }
  }
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0): the rows have landed
  if (unit >= 0) add_relaxed(&b.rows_in[unit], 1u);
  return true;
}

// Mover entry past our tokens: a chunk of kBwdMoveRows gradient rows peer q
// sent us, one row per wave at a time, into the grouped gradient rows.
__device__ __forceinline__ void bwd_move_peer(const BwdParams& b, const CombineMeta& M, const BwdLds& B, int i) {
  const CombineParams& p = b.c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int q = 0;
  while (q + 1 <= p.world && B.chunk_base[q + 1] <= i) ++q;
  const int r0 = (i - B.chunk_base[q]) * kBwdMoveRows;
  const int n_q = B.cum[q][p.E_loc];
  for (int rr = wave; rr < kBwdMoveRows; rr += nw) {
    const int r = r0 + rr;
    if (r >= n_q) break;
    int el = 0;
    while (el + 1 < p.E_loc && B.cum[q][el + 1] <= r) ++el;
    const int64_t grow = (int64_t)M.go[el] + B.before[q][el] + (r - B.cum[q][el]);
    wave_copy_row_dev_dst(b.dres + grow * p.H, b.peer_send_grad[q] + (int64_t)r * p.H, p.H * 2);
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
    if (lane == 0) add_relaxed(&b.rows_in[M.ub[el] + ((int)grow - M.go[el]) / kBwdUnit], 1u);
  }
}

// First-stage entry: F columns [blk*FB, +FB) of unit x.  SH: the dH tile
// (N x K weights: Wd rows); SD: the SwiGLU-layout tile (gate and up blocks
// of the same 128 columns), whose epilogue reads dH back.
template <class SH, class SD, int RING, int FB>
__device__ __forceinline__ void bwd_stage1(const BwdParams& b, const Unit& x, int blk, f32x16 (&ah)[SH::TM][SH::TN],
                                           f32x16 (&ad)[SD::TM][SD::TN]) {
  static_assert(SH::BNT && !SD::BNT && SH::BM == SD::BM && SH::BN == FB && SD::BN == 2 * kBwdFCols &&
                    FB % kBwdFCols == 0,
                "dH tile of FB columns, SwiGLU tiles of 128");
  const CombineParams& p = b.c;
  const int64_t H = p.H, F = p.F;
  const int64_t row0 = x.row0;
  const int m = x.m_valid;
  const int64_t woff = (int64_t)x.el * H * F;
  // dH = dres . Wd^T; the gradient rows come from this launch's movers
  tile_mainloop<SH, false, true, RING>(ah, b.dres + row0 * H, H, m, BSrc{p.wd + woff + (int64_t)blk * FB * H, nullptr, H},
                                       p.H);
  float* dhp = b.dh + row0 * F + (int64_t)blk * FB;
  const DevBuf db(dhp);
  tile_foreach4<SH>(ah, [&](int r, int c, f32x4 v) {
    if (r < m) db.st128((uint32_t)(r * F + c) * 4u, __builtin_bit_cast(u32x4, v));
  });
  KOS_WAITCNT(0, 0);
  lds_barrier();   // the whole dH block is stored before any wave reads it back
#pragma unroll 1
  for (int hf = 0; hf < FB / kBwdFCols; ++hf) {
    const int64_t c0 = (int64_t)blk * FB + hf * kBwdFCols;
    // g and u of the forward, recomputed (the grouped input is resident)
    tile_mainloop<SD, true, false, RING>(ad, p.xg + row0 * H, H, m, BSrc{p.wg + woff + c0, p.wu + woff + c0, F}, p.H);
    // dU = dH * silu(g), dG = dH * u * silu'(g), silu'(g) = s (1 + g (1 - s)),
    // s = 1 / (1 + e^-g); in place of g and u.  Lane l holds, in block
    // (i, j) of the gate half, rows wm*WM + i*32 + l%32 and four columns
    // from wn*WN/2 + j*32 + 8*q + 4*(l/32) per group q.
    {
      const WaveCtx w = wave_ctx();
      const int wm = w.wave / SD::WGN, wn = w.wave % SD::WGN;
#pragma unroll
      for (int i = 0; i < SD::TM; ++i) {
        const int row = wm * SD::WM + i * 32 + (w.lane & 31);
        const int rr = row < m ? row : m - 1;   // rows past the unit are computed, never stored
#pragma unroll
        for (int j = 0; j < SD::TN / 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * (SD::WN / 2) + j * 32 + q * 8 + (w.lane >> 5) * 4;
            const f32x4 d = __builtin_bit_cast(f32x4, db.ld128((uint32_t)(rr * F + hf * kBwdFCols + col) * 4u));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float g = ad[i][j][4 * q + e], u = ad[i][j + SD::TN / 2][4 * q + e];
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
              ad[i][j][4 * q + e] = d[e] * u * (sg * (1.0f + g * (1.0f - sg)));
              ad[i][j + SD::TN / 2][4 * q + e] = d[e] * (g * sg);
            }
            // one group at a time: keeps the loads of later groups from
            // being hoisted here (each would hold four more registers)
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    }
    // read by this launch's second-stage tiles: device-coherent stores
    tile_store_rows_pair<SD, RING, true>(ad, b.dg + row0 * F + c0, b.du + row0 * F + c0, F, m);
  }
}

// First-stage entry with the forward's g and u at hand (bf16, as the
// forward's tiles kept them): F columns [blk*FB, +FB) of unit x,
// dH = dres . Wd^T in registers (stored to dh when given), then dU and dG
// from the saved g and u, each through the LDS ring in a pass of its own
// (dH stays in the accumulators; the second pass reads g and u again, from
// the cache).
template <class SH, int RING, int FB>
__device__ __forceinline__ void bwd_stage1_saved(const BwdParams& b, const Unit& x, int blk,
                                                 f32x16 (&ah)[SH::TM][SH::TN]) {
  static_assert(SH::BNT && SH::BN == FB, "dH tile of FB columns (N x K weights: Wd rows)");
  const CombineParams& p = b.c;
  const int64_t H = p.H, F = p.F;
  const int64_t row0 = x.row0;
  const int m = x.m_valid;
  const int64_t c0 = (int64_t)blk * FB;
  const int64_t woff = (int64_t)x.el * H * F;
  tile_mainloop<SH, false, true, RING>(ah, b.dres + row0 * H, H, m, BSrc{p.wd + woff + c0 * H, nullptr, H}, p.H);
  if (b.dh) {
    float* dhp = b.dh + row0 * F + c0;
    tile_foreach4<SH>(ah, [&](int r, int c, f32x4 v) {
      if (r < m) *reinterpret_cast<f32x4*>(dhp + r * F + c) = v;
    });
  }
  const WaveCtx w = wave_ctx();
  const int wm = w.wave / SH::WGN, wn = w.wave % SH::WGN;
  const uint16_t* gp = b.g_in + row0 * F + c0;
  const uint16_t* up = b.u_in + row0 * F + c0;
  // the lane's g and u pieces of one 32-row block of the tile, loaded
  // together when the block's first group is reached (one wait per block)
  u32x2 gs[SH::TN][4], us[SH::TN][4];
  auto load_block = [&](int i, bool with_u) {
    const int row = wm * SH::WM + i * 32 + (w.lane & 31);
    const int64_t rr = row < m ? row : m - 1;   // rows past the unit are computed, never stored
#pragma unroll
    for (int j = 0; j < SH::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * SH::WN + j * 32 + q * 8 + (w.lane >> 5) * 4;
        gs[j][q] = *reinterpret_cast<const u32x2*>(gp + rr * F + col);
        if (with_u) us[j][q] = *reinterpret_cast<const u32x2*>(up + rr * F + col);
      }
  };
  auto unpack = [](u32x2 v, float (&f)[4]) {
    f[0] = __builtin_bit_cast(float, v.x << 16);
    f[1] = __builtin_bit_cast(float, v.x & 0xFFFF0000u);
    f[2] = __builtin_bit_cast(float, v.y << 16);
    f[3] = __builtin_bit_cast(float, v.y & 0xFFFF0000u);
  };
  // dU = dH * silu(g), silu(g) = g s, s = 1 / (1 + e^-g)
  tile_store_rows_fn<SH, RING, true, FB>(b.du + row0 * F + c0, F, m, [&](int i, int j, int q) {
    if (j == 0 && q == 0) load_block(i, false);
    float g[4];
    unpack(gs[j][q], g);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ah[i][j][4 * q + e] * (g[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e])));
    return v;
  });
  KOS_WAITCNT(0, 0);
  lds_barrier();   // every wave has read dU out of the ring
  // dG = dH * u * silu'(g), silu'(g) = s (1 + g (1 - s))
  tile_store_rows_fn<SH, RING, true, FB>(b.dg + row0 * F + c0, F, m, [&](int i, int j, int q) {
    if (j == 0 && q == 0) load_block(i, true);
    float g[4], u[4];
    unpack(gs[j][q], g);
    unpack(us[j][q], u);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[e]));
      v[e] = ah[i][j][4 * q + e] * u[e] * (sg * (1.0f + g[e] * (1.0f - sg)));
    }
    return v;
  });
}

// Second-stage tile: H columns [nh*256, +256) of unit x's dX.
template <class S, int RING>
__device__ __forceinline__ void bwd_tile2(const BwdParams& b, const Unit& x, int nh, f32x16 (&acc)[S::TM][S::TN]) {
  static_assert(S::BNT && S::BN == kBwdHCols, "dX tile reads N x K weights (Wg, Wu rows)");
  const CombineParams& p = b.c;
  const int64_t H = p.H, F = p.F;
  const int64_t woff = (int64_t)x.el * H * F + (int64_t)nh * kBwdHCols * F;
  // one K loop over [dG | dU] . [Wg^T ; Wu^T]
  tile_mainloop<S, false, true, RING, true>(acc, b.dg + (int64_t)x.row0 * F, F, x.m_valid, BSrc{p.wg + woff, nullptr, F},
                                            2 * p.F, b.du + (int64_t)x.row0 * F, p.wu + woff, p.F);
  // read by pushes and the fold of this launch
  tile_store_rows<S, RING, true>(acc, p.yg + (int64_t)x.row0 * H + nh * kBwdHCols, H, x.m_valid);
}

// dw[j] = <dy row, res row j> for j < k, fp32, in every lane.  resp: lane
// j's result row (bf16).  Eight rows at a time (the row chunks of one pass
// stay in registers).
template <int KN>
__device__ __forceinline__ void pair_dots(int H, int k, uint64_t resp, const uint16_t* dyrow, int lane,
                                          float (&dw)[KN]) {
  static_assert(KN % 8 == 0, "groups of eight rows");
  const u32x4* dyv = reinterpret_cast<const u32x4*>(dyrow);
  const int nc = H / 8;
#pragma unroll
  for (int g = 0; g < KN; g += 8) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) dw[g + jj] = 0.f;
    if (g >= k) continue;
    const u32x4* rows[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      rows[jj] = reinterpret_cast<const u32x4*>(readlane_u64(resp, g + jj < k ? g + jj : g));
    float acc[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[jj] = 0.f;
    for (int c = lane; c < nc; c += 64) {
      const u32x4 a = dyv[c];
      u32x4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (g + jj < k) v[jj] = rows[jj][c];
      const uint32_t qa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (g + jj >= k) break;
        const uint32_t qv[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[jj] += __builtin_bit_cast(float, qa[m] << 16) * __builtin_bit_cast(float, qv[m] << 16);
          acc[jj] += __builtin_bit_cast(float, qa[m] & 0xFFFF0000u) * __builtin_bit_cast(float, qv[m] & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      float t = acc[jj];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
      dw[g + jj] = g + jj < k ? t : 0.f;
    }
  }
}

// Token t's data gradient and router gradient, one wave.  Lane j < k
// resolves pair j: its dX row (local: a grouped row, gated on the unit's
// second-stage tiles; remote: what its rank returned) and its forward
// result.  Returns false (wave-uniform) on abort, time-out or bad routing.
template <int KN, int CB>
__device__ __forceinline__ bool bwd_fold_token(const BwdParams& b, const CombineMeta& M, int t, uint32_t info) {
  const CombineParams& p = b.c;
  const int lane = threadIdx.x & 63;
  const int k = p.k;
  bool local = false, bad = false;
  int u = 0, e = -1;
  uint64_t dxp = 0, resp = 0;
  float wj = 0.f;
  if (lane < k) {
    const int64_t o = (int64_t)t * k + lane;
    e = p.topk_idx[o];
    const int pos = p.perm[o];
    wj = p.topk_w[o];
    bad = e < 0 || e >= p.E || pos < M.off[e] || pos >= M.off[e + 1];
    if (!bad) {
      const int d = e / p.E_loc;
      if (d == p.rank) {
        const int el = e - p.rank * p.E_loc;
        const int grow = M.go[el] + M.before[el] + (pos - M.off[e]);
        bad = grow >= M.go[el + 1];
        local = true;
        u = M.ub[el] + (grow - M.go[el]) / kBwdUnit;
        dxp = reinterpret_cast<uint64_t>(p.yg + (int64_t)grow * p.H);
        resp = reinterpret_cast<uint64_t>(b.y_fwd + (int64_t)grow * p.H);
      } else {
        const int64_t r = pos - M.off[d * p.E_loc];
        dxp = reinterpret_cast<uint64_t>(p.peer_return[d] + r * p.H);
        resp = reinterpret_cast<uint64_t>(b.peer_return_fwd[d] + r * p.H);
      }
    }
  }
  if (__any(bad)) {
    if (lane == 0) raise_error(p.ws, KOS_ERR_ARG, 0x00B50000u | (uint32_t)(t & 0xFFFF));
    return false;
  }
  const uint32_t* t2_done = p.ctr + p.u_max;
  uint32_t it = 0;
  for (;;) {
    const bool ready = !local || ld_relaxed(&t2_done[u]) >= (uint32_t)p.D;
    if (__all(ready)) break;
    if (aborted(p.ws)) return false;
    if (++it >= p.spin_limit) {
      if (lane == 0) raise_error(p.ws, KOS_ERR_TIMEOUT, info);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  fold_token_rows<KN, CB>(p.H, k, dxp, 1.0f, p.y + (int64_t)t * p.H, lane);
  // router gradient: dlogits[idx_j] = w_j (dw_j - sum_i w_i dw_i)
  float dw[KN];
  pair_dots<KN>(p.H, k, resp, b.dy + (int64_t)t * p.H, lane, dw);
  float w[KN], s = 0.f;
  int idx[KN];
#pragma unroll
  for (int j = 0; j < KN; ++j) {
    w[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, wj), j));
    idx[j] = __builtin_amdgcn_readlane(e, j);
    if (j < k) s += w[j] * dw[j];
  }
  float* row = b.dlogits + (int64_t)t * p.E;
  for (int ee = lane; ee < p.E; ee += 64) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < KN; ++j)
      if (j < k && idx[j] == ee) v = w[j] * (dw[j] - s);
    row[ee] = v;
  }
  return true;
}

// The tiles of a unit's rows (BM = 256, or 128 / 64 for an expert's last
// unit when its rows fit): dX (N x K weights), dH over FB columns of F
// (N x K weights), g and u over 128 columns (SwiGLU layout).  Eight waves.
template <int BM, int FB>
struct BwdShapes {
  using X = TileShape<BM, kBwdHCols, 4, 2, 4, true>;
  using DH = TileShape<BM, FB, 4, 2, 4, true>;
  using GU = TileShape<BM, 2 * kBwdFCols, 4, 2, 4>;
};

// SAVED: the first stage reads the forward's kept g and u (g_in, u_in)
// instead of recomputing them.
template <int FB, bool SAVED>
__global__ __launch_bounds__(512, 1) void moe_layer_bwd_kernel(BwdParams args) {
  using B256 = BwdShapes<kBwdUnit, FB>;
  using B128 = BwdShapes<128, FB>;
  using B64 = BwdShapes<64, FB>;
  static_assert(B256::X::NT == 512 && B256::DH::NT == 512 && B256::GU::NT == 512 && 512 / 64 == kBwdMoveTokens,
                "one workgroup shape; a mover entry holds one token per wave");
  constexpr int RING = B256::X::STAGE_BYTES;
  static_assert(B256::DH::STAGE_BYTES <= RING && B256::GU::STAGE_BYTES <= RING, "the dX tile's stage is the largest");
  __shared__ CombineMeta M;
  __shared__ BwdLds B;
  __shared__ WgSlots slots;
  __shared__ BwdParams ps;   // the parameter block, read from LDS where needed
  if (threadIdx.x == 0) ps = args;
  __syncthreads();
  const CombineParams& p = ps.c;
  WsHeader* h = p.ws;
  uint32_t* t1_done = p.ctr;
  uint32_t* t2_done = p.ctr + p.u_max;
  Tracer tr(p.trace);
  const uint32_t ticket = wg_ticket(h, &slots);
  bool ok = bwd_meta(ps, M, B, &slots);

  // ---- movers -------------------------------------------------------------
  if (ok) {
    const int n_own = B.chunk_base[0], n_entries = B.chunk_base[p.world];
    const int wave = threadIdx.x >> 6;
    for (;;) {
      const uint32_t i = wg_claim(&h->head[0], h, &slots);
      if (i >= (uint32_t)n_entries) break;
      const uint64_t t0 = tr.now();
      if ((int)i < n_own) {
        const int t = (int)i * kBwdMoveTokens + wave;
        if (t < p.T) bwd_move_token(ps, M, t);   // an error stops the queues at the next claim
      } else {
        bwd_move_peer(ps, M, B, (int)i);
      }
      tr.put_wg(KOS_TR_MOVE, i, t0);
    }
  }

  // ---- tiles, two-way with pushes ------------------------------------------
  const int U = ok ? M.ub[p.E_loc] : 0;
  constexpr int kSlabs = kBwdUnit / kPushRows;
  const int n_push = U * kSlabs;
  if (ok) {
    f32x16 ax[B256::X::TM][B256::X::TN], ax1[B128::X::TM][B128::X::TN], ax2[B64::X::TM][B64::X::TN];
    f32x16 ah[B256::DH::TM][B256::DH::TN], ah1[B128::DH::TM][B128::DH::TN], ah2[B64::DH::TM][B64::DH::TN];
    f32x16 ad[B256::GU::TM][B256::GU::TN], ad1[B128::GU::TM][B128::GU::TN], ad2[B64::GU::TM][B64::GU::TN];
    const int n_tiles = U * (p.G + p.D);
    for (;;) {
      for (;;) {   // push while the head of the push queue is ready
        __syncthreads();
        if (threadIdx.x == 0) {
          uint32_t hd = ld_relaxed(&h->head[2]);
          uint32_t got = kNoEntry;
          if (hd < (uint32_t)n_push && ld_relaxed(&t2_done[hd / kSlabs]) >= (uint32_t)p.D &&
              __hip_atomic_compare_exchange_strong(&h->head[2], &hd, hd + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT))
            got = hd;
          slots.claim = got;
        }
        __syncthreads();
        const uint32_t got = slots.claim;
        if (got == kNoEntry) break;
        const uint64_t t0 = tr.now();
        push_slab(p, M, unit_of<kBwdUnit>(M, p.E_loc, (int)got / kSlabs), (int)got % kSlabs);
        tr.put_wg(KOS_TR_PUSH, got, t0);
      }
      const uint32_t j = wg_claim(&h->head[1], h, &slots);
      if (j >= (uint32_t)n_tiles) break;
      const CombineTile ct = combine_tile_of((int)j, U, p.G, p.D, p.L, true, true);
      const Unit x = unit_of<kBwdUnit>(M, p.E_loc, ct.u);
      uint64_t t0 = tr.now();
      if (!ct.down) {
        if (!wg_observe(&ps.rows_in[ct.u], (uint32_t)x.m_valid, h, p.spin_limit, j, &slots)) {
          ok = false;
          break;
        }
        tr.put(KOS_TR_WAIT, j, t0);
        t0 = tr.now();
        if constexpr (SAVED) {
          if (x.m_valid > 128) bwd_stage1_saved<typename B256::DH, RING, FB>(ps, x, ct.nt, ah);
          else if (x.m_valid > 64) bwd_stage1_saved<typename B128::DH, RING, FB>(ps, x, ct.nt, ah1);
          else bwd_stage1_saved<typename B64::DH, RING, FB>(ps, x, ct.nt, ah2);
        } else {
          if (x.m_valid > 128) bwd_stage1<typename B256::DH, typename B256::GU, RING, FB>(ps, x, ct.nt, ah, ad);
          else if (x.m_valid > 64) bwd_stage1<typename B128::DH, typename B128::GU, RING, FB>(ps, x, ct.nt, ah1, ad1);
          else bwd_stage1<typename B64::DH, typename B64::GU, RING, FB>(ps, x, ct.nt, ah2, ad2);
        }
        wg_publish(&t1_done[ct.u], 1u);
        tr.put(KOS_TR_TILE, j, t0);
      } else {
        if (!wg_observe(&t1_done[ct.u], (uint32_t)p.G, h, p.spin_limit, j, &slots)) {
          ok = false;
          break;
        }
        tr.put(KOS_TR_WAIT, j, t0);
        t0 = tr.now();
        if (x.m_valid > 128) bwd_tile2<typename B256::X, RING>(ps, x, ct.nt, ax);
        else if (x.m_valid > 64) bwd_tile2<typename B128::X, RING>(ps, x, ct.nt, ax1);
        else bwd_tile2<typename B64::X, RING>(ps, x, ct.nt, ax2);
        wg_publish(&t2_done[ct.u], 1u);
        tr.put(KOS_TR_TILE2, j, t0);
      }
    }
  }

  // ---- pushes left over, in unit order -------------------------------------
  if (ok) {
    for (;;) {
      const uint32_t i = wg_claim(&h->head[2], h, &slots);
      if (i >= (uint32_t)n_push) break;
      const int u = (int)i / kSlabs;
      uint64_t t0 = tr.now();
      if (!wg_observe(&t2_done[u], (uint32_t)p.D, h, p.spin_limit, 0x20000000u | i, &slots)) {
        ok = false;
        break;
      }
      tr.put(KOS_TR_WAIT, i, t0);
      t0 = tr.now();
      push_slab(p, M, unit_of<kBwdUnit>(M, p.E_loc, u), (int)i % kSlabs);
      tr.put_wg(KOS_TR_PUSH, i, t0);
    }
  }

  // ---- fold: dx and the router gradient -------------------------------------
  if (ok) {
    const int nfb = (p.T + kFoldTokens - 1) / kFoldTokens;
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (;;) {
      const uint32_t i = wg_claim(&h->head[3], h, &slots);
      if (i >= (uint32_t)nfb) break;
      const uint64_t t0 = tr.now();
      const int tb = (int)i * kFoldTokens, te = min(p.T, tb + kFoldTokens);
      const int ks = __builtin_amdgcn_readfirstlane(p.k);
      for (int t = tb + wave; t < te; t += nw) {
        const uint32_t info = 0x40000000u | i;
        const bool done = ks <= 8 ? bwd_fold_token<8, 2>(ps, M, t, info) : bwd_fold_token<kMoeMaxTopk, 1>(ps, M, t, info);
        if (!done) break;   // the error is recorded; the next claim stops this workgroup
      }
      tr.put(KOS_TR_FOLD, i, t0);
    }
  }
  tr.finish(ticket);
  wg_exit(h, ps.rows_in, ps.n_counters, &slots);
}


}  // namespace kos

using namespace kos;

extern "C" kos_status kos_moe_layer_bwd(const kos_moe_shape* s, const void* dy, const int32_t* topk_idx,
                                        const float* topk_w, const int32_t* perm, const int32_t* counts,
                                        const int32_t* peer_counts, const void* x_grouped, int64_t grouped_cap,
                                        const int32_t* grouped_offsets, const int32_t* row_src,
                                        const void* y_grouped, const void* const* peer_return, const void* w_gate,
                                        const void* w_up, const void* w_down, const void* gate_saved,
                                        const void* up_saved, const void* const* peer_send_grad,
                                        void* const* out_send_grad, const int64_t* send_caps, void* dres_grouped,
                                        void* dg, void* du, float* dh, void* dx_grouped,
                                        const void* const* peer_return_grad,
                                        void* const* out_return_grad, const int64_t* return_caps, void* dx,
                                        float* dlogits, const kos_opts* opts, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (!s) return fail(KOS_ERR_ARG, "shape is NULL");
  const int R = s->world, r = s->rank;
  if (R < 1 || R > 8) return fail(KOS_ERR_ARG, "world %d outside [1, 8]", R);
  if (r < 0 || r >= R) return fail(KOS_ERR_ARG, "rank %d outside [0, %d)", r, R);
  if (s->reserved) return fail(KOS_ERR_ARG, "reserved must be 0");
  if (s->tokens < 0 || s->hidden <= 0 || s->hidden % kBwdHCols || s->ffn <= 0 || s->ffn % kBwdFCols ||
      s->experts <= 0 || s->experts > kMoeMaxExperts || s->experts % R || s->experts / R > kMoeMaxLocal ||
      s->topk < 1 || s->topk > kMoeMaxTopk || s->topk > s->experts)
    return fail(KOS_ERR_SHAPE, "unsupported expert-layer shape (hidden %% %d, ffn %% %d)", kBwdHCols, kBwdFCols);
  const bool no_tokens = s->tokens == 0;
  if ((!no_tokens && (!dy || !topk_idx || !topk_w || !perm || !dx || !dlogits)) || !counts || !peer_counts ||
      !x_grouped || !grouped_offsets || !row_src || !y_grouped || !w_gate || !w_up || !w_down || !dres_grouped ||
      !dg || !du || (!dh && !gate_saved) || !dx_grouped)
    return fail(KOS_ERR_ARG, "null buffer");
  if ((gate_saved == nullptr) != (up_saved == nullptr))
    return fail(KOS_ERR_ARG, "gate_saved and up_saved are given together or not at all");
  if (R > 1 && (!peer_return || !peer_send_grad || !out_send_grad || !send_caps || !peer_return_grad ||
                !out_return_grad || !return_caps))
    return fail(KOS_ERR_ARG, "a peer array is NULL");
  for (int q = 0; q < R; ++q) {
    if (q == r) continue;
    if (send_caps[q] < 0 || return_caps[q] < 0) return fail(KOS_ERR_ARG, "negative capacity for rank %d", q);
    // NULL is allowed where nothing travels (checked on the device)
    if (!aligned16(peer_return[q]) || !aligned16(peer_send_grad[q]) || !aligned16(out_send_grad[q]) ||
        !aligned16(peer_return_grad[q]) || !aligned16(out_return_grad[q]))
      return fail(KOS_ERR_ALIGN, "peer buffer not aligned");
  }
  if (!aligned16(dy) || !aligned16(x_grouped) || !aligned16(y_grouped) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(dres_grouped) || !aligned16(dg) || !aligned16(du) || !aligned16(dh) ||
      !aligned16(dx_grouped) || !aligned16(dx) || !aligned16(gate_saved) || !aligned16(up_saved))
    return fail(KOS_ERR_ALIGN, "buffers must be 16-byte aligned");
  if (grouped_cap < 0 || grouped_cap > (int64_t(1) << 31) - 1) return fail(KOS_ERR_ARG, "bad grouped_cap");
  // tiles address one expert's weights and the grouped rows through 32-bit
  // buffer offsets
  if ((int64_t)s->hidden * s->ffn * 2 >= (int64_t(1) << 31))
    return fail(KOS_ERR_SHAPE, "one expert's weight (hidden x ffn bf16) must be smaller than 2 GiB");
  if (grouped_cap * s->hidden * 2 >= (int64_t(1) << 31))
    return fail(KOS_ERR_SHAPE, "grouped_cap x hidden x 2 bytes must stay below 2 GiB");
  kos_status st = check_workspace(ws, ws_bytes);
  if (st != KOS_OK) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != KOS_OK) return st;
  kos_opts o;
  if ((st = resolve_opts(opts, dev, CrewDefaults{16, 8, 16, 8}, &o)) != KOS_OK) return st;
  if (o.mode != KOS_MODE_FUSED || o.policy != KOS_POLICY_DEFAULT)
    return fail(KOS_ERR_UNSUPPORTED, "the backward layer is fused, two-way only");

  BwdParams b{};
  CombineParams& p = b.c;
  p.world = R;
  p.rank = r;
  p.T = s->tokens;
  p.H = s->hidden;
  p.E = s->experts;
  p.k = s->topk;
  p.F = s->ffn;
  p.E_loc = s->experts / R;
  p.xg = static_cast<const uint16_t*>(x_grouped);
  p.go_in = grouped_offsets;
  p.row_src = row_src;
  p.wg = static_cast<const uint16_t*>(w_gate);
  p.wu = static_cast<const uint16_t*>(w_up);
  p.wd = static_cast<const uint16_t*>(w_down);
  p.topk_idx = topk_idx;
  p.topk_w = topk_w;
  p.counts = counts;
  p.perm = perm;
  p.peer_counts = peer_counts;
  for (int q = 0; q < R; ++q) {
    const bool me = q == r;
    p.peer_return[q] = me ? nullptr : static_cast<const uint16_t*>(peer_return_grad[q]);
    p.out_return[q] = me ? nullptr : static_cast<uint16_t*>(out_return_grad[q]);
    p.return_cap[q] = me ? 0 : return_caps[q];
    b.peer_return_fwd[q] = me ? nullptr : static_cast<const uint16_t*>(peer_return[q]);
    b.peer_send_grad[q] = me ? nullptr : static_cast<const uint16_t*>(peer_send_grad[q]);
    b.out_send_grad[q] = me ? nullptr : static_cast<uint16_t*>(out_send_grad[q]);
    b.send_cap[q] = me ? 0 : send_caps[q];
  }
  p.yg = static_cast<uint16_t*>(dx_grouped);
  p.y = static_cast<uint16_t*>(dx);
  const int FB = s->ffn % 256 == 0 ? 256 : kBwdFCols;   // F columns per first-stage entry
  p.G = s->ffn / FB;
  p.D = s->hidden / kBwdHCols;
  p.L = (o.grid + p.G - 1) / p.G;
  p.u_max = (int32_t)((grouped_cap + kBwdUnit - 1) / kBwdUnit) + p.E_loc;
  p.grouped_cap = (int32_t)grouped_cap;
  p.do_gu = p.do_dn = p.do_push = p.do_fold = 1;
  p.two_way = 1;
  p.wait_flags = 1;
  p.spin_limit = o.spin_limit;
  p.ws = static_cast<WsHeader*>(ws);
  p.trace = trace_slot(ws, o.trace, 0);
  b.dy = static_cast<const uint16_t*>(dy);
  b.y_fwd = static_cast<const uint16_t*>(y_grouped);
  b.dres = static_cast<uint16_t*>(dres_grouped);
  b.dg = static_cast<uint16_t*>(dg);
  b.du = static_cast<uint16_t*>(du);
  b.dh = dh;
  b.g_in = static_cast<const uint16_t*>(gate_saved);
  b.u_in = static_cast<const uint16_t*>(up_saved);
  b.dlogits = dlogits;
  uint32_t* base = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kCountersOffset);
  b.rows_in = base;
  p.ctr = base + p.u_max;   // t1_done, t2_done
  b.n_counters = 3 * (uint32_t)p.u_max;
  if ((size_t)b.n_counters > kMaxCounters) return fail(KOS_ERR_SHAPE, "grouped_cap too large for the workspace");

  hipStream_t strm = static_cast<hipStream_t>(stream);
  const bool saved = gate_saved != nullptr;
  if (FB == 256 && saved)
    hipLaunchKernelGGL((moe_layer_bwd_kernel<256, true>), dim3(o.grid), dim3(512), 0, strm, b);
  else if (FB == 256)
    hipLaunchKernelGGL((moe_layer_bwd_kernel<256, false>), dim3(o.grid), dim3(512), 0, strm, b);
  else if (saved)
    hipLaunchKernelGGL((moe_layer_bwd_kernel<kBwdFCols, true>), dim3(o.grid), dim3(512), 0, strm, b);
  else
    hipLaunchKernelGGL((moe_layer_bwd_kernel<kBwdFCols, false>), dim3(o.grid), dim3(512), 0, strm, b);
  return launch_status("moe_layer_bwd launch");
}
