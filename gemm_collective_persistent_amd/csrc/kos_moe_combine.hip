// Expert layer, combine direction, as one persistent kernel: grouped SwiGLU
// expert GEMMs, results pushed back to the ranks that sent the rows, and the
// weighted fold of our own tokens [KOSMOS arXiv abstract: the whole expert
// layer, routing through the final weighted sum, in one launch per
// direction; KOSMOS explainer, "KOSMOS removes the manager": roles switch
// both ways here -- between tiles a workgroup sends back a finished result
// if one is waiting, else it computes the next tile].
//
// Work units: (local expert e, row block of BM grouped rows), expert-major.
// Per unit: G gate/up tiles (each BN/2 columns of h = bf16(silu(X.Wg) *
// (X.Wu)), gate and up computed in one MFMA tile) and D down tiles (BN
// columns of Y = bf16(h.Wd)), the down tiles gated on the unit's G gate/up
// tiles.
// Queues:
//   head[1]  tiles, consumer-ordered with a lag of L units: the gate/up
//            tiles of units 0..L-1, then for each unit i the gate/up tiles
//            of unit i+L followed by the down tiles of unit i -- a down tile
//            is claimed about a wave of tiles after the tiles it needs.
//   head[2]  push entries, kPushRows-row slabs of each unit, in unit order:
//            rows whose source is another rank are copied to that rank's
//            return buffer once the unit's D down tiles are done.  Between
//            tiles a workgroup takes the head entry if it is ready, else
//            builds the next tile.
//   head[3]  fold entries, kFoldTokens tokens each, one token per wave at a
//            time: y[t] = bf16(sum_j w[t,j] * res(t,j)), fp32, j ascending;
//            local results gated on their unit's down tiles, remote results
//            read from what the peers returned.
#include "kos_host.h"
#include "kos_moe.h"
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

// Tile entry j of the queue -> (is_down, unit, column tile).
__device__ __forceinline__ void decode_tile(const CombineParams& p, int U, int j, bool& down, int& u, int& nt) {
  if (p.do_gu && !p.do_dn) {
    down = false;
    u = j / p.G;
    nt = j % p.G;
    return;
  }
  if (!p.do_gu) {
    down = true;
    u = j / p.D;
    nt = j % p.D;
    return;
  }
  const int L = min(p.L, U);
  const int head = L * p.G;
  if (j < head) {
    down = false;
    u = j / p.G;
    nt = j % p.G;
    return;
  }
  const int jj = j - head;
  const int nfull = max(U - p.L, 0);
  const int GD = p.G + p.D;
  if (jj < nfull * GD) {
    const int i = jj / GD, r = jj % GD;
    if (r < p.G) {
      down = false;
      u = i + p.L;
      nt = r;
    } else {
      down = true;
      u = i;
      nt = r - p.G;
    }
    return;
  }
  const int jj2 = jj - nfull * GD;
  down = true;
  u = nfull + jj2 / p.D;
  nt = jj2 % p.D;
}

template <class S, int RING>
__device__ __forceinline__ void gate_up_tile(const CombineParams& p, const Unit& x, int nt, f32x16 (&acc)[S::TM][S::TN]) {
  constexpr int HN = S::BN / 2;    // h columns per tile
  const int64_t H = p.H, F = p.F;
  BSrc b{p.wg + (int64_t)x.el * H * F + (int64_t)nt * HN, p.wu + (int64_t)x.el * H * F + (int64_t)nt * HN, F};
  tile_mainloop<S, true, false, RING>(acc, p.xg + (int64_t)x.row0 * H, H, x.m_valid, b, p.H);
  // read by this launch's down tiles: device-coherent stores
  tile_store_rows<S, RING, true, true>(acc, p.h + (int64_t)x.row0 * F + (int64_t)nt * HN, F, x.m_valid);
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
// wave at a time.
__device__ __forceinline__ void push_slab(const CombineParams& p, const CombineMeta& M, const Unit& x, int slab) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const DevBuf yb(p.yg);
  const int r1 = min(x.m_valid, (slab + 1) * kPushRows);
  for (int r = slab * kPushRows + wave; r < r1; r += nw) {
    const int64_t grow = (int64_t)x.row0 + r;
    const int src = p.row_src[grow * 2];
    if (src == p.rank) continue;
    const int64_t i = p.row_src[grow * 2 + 1];
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
// false (wave-uniform) on abort or time-out.
template <int BM>
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
    const int e = p.topk_idx[(int64_t)t * k + lane];
    const int pos = p.perm[(int64_t)t * k + lane];
    wj = p.topk_w[(int64_t)t * k + lane];
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

template <int BM>
__device__ __forceinline__ bool fold_block(const CombineParams& p, const CombineMeta& M, int fb, WgSlots* s) {
  const int t0 = fb * kFoldTokens;
  const int t1 = min(p.T, t0 + kFoldTokens);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (threadIdx.x == 0) s->ok = 1;
  __syncthreads();
  for (int t = t0 + wave; t < t1; t += nw)
    if (!fold_token_wave<BM>(p, M, t, 0x40000000u | (uint32_t)fb)) {
      if ((threadIdx.x & 63) == 0) s->ok = 0;
      break;
    }
  __syncthreads();
  return s->ok != 0;
}

// S: the unit's tile (BM rows of one expert).  ST, ST2: tiles of the same
// width and fewer rows for an expert's last unit when its rows fit (less
// work spent on rows past the end; ST2 == ST when there is one tail size).
// COH: one launch produces and consumes h and Y (fused and fixed-crew
// modes).
template <class S, class ST, class ST2, bool COH>
__global__ __launch_bounds__(S::NT, 1) void moe_combine_kernel(CombineParams args) {
  constexpr int BM = S::BM;
  static_assert(ST::BN == S::BN && ST::BM < S::BM && ST::NT == S::NT, "tail tile: same width, fewer rows");
  static_assert(ST2::BN == S::BN && ST2::BM <= ST::BM && ST2::NT == S::NT, "second tail: no more rows than the first");
  constexpr bool kTail2 = ST2::BM < ST::BM;
  __shared__ CombineMeta M;
  __shared__ WgSlots slots;
  // The parameter block lives in LDS: the role code reads the fields it needs
  // when it needs them instead of pinning ~40 pointers in scalar registers.
  __shared__ CombineParams ps;
  if (threadIdx.x == 0) ps = args;
  __syncthreads();
  const CombineParams& p = ps;
  WsHeader* h = p.ws;
  if (!load_combine_meta<BM>(p, M, &slots)) {   // a peer buffer it needs is NULL (every workgroup agrees)
    wg_exit(h, p.ctr, 2 * p.u_max, &slots);
    return;
  }
  const int U = M.ub[p.E_loc];
  constexpr int kPushSlabs = (BM + kPushRows - 1) / kPushRows;
  const int n_push = U * kPushSlabs;
  uint32_t* gu_done = p.ctr;
  uint32_t* dn_done = p.ctr + p.u_max;
  Tracer tr(p.trace);
  const uint32_t ticket = wg_ticket(h, &slots);
  const bool crew = p.n_crew > 0 && ticket < (uint32_t)p.n_crew;
  bool failed = false;

  // ---- builder role (two-way: push any ready result between tiles) -------
  if (!crew && (p.do_gu || p.do_dn)) {
    f32x16 acc[S::TM][S::TN];
    f32x16 acc_t[ST::TM][ST::TN];
    f32x16 acc_t2[ST2::TM][ST2::TN];
    constexpr int RB = S::STAGE_BYTES;
    const int n_entries = (p.do_gu && p.do_dn) ? U * (p.G + p.D) : (p.do_gu ? U * p.G : U * p.D);
    for (;;) {
      if (p.two_way && p.do_push) {
        for (;;) {   // push while the head of the push queue is ready
          __syncthreads();
          if (threadIdx.x == 0) {
            uint32_t hd = ld_relaxed(&h->head[2]);
            uint32_t got = kNoEntry;
            if (hd < (uint32_t)n_push && ld_relaxed(&dn_done[hd / kPushSlabs]) >= (uint32_t)p.D &&
                __hip_atomic_compare_exchange_strong(&h->head[2], &hd, hd + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
              got = hd;
            slots.claim = got;
          }
          __syncthreads();
          const uint32_t got = slots.claim;
          if (got == kNoEntry) break;
          const uint64_t t0 = tr.now();
          push_slab(p, M, unit_of<BM>(M, p.E_loc, (int)got / kPushSlabs), (int)got % kPushSlabs);
          tr.put(KOS_TR_PUSH, got, t0);
        }
      }
      const uint32_t j = wg_claim(&h->head[1], h, &slots);
      if (j >= (uint32_t)n_entries) break;
      bool down;
      int u, nt;
      decode_tile(p, U, (int)j, down, u, nt);
      const Unit x = unit_of<BM>(M, p.E_loc, u);
      const bool tail = x.m_valid <= ST::BM;
      const bool tail2 = kTail2 && x.m_valid <= ST2::BM;
      uint64_t t0 = tr.now();
      if (!down) {
        if (tail2) gate_up_tile<ST2, RB>(p, x, nt, acc_t2);
        else if (tail) gate_up_tile<ST, RB>(p, x, nt, acc_t);
        else gate_up_tile<S, RB>(p, x, nt, acc);
        wg_publish(&gu_done[u], 1u);
        tr.put(KOS_TR_TILE, j, t0);
      } else {
        if (p.wait_flags && p.do_gu) {
          if (!wg_observe(&gu_done[u], (uint32_t)p.G, h, p.spin_limit, j, &slots)) {
            failed = true;
            break;
          }
          tr.put(KOS_TR_WAIT, j, t0);
          t0 = tr.now();
        }
        if (tail2) down_tile<ST2, COH, RB>(p, x, nt, acc_t2);
        else if (tail) down_tile<ST, COH, RB>(p, x, nt, acc_t);
        else down_tile<S, COH, RB>(p, x, nt, acc);
        wg_publish(&dn_done[u], 1u);
        tr.put(KOS_TR_TILE2, j, t0);
      }
    }
    if (p.n_crew > 0) {   // fixed crew: builders only build
      tr.finish(ticket);
      wg_exit(h, p.ctr, 2 * p.u_max, &slots);
      return;
    }
  }

  // ---- pusher role (drain, in unit order) --------------------------------
  if (!failed && p.do_push) {
    for (;;) {
      const uint32_t i = wg_claim(&h->head[2], h, &slots);
      if (i >= (uint32_t)n_push) break;
      const int u = (int)i / kPushSlabs;
      uint64_t t0 = tr.now();
      if (p.wait_flags) {
        if (!wg_observe(&dn_done[u], (uint32_t)p.D, h, p.spin_limit, 0x20000000u | i, &slots)) break;
        tr.put(KOS_TR_WAIT, i, t0);
        t0 = tr.now();
      }
      push_slab(p, M, unit_of<BM>(M, p.E_loc, u), (int)i % kPushSlabs);
      tr.put(KOS_TR_PUSH, i, t0);
    }
  }

  // ---- fold role ---------------------------------------------------------
  if (!failed && p.do_fold) {
    const int nfb = (p.T + kFoldTokens - 1) / kFoldTokens;
    for (;;) {
      const uint32_t i = wg_claim(&h->head[3], h, &slots);
      if (i >= (uint32_t)nfb) break;
      const uint64_t t0 = tr.now();
      if (!fold_block<BM>(p, M, (int)i, &slots)) break;
      tr.put(KOS_TR_FOLD, i, t0);
    }
  }
  tr.finish(ticket);
  wg_exit(h, p.ctr, 2 * p.u_max, &slots);
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

using namespace kos;

extern "C" kos_status kos_moe_combine(const kos_moe_shape* s, const void* x_grouped, const int32_t* grouped_offsets,
                                      const int32_t* row_src, int64_t grouped_cap, const void* w_gate,
                                      const void* w_up, const void* w_down, const int32_t* topk_idx,
                                      const float* topk_w, const int32_t* counts, const int32_t* perm,
                                      const int32_t* peer_counts, const void* const* peer_return, void* h,
                                      void* y_grouped, void* const* out_return, const int64_t* return_caps,
                                      void* y, const kos_opts* opts,
                                      void* ws, size_t ws_bytes, void* stream) {
  if (!s) return fail(KOS_ERR_ARG, "shape is NULL");
  const bool big = s->hidden % CombineTileBig::BN == 0 && s->ffn % (CombineTileBig::BN / 2) == 0;
  using S = CombineTileSmall;   // the checks below use the small tile's divisibility
  const int R = s->world, r = s->rank;
  if (R < 1 || R > 8) return fail(KOS_ERR_ARG, "world %d outside [1, 8]", R);
  if (r < 0 || r >= R) return fail(KOS_ERR_ARG, "rank %d outside [0, %d)", r, R);
  if (s->reserved) return fail(KOS_ERR_ARG, "reserved must be 0");
  if (s->tokens < 0 || s->hidden <= 0 || s->hidden % S::BN || s->ffn <= 0 || s->ffn % (S::BN / 2) ||
      s->experts <= 0 || s->experts > kMoeMaxExperts || s->experts % R || s->experts / R > kMoeMaxLocal ||
      s->topk < 1 || s->topk > kMoeMaxTopk || s->topk > s->experts)
    return fail(KOS_ERR_SHAPE, "unsupported expert-layer shape (hidden %% %d, ffn %% %d)", S::BN, S::BN / 2);
  // per-token buffers may be NULL for an empty batch (nothing reads them)
  const bool no_tokens = s->tokens == 0;
  if (!x_grouped || !grouped_offsets || !row_src || !w_gate || !w_up || !w_down ||
      (!no_tokens && (!topk_idx || !topk_w || !perm || !y)) || !counts || !peer_counts || !h || !y_grouped)
    return fail(KOS_ERR_ARG, "null buffer");
  if (R > 1 && (!peer_return || !out_return || !return_caps))
    return fail(KOS_ERR_ARG, "peer_return / out_return / return_caps is NULL");
  for (int q = 0; q < R; ++q) {
    if (q == r) continue;
    // NULL is allowed where nothing travels (checked on the device)
    if (!aligned16(peer_return[q]) || !aligned16(out_return[q])) return fail(KOS_ERR_ALIGN, "peer buffer not aligned");
  }
  if (!aligned16(x_grouped) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(h) ||
      !aligned16(y_grouped) || !aligned16(y))
    return fail(KOS_ERR_ALIGN, "buffers must be 16-byte aligned");
  if (grouped_cap < 0 || grouped_cap > (int64_t(1) << 31) - 1) return fail(KOS_ERR_ARG, "bad grouped_cap");
  // the tiles address one expert's weights through 32-bit buffer offsets
  if ((int64_t)s->hidden * s->ffn * 2 >= (int64_t(1) << 31))
    return fail(KOS_ERR_SHAPE, "one expert's weight (hidden x ffn bf16) must be smaller than 2 GiB");
  // the grouped results are read back through 32-bit byte offsets
  if (grouped_cap * s->hidden * 2 >= (int64_t(1) << 31))
    return fail(KOS_ERR_SHAPE, "grouped_cap x hidden x 2 bytes must stay below 2 GiB");
  kos_status st = check_workspace(ws, ws_bytes);
  if (st != KOS_OK) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != KOS_OK) return st;
  kos_opts o;
  if ((st = resolve_opts(opts, dev, CrewDefaults{16, 8, 16, 8}, &o)) != KOS_OK) return st;

  CombineParams p{};
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
    p.peer_return[q] = q == r ? nullptr : static_cast<const uint16_t*>(peer_return[q]);
    p.out_return[q] = q == r ? nullptr : static_cast<uint16_t*>(out_return[q]);
    p.return_cap[q] = q == r ? 0 : return_caps[q];
  }
  p.h = static_cast<uint16_t*>(h);
  p.yg = static_cast<uint16_t*>(y_grouped);
  p.y = static_cast<uint16_t*>(y);
  const int BMt = big ? CombineTileBig::BM : CombineTileSmall::BM;
  const int BNt = big ? CombineTileBig::BN : CombineTileSmall::BN;
  p.G = s->ffn / (BNt / 2);
  p.D = s->hidden / BNt;
  p.L = (o.grid + p.G - 1) / p.G;
  p.u_max = (int32_t)((grouped_cap + BMt - 1) / BMt) + p.E_loc;
  p.grouped_cap = (int32_t)grouped_cap;
  if ((size_t)2 * p.u_max > kMaxCounters) return fail(KOS_ERR_SHAPE, "grouped_cap too large for the workspace");
  p.spin_limit = o.spin_limit;
  p.ws = static_cast<WsHeader*>(ws);
  p.ctr = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kCountersOffset);
  p.trace = trace_slot(ws, o.trace, 0);

  hipStream_t strm = static_cast<hipStream_t>(stream);
  auto launch = [&](const CombineParams& q, const char* what) {
    const bool coh = q.wait_flags != 0;
    if (big && coh)
      hipLaunchKernelGGL((moe_combine_kernel<CombineTileBig, CombineTailBig, CombineTail2Big, true>), dim3(o.grid), dim3(CombineTileBig::NT), 0, strm,
                         q);
    else if (big)
      hipLaunchKernelGGL((moe_combine_kernel<CombineTileBig, CombineTailBig, CombineTail2Big, false>), dim3(o.grid), dim3(CombineTileBig::NT), 0,
                         strm, q);
    else if (coh)
      hipLaunchKernelGGL((moe_combine_kernel<CombineTileSmall, CombineTailSmall, CombineTailSmall, true>), dim3(o.grid), dim3(CombineTileSmall::NT), 0,
                         strm, q);
    else
      hipLaunchKernelGGL((moe_combine_kernel<CombineTileSmall, CombineTailSmall, CombineTailSmall, false>), dim3(o.grid), dim3(CombineTileSmall::NT), 0,
                         strm, q);
    return launch_status(what);
  };
  if (o.mode == KOS_MODE_UNFUSED) {
    // four launches: gate/up GEMMs, down GEMMs, push, fold
    CombineParams a = p;
    a.do_gu = 1;
    if ((st = launch(a, "moe_combine gate/up launch")) != KOS_OK) return st;
    CombineParams b = p;
    b.trace = trace_slot(ws, o.trace, 1);
    b.do_dn = 1;
    if ((st = launch(b, "moe_combine down launch")) != KOS_OK) return st;
    CombineParams c = p;
    c.trace = trace_slot(ws, o.trace, 2);
    c.do_push = 1;
    if ((st = launch(c, "moe_combine push launch")) != KOS_OK) return st;
    CombineParams d = p;
    d.trace = trace_slot(ws, o.trace, 3);
    d.do_fold = 1;
    return launch(d, "moe_combine fold launch");
  }
  p.do_gu = p.do_dn = p.do_push = p.do_fold = 1;
  p.wait_flags = 1;
  if (o.mode == KOS_MODE_FIXED) {
    if (o.n_movers < 1 || o.n_movers >= o.grid)
      return fail(KOS_ERR_ARG, "n_movers %d must be in [1, grid %d)", o.n_movers, o.grid);
    p.n_crew = o.n_movers;
    p.two_way = 0;
  } else {
    p.two_way = 1;
  }
  return launch(p, "moe_combine launch");
}
