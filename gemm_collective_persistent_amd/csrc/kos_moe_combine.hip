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
#include "kos_moe_combine.h"

namespace kos {

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
          tr.put_wg(KOS_TR_PUSH, got, t0);
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
      tr.put_wg(KOS_TR_PUSH, i, t0);
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

}  // namespace kos

using namespace kos;

extern "C" kos_status kos_moe_combine(const kos_moe_shape* s, const void* x_grouped, const int32_t* grouped_offsets,
                                      const int32_t* row_src, int64_t grouped_cap, const void* w_gate,
                                      const void* w_up, const void* w_down, const int32_t* topk_idx,
                                      const float* topk_w, const int32_t* counts, const int32_t* perm,
                                      const int32_t* peer_counts, const void* const* peer_return, void* h,
                                      void* gate_save, void* up_save, void* y_grouped,
                                      void* const* out_return, const int64_t* return_caps,
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
      !aligned16(y_grouped) || !aligned16(y) || !aligned16(gate_save) || !aligned16(up_save))
    return fail(KOS_ERR_ALIGN, "buffers must be 16-byte aligned");
  if ((gate_save == nullptr) != (up_save == nullptr))
    return fail(KOS_ERR_ARG, "gate_save and up_save are given together or not at all");
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
  p.g_save = static_cast<uint16_t*>(gate_save);
  p.u_save = static_cast<uint16_t*>(up_save);
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
    p.two_way = o.policy == KOS_POLICY_DEFAULT;   // swapped: one-way, pushes once the tiles run out
  }
  return launch(p, "moe_combine launch");
}
