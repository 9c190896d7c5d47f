// The whole expert layer, forward direction, as ONE persistent kernel:
// router -> permutation -> token movement -> grouped SwiGLU expert GEMMs ->
// results pushed back -> weighted fold [KOSMOS arXiv abstract: the whole
// expert layer, routing through the final weighted sum, runs in one launch
// per direction; KOSMOS explainer, "KOSMOS removes the manager": workgroups
// take the next entry of queues ordered by what consumers need, and in the
// combine step switch both ways between sending results back and building
// tiles].
//
// The same steps as kos_moe_dispatch followed by kos_moe_combine (the
// shared pieces are in kos_moe_dispatch.h and kos_moe_combine.h), with the
// launch boundary between them replaced by ready counters: a workgroup runs
// through the queues in this order, taking entries until each runs out.
//   head[0]  router entries (16 tokens each)         -> ctr[0] counts them
//   head[1]  scan entries (one per expert), gated on every router entry
//                                                      -> ctr[1] counts them
//   then every workgroup waits for ctr[1] (all experts scanned) and builds
//   the layer's bookkeeping (packed and grouped offsets) in its LDS
//   head[2]  mover entries: our tokens to the peers' send buffers or straight
//            into the grouped input, the peers' rows into the grouped input;
//            each grouped row, once stored, bumps rows_in[its unit]
//   head[3]  tiles of the grouped SwiGLU GEMMs, in the combine's lagged
//            consumer order; a unit's gate/up tiles wait until rows_in holds
//            all its rows, its down tiles until its gate/up tiles are done;
//            between tiles a workgroup takes the push queue's head if ready
//   head[4]  push entries (results of rows a peer sent us, back to it)
//   head[5]  fold entries (our tokens: the weighted sum of their k results),
//            after every mover entry of our tokens is done (the fold reads
//            the packed positions they write) and each local result's unit
//            is built
// Every wait is on work that sits earlier in some workgroup's queue order
// and was already claimed by a running workgroup, so no wait is circular
// (all workgroups are resident: one per compute unit).
#include "kos_host.h"
#include "kos_moe_combine.h"
#include "kos_moe_dispatch.h"

namespace kos {

struct LayerParams {
  DispatchParams d;    // router, scan, movers (x_grouped, row_src, perm, ... as the dispatch)
  CombineParams c;     // tiles, pushes, fold (as the combine; its ctr = gu_done, dn_done)
  uint32_t* base;      // counters: [0] routed entries, [1] scanned experts, [2] own-token mover
                       // entries done, [3, 3 + u_max) rows_in
  uint32_t n_counters; // 3 + 3 * u_max: what the last workgroup out resets
};

// The combine's bookkeeping, taken from the dispatch's (both in LDS):
// grouped offsets, rows of lower ranks per local expert, our packed
// offsets, rows each rank sent us, and the units of each local expert.
// Also checks the return buffers against the rows each peer sent and the
// peer buffers that results travel through.  Returns false (every thread)
// after recording an error.
template <int BM>
__device__ __forceinline__ bool layer_meta(const CombineParams& p, const DispatchLds& L, CombineMeta& M, WgSlots* s) {
  for (int el = threadIdx.x; el <= p.E_loc; el += blockDim.x) M.go[el] = L.go[el];
  for (int el = threadIdx.x; el < p.E_loc; el += blockDim.x) M.before[el] = L.before[p.rank][el];
  for (int e = threadIdx.x; e <= p.E; e += blockDim.x) M.off[e] = L.off[e];
  if (threadIdx.x < 8) M.recv[threadIdx.x] = threadIdx.x < p.world ? L.cum[threadIdx.x][p.E_loc] : 0;
  if (threadIdx.x == 0) {
    s->ok = 1;
    M.ub[0] = 0;
    for (int el = 0; el < p.E_loc; ++el) {
      const int n = L.go[el + 1] - L.go[el];
      M.ub[el + 1] = M.ub[el] + (n + BM - 1) / BM;
    }
  }
  __syncthreads();
  const int q = threadIdx.x;
  if (q < p.world && q != p.rank) {
    const int sent = M.off[(q + 1) * p.E_loc] - M.off[q * p.E_loc];   // results q returns
    if ((sent > 0 && p.peer_return[q] == nullptr) || (M.recv[q] > 0 && p.out_return[q] == nullptr)) {
      raise_error(p.ws, KOS_ERR_ARG, 0x00C00000u);
      s->ok = 0;
    }
    if (M.recv[q] > p.return_cap[q]) {
      raise_error(p.ws, KOS_ERR_CAPACITY, 0x00F00000u | (uint32_t)q);
      s->ok = 0;
    }
  }
  __syncthreads();
  return s->ok != 0;
}

// SAVE: the gate/up tiles also keep g and u (gate_save, up_save given).
template <class S, class ST, class ST2, bool SAVE>
__global__ __launch_bounds__(S::NT, 1) void moe_layer_kernel(LayerParams args) {
  constexpr int BM = S::BM, NW = S::NT / 64;
  constexpr int MT = NW;                           // our tokens per mover entry: one per wave
  static_assert(ST::BN == S::BN && ST::BM < S::BM && ST::NT == S::NT, "tail tile: same width, fewer rows");
  static_assert(ST2::BN == S::BN && ST2::BM <= ST::BM && ST2::NT == S::NT, "second tail: no more rows than the first");
  constexpr bool kTail2 = ST2::BM < ST::BM;
  __shared__ DispatchLds L;
  __shared__ CombineMeta M;
  __shared__ WgSlots slots;
  // The parameter block lives in LDS (the roles read the fields they need
  // when they need them).
  __shared__ LayerParams ps;
  if (threadIdx.x == 0) ps = args;
  __syncthreads();
  const DispatchParams& d = ps.d;
  const CombineParams& p = ps.c;
  WsHeader* h = d.ws;
  uint32_t* own_moved = ps.base + 2;
  uint32_t* rows_in = ps.base + 3;
  uint32_t* gu_done = p.ctr;
  uint32_t* dn_done = p.ctr + p.u_max;
  Tracer tr(d.trace);
  const uint32_t ticket = wg_ticket(h, &slots);
  dispatch_prologue<MT>(d, L);

  // ---- router, then scan --------------------------------------------------
  const uint32_t n_route = (uint32_t)d.nblk * 4;
  for (;;) {
    const uint32_t b4 = wg_claim(&h->head[0], h, &slots);
    if (b4 >= n_route) break;
    const uint64_t t0 = tr.now();
    route_any<NW>(d, (int)b4, L);
    wg_publish(&d.ctr[0], 1u);
    tr.put(KOS_TR_ROUTE, b4, t0);
  }
  bool ok = true;
  for (;;) {
    const uint32_t e = wg_claim(&h->head[1], h, &slots);
    if (e >= (uint32_t)d.E) break;
    uint64_t t0 = tr.now();
    if (!wg_observe(&d.ctr[0], n_route, h, d.spin_limit, 0xFFFE0000u | e, &slots)) {
      ok = false;
      break;
    }
    tr.put(KOS_TR_WAIT, e, t0);
    t0 = tr.now();
    scan_expert(d, L, (int)e);
    wg_publish(&d.ctr[1], 1u);
    tr.put(KOS_TR_SCAN, e, t0);
  }

  // ---- the layer's bookkeeping, in every workgroup -------------------------
  const uint64_t tw = tr.now();
  if (ok) ok = wg_observe(&d.ctr[1], (uint32_t)d.E, h, d.spin_limit, 0xFFFF0000u, &slots);
  if (ok) ok = load_meta(d, L, &slots, ticket == 0);
  if (ok) ok = layer_meta<BM>(p, L, M, &slots);
  tr.put(KOS_TR_WAIT, 0xFFFFFF, tw);

  // ---- movers -------------------------------------------------------------
  if (ok) {
    const int n_entries = L.n_entries;
    const int lane = threadIdx.x & 63;
    for (;;) {
      const uint32_t i = wg_claim(&h->head[2], h, &slots);
      if (i >= (uint32_t)n_entries) break;
      const uint64_t t0 = tr.now();
      move_entry<MT, true>(d, L, (int)i, [&](int grow, int el) {
        if (lane == 0) add_relaxed(&rows_in[M.ub[el] + (grow - M.go[el]) / BM], 1u);
      });
      // our tokens' packed positions (perm) are read by the fold
      if ((int)i < d.nblk * (kMoeTokBlock / MT)) wg_publish(own_moved, 1u);
      tr.put_wg(KOS_TR_MOVE, i, t0);
    }
  }

  // ---- builders, two-way with pushes --------------------------------------
  const int U = ok ? M.ub[p.E_loc] : 0;
  constexpr int kPushSlabs = (BM + kPushRows - 1) / kPushRows;
  const int n_push = U * kPushSlabs;
  if (ok) {
    f32x16 acc[S::TM][S::TN];
    f32x16 acc_t[ST::TM][ST::TN];
    f32x16 acc_t2[ST2::TM][ST2::TN];
    constexpr int RB = S::STAGE_BYTES;
    const int n_entries = U * (p.G + p.D);
    for (;;) {
      for (;;) {   // push while the head of the push queue is ready
        __syncthreads();
        if (threadIdx.x == 0) {
          uint32_t hd = ld_relaxed(&h->head[4]);
          uint32_t got = kNoEntry;
          if (hd < (uint32_t)n_push && ld_relaxed(&dn_done[hd / kPushSlabs]) >= (uint32_t)p.D &&
              __hip_atomic_compare_exchange_strong(&h->head[4], &hd, hd + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT))
            got = hd;
          slots.claim = got;
        }
        __syncthreads();
        const uint32_t got = slots.claim;
        if (got == kNoEntry) break;
        const uint64_t t0 = tr.now();
        push_slab<true>(p, M, unit_of<BM>(M, p.E_loc, (int)got / kPushSlabs), (int)got % kPushSlabs);
        tr.put_wg(KOS_TR_PUSH, got, t0);
      }
      const uint32_t j = wg_claim(&h->head[3], h, &slots);
      if (j >= (uint32_t)n_entries) break;
      bool down;
      int u, nt;
      decode_tile(p, U, (int)j, down, u, nt);
      const Unit x = unit_of<BM>(M, p.E_loc, u);
      const bool tail = x.m_valid <= ST::BM;
      const bool tail2 = kTail2 && x.m_valid <= ST2::BM;
      uint64_t t0 = tr.now();
      if (!down) {
        // the unit's grouped rows, stored by this launch's movers
        if (!wg_observe(&rows_in[u], (uint32_t)x.m_valid, h, p.spin_limit, j, &slots)) {
          ok = false;
          break;
        }
        tr.put(KOS_TR_WAIT, j, t0);
        t0 = tr.now();
        if (tail2) gate_up_tile<ST2, RB, true, SAVE>(p, x, nt, acc_t2);
        else if (tail) gate_up_tile<ST, RB, true, SAVE>(p, x, nt, acc_t);
        else gate_up_tile<S, RB, true, SAVE>(p, x, nt, acc);
        wg_publish(&gu_done[u], 1u);
        tr.put(KOS_TR_TILE, j, t0);
      } else {
        if (!wg_observe(&gu_done[u], (uint32_t)p.G, h, p.spin_limit, j, &slots)) {
          ok = false;
          break;
        }
        tr.put(KOS_TR_WAIT, j, t0);
        t0 = tr.now();
        if (tail2) down_tile<ST2, true, RB>(p, x, nt, acc_t2);
        else if (tail) down_tile<ST, true, RB>(p, x, nt, acc_t);
        else down_tile<S, true, RB>(p, x, nt, acc);
        wg_publish(&dn_done[u], 1u);
        tr.put(KOS_TR_TILE2, j, t0);
      }
    }
  }

  // ---- pushes left over, in unit order -------------------------------------
  if (ok) {
    for (;;) {
      const uint32_t i = wg_claim(&h->head[4], h, &slots);
      if (i >= (uint32_t)n_push) break;
      const int u = (int)i / kPushSlabs;
      uint64_t t0 = tr.now();
      if (!wg_observe(&dn_done[u], (uint32_t)p.D, h, p.spin_limit, 0x20000000u | i, &slots)) {
        ok = false;
        break;
      }
      tr.put(KOS_TR_WAIT, i, t0);
      t0 = tr.now();
      push_slab<true>(p, M, unit_of<BM>(M, p.E_loc, u), (int)i % kPushSlabs);
      tr.put_wg(KOS_TR_PUSH, i, t0);
    }
  }

  // ---- fold ----------------------------------------------------------------
  // the fold reads every pair's packed position, written by the movers of
  // our tokens (a token whose results all come from peers waits on no tile)
  if (ok) {
    const uint64_t t0 = tr.now();
    ok = wg_observe(own_moved, (uint32_t)(d.nblk * (kMoeTokBlock / MT)), h, p.spin_limit, 0x30000000u, &slots);
    tr.put(KOS_TR_WAIT, 0xFFFFFE, t0);
  }
  if (ok) {
    const int nfb = (p.T + kFoldTokens - 1) / kFoldTokens;
    for (;;) {
      const uint32_t i = wg_claim(&h->head[5], h, &slots);
      if (i >= (uint32_t)nfb) break;
      const uint64_t t0 = tr.now();
      if (!fold_block<BM, true>(p, M, (int)i, &slots)) break;
      tr.put(KOS_TR_FOLD, i, t0);
    }
  }
  tr.finish(ticket);
  wg_exit(h, ps.base, ps.n_counters, &slots);
}

}  // namespace kos

using namespace kos;

extern "C" kos_status kos_moe_layer(const kos_moe_shape* s, const void* x, const float* logits,
                                    const void* const* peer_send, const int32_t* peer_counts,
                                    const void* w_gate, const void* w_up, const void* w_down,
                                    const void* const* peer_return, int32_t* topk_idx, float* topk_w,
                                    int32_t* counts, int32_t* perm, void* const* out_send,
                                    const int64_t* send_caps, void* x_grouped, int64_t grouped_cap,
                                    int32_t* grouped_offsets, int32_t* row_src, void* h, void* gate_save,
                                    void* up_save, void* y_grouped, void* const* out_return,
                                    const int64_t* return_caps, void* y, const kos_opts* opts, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!s) return fail(KOS_ERR_ARG, "shape is NULL");
  const int R = s->world, r = s->rank;
  if (R < 1 || R > 8) return fail(KOS_ERR_ARG, "world %d outside [1, 8]", R);
  if (r < 0 || r >= R) return fail(KOS_ERR_ARG, "rank %d outside [0, %d)", r, R);
  if (s->reserved) return fail(KOS_ERR_ARG, "reserved must be 0");
  using Sm = CombineTileSmall;   // the checks use the small tile's divisibility
  if (s->tokens < 0 || s->hidden <= 0 || s->hidden % Sm::BN || s->ffn <= 0 || s->ffn % (Sm::BN / 2) ||
      s->experts <= 0 || s->experts > kMoeMaxExperts || s->experts % R || s->experts / R > kMoeMaxLocal ||
      s->topk < 1 || s->topk > kMoeMaxTopk || s->topk > s->experts)
    return fail(KOS_ERR_SHAPE, "unsupported expert-layer shape (hidden %% %d, ffn %% %d)", Sm::BN, Sm::BN / 2);
  const bool no_tokens = s->tokens == 0;
  if ((!no_tokens && (!x || !logits || !topk_idx || !topk_w || !perm || !y)) || !peer_counts || !counts ||
      !x_grouped || !grouped_offsets || !row_src || !w_gate || !w_up || !w_down || !h || !y_grouped)
    return fail(KOS_ERR_ARG, "null buffer");
  if (R > 1 && (!peer_send || !out_send || !send_caps || !peer_return || !out_return || !return_caps))
    return fail(KOS_ERR_ARG, "a peer array is NULL");
  for (int q = 0; q < R; ++q) {
    if (q == r) continue;
    if (send_caps[q] < 0) return fail(KOS_ERR_ARG, "send_caps[%d] is negative", q);
    // NULL is allowed where nothing travels (checked on the device)
    if (!aligned16(peer_send[q]) || !aligned16(out_send[q]) || !aligned16(peer_return[q]) ||
        !aligned16(out_return[q]))
      return fail(KOS_ERR_ALIGN, "peer buffer not aligned");
  }
  if (!aligned16(x) || !aligned16(x_grouped) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(h) || !aligned16(y_grouped) || !aligned16(y) || !aligned16(gate_save) || !aligned16(up_save))
    return fail(KOS_ERR_ALIGN, "buffers must be 16-byte aligned");
  if ((gate_save == nullptr) != (up_save == nullptr))
    return fail(KOS_ERR_ARG, "gate_save and up_save are given together or not at all");
  if (grouped_cap < 0 || grouped_cap > (int64_t(1) << 31) - 1) return fail(KOS_ERR_ARG, "bad grouped_cap");
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
    return fail(KOS_ERR_UNSUPPORTED, "the single-launch layer is fused, two-way only (the two calls are the baseline)");

  const bool big = s->hidden % CombineTileBig::BN == 0 && s->ffn % (CombineTileBig::BN / 2) == 0;
  LayerParams lp{};
  DispatchParams& d = lp.d;
  d.world = R;
  d.rank = r;
  d.T = s->tokens;
  d.H = s->hidden;
  d.E = s->experts;
  d.k = s->topk;
  d.E_loc = s->experts / R;
  d.x = static_cast<const uint16_t*>(x);
  d.logits = logits;
  for (int q = 0; q < R; ++q) {
    d.peer_send[q] = q == r ? nullptr : static_cast<const uint16_t*>(peer_send[q]);
    d.out_send[q] = q == r ? nullptr : static_cast<uint16_t*>(out_send[q]);
    d.send_cap[q] = q == r ? 0 : send_caps[q];
  }
  d.peer_counts = peer_counts;
  d.topk_idx = topk_idx;
  d.topk_w = topk_w;
  d.counts = counts;
  d.perm = perm;
  d.x_grouped = static_cast<uint16_t*>(x_grouped);
  d.grouped_cap = grouped_cap;
  d.grouped_offsets = grouped_offsets;
  d.row_src = row_src;
  d.nblk = (s->tokens + kMoeTokBlock - 1) / kMoeTokBlock;
  d.do_route = d.do_copy = d.wait_scan = 1;
  d.spin_limit = o.spin_limit;
  d.ws = static_cast<WsHeader*>(ws);
  d.trace = trace_slot(ws, o.trace, 0);
  uint32_t* base = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kCountersOffset);
  d.ctr = base;
  char* scratch = static_cast<char*>(ws) + kScratchOffset;
  const size_t mask_bytes = (size_t)d.nblk * d.E * 8, base_bytes = (size_t)d.nblk * d.E * 4;
  if (d.nblk > 1024 || mask_bytes + base_bytes > kScratchBytes)
    return fail(KOS_ERR_SHAPE, "too many tokens (at most 65536) or tokens x experts for the workspace");
  d.masks = reinterpret_cast<unsigned long long*>(scratch);
  d.base = reinterpret_cast<int32_t*>(scratch + mask_bytes);

  CombineParams& p = lp.c;
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
  p.do_gu = p.do_dn = p.do_push = p.do_fold = 1;
  p.two_way = 1;
  p.wait_flags = 1;
  p.spin_limit = o.spin_limit;
  p.ws = d.ws;
  p.trace = d.trace;
  p.ctr = base + 3 + p.u_max;   // gu_done, dn_done
  lp.base = base;
  lp.n_counters = 3 + 3 * (uint32_t)p.u_max;
  if ((size_t)lp.n_counters > kMaxCounters) return fail(KOS_ERR_SHAPE, "grouped_cap too large for the workspace");

  hipStream_t strm = static_cast<hipStream_t>(stream);
  const bool save = gate_save != nullptr;
  if (big && save)
    hipLaunchKernelGGL((moe_layer_kernel<CombineTileBig, CombineTailBig, CombineTail2Big, true>), dim3(o.grid),
                       dim3(CombineTileBig::NT), 0, strm, lp);
  else if (big)
    hipLaunchKernelGGL((moe_layer_kernel<CombineTileBig, CombineTailBig, CombineTail2Big, false>), dim3(o.grid),
                       dim3(CombineTileBig::NT), 0, strm, lp);
  else if (save)
    hipLaunchKernelGGL((moe_layer_kernel<CombineTileSmall, CombineTailSmall, CombineTailSmall, true>), dim3(o.grid),
                       dim3(CombineTileSmall::NT), 0, strm, lp);
  else
    hipLaunchKernelGGL((moe_layer_kernel<CombineTileSmall, CombineTailSmall, CombineTailSmall, false>),
                       dim3(o.grid), dim3(CombineTileSmall::NT), 0, strm, lp);
  return launch_status("moe_layer launch");
}
