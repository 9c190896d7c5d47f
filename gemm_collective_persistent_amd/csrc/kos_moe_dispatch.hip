// Expert layer, dispatch direction, as one persistent kernel: router ->
// permutation -> token movement [KOSMOS arXiv abstract: the whole expert
// layer, routing through the final weighted sum, runs in one launch per
// direction; KOSMOS explainer, "Start with the problem": each token's row is
// sent to the rank that owns its expert].
//
// Queues and counters:
//   head[0]      router entries, one per quarter (16 tokens) of a block of
//                64 tokens: top-k of each token's logits (descending, ties
//                to the lowest expert index), softmax over the k, and, per
//                expert, the 16-bit quarter of the block's 64-bit mask of
//                tokens routed to it (order-free, so the result is
//                deterministic).
//   counter[0]   routed entries.
//   head[2]      scan entries, one per expert (once counter[0] is
//                complete): the expert's count and, per block, the pairs of
//                that expert in earlier blocks; counter[1] counts them.
//                Every mover then scans the counts itself (packed offsets,
//                grouped offsets of our local experts, capacity checks).
//   head[1]      mover entries (after counter[1]): kMoveTokens of our
//                tokens -- pair (t, j) of expert e lands at off[e] +
//                base[block][e] + popcount(mask & tokens before t); the row
//                goes to the send buffer of e's rank, or straight into the
//                grouped input when e is local -- then kMoveRows-row chunks of
//                each peer's rows, pulled into the grouped input.  Entries
//                are small (at most about 1 MB of traffic: one of our
//                tokens, or two peer rows, per wave) so that the workgroups
//                run out of them together.
#include "kos_host.h"
#include "kos_moe_dispatch.h"

namespace kos {

constexpr int kMoveTokens = 8;    // our tokens per mover entry (one per wave)

template <int NT>
__global__ __launch_bounds__(NT, 1) void moe_dispatch_kernel(DispatchParams args) {
  __shared__ DispatchLds L;
  __shared__ WgSlots slots;
  // The parameter block lives in LDS: each role reads the fields it needs
  // when it needs them instead of pinning them all in scalar registers.
  __shared__ DispatchParams ps;
  if (threadIdx.x == 0) ps = args;
  __syncthreads();
  const DispatchParams& p = ps;
  WsHeader* h = p.ws;
  Tracer tr(p.trace);
  const uint32_t ticket = wg_ticket(h, &slots);

  dispatch_prologue<kMoveTokens>(p, L);

  // ---- router role, then one scan entry per expert ---------------------
  if (p.do_route) {
    const uint32_t n_route = (uint32_t)p.nblk * 4;
    for (;;) {
      const uint32_t b4 = wg_claim(&h->head[0], h, &slots);
      if (b4 >= n_route) break;
      const uint64_t t0 = tr.now();
      route_any<NT / 64>(p, (int)b4, L);
      // this entry's device-coherent stores have completed: count it
      wg_publish(&p.ctr[0], 1u);
      tr.put(KOS_TR_ROUTE, b4, t0);
    }
    for (;;) {
      const uint32_t e = wg_claim(&h->head[2], h, &slots);
      if (e >= (uint32_t)p.E) break;
      uint64_t t0 = tr.now();
      if (!wg_observe(&p.ctr[0], n_route, h, p.spin_limit, 0xFFFE0000u | e, &slots)) break;
      tr.put(KOS_TR_WAIT, e, t0);
      t0 = tr.now();
      scan_expert(p, L, (int)e);
      wg_publish(&p.ctr[1], 1u);
      tr.put(KOS_TR_SCAN, e, t0);
    }
  }

  // ---- mover role -------------------------------------------------------
  if (p.do_copy) {
    const int n_entries = L.n_entries;
    const uint64_t tw = tr.now();
    bool go_on = !p.wait_scan || wg_observe(&p.ctr[1], (uint32_t)p.E, h, p.spin_limit, 0xFFFF0000u, &slots);
    if (go_on) go_on = load_meta(p, L, &slots, ticket == 0);
    tr.put(KOS_TR_WAIT, 0xFFFFFF, tw);
    for (;;) {
      if (!go_on) break;
      const uint32_t i = wg_claim(&h->head[1], h, &slots);
      if (i >= (uint32_t)n_entries) break;
      const uint64_t t0 = tr.now();
      move_entry<kMoveTokens, false>(p, L, (int)i, [](int, int) {});
      tr.put_wg(KOS_TR_MOVE, i, t0);
    }
  }
  tr.finish(ticket);
  wg_exit(h, p.ctr, 2, &slots);
}

}  // namespace kos

using namespace kos;

extern "C" kos_status kos_moe_dispatch(const kos_moe_shape* s, const void* x, const float* logits,
                                       const void* const* peer_send, const int32_t* peer_counts, int32_t* topk_idx,
                                       float* topk_w, int32_t* counts, int32_t* perm, void* const* out_send,
                                       const int64_t* send_caps, void* x_grouped, int64_t grouped_cap,
                                       int32_t* grouped_offsets, int32_t* row_src, const kos_opts* opts, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!s) return fail(KOS_ERR_ARG, "shape is NULL");
  const int R = s->world, r = s->rank;
  if (R < 1 || R > 8) return fail(KOS_ERR_ARG, "world %d outside [1, 8]", R);
  if (r < 0 || r >= R) return fail(KOS_ERR_ARG, "rank %d outside [0, %d)", r, R);
  if (s->reserved) return fail(KOS_ERR_ARG, "reserved must be 0");
  if (s->tokens < 0 || s->hidden <= 0 || s->hidden % 64 || s->experts <= 0 || s->experts > kMoeMaxExperts ||
      s->experts % R || s->experts / R > kMoeMaxLocal || s->topk < 1 || s->topk > kMoeMaxTopk ||
      s->topk > s->experts || s->ffn <= 0)
    return fail(KOS_ERR_SHAPE, "unsupported expert-layer shape");
  // per-token buffers may be NULL for an empty batch (nothing reads them)
  const bool no_tokens = s->tokens == 0;
  if ((!no_tokens && (!x || !logits || !topk_idx || !topk_w || !perm)) || !peer_counts || !counts || !x_grouped ||
      !grouped_offsets || !row_src)
    return fail(KOS_ERR_ARG, "null buffer");
  if (R > 1 && (!peer_send || !out_send || !send_caps))
    return fail(KOS_ERR_ARG, "peer_send / out_send / send_caps is NULL");
  for (int q = 0; q < R; ++q)
    if (q != r && send_caps[q] < 0) return fail(KOS_ERR_ARG, "send_caps[%d] is negative", q);
  for (int q = 0; q < R; ++q) {
    if (q == r) continue;
    // NULL is allowed where nothing travels (checked on the device)
    if (!aligned16(peer_send[q]) || !aligned16(out_send[q])) return fail(KOS_ERR_ALIGN, "peer buffer not aligned");
  }
  if (!aligned16(x) || !aligned16(x_grouped)) return fail(KOS_ERR_ALIGN, "row buffers must be 16-byte aligned");
  if (grouped_cap < 0 || grouped_cap > (int64_t(1) << 31) - 1)
    return fail(KOS_ERR_ARG, "bad capacity");
  kos_status st = check_workspace(ws, ws_bytes);
  if (st != KOS_OK) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != KOS_OK) return st;
  kos_opts o;
  if ((st = resolve_opts(opts, dev, CrewDefaults{16, 8, 16, 8}, &o)) != KOS_OK) return st;
  if (o.mode == KOS_MODE_FIXED) return fail(KOS_ERR_UNSUPPORTED, "dispatch has no compute role to split from");

  DispatchParams p{};
  p.world = R;
  p.rank = r;
  p.T = s->tokens;
  p.H = s->hidden;
  p.E = s->experts;
  p.k = s->topk;
  p.E_loc = s->experts / R;
  p.x = static_cast<const uint16_t*>(x);
  p.logits = logits;
  for (int q = 0; q < R; ++q) {
    p.peer_send[q] = q == r ? nullptr : static_cast<const uint16_t*>(peer_send[q]);
    p.out_send[q] = q == r ? nullptr : static_cast<uint16_t*>(out_send[q]);
  }
  p.peer_counts = peer_counts;
  p.topk_idx = topk_idx;
  p.topk_w = topk_w;
  p.counts = counts;
  p.perm = perm;
  for (int q = 0; q < R; ++q) p.send_cap[q] = q == r ? 0 : send_caps[q];
  p.x_grouped = static_cast<uint16_t*>(x_grouped);
  p.grouped_cap = grouped_cap;
  p.grouped_offsets = grouped_offsets;
  p.row_src = row_src;
  p.nblk = (s->tokens + kMoeTokBlock - 1) / kMoeTokBlock;
  p.spin_limit = o.spin_limit;
  p.ws = static_cast<WsHeader*>(ws);
  p.trace = trace_slot(ws, o.trace, 0);
  p.ctr = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kCountersOffset);
  char* scratch = static_cast<char*>(ws) + kScratchOffset;
  const size_t mask_bytes = (size_t)p.nblk * p.E * 8, base_bytes = (size_t)p.nblk * p.E * 4;
  if (p.nblk > 1024 || mask_bytes + base_bytes > kScratchBytes)
    return fail(KOS_ERR_SHAPE, "too many tokens (at most 65536) or tokens x experts for the workspace");
  p.masks = reinterpret_cast<unsigned long long*>(scratch);
  p.base = reinterpret_cast<int32_t*>(scratch + mask_bytes);

  hipStream_t strm = static_cast<hipStream_t>(stream);
  constexpr int NT = 512;   // eight waves: two rows in flight per SIMD while moving
  if (o.mode == KOS_MODE_UNFUSED) {
    DispatchParams a = p;   // launch 1: router + scan
    a.do_route = 1;
    a.do_copy = 0;
    hipLaunchKernelGGL(moe_dispatch_kernel<NT>, dim3(o.grid), dim3(NT), 0, strm, a);
    if ((st = launch_status("moe_dispatch route launch")) != KOS_OK) return st;
    DispatchParams b = p;   // launch 2: token movement
    b.trace = trace_slot(ws, o.trace, 1);
    b.do_route = 0;
    b.do_copy = 1;
    b.wait_scan = 0;
    hipLaunchKernelGGL(moe_dispatch_kernel<NT>, dim3(o.grid), dim3(NT), 0, strm, b);
    return launch_status("moe_dispatch copy launch");
  }
  p.do_route = 1;
  p.do_copy = 1;
  p.wait_scan = 1;
  hipLaunchKernelGGL(moe_dispatch_kernel<NT>, dim3(o.grid), dim3(NT), 0, strm, p);
  return launch_status("moe_dispatch launch");
}
