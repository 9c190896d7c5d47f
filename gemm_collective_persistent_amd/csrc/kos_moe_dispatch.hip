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
//                are small (about 0.5 MB of traffic) so that the workgroups
//                run out of them together.
#include "kos_host.h"
#include "kos_moe.h"

namespace kos {

constexpr int kMoveTokens = 4;    // our tokens per mover entry
constexpr int kMoveRows = 16;     // peer rows per mover entry
constexpr int kMoveSubs = kMoeTokBlock / kMoveTokens;   // own entries per 64-token block

struct DispatchParams {
  int32_t world, rank, T, H, E, k, E_loc;
  const uint16_t* x;
  const float* logits;
  const uint16_t* peer_send[8];
  const int32_t* peer_counts;   // [world, E_loc]
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* perm;
  uint16_t* out_send[8];
  int64_t send_cap[8];          // rows out_send[d] holds
  uint16_t* x_grouped;
  int64_t grouped_cap;
  int32_t* grouped_offsets;
  int32_t* row_src;
  int32_t nblk;
  int32_t do_route, do_copy, wait_scan;
  uint32_t spin_limit;
  WsHeader* ws;
  kos_trace_rec* trace;          // null: tracing off
  uint32_t* ctr;                 // [0] routed blocks, [1] scan done
  unsigned long long* masks;     // scratch [nblk, E]
  int32_t* base;                 // scratch [nblk, E]: pairs of expert e in blocks before b
};

struct DispatchLds {
  uint32_t m[kMoeMaxExperts];           // router: 16-bit token masks of one entry
  int32_t cnt[kMoeMaxExperts];          // scan: per-expert counts
  int32_t wave_tot[4];
  int32_t off[kMoeMaxExperts + 1];
  int32_t pc[8][kMoeMaxLocal];          // peer counts (row `rank` = our own local counts after the scan)
  int32_t cum[8][kMoeMaxLocal + 1];     // per-source prefix over local experts
  int32_t before[8][kMoeMaxLocal];      // rows of sources < p, per local expert
  int32_t go[kMoeMaxLocal + 1];         // grouped offsets
  int32_t chunk_base[9];                // first peer entry of each source
};

// Order-preserving key of a (logit, expert) candidate: larger logit first,
// equal logits (+0 and -0 included) to the lower expert index.  Key 0 means
// "no candidate" (every real key is larger).
__device__ __forceinline__ uint64_t cand_key(float v, int e) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);   // -0 -> +0
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~e;
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __builtin_bit_cast(float, (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)~(uint32_t)k; }

// One step of a wave-wide maximum over 64-bit keys through DPP lane moves;
// lanes outside ROW_MASK keep their own key.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t key_max_dpp(uint64_t k) {
  const int lo = (int)(uint32_t)k, hi = (int)(uint32_t)(k >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > k ? o : k;
}

// Largest key of the wave, in every lane: within quads (swap 1, swap 2),
// within rows of 16 (half-row mirror, row mirror), then across rows
// (broadcast of lane 15 into rows 1 and 3, of lane 31 into rows 2 and 3),
// leaving the maximum in lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = key_max_dpp<0xB1, 0xF>(k);    // quad_perm [1,0,3,2]
  k = key_max_dpp<0x4E, 0xF>(k);    // quad_perm [2,3,0,1]
  k = key_max_dpp<0x141, 0xF>(k);   // row_half_mirror
  k = key_max_dpp<0x140, 0xF>(k);   // row_mirror
  k = key_max_dpp<0x142, 0xA>(k);   // row_bcast:15
  k = key_max_dpp<0x143, 0xC>(k);   // row_bcast:31
  return readlane_u64(k, 63);
}

// Sum over the wave (every lane gets it).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Router entry `b4`: tokens [16*b4, 16*b4 + 16) = quarter b4 % 4 of block b4 / 4.
// Each wave takes every 4th token; all its tokens' logits are loaded
// before the first selection.  NV: 64-logit slots per lane (E <= 64*NV).
// Lane j keeps the j-th selection of the token being routed.
template <int NV>
__device__ __forceinline__ void route_entry(const DispatchParams& p, int b4, DispatchLds& L) {
  constexpr int QT = kMoeTokBlock / 4;
  constexpr int TPW = QT / 4;                 // tokens per wave (4 waves)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) L.m[e] = 0u;
  __syncthreads();
  float v[TPW][NV];
#pragma unroll
  for (int x = 0; x < TPW; ++x) {
    const int t = b4 * QT + wave + 4 * x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      v[x][i] = (t < p.T && e < p.E) ? p.logits[(int64_t)t * p.E + e] : 0.f;
    }
  }
  const int k = p.k;
  // the wave's TPW tokens select side by side (independent reduction
  // chains interleave); tokens past T select garbage and store nothing
  uint32_t taken[TPW];
  float my_v[TPW];   // selection `lane` (lanes < k)
  int my_i[TPW];
#pragma unroll
  for (int x = 0; x < TPW; ++x) {
    taken[x] = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i >= p.E) taken[x] |= 1u << i;
    my_v[x] = 0.f;
    my_i[x] = 0;
  }
  for (int j = 0; j < k; ++j) {
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
      // this lane's best remaining candidate, then the wave's
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const uint64_t kk = ((taken[x] >> i) & 1u) ? 0 : cand_key(v[x][i], lane + 64 * i);
        best = kk > best ? kk : best;
      }
      const uint64_t win = wave_max_key(best);
      const int wi = key_index(win);
      if (lane == j) {
        my_v[x] = key_value(win);
        my_i[x] = wi;
      }
      if ((wi & 63) == lane) taken[x] |= 1u << (wi >> 6);
    }
  }
#pragma unroll
  for (int x = 0; x < TPW; ++x) {
    const int tl = wave + 4 * x;
    const int t = b4 * QT + tl;
    // softmax over the k selected logits (largest first)
    const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, my_v[x])));
    const float z = lane < k ? expf(my_v[x] - v0) : 0.f;
    const float w = z / wave_sum(z);
    if (t < p.T && lane < k) {
      // read by other workgroups of this launch: device-coherent stores
      st_dev_b32(&p.topk_idx[(int64_t)t * k + lane], (uint32_t)my_i[x]);
      st_dev_b32(&p.topk_w[(int64_t)t * k + lane], __builtin_bit_cast(uint32_t, w));
      atomicOr(&L.m[my_i[x]], 1u << tl);
    }
  }
  __syncthreads();
  // quarter q of the block's 64-bit mask: its 16-bit lane q (little endian),
  // stored device-coherent (the scan runs in another workgroup)
  const int b = b4 >> 2, q = b4 & 3;
  const DevBuf mb(p.masks + (int64_t)b * p.E);
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) mb.st16((uint32_t)(e * 8 + q * 2), (uint16_t)L.m[e]);
}

// Scan entry: expert e, once every router entry is counted.  Its block
// masks -> per-block counts -> exclusive prefix over the blocks:
// base[b][e] = pairs of e in blocks before b (relative to e's packed
// offset), counts[e] = total.  Stored device-coherent (movers of this launch
// read them after counter[1]).  nblk <= 1024.
__device__ __forceinline__ void scan_expert(const DispatchParams& p, DispatchLds& L, int e) {
  for (int b = threadIdx.x; b < p.nblk; b += blockDim.x)
    L.cnt[b] = __popcll(ld_dev_b64(&p.masks[(int64_t)b * p.E + e]));
  __syncthreads();
  block_exclusive_scan(L.cnt, L.off, p.nblk, L.wave_tot);
  for (int b = threadIdx.x; b < p.nblk; b += blockDim.x) st_dev_b32(&p.base[(int64_t)b * p.E + e], (uint32_t)L.off[b]);
  if (threadIdx.x == 0) st_dev_b32(&p.counts[e], (uint32_t)L.off[p.nblk]);
  __syncthreads();
}

// After counter[1] (every expert scanned): the packed offsets (exclusive
// scan of the counts), our local experts' grouped offsets and the
// per-source prefixes, in LDS; every mover computes the same values.
// Capacity checks: an overflow records KOS_ERR_CAPACITY and returns false
// (every thread).  `writer` stores the grouped offsets (an output).
__device__ __forceinline__ bool load_meta(const DispatchParams& p, DispatchLds& L, WgSlots* slots, bool writer) {
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) L.cnt[e] = (int32_t)ld_dev_b32(&p.counts[e]);
  __syncthreads();
  block_exclusive_scan(L.cnt, L.off, p.E, L.wave_tot);
  for (int el = threadIdx.x; el < p.E_loc; el += blockDim.x) {
    const int ge = p.rank * p.E_loc + el;
    L.pc[p.rank][el] = L.off[ge + 1] - L.off[ge];
  }
  __syncthreads();
  for (int el = threadIdx.x; el < p.E_loc; el += blockDim.x) {
    int run = 0;
    for (int q = 0; q < p.world; ++q) {
      L.before[q][el] = run;
      run += L.pc[q][el];
    }
  }
  if (threadIdx.x == 0) {
    bool over = false;
    bool null_send = false;
    for (int d = 0; d < p.world; ++d) {
      if (d == p.rank) continue;
      const int sent = L.off[(d + 1) * p.E_loc] - L.off[d * p.E_loc];
      if (sent > p.send_cap[d]) over = true;
      if (sent > 0 && p.out_send[d] == nullptr) null_send = true;   // rows for a NULL buffer
    }
    int64_t go = 0;
    for (int el = 0; el < p.E_loc; ++el) {
      L.go[el] = (int32_t)go;
      for (int q = 0; q < p.world; ++q) go += L.pc[q][el];
    }
    L.go[p.E_loc] = (int32_t)go;
    if (go > p.grouped_cap) over = true;
    if (over) raise_error(p.ws, KOS_ERR_CAPACITY, (uint32_t)go);
    if (null_send) raise_error(p.ws, KOS_ERR_ARG, 0x00B00000u);
    slots->ok = over || null_send ? 0 : 1;
  }
  __syncthreads();
  if (writer && slots->ok)
    for (int el = threadIdx.x; el <= p.E_loc; el += blockDim.x) p.grouped_offsets[el] = L.go[el];
  return slots->ok != 0;
}

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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = NT / 64;
  Tracer tr(p.trace);
  const uint32_t ticket = wg_ticket(h, &slots);

  // peer counts (inputs) and the per-source prefixes
  for (int i = threadIdx.x; i < p.world * p.E_loc; i += NT) {
    const int q = i / p.E_loc, el = i % p.E_loc;
    L.pc[q][el] = q == p.rank ? 0 : p.peer_counts[i];
  }
  __syncthreads();
  // a peer whose send buffer is NULL must send nothing: else this
  // workgroup takes its rows as absent (never reads the NULL buffer) and
  // the call reports KOS_ERR_ARG
  if (threadIdx.x < p.world && threadIdx.x != p.rank && p.peer_send[threadIdx.x] == nullptr) {
    bool any = false;
    for (int el = 0; el < p.E_loc; ++el) any |= L.pc[threadIdx.x][el] != 0;
    if (any) {
      raise_error(p.ws, KOS_ERR_ARG, 0x00A00000u | threadIdx.x);
      for (int el = 0; el < p.E_loc; ++el) L.pc[threadIdx.x][el] = 0;
    }
  }
  __syncthreads();
  if (threadIdx.x < p.world) {
    const int q = threadIdx.x;
    int run = 0;
    for (int el = 0; el < p.E_loc; ++el) {
      L.cum[q][el] = run;
      run += L.pc[q][el];
    }
    L.cum[q][p.E_loc] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int nb = p.nblk * kMoveSubs;
    for (int q = 0; q < p.world; ++q) {
      L.chunk_base[q] = nb;
      if (q != p.rank) nb += (L.cum[q][p.E_loc] + kMoveRows - 1) / kMoveRows;
    }
    L.chunk_base[p.world] = nb;
  }
  __syncthreads();

  // ---- router role, then one scan entry per expert ---------------------
  if (p.do_route) {
    const uint32_t n_route = (uint32_t)p.nblk * 4;
    for (;;) {
      const uint32_t b4 = wg_claim(&h->head[0], h, &slots);
      if (b4 >= n_route) break;
      const uint64_t t0 = tr.now();
      if (p.E <= 64) route_entry<1>(p, (int)b4, L);
      else if (p.E <= 128) route_entry<2>(p, (int)b4, L);
      else if (p.E <= 256) route_entry<4>(p, (int)b4, L);
      else if (p.E <= 512) route_entry<8>(p, (int)b4, L);
      else route_entry<16>(p, (int)b4, L);
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
    const int n_entries = L.chunk_base[p.world];
    const uint64_t tw = tr.now();
    bool go_on = !p.wait_scan || wg_observe(&p.ctr[1], (uint32_t)p.E, h, p.spin_limit, 0xFFFF0000u, &slots);
    if (go_on) go_on = load_meta(p, L, &slots, ticket == 0);
    tr.put(KOS_TR_WAIT, 0xFFFFFF, tw);
    for (;;) {
      if (!go_on) break;
      const uint32_t i = wg_claim(&h->head[1], h, &slots);
      if (i >= (uint32_t)n_entries) break;
      const uint64_t t0 = tr.now();
      const int H = p.H;
      const int row_bytes = H * 2;
      if ((int)i < p.nblk * kMoveSubs) {
        // kMoveTokens of our tokens, one token per wave at a time
        const int b = (int)i / kMoveSubs, q = (int)i % kMoveSubs;
        for (int tq = wave; tq < kMoveTokens; tq += nw) {
          const int tl = q * kMoveTokens + tq;
          const int t = b * kMoeTokBlock + tl;
          if (t >= p.T) break;
          uint16_t* dst[kMoeMaxTopk];
#pragma unroll
          for (int j = 0; j < kMoeMaxTopk; ++j) {
            if (j >= p.k) break;
            const int e = (int)ld_dev_b32(&p.topk_idx[(int64_t)t * p.k + j]);
            const unsigned long long m = ld_dev_b64(&p.masks[(int64_t)b * p.E + e]);
            const int pos = L.off[e] + (int)ld_dev_b32(&p.base[(int64_t)b * p.E + e]) + __popcll(m & ((1ull << tl) - 1ull));
            const int d = e / p.E_loc;
            if (lane == j) p.perm[(int64_t)t * p.k + j] = pos;
            if (d != p.rank) {
              dst[j] = p.out_send[d] + (int64_t)(pos - L.off[d * p.E_loc]) * H;
            } else {
              const int el = e - p.rank * p.E_loc;
              const int64_t grow = (int64_t)L.go[el] + L.before[p.rank][el] + (pos - L.off[e]);
              dst[j] = p.x_grouped + grow * H;
              if (lane == 0) {
                p.row_src[grow * 2] = p.rank;
                p.row_src[grow * 2 + 1] = pos - L.off[p.rank * p.E_loc];
              }
            }
          }
          // the whole row in registers (up to 16 chunks per lane per pass),
          // then one copy per destination
          const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (int64_t)t * H);
          const int nc = row_bytes / 16;
          constexpr int U = 16;
          for (int c0 = lane; c0 < nc; c0 += U * 64) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
              if (c0 + u * 64 < nc) v[u] = src[c0 + u * 64];
#pragma unroll
            for (int j = 0; j < kMoeMaxTopk; ++j) {
              if (j >= p.k) break;
              u32x4* d = reinterpret_cast<u32x4*>(wave_uniform(dst[j]));
#pragma unroll
              for (int u = 0; u < U; ++u)
                if (c0 + u * 64 < nc) d[c0 + u * 64] = v[u];
            }
          }
        }
      } else {
        // a chunk of kMoveRows rows peer q sent us, pulled into the grouped input
        int q = 0;
        while (q + 1 <= p.world && L.chunk_base[q + 1] <= (int)i) ++q;
        const int r0 = ((int)i - L.chunk_base[q]) * kMoveRows;
        const int n_q = L.cum[q][p.E_loc];
        for (int rr = wave; rr < kMoveRows; rr += nw) {
          const int r = r0 + rr;
          if (r >= n_q) break;
          int el = 0;
          while (el + 1 < p.E_loc && L.cum[q][el + 1] <= r) ++el;
          const int64_t grow = (int64_t)L.go[el] + L.before[q][el] + (r - L.cum[q][el]);
          wave_copy_row(p.x_grouped + grow * H, p.peer_send[q] + (int64_t)r * H, row_bytes);
          if (lane == 0) {
            p.row_src[grow * 2] = q;
            p.row_src[grow * 2 + 1] = r;
          }
        }
      }
      tr.put(KOS_TR_MOVE, i, t0);
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
  constexpr int NT = 256;
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
