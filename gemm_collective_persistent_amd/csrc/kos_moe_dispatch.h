// Expert layer, dispatch-direction pieces shared by the dispatch kernel and
// the single-launch expert layer: the router, the per-expert scan, the
// layer's bookkeeping and the token movers (see kos_moe_dispatch.hip for
// the queues they run under).
#pragma once

#include "kos_moe.h"

namespace kos {

constexpr int kMoveRows = 16;     // peer rows per mover entry

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
  int32_t wave_tot[16];
  int32_t off[kMoeMaxExperts + 1];
  int32_t pc[8][kMoeMaxLocal];          // peer counts (row `rank` = our own local counts after the scan)
  int32_t cum[8][kMoeMaxLocal + 1];     // per-source prefix over local experts
  int32_t before[8][kMoeMaxLocal];      // rows of sources < p, per local expert
  int32_t go[kMoeMaxLocal + 1];         // grouped offsets
  int32_t go_over;                      // the grouped rows exceed grouped_cap
  int32_t own_entries;                  // mover entries of our own tokens
  int32_t n_entries;                    // all mover entries
  int32_t chunk_base[9];                // first entry of each source's rows
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
// Each of the NW waves takes every NW-th token; all its tokens' logits are
// loaded before the first selection.  NV: 64-logit slots per lane (E <=
// 64*NV).  Lane j keeps the j-th selection of the token being routed.
template <int NV, int NW>
__device__ __forceinline__ void route_entry(const DispatchParams& p, int b4, DispatchLds& L) {
  constexpr int QT = kMoeTokBlock / 4;
  constexpr int TPW = QT / NW;                // tokens per wave
  static_assert(QT % NW == 0, "whole tokens per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) L.m[e] = 0u;
  __syncthreads();
  float v[TPW][NV];
#pragma unroll
  for (int x = 0; x < TPW; ++x) {
    const int t = b4 * QT + wave + NW * x;
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
    const int tl = wave + NW * x;
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
  // one lane per local expert (E_loc <= 64): the rows of the sources before
  // q, then the grouped offsets as a wave-wide exclusive prefix of the
  // experts' totals, in 64 bits so that the capacity check sees any overflow
  // (a single thread walking every (expert, source) pair took ~10 us)
  if (threadIdx.x < 64) {
    const int el = threadIdx.x;
    int64_t run = 0;
    if (el < p.E_loc)
      for (int q = 0; q < p.world; ++q) {
        L.before[q][el] = (int32_t)run;
        run += L.pc[q][el];
      }
    int64_t incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t o = __shfl_up(incl, d);
      if (el >= d) incl += o;
    }
    if (el < p.E_loc) L.go[el] = (int32_t)(incl - run);
    if (el == p.E_loc - 1) {
      L.go[p.E_loc] = (int32_t)incl;
      L.go_over = incl > p.grouped_cap ? 1 : 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    bool over = L.go_over != 0;
    bool null_send = false;
    for (int d = 0; d < p.world; ++d) {
      if (d == p.rank) continue;
      const int sent = L.off[(d + 1) * p.E_loc] - L.off[d * p.E_loc];
      if (sent > p.send_cap[d]) over = true;
      if (sent > 0 && p.out_send[d] == nullptr) null_send = true;   // rows for a NULL buffer
    }
    if (over) raise_error(p.ws, KOS_ERR_CAPACITY, (uint32_t)L.go[p.E_loc]);
    if (null_send) raise_error(p.ws, KOS_ERR_ARG, 0x00B00000u);
    slots->ok = over || null_send ? 0 : 1;
  }
  __syncthreads();
  if (writer && slots->ok)
    for (int el = threadIdx.x; el <= p.E_loc; el += blockDim.x) p.grouped_offsets[el] = L.go[el];
  return slots->ok != 0;
}


// A router entry for any expert count (the logit slots per lane chosen by E).
template <int NW>
__device__ __forceinline__ void route_any(const DispatchParams& p, int b4, DispatchLds& L) {
  if (p.E <= 64) route_entry<1, NW>(p, b4, L);
  else if (p.E <= 128) route_entry<2, NW>(p, b4, L);
  else if (p.E <= 256) route_entry<4, NW>(p, b4, L);
  else if (p.E <= 512) route_entry<8, NW>(p, b4, L);
  else route_entry<16, NW>(p, b4, L);
}

// Every workgroup's copy of the peers' counts (row `rank` zero) and their
// per-source prefixes, in LDS, and the first mover entry of each source's
// rows (MT of our tokens per own entry).  A peer whose send buffer is NULL
// must send nothing: else this workgroup takes its rows as absent (never
// reads the NULL buffer) and the call reports KOS_ERR_ARG.
template <int MT>
__device__ __forceinline__ void dispatch_prologue(const DispatchParams& p, DispatchLds& L) {
  for (int i = threadIdx.x; i < p.world * p.E_loc; i += blockDim.x) {
    const int q = i / p.E_loc, el = i % p.E_loc;
    L.pc[q][el] = q == p.rank ? 0 : p.peer_counts[i];
  }
  __syncthreads();
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
  // peer rows are pulled source after source, each source's rows in its own
  // (expert-major) order: long contiguous reads of each peer's buffer
  // (pulling them in the grouped input's expert-then-source order instead
  // was measured slower, for the dispatch and for the single-launch layer)
  if (threadIdx.x == 0) {
    const int own = p.nblk * (kMoeTokBlock / MT);
    int nb = own;
    for (int q = 0; q < p.world; ++q) {
      L.chunk_base[q] = nb;
      if (q != p.rank) nb += (L.cum[q][p.E_loc] + kMoveRows - 1) / kMoveRows;
    }
    L.chunk_base[p.world] = nb;
    L.own_entries = own;
    L.n_entries = nb;
  }
  __syncthreads();
}

// Waits until this wave's stores have completed (vmcnt 0): what a wave
// publishes afterwards is ordered after them.
__device__ __forceinline__ void wave_stores_done() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8)); }

// Mover entry i (after load_meta).  Entries below nblk * 64/MT are MT of
// our tokens each, one token per wave at a time: pair (t, j) of expert e
// lands at its packed position, in the send buffer of e's rank or, when e is
// local, straight in the grouped input.  The rest are kMoveRows-row chunks
// of what each peer sent us, pulled into the grouped input.  COH: the
// grouped rows and their provenance are read later in the same launch --
// device-coherent stores, and sink(grouped row, local expert) is called (by
// every lane of the wave) once each row's stores have completed.
template <int MT, bool COH, class Sink>
__device__ __forceinline__ void move_entry(const DispatchParams& p, const DispatchLds& L, int i, Sink&& sink) {
  constexpr int SUBS = kMoeTokBlock / MT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int H = p.H;
  const int row_bytes = H * 2;
  if (i < p.nblk * SUBS) {
    const int b = i / SUBS, q = i % SUBS;
    for (int tq = wave; tq < MT; tq += nw) {
      const int tl = q * MT + tq;
      const int t = b * kMoeTokBlock + tl;
      if (t >= p.T) break;
      uint16_t* dst[kMoeMaxTopk];
      int gr[kMoeMaxTopk];   // grouped row of a local destination, else -1
      int ge[kMoeMaxTopk];   // its local expert
#pragma unroll
      for (int j = 0; j < kMoeMaxTopk; ++j) {
        gr[j] = -1;
        ge[j] = 0;
        if (j >= p.k) break;
        const int e = (int)ld_dev_b32(&p.topk_idx[(int64_t)t * p.k + j]);
        const unsigned long long m = ld_dev_b64(&p.masks[(int64_t)b * p.E + e]);
        const int pos = L.off[e] + (int)ld_dev_b32(&p.base[(int64_t)b * p.E + e]) + __popcll(m & ((1ull << tl) - 1ull));
        const int d = e / p.E_loc;
        if (lane == j) {
          if constexpr (COH) st_dev_b32(&p.perm[(int64_t)t * p.k + j], (uint32_t)pos);
          else p.perm[(int64_t)t * p.k + j] = pos;
        }
        if (d != p.rank) {
          dst[j] = p.out_send[d] + (int64_t)(pos - L.off[d * p.E_loc]) * H;
        } else {
          const int el = e - p.rank * p.E_loc;
          const int64_t grow = (int64_t)L.go[el] + L.before[p.rank][el] + (pos - L.off[e]);
          gr[j] = (int)grow;
          ge[j] = el;
          dst[j] = p.x_grouped + grow * H;
          const int src_row = pos - L.off[p.rank * p.E_loc];
          if constexpr (COH) {
            if (lane == 0) st_dev_b32(&p.row_src[grow * 2], (uint32_t)p.rank);
            if (lane == 1) st_dev_b32(&p.row_src[grow * 2 + 1], (uint32_t)src_row);
          } else if (lane == 0) {
            p.row_src[grow * 2] = p.rank;
            p.row_src[grow * 2 + 1] = src_row;
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
          if (COH && gr[j] >= 0) {
            const DevBuf db(dst[j]);
#pragma unroll
            for (int u = 0; u < U; ++u)
              if (c0 + u * 64 < nc) db.st128((uint32_t)(c0 + u * 64) * 16u, v[u]);
          } else {
            u32x4* d = reinterpret_cast<u32x4*>(wave_uniform(dst[j]));
#pragma unroll
            for (int u = 0; u < U; ++u)
              if (c0 + u * 64 < nc) d[c0 + u * 64] = v[u];
          }
        }
      }
      if constexpr (COH) {
        wave_stores_done();
#pragma unroll
        for (int j = 0; j < kMoeMaxTopk; ++j) {
          if (j >= p.k) break;
          if (gr[j] >= 0) sink(gr[j], ge[j]);
        }
      }
    }
  } else {
    // a chunk of kMoveRows rows peer q sent us, pulled into the grouped input
    int q = 0;
    while (q + 1 <= p.world && L.chunk_base[q + 1] <= i) ++q;
    const int r0 = (i - L.chunk_base[q]) * kMoveRows;
    const int n_q = L.cum[q][p.E_loc];
    for (int rr = wave; rr < kMoveRows; rr += nw) {
      const int r = r0 + rr;
      if (r >= n_q) break;
      int el = 0;
      while (el + 1 < p.E_loc && L.cum[q][el + 1] <= r) ++el;
      const int64_t grow = (int64_t)L.go[el] + L.before[q][el] + (r - L.cum[q][el]);
      if constexpr (COH) {
        wave_copy_row_dev_dst(p.x_grouped + grow * H, p.peer_send[q] + (int64_t)r * H, row_bytes);
        if (lane == 0) st_dev_b32(&p.row_src[grow * 2], (uint32_t)q);
        if (lane == 1) st_dev_b32(&p.row_src[grow * 2 + 1], (uint32_t)r);
        wave_stores_done();
        sink((int)grow, el);
      } else {
        wave_copy_row(p.x_grouped + grow * H, p.peer_send[q] + (int64_t)r * H, row_bytes);
        if (lane == 0) {
          p.row_src[grow * 2] = q;
          p.row_src[grow * 2 + 1] = r;
        }
      }
    }
  }
}

}  // namespace kos
