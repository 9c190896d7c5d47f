// GEMM + reduce-scatter as one persistent kernel (one rank's share).
//
// [KOSMOS explainer, "Start with the problem"]: after a row-parallel GEMM
// each rank's partial sums are split by rows over the ranks and summed.
// ["Role switching only works if ..."]: tiles come out one band of rows at a
// time, covering that band in every rank's chunk, so summing can begin once
// the first band exists; finishing one chunk before the next is the slower
// ablation.  ["KOSMOS removes the manager"]: a builder that finds no tile
// left turns reducer for good (one-way switch).
//
// Chunk c = rows [c*mc, (c+1)*mc), mc = m/world; band b of a chunk = its
// rows [b*BM, (b+1)*BM).
// Queues:
//   head[1]  tiles.  Band order: band b, then chunk c ascending, then
//            column tile.  Row order: chunk c, then band, then column tile.
//            Every tile stores its fp32 partial into `partial` (rows of
//            chunk c != rank stand for the push into rank c's inbox); tiles
//            of our own chunk then bump ready[band * tiles_n + col].
//   head[2]  reduce entries (band b, column tile, 32-row slab) of our own
//            chunk, in that order: y = sum_p X_p in ascending p (fp32),
//            X_rank = partial[chunk rank], X_p = peer_slices[p].  Gated on
//            the ready counter of our own tile at (b, column).  The peers'
//            slices of a band are taken as ready together with ours: every
//            rank runs the same order at the same pace.
//
// MXFP8 variant (same kernel, MX tile shape): A and W are E4M3 rows with
// slab-packed E8M0 scales (kos_tile_mx.h); partials and the reduction stay
// fp32.
#include <algorithm>

#include "kos_host.h"
#include "kos_order.h"
#include "kos_tile.h"
#include "kos_tile_mx.h"

namespace kos {

struct RsParams {
  int32_t world, rank;
  int32_t m, k, n, mc;
  // operands as bytes: bf16 A m x k and W k x n, or E4M3 A m x k and W n x k
  const char* a;
  const char* w;
  const uint8_t* a_sc;   // MX only: slab-packed scales
  const uint8_t* w_sc;
  const float* peers[8];
  float* partial;
  float* y;
  int32_t row_order;
  int32_t n_reducers;       // tickets below this start as reducers
  int32_t builders_switch;  // builders become reducers when tiles run out
  int32_t do_build, do_reduce, wait_flags;
  int32_t builders_reduce;  // two-way: builders take ready reduce entries between tiles
  uint32_t spin_limit;
  int32_t bands;            // mc / BM
  int32_t tiles_n;          // n / BN
  int32_t n_tiles, n_reduce;
  WsHeader* ws;
  uint32_t* ready;
  kos_trace_rec* trace;     // null: tracing off
};

// Rows of one reduce entry: a slab of kSlabRows rows of one output tile.
constexpr int kSlabRows = 32;

// y[slab rows, tile cols] = sum over ranks, ascending, in fp32.  Each pass
// issues every load first (U float4 per source per thread, up to 8 x U in
// flight), then adds and stores.
template <int BN>
__device__ __forceinline__ void reduce_entry(const RsParams& p, int64_t r0, int col_tile) {
  const int64_t N = p.n;
  const int64_t c0 = (int64_t)col_tile * BN;
  constexpr int V = BN / 4;                              // float4 per row
  constexpr int E = kSlabRows * V;                       // float4 per slab
  constexpr int U = 4;
  const float* src[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    src[q] = q >= p.world ? nullptr
                          : (q == p.rank ? p.partial + ((int64_t)p.rank * p.mc + r0) * N + c0
                                         : p.peers[q] + r0 * N + c0);
  float* dst = p.y + r0 * N + c0;
  const DevBuf ob(src[p.rank]);
  for (int e0 = threadIdx.x; e0 < E; e0 += U * blockDim.x) {
    int64_t off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * (int)blockDim.x;
      ok[u] = e < E;
      off[u] = (int64_t)(e / V) * N + (e % V) * 4;
    }
    // peers' slices (plain loads) and our own staged rows (device-coherent:
    // written by builders of this launch) into separate registers, all
    // issued before the first add
    f32x4 x[8][U];
    f32x4 own[U];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q >= p.world) break;
      if (q == p.rank) continue;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ok[u]) x[q][u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src[q] + off[u]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) own[u] = __builtin_bit_cast(f32x4, ob.ld128((uint32_t)off[u] * 4u));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q >= p.world) break;
        a += q == p.rank ? own[u] : x[q][u];
      }
      *reinterpret_cast<f32x4*>(dst + off[u]) = a;
    }
  }
}

template <class S>
__global__ __launch_bounds__(S::NT, 1) void gemm_rs_kernel(RsParams args) {
  constexpr int BM = S::BM, BN = S::BN;
  __shared__ WgSlots slots;
  // The parameter block lives in LDS: each role reads the fields it needs
  // when it needs them instead of pinning them all in scalar registers.
  __shared__ RsParams ps;
  if (threadIdx.x == 0) ps = args;
  __syncthreads();
  const RsParams& p = ps;
  WsHeader* h = p.ws;
  const int64_t K = p.k, N = p.n;
  Tracer tr(p.trace);
  const uint32_t ticket = wg_ticket(h, &slots);
  const bool starts_reducer = p.do_reduce && ticket < (uint32_t)p.n_reducers;

  constexpr int SLABS = BM / kSlabRows;
  const uint32_t n_red = (uint32_t)p.n_reduce * SLABS;
  // one reduce entry (its tile is ready): a slab of our chunk's output
  auto do_reduce = [&](uint32_t i, uint64_t t0) {
    const RsReduce re = rs_reduce_of((int)i, p.tiles_n, SLABS);
    reduce_entry<BN>(p, (int64_t)re.band * BM + re.slab * kSlabRows, re.col);
    tr.put_wg(KOS_TR_REDUCE, i, t0);
  };

  // ---- builder role -----------------------------------------------------
  if (p.do_build && !starts_reducer) {
    f32x16 acc[S::TM][S::TN];
    for (;;) {
      if (p.builders_reduce) {   // two-way: reduce while the reduce queue's head is ready
        for (;;) {
          __syncthreads();
          if (threadIdx.x == 0) {
            uint32_t hd = ld_relaxed(&h->head[2]);
            uint32_t got = kNoEntry;
            if (hd < n_red) {
              const RsReduce re = rs_reduce_of((int)hd, p.tiles_n, SLABS);
              if (ld_relaxed(&p.ready[re.band * p.tiles_n + re.col]) >= 1u &&
                  __hip_atomic_compare_exchange_strong(&h->head[2], &hd, hd + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT))
                got = hd;
            }
            slots.claim = got;
          }
          __syncthreads();
          const uint32_t got = slots.claim;
          if (got == kNoEntry) break;
          do_reduce(got, tr.now());
        }
      }
      const uint32_t j = wg_claim(&h->head[1], h, &slots);
      if (j >= (uint32_t)p.n_tiles) break;
      const uint64_t t0 = tr.now();
      const RsTile tile = rs_tile_of((int)j, p.row_order != 0, p.world, p.bands, p.tiles_n);
      const int band = tile.band, chunk = tile.chunk, col = tile.col;
      const int64_t row0 = (int64_t)chunk * p.mc + (int64_t)band * BM;
      if constexpr (S::MX) {
        const MxSrc a{reinterpret_cast<const uint8_t*>(p.a) + row0 * K, p.a_sc + row0 * 2, K, 2 * (int64_t)p.m};
        const MxSrc b{reinterpret_cast<const uint8_t*>(p.w) + (int64_t)col * BN * K, p.w_sc + (int64_t)col * BN * 2, K,
                      2 * N};
        tile_mainloop_mx<S>(acc, a, BM, b, BN, p.k);
      } else {
        // W k x n, or (BNT) n x k
        const BSrc b = S::BNT ? BSrc{reinterpret_cast<const uint16_t*>(p.w) + (int64_t)col * BN * K, nullptr, K}
                              : BSrc{reinterpret_cast<const uint16_t*>(p.w) + (int64_t)col * BN, nullptr, N};
        tile_mainloop<S>(acc, reinterpret_cast<const uint16_t*>(p.a) + row0 * K, K, BM, b, p.k);
      }
      float* P = p.partial + row0 * N + (int64_t)col * BN;
      // whole rows of the tile through the (now free) LDS ring
      if (chunk == p.rank) {   // read by this launch's reducers: device-coherent stores
        tile_store_out<S, ring_bytes<S>(), true, float, ring_bufs<S>()>(acc, P, N, BM);
        wg_publish(&p.ready[band * p.tiles_n + col], 1u);
      } else {
        tile_store_out<S, ring_bytes<S>(), false, float, ring_bufs<S>()>(acc, P, N, BM);
      }
      tr.put(KOS_TR_TILE, j, t0);
    }
    if (!p.builders_switch || !p.do_reduce) {
      tr.finish(ticket);
      wg_exit(h, p.ready, p.bands * p.tiles_n, &slots);
      return;
    }
  }

  // ---- reducer role -----------------------------------------------------
  if (p.do_reduce) {
    for (;;) {
      const uint32_t i = wg_claim(&h->head[2], h, &slots);
      if (i >= n_red) break;
      const RsReduce re = rs_reduce_of((int)i, p.tiles_n, SLABS);
      uint64_t t0 = tr.now();
      if (p.wait_flags) {
        if (!wg_observe(&p.ready[re.band * p.tiles_n + re.col], 1u, h, p.spin_limit, i, &slots)) break;
        tr.put(KOS_TR_WAIT, i, t0);
        t0 = tr.now();
      }
      do_reduce(i, t0);
    }
  }
  tr.finish(ticket);
  wg_exit(h, p.ready, p.bands * p.tiles_n, &slots);
}

template <class S>
static kos_status launch_rs(const RsParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_rs_kernel<S>), dim3(grid), dim3(S::NT), 0, stream, p);
  return launch_status("gemm_rs launch");
}

template <bool BNT>
static kos_status launch_rs_tile(int bm, int bn, const RsParams& p, int grid, hipStream_t s) {
  if (bm == 256 && bn == 256) return launch_rs<TileShape<256, 256, 4, 2, 4, BNT>>(p, grid, s);
  if (bm == 256 && bn == 128) return launch_rs<TileShape<256, 128, 4, 2, 2, BNT>>(p, grid, s);
  if (bm == 128 && bn == 128) return launch_rs<TileShape<128, 128, 4, 2, 2, BNT>>(p, grid, s);
  return launch_rs<TileShape<64, 64, 4, 2, 2, BNT>>(p, grid, s);
}

}  // namespace kos

using namespace kos;

namespace kos {

// Arguments of one call: bf16 (W k x n, or wt: n x k) or MX.
struct RsCall {
  bool mx, wt;
  int32_t world, rank;
  int64_t m, k, n;
  const void* a;
  const void* a_sc;
  const void* w;
  const void* w_sc;
  const float* const* peer_slices;
  float* partial;
  float* y;
  const kos_opts* opts;
  void* ws;
  size_t ws_bytes;
  void* stream;
};

static kos_status gemm_rs_run(const RsCall& c) {
  const int32_t world = c.world, rank = c.rank;
  const int64_t m = c.m, k = c.k, n = c.n;
  const void *a = c.a, *w = c.w;
  const float* const* peer_slices = c.peer_slices;
  float *partial = c.partial, *y = c.y;
  const kos_opts* opts = c.opts;
  void* ws = c.ws;
  const size_t ws_bytes = c.ws_bytes;
  void* stream = c.stream;
  if (world < 1 || world > 8) return fail(KOS_ERR_ARG, "world %d outside [1, 8]", world);
  if (rank < 0 || rank >= world) return fail(KOS_ERR_ARG, "rank %d outside [0, %d)", rank, world);
  if (!a || !w || !partial || !y) return fail(KOS_ERR_ARG, "null buffer");
  if (c.mx && (!c.a_sc || !c.w_sc)) return fail(KOS_ERR_ARG, "null scale buffer");
  if (world > 1 && !peer_slices) return fail(KOS_ERR_ARG, "peer_slices is NULL");
  for (int p = 0; p < world; ++p)
    if (p != rank && !peer_slices[p]) return fail(KOS_ERR_ARG, "peer_slices[%d] is NULL", p);
  if (c.mx) {
    if (m <= 0 || k <= 0 || n <= 0 || m % world || (m / world) % 256 || k % 256 || n % 256)
      return fail(KOS_ERR_SHAPE, "MX: m %lld (m/world), k %lld, n %lld must be positive multiples of 256",
                  (long long)m, (long long)k, (long long)n);
  } else if (m <= 0 || k <= 0 || n <= 0 || m % world || (m / world) % 64 || k % 64 || n % 64) {
    return fail(KOS_ERR_SHAPE, "m %lld (m/world a multiple of 64), k %lld, n %lld (multiples of 64) unsupported",
                (long long)m, (long long)k, (long long)n);
  }
  if (m > (int64_t(1) << 30) || k > (1 << 20) || n > (1 << 20)) return fail(KOS_ERR_SHAPE, "sizes too large");
  // the tiles address W (bf16) and the scale slabs through 32-bit offsets
  // (n <= 2^20 keeps a tile's 256 output rows, fp32, below 1 GiB of offsets)
  if (!c.mx && k * n * 2 >= (int64_t(1) << 31)) return fail(KOS_ERR_SHAPE, "w (bf16) must be smaller than 2 GiB");
  if (c.mx && (k / 64) * 2 * std::max(m, n) >= (int64_t(1) << 31))
    return fail(KOS_ERR_SHAPE, "MX scale arrays must be smaller than 2 GiB");
  if (!aligned16(a) || !aligned16(w) || !aligned16(partial) || !aligned16(y))
    return fail(KOS_ERR_ALIGN, "buffers must be 16-byte aligned");
  if (c.mx && (!aligned16(c.a_sc) || !aligned16(c.w_sc))) return fail(KOS_ERR_ALIGN, "scale buffers must be 16-byte aligned");
  for (int p = 0; p < world; ++p)
    if (p != rank && !aligned16(peer_slices[p])) return fail(KOS_ERR_ALIGN, "peer_slices[%d] not aligned", p);
  kos_status st = check_workspace(ws, ws_bytes);
  if (st != KOS_OK) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != KOS_OK) return st;
  kos_opts o;
  // FUSED: nobody waits idle for the first band; builders switch to reducing
  // when the tiles run out.  FIXED: a reserved reduction crew.
  if ((st = resolve_opts(opts, dev, CrewDefaults{0, 0, 16, 8}, &o)) != KOS_OK) return st;

  const int64_t mc = m / world;
  int bm = 64, bn = 64;
  if (c.mx || (mc % 256 == 0 && n % 256 == 0)) bm = 256, bn = 256;
  else if (mc % 256 == 0 && n % 128 == 0) bm = 256, bn = 128;
  else if (mc % 128 == 0 && n % 128 == 0) bm = 128, bn = 128;

  RsParams p{};
  p.world = world;
  p.rank = rank;
  p.m = (int32_t)m;
  p.k = (int32_t)k;
  p.n = (int32_t)n;
  p.mc = (int32_t)mc;
  p.a = static_cast<const char*>(a);
  p.w = static_cast<const char*>(w);
  p.a_sc = static_cast<const uint8_t*>(c.a_sc);
  p.w_sc = static_cast<const uint8_t*>(c.w_sc);
  for (int q = 0; q < world; ++q) p.peers[q] = q == rank ? nullptr : peer_slices[q];
  p.partial = partial;
  p.y = y;
  p.row_order = o.rs_order == KOS_RS_ROW;
  p.spin_limit = o.spin_limit;
  p.bands = (int32_t)(mc / bm);
  p.tiles_n = (int32_t)(n / bn);
  p.n_tiles = world * p.bands * p.tiles_n;
  p.n_reduce = p.bands * p.tiles_n;
  p.ws = static_cast<WsHeader*>(ws);
  p.ready = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kCountersOffset);
  p.trace = trace_slot(ws, o.trace, 0);
  if ((size_t)p.n_reduce > kMaxCounters) return fail(KOS_ERR_SHAPE, "too many output tiles");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = o.grid;
  auto launch = [&](const RsParams& q) {
    return c.mx ? launch_rs<TileShapeMX<256, 256>>(q, grid, s)
                : c.wt ? launch_rs_tile<true>(bm, bn, q, grid, s) : launch_rs_tile<false>(bm, bn, q, grid, s);
  };
  if (o.mode == KOS_MODE_UNFUSED) {
    RsParams gm = p;            // launch 1: the whole GEMM
    gm.do_build = 1;
    gm.do_reduce = 0;
    gm.n_reducers = 0;
    if ((st = launch(gm)) != KOS_OK) return st;
    RsParams rd = p;            // launch 2: the whole reduction
    rd.trace = trace_slot(ws, o.trace, 1);
    rd.do_build = 0;
    rd.do_reduce = 1;
    rd.n_reducers = grid;
    rd.wait_flags = 0;
    return launch(rd);
  }
  // The crew that starts reducing (FUSED, may be empty) or only reduces (FIXED).
  const int min_crew = o.mode == KOS_MODE_FUSED ? 0 : 1;
  if (o.n_movers < min_crew || o.n_movers >= grid)
    return fail(KOS_ERR_ARG, "n_movers %d must be in [%d, grid %d)", o.n_movers, min_crew, grid);
  p.n_reducers = o.n_movers;
  p.builders_switch = o.mode == KOS_MODE_FUSED;
  p.builders_reduce = o.mode == KOS_MODE_FUSED && o.policy == KOS_POLICY_SWAPPED;
  p.do_build = 1;
  p.do_reduce = 1;
  p.wait_flags = 1;
  return launch(p);
}

}  // namespace kos

using namespace kos;

extern "C" kos_status kos_gemm_rs(int32_t world, int32_t rank, int64_t m, int64_t k, int64_t n, const void* a,
                                  const void* w, const float* const* peer_slices, float* partial, float* y,
                                  const kos_opts* opts, void* ws, size_t ws_bytes, void* stream) {
  return gemm_rs_run(RsCall{false, false, world, rank, m, k, n, a, nullptr, w, nullptr, peer_slices, partial, y, opts,
                            ws, ws_bytes, stream});
}

extern "C" kos_status kos_gemm_rs_wt(int32_t world, int32_t rank, int64_t m, int64_t k, int64_t n, const void* a,
                                     const void* w_t, const float* const* peer_slices, float* partial, float* y,
                                     const kos_opts* opts, void* ws, size_t ws_bytes, void* stream) {
  return gemm_rs_run(RsCall{false, true, world, rank, m, k, n, a, nullptr, w_t, nullptr, peer_slices, partial, y, opts,
                            ws, ws_bytes, stream});
}

extern "C" kos_status kos_gemm_rs_mx(int32_t world, int32_t rank, int64_t m, int64_t k, int64_t n, const void* a,
                                     const void* a_scales, const void* w, const void* w_scales,
                                     const float* const* peer_slices, float* partial, float* y,
                                     const kos_opts* opts, void* ws, size_t ws_bytes, void* stream) {
  return gemm_rs_run(RsCall{true, false, world, rank, m, k, n, a, a_scales, w, w_scales, peer_slices, partial, y, opts, ws,
                            ws_bytes, stream});
}
