// All-gather + GEMM as one persistent kernel (one rank's share).
//
// [KOSMOS explainer, "Start with the problem"]: under TP+SP the GEMM's
// input is first collected from every rank.  ["Role switching only works
// if ..."]: the tiles of the shard held locally go first, while the movers
// bring the other shards over in the order the tiles will consume them.
// ["KOSMOS removes the manager"]: a mover with no transfer left turns
// builder for good (one-way switch).
//
// Queues (heads in the workspace):
//   head[0]  move entries: remote shards in consumption order (rank+1,
//            rank+2, ... mod world), row blocks ascending, each row block cut
//            into equal slices; then the local shard's copy into the
//            gathered output (nobody waits for it).
//   head[1]  tiles: local shard first, then the remote shards in the same
//            order; within a shard row block ascending, then column tile.
// Ready counter per (shard, row block): the number of its slices landed.
//
// MXFP8 variant (same kernel, MX tile shape): the shards are E4M3 rows with
// slab-packed E8M0 scales (kos_tile_mx.h); a move copies a slice's rows and
// then its scales in every slab before it is counted.
#include <algorithm>
#include <mutex>

#include "kos_host.h"
#include "kos_order.h"
#include "kos_tile.h"
#include "kos_tile_mx.h"

namespace kos {

struct AgParams {
  int32_t world, rank;
  int32_t m_local, k, n;
  // operands as bytes: bf16 rows of 2k bytes (W k x n), or E4M3 rows of k
  // bytes (W n x k)
  const char* a_local;
  const char* peers[8];
  const char* w;
  char* gathered;
  // MX only: slab-packed scales of the same rows (slab stride 2 x rows)
  const uint8_t* sc_local;
  const uint8_t* sc_peers[8];
  const uint8_t* w_sc;
  uint8_t* sc_gathered;
  void* c;
  int32_t c_f32;
  int32_t n_movers;       // tickets below this start as movers
  int32_t movers_switch;  // movers become builders when moves run out
  int32_t do_build;       // this launch builds tiles
  int32_t wait_flags;     // builders wait for remote row blocks
  int32_t builders_move;  // two-way: builders take move entries between tiles
  uint32_t spin_limit;
  int32_t rb_per_shard;   // m_local / BM
  int32_t tiles_n;        // n / BN
  int32_t rows_per_move;  // rows of one move entry (divides BM)
  int32_t moves_per_rb;   // BM / rows_per_move
  int32_t n_move;         // move entries (remote + local)
  int32_t n_tiles;
  WsHeader* ws;
  uint32_t* ready;
  kos_trace_rec* trace;   // null: tracing off
  int32_t hand_over;      // the library's static scratch: hand the status over at exit
  int32_t* status_out;    // where (may be null)
};

// One output tile's K loop over the BM rows of A at `a_rows` (bytes) and
// column tile nt of W.  MX: `a_sc` is the rows' slab-0 scales, `a_slab` the
// slab stride of that scale array.  COH: the rows were written by this
// launch.
template <class S, bool COH>
__device__ __forceinline__ void build_tile(f32x16 (&acc)[S::TM][S::TN], const AgParams& p, const char* a_rows,
                                           const uint8_t* a_sc, int64_t a_slab, int nt) {
  const int64_t K = p.k, N = p.n;
  if constexpr (S::MX) {
    const MxSrc a{reinterpret_cast<const uint8_t*>(a_rows), a_sc, K, a_slab};
    const MxSrc b{reinterpret_cast<const uint8_t*>(p.w) + (int64_t)nt * S::BN * K, p.w_sc + (int64_t)nt * S::BN * 2,
                  K, 2 * N};
    tile_mainloop_mx<S, COH>(acc, a, S::BM, b, S::BN, p.k);
  } else {
    // W k x n, or (BNT) n x k
    const BSrc b = S::BNT ? BSrc{reinterpret_cast<const uint16_t*>(p.w) + (int64_t)nt * S::BN * K, nullptr, K}
                          : BSrc{reinterpret_cast<const uint16_t*>(p.w) + (int64_t)nt * S::BN, nullptr, N};
    tile_mainloop<S, false, COH>(acc, reinterpret_cast<const uint16_t*>(a_rows), K, S::BM, b, p.k);
  }
}

// The scales of `rows` rows (a multiple of 8) in each of `slabs` slabs:
// 2*rows bytes at dst + s*dst_slab from src + s*src_slab, 16-byte pieces,
// device-coherent stores (the entry point keeps slabs*dst_slab below 2^31).
__device__ inline void copy_scale_rows(uint8_t* dst, const uint8_t* src, int rows, int slabs, int64_t dst_slab,
                                       int64_t src_slab) {
  const int per = rows * 2 / 16;
  const int n = slabs * per;
  const DevBuf d(dst);
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const int sl = t / per, c = t % per;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + sl * src_slab) + c);
    d.st128((uint32_t)(sl * dst_slab) + c * 16u, v);
  }
}

template <class S>
__global__ __launch_bounds__(S::NT, 1) void ag_gemm_kernel(AgParams args) {
  constexpr int BM = S::BM, BN = S::BN;
  __shared__ WgSlots slots;
  // The parameter block lives in LDS: each role reads the fields it needs
  // when it needs them instead of pinning them all in scalar registers.
  __shared__ AgParams ps;
  if (threadIdx.x == 0) ps = args;
  __syncthreads();
  const AgParams& p = ps;
  WsHeader* h = p.ws;
  const int64_t K = p.k, N = p.n;
  const int64_t RB = S::MX ? K : 2 * K;   // bytes per A row
  Tracer tr(p.trace);
  const uint32_t ticket = wg_ticket(h, &slots);

  // one move entry: a slice of a shard's row block into the gathered rows
  auto do_move = [&](uint32_t i) {
    const uint64_t t0 = tr.now();
    const AgMove mv = ag_move_of((int)i, p.world, p.rank, p.rb_per_shard, p.moves_per_rb);
    const int shard = mv.shard, rb = mv.rb;
    const char* src_shard = shard == p.rank ? p.a_local : p.peers[shard];
    const int64_t row = (int64_t)rb * BM + (int64_t)mv.sub * p.rows_per_move;
    wg_copy_dev(p.gathered + ((int64_t)shard * p.m_local + row) * RB, src_shard + row * RB,
                (size_t)p.rows_per_move * RB);
    if constexpr (S::MX)
      copy_scale_rows(p.sc_gathered + ((int64_t)shard * p.m_local + row) * 2,
                      (shard == p.rank ? p.sc_local : p.sc_peers[shard]) + row * 2, p.rows_per_move, K / 64,
                      (int64_t)p.world * p.m_local * 2, (int64_t)p.m_local * 2);
    wg_publish(&p.ready[shard * p.rb_per_shard + rb], 1u);
    tr.put(KOS_TR_MOVE, i, t0);
  };

  // ---- mover role -------------------------------------------------------
  if (ticket < (uint32_t)p.n_movers) {
    for (;;) {
      const uint32_t i = wg_claim(&h->head[0], h, &slots);
      if (i >= (uint32_t)p.n_move) break;
      do_move(i);
    }
    if (!p.movers_switch) {
      tr.finish(ticket);
      wg_exit(h, p.ready, p.world * p.rb_per_shard, &slots, p.hand_over, p.status_out);
      return;
    }
  }

  // ---- builder role -----------------------------------------------------
  if (p.do_build) {
    f32x16 acc[S::TM][S::TN];
    for (;;) {
      if (p.builders_move) {   // two-way: while move entries are left, take one between tiles
        __syncthreads();
        if (threadIdx.x == 0) slots.aux[0] = ld_relaxed(&h->head[0]) < (uint32_t)p.n_move;
        __syncthreads();
        if (slots.aux[0]) {
          const uint32_t i = wg_claim(&h->head[0], h, &slots);
          if (i < (uint32_t)p.n_move) {
            do_move(i);
            continue;
          }
        }
      }
      const uint32_t j = wg_claim(&h->head[1], h, &slots);
      if (j >= (uint32_t)p.n_tiles) break;
      const AgTile tile = ag_tile_of((int)j, p.world, p.rank, p.rb_per_shard, p.tiles_n);
      const int q = tile.q, rb = tile.rb, nt = tile.nt, shard = tile.shard;
      uint64_t t0 = tr.now();
      if (q == 0) {
        build_tile<S, false>(acc, p, p.a_local + (int64_t)rb * BM * RB, p.sc_local + (int64_t)rb * BM * 2,
                             (int64_t)p.m_local * 2, nt);
      } else {
        const int64_t r0 = (int64_t)shard * p.m_local + (int64_t)rb * BM;
        const char* A = p.gathered + r0 * RB;
        const uint8_t* As = p.sc_gathered + r0 * 2;
        const int64_t slab = (int64_t)p.world * p.m_local * 2;
        if (p.wait_flags) {
          // rows written by movers of this launch: wait for them, read device-coherent
          if (!wg_observe(&p.ready[shard * p.rb_per_shard + rb], (uint32_t)p.moves_per_rb, h, p.spin_limit, j,
                          &slots))
            break;
          tr.put(KOS_TR_WAIT, j, t0);
          t0 = tr.now();
          build_tile<S, true>(acc, p, A, As, slab, nt);
        } else {
          build_tile<S, false>(acc, p, A, As, slab, nt);
        }
      }
      const int64_t row0 = (int64_t)shard * p.m_local + (int64_t)rb * BM;
      const int64_t col0 = (int64_t)nt * BN;
      if (p.c_f32) {
        float* C = reinterpret_cast<float*>(p.c) + row0 * N + col0;
        tile_foreach4<S>(acc, [&](int r, int c, f32x4 v) { *reinterpret_cast<f32x4*>(&C[r * N + c]) = v; });
      } else {   // whole rows of the tile through the (now free) LDS ring
        tile_store_out<S, ring_bytes<S>(), false, uint16_t, ring_bufs<S>()>(
            acc, reinterpret_cast<uint16_t*>(p.c) + row0 * N + col0, N, BM);
      }
      tr.put(KOS_TR_TILE, j, t0);
    }
  }
  tr.finish(ticket);
  wg_exit(h, p.ready, p.world * p.rb_per_shard, &slots, p.hand_over, p.status_out);
}

template <class S>
static kos_status launch_ag(const AgParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((ag_gemm_kernel<S>), dim3(grid), dim3(S::NT), 0, stream, p);
  return launch_status("ag_gemm launch");
}

template <bool BNT>
static kos_status launch_ag_tile(int bm, int bn, const AgParams& p, int grid, hipStream_t s) {
  if (bm == 256 && bn == 256) return launch_ag<TileShape<256, 256, 4, 2, 4, BNT>>(p, grid, s);
  if (bm == 256 && bn == 192) return launch_ag<TileShape<256, 192, 4, 2, 2, BNT>>(p, grid, s);
  if (bm == 256 && bn == 128) return launch_ag<TileShape<256, 128, 4, 2, 2, BNT>>(p, grid, s);
  if (bm == 128 && bn == 128) return launch_ag<TileShape<128, 128, 4, 2, 2, BNT>>(p, grid, s);
  return launch_ag<TileShape<64, 64, 4, 2, 2, BNT>>(p, grid, s);
}

// The largest tile (fewest operand re-reads) that divides the shard rows and
// the columns and still gives every workgroup at least one tile.
static void pick_ag_tile(int64_t world, int64_t m_local, int64_t n, int grid, int* bm, int* bn) {
  static const int cand[][2] = {{256, 256}, {256, 192}, {256, 128}, {128, 128}, {64, 64}};
  for (const auto& c : cand) {
    if (m_local % c[0] || n % c[1]) continue;
    const int64_t tiles = world * (m_local / c[0]) * (n / c[1]);
    if (tiles >= grid || (c[0] == 64 && c[1] == 64)) {
      *bm = c[0];
      *bn = c[1];
      return;
    }
  }
  // no tile gives one per workgroup: the largest that divides
  for (const auto& c : cand)
    if (m_local % c[0] == 0 && n % c[1] == 0) {
      *bm = c[0];
      *bn = c[1];
      return;
    }
}

}  // namespace kos

using namespace kos;

namespace kos {

// Arguments of one call: bf16 (W k x n, or wt: n x k) or MX.
struct AgCall {
  bool mx, wt;
  int32_t world, rank;
  int64_t m_local, k, n;
  const void* a_local;
  const void* const* a_peers;
  const void* w;
  void* a_gathered;
  const void* sc_local;
  const void* const* sc_peers;
  const void* w_sc;
  void* sc_gathered;
  void* c;
  int32_t c_dtype;
  const kos_opts* opts;
  void* ws;
  size_t ws_bytes;
  void* stream;
  bool noalloc;           // no caller workspace: the library's static scratch
  int32_t* status_out;    // noalloc: the call's device-side status goes here
};

// ---------------------------------------------------------------------------
// the allocation-free variant's scratch: a file-scope device array (one copy
// per GPU, held until the process ends) laid out like the head of a
// workspace -- the 256-byte header, then the ready counters at
// kCountersOffset -- for callers that cannot allocate.  Host code never
// passes the array's name to a kernel (on the host it only stands for the
// symbol); it uses the device address hipGetSymbolAddress returns, looked up
// once per device with that device current.
// ---------------------------------------------------------------------------

constexpr size_t kStaticCounters = 16384;   // ready counters: world x row blocks
constexpr size_t kStaticScratchBytes = kCountersOffset + kStaticCounters * sizeof(uint32_t);   // 68 KiB
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void scratch_clear_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];       // per device: the array's device address
bool g_scratch_clear[64];      // per device: zeroed once (by a fill kernel, never a memset)
}  // namespace

// The scratch of the current device, zeroed before its first use (on
// `stream`, ahead of the caller's launch).  Every call leaves it zeroed
// again (the last workgroup out resets it).
static kos_status static_scratch(const DeviceInfo& dev, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  const int d = dev.device;
  if (!g_scratch_ptr[d]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KOS_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[d] = ptr;
  }
  if (!g_scratch_clear[d]) {
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(16), dim3(256), 0, stream,
                       static_cast<uint32_t*>(g_scratch_ptr[d]), (uint32_t)(kStaticScratchBytes / 4));
    kos_status st = launch_status("static scratch clear");
    if (st != KOS_OK) return st;
    g_scratch_clear[d] = true;
  }
  *out = g_scratch_ptr[d];
  return KOS_OK;
}

static kos_status ag_gemm_run(const AgCall& a) {
  const int32_t world = a.world, rank = a.rank;
  const int64_t m_local = a.m_local, k = a.k, n = a.n;
  if (world < 1 || world > 8) return fail(KOS_ERR_ARG, "world %d outside [1, 8]", world);
  if (rank < 0 || rank >= world) return fail(KOS_ERR_ARG, "rank %d outside [0, %d)", rank, world);
  if (a.c_dtype != KOS_BF16 && a.c_dtype != KOS_F32) return fail(KOS_ERR_ARG, "bad c_dtype %d", a.c_dtype);
  if (!a.a_local || !a.w || !a.a_gathered || !a.c) return fail(KOS_ERR_ARG, "null buffer");
  if (a.mx && (!a.sc_local || !a.w_sc || !a.sc_gathered)) return fail(KOS_ERR_ARG, "null scale buffer");
  if (world > 1 && (!a.a_peers || (a.mx && !a.sc_peers))) return fail(KOS_ERR_ARG, "peer array is NULL");
  for (int p = 0; p < world; ++p) {
    if (p == rank) continue;
    if (!a.a_peers[p]) return fail(KOS_ERR_ARG, "a_peers[%d] is NULL", p);
    if (a.mx && !a.sc_peers[p]) return fail(KOS_ERR_ARG, "a_peer_scales[%d] is NULL", p);
  }
  if (a.mx) {
    if (m_local <= 0 || k <= 0 || n <= 0 || m_local % 256 || k % 256 || n % 256)
      return fail(KOS_ERR_SHAPE, "MX: m_local %lld, k %lld, n %lld must be positive multiples of 256",
                  (long long)m_local, (long long)k, (long long)n);
  } else if (m_local <= 0 || k <= 0 || n <= 0 || m_local % 64 || k % 64 || n % 64) {
    return fail(KOS_ERR_SHAPE, "m_local %lld, k %lld, n %lld must be positive multiples of 64", (long long)m_local,
                (long long)k, (long long)n);
  }
  if (m_local * world > (int64_t(1) << 30) || k > (1 << 20) || n > (1 << 20))
    return fail(KOS_ERR_SHAPE, "sizes too large");
  // the tiles address W (bf16) and the scale slabs through 32-bit offsets
  // (n <= 2^20 keeps a tile's 256 output rows, fp32, below 1 GiB of offsets)
  if (!a.mx && k * n * 2 >= (int64_t(1) << 31)) return fail(KOS_ERR_SHAPE, "w (bf16) must be smaller than 2 GiB");
  if (a.mx && (k / 64) * 2 * std::max<int64_t>(m_local * world, n) >= (int64_t(1) << 31))
    return fail(KOS_ERR_SHAPE, "MX scale arrays must be smaller than 2 GiB");
  if (!aligned16(a.a_local) || !aligned16(a.w) || !aligned16(a.a_gathered) || !aligned16(a.c))
    return fail(KOS_ERR_ALIGN, "buffers must be 16-byte aligned");
  if (a.mx && (!aligned16(a.sc_local) || !aligned16(a.w_sc) || !aligned16(a.sc_gathered)))
    return fail(KOS_ERR_ALIGN, "scale buffers must be 16-byte aligned");
  for (int p = 0; p < world; ++p) {
    if (p == rank) continue;
    if (!aligned16(a.a_peers[p])) return fail(KOS_ERR_ALIGN, "a_peers[%d] not 16-byte aligned", p);
    if (a.mx && !aligned16(a.sc_peers[p])) return fail(KOS_ERR_ALIGN, "a_peer_scales[%d] not 16-byte aligned", p);
  }
  kos_status st = a.noalloc ? KOS_OK : check_workspace(a.ws, a.ws_bytes);
  if (st != KOS_OK) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != KOS_OK) return st;
  if (a.noalloc && a.opts && a.opts->trace)
    return fail(KOS_ERR_ARG, "the allocation-free entry point has no trace region");
  if (a.noalloc && (reinterpret_cast<uintptr_t>(a.status_out) & 3u))
    return fail(KOS_ERR_ALIGN, "status_out must be 4-byte aligned");
  kos_opts o;
  // Movers over device memory: half the grid saturates HBM copy bandwidth
  // and the other half builds the local shard meanwhile; over PCIe sixteen
  // workgroups keep enough requests in flight to fill the link.
  if ((st = resolve_opts(a.opts, dev, CrewDefaults{kCrewHalfGrid, 16, 16, 8}, &o)) != KOS_OK) return st;

  int bm = 256, bn = 256;
  if (a.mx) {
    // 256 x 192 MX tiles where they take fewer rounds of the grid, counted
    // in tile columns (the QKV shard: 256 tiles of 192 columns fill every
    // compute unit once, 256-column tiles only 192 of them)
    const int64_t rounds256 = (world * (m_local / 256) * (n / 256) + o.grid - 1) / o.grid;
    const int64_t rounds192 = (world * (m_local / 256) * (n / 192) + o.grid - 1) / o.grid;
    if (n % 192 == 0 && rounds192 * 192 < rounds256 * 256) bn = 192;
  } else {
    pick_ag_tile(world, m_local, n, o.grid, &bm, &bn);
  }
  const int64_t row_bytes = a.mx ? k : 2 * k;

  AgParams p{};
  p.world = world;
  p.rank = rank;
  p.m_local = (int32_t)m_local;
  p.k = (int32_t)k;
  p.n = (int32_t)n;
  p.a_local = static_cast<const char*>(a.a_local);
  for (int q = 0; q < world; ++q) p.peers[q] = q == rank ? nullptr : static_cast<const char*>(a.a_peers[q]);
  p.w = static_cast<const char*>(a.w);
  p.gathered = static_cast<char*>(a.a_gathered);
  if (a.mx) {
    p.sc_local = static_cast<const uint8_t*>(a.sc_local);
    for (int q = 0; q < world; ++q) p.sc_peers[q] = q == rank ? nullptr : static_cast<const uint8_t*>(a.sc_peers[q]);
    p.w_sc = static_cast<const uint8_t*>(a.w_sc);
    p.sc_gathered = static_cast<uint8_t*>(a.sc_gathered);
  }
  p.c = a.c;
  p.c_f32 = a.c_dtype == KOS_F32;
  p.spin_limit = o.spin_limit;
  p.rb_per_shard = (int32_t)(m_local / bm);
  p.tiles_n = (int32_t)(n / bn);
  // Move entries of about 128 KiB: whole rows, dividing the row block (MX:
  // a power of two of at least 8 rows, whole 16-byte pieces of scales).
  int rows = (int)((128 * 1024) / row_bytes);
  if (rows < 1) rows = 1;
  if (rows > bm) rows = bm;
  if (a.mx) {
    int r = 8;
    while (r * 2 <= rows) r *= 2;
    rows = r;
  }
  while (bm % rows) --rows;
  p.rows_per_move = rows;
  p.moves_per_rb = bm / rows;
  p.n_move = world * p.rb_per_shard * p.moves_per_rb;
  p.n_tiles = world * p.rb_per_shard * p.tiles_n;
  if ((size_t)world * p.rb_per_shard > (a.noalloc ? kStaticCounters : kMaxCounters))
    return fail(KOS_ERR_SHAPE, "too many row blocks (%lld) for the %s", (long long)world * p.rb_per_shard,
                a.noalloc ? "static scratch" : "workspace");
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  void* ws = a.ws;
  if (a.noalloc && (st = static_scratch(dev, s, &ws)) != KOS_OK) return st;
  p.ws = static_cast<WsHeader*>(ws);
  p.ready = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kCountersOffset);
  p.trace = a.noalloc ? nullptr : trace_slot(ws, o.trace, 0);
  p.hand_over = a.noalloc;
  p.status_out = a.status_out;

  // A single rank whose gathered output is its own shard has nothing to move.
  const bool nothing_to_move =
      world == 1 && a.a_gathered == a.a_local && (!a.mx || a.sc_gathered == a.sc_local);
  if (nothing_to_move) p.n_move = 0;

  const int grid = o.grid;
  auto launch = [&](const AgParams& q) {
    if (a.mx)
      return bn == 192 ? launch_ag<TileShapeMX<256, 192, 4, 2>>(q, grid, s) : launch_ag<TileShapeMX<256, 256>>(q, grid, s);
    return a.wt ? launch_ag_tile<true>(bm, bn, q, grid, s) : launch_ag_tile<false>(bm, bn, q, grid, s);
  };
  if (o.mode == KOS_MODE_UNFUSED && nothing_to_move) {
    AgParams gm = p;           // the GEMM alone
    gm.n_movers = 0;
    gm.do_build = 1;
    gm.wait_flags = 0;
    return launch(gm);
  }
  if (o.mode == KOS_MODE_UNFUSED) {
    AgParams mv = p;           // launch 1: the whole all-gather
    mv.n_movers = grid;
    mv.movers_switch = 0;
    mv.do_build = 0;
    if ((st = launch(mv)) != KOS_OK) return st;
    AgParams gm = p;           // launch 2: the whole GEMM
    gm.trace = a.noalloc ? nullptr : trace_slot(ws, o.trace, 1);
    gm.n_movers = 0;
    gm.n_move = 0;
    gm.do_build = 1;
    gm.wait_flags = 0;
    return launch(gm);
  }
  if (o.n_movers < 1 || o.n_movers >= grid)
    return fail(KOS_ERR_ARG, "n_movers %d must be in [1, grid %d)", o.n_movers, grid);
  // FUSED: a mover without an entry turns builder at once, so a crew larger
  // than the move entries only makes the first workgroups to arrive (the
  // movers) reach the tiles last; start no more movers than there are moves
  p.n_movers = o.mode == KOS_MODE_FUSED ? std::max(1, std::min(o.n_movers, p.n_move)) : o.n_movers;
  p.movers_switch = o.mode == KOS_MODE_FUSED;
  p.builders_move = o.mode == KOS_MODE_FUSED && o.policy == KOS_POLICY_SWAPPED;
  p.do_build = 1;
  p.wait_flags = 1;
  return launch(p);
}

}  // namespace kos

using namespace kos;

extern "C" kos_status kos_ag_gemm(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                                  const void* a_local, const void* const* a_peers, const void* w,
                                  void* a_gathered, void* c, int32_t c_dtype, const kos_opts* opts, void* ws,
                                  size_t ws_bytes, void* stream) {
  return ag_gemm_run(AgCall{false, false, world, rank, m_local, k, n, a_local, a_peers, w, a_gathered, nullptr,
                            nullptr, nullptr, nullptr, c, c_dtype, opts, ws, ws_bytes, stream, false, nullptr});
}

extern "C" kos_status kos_ag_gemm_wt(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                                     const void* a_local, const void* const* a_peers, const void* w_t,
                                     void* a_gathered, void* c, int32_t c_dtype, const kos_opts* opts, void* ws,
                                     size_t ws_bytes, void* stream) {
  return ag_gemm_run(AgCall{false, true, world, rank, m_local, k, n, a_local, a_peers, w_t, a_gathered, nullptr,
                            nullptr, nullptr, nullptr, c, c_dtype, opts, ws, ws_bytes, stream, false, nullptr});
}

extern "C" kos_status kos_ag_gemm_mx(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                                     const void* a_local, const void* a_local_scales, const void* const* a_peers,
                                     const void* const* a_peer_scales, const void* w, const void* w_scales,
                                     void* a_gathered, void* a_gathered_scales, void* c, int32_t c_dtype,
                                     const kos_opts* opts, void* ws, size_t ws_bytes, void* stream) {
  return ag_gemm_run(AgCall{true, false, world, rank, m_local, k, n, a_local, a_peers, w, a_gathered, a_local_scales,
                            a_peer_scales, w_scales, a_gathered_scales, c, c_dtype, opts, ws, ws_bytes, stream, false, nullptr});
}

extern "C" kos_status kos_ag_gemm_noalloc(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                                          const void* a_local, const void* const* a_peers, const void* w,
                                          void* a_gathered, void* c, int32_t c_dtype, const kos_opts* opts,
                                          int32_t* status_out, void* stream) {
  return ag_gemm_run(AgCall{false, false, world, rank, m_local, k, n, a_local, a_peers, w, a_gathered, nullptr,
                            nullptr, nullptr, nullptr, c, c_dtype, opts, nullptr, 0, stream, true, status_out});
}
