// Queue orders of the persistent kernels: which piece of work entry i of a
// queue is.  The order is the schedule -- entries are laid out in the order
// their consumers need them, and whoever is free takes the next one
// [KOSMOS explainer, "Role switching only works if ..."].
//
// Plain constexpr C++ (usable in device code and in host code alike): the
// kernels decode their entries with these functions, and the host-side
// protocol model of the tests runs the same orders.
#pragma once

namespace kos {

// ---- all-gather + GEMM ----------------------------------------------------

// Move entry i: remote shards first, in the order the tiles consume them
// (rank+1, rank+2, ... mod world), each shard's row blocks ascending, each
// row block cut into `moves_per_rb` slices; then the local shard's copy into
// the gathered output (which no tile waits for).
struct AgMove {
  int shard;   // whose rows
  int rb;      // row block of that shard
  int sub;     // slice of the row block
};
constexpr AgMove ag_move_of(int i, int world, int rank, int rb_per_shard, int moves_per_rb) {
  const int per_shard = rb_per_shard * moves_per_rb;
  const int n_remote = (world - 1) * per_shard;
  int shard = rank, rem = i - n_remote;
  if (i < n_remote) {
    shard = (rank + 1 + i / per_shard) % world;
    rem = i % per_shard;
  }
  return AgMove{shard, rem / moves_per_rb, rem % moves_per_rb};
}

// Tile entry j: the local shard's tiles first, then the remote shards in the
// movers' order; within a shard row block ascending, then column tile.
// q = 0 is the local shard (never waits), q > 0 the q-th remote one.
struct AgTile {
  int q, shard, rb, nt;
};
constexpr AgTile ag_tile_of(int j, int world, int rank, int rb_per_shard, int tiles_n) {
  const int per_q = rb_per_shard * tiles_n;
  const int q = j / per_q, rem = j % per_q;
  return AgTile{q, (rank + q) % world, rem / tiles_n, rem % tiles_n};
}

// ---- GEMM + reduce-scatter ------------------------------------------------

// Tile entry j.  Band order: band b (BM rows of every chunk), then chunk c
// ascending, then column tile -- the first band of every rank's chunk is
// done before any second band.  Row order (the ablation): chunk after
// chunk, each band by band.
struct RsTile {
  int band, chunk, col;
};
constexpr RsTile rs_tile_of(int j, bool row_order, int world, int bands, int tiles_n) {
  if (!row_order) {
    const int per_band = world * tiles_n;
    const int rem = j % per_band;
    return RsTile{j / per_band, rem / tiles_n, rem % tiles_n};
  }
  const int per_chunk = bands * tiles_n;
  const int rem = j % per_chunk;
  return RsTile{rem / tiles_n, j / per_chunk, rem % tiles_n};
}

// Reduce entry i of our own chunk: (band, column tile, slab of `slab_rows`
// rows), in that order; gated on our tile (band, column).
struct RsReduce {
  int band, col, slab;
};
constexpr RsReduce rs_reduce_of(int i, int tiles_n, int slabs) {
  const int tile = i / slabs;
  return RsReduce{tile / tiles_n, tile % tiles_n, i % slabs};
}

// ---- expert combine ---------------------------------------------------------

// Tile entry j of the grouped SwiGLU GEMMs over U units (expert, row block),
// G gate/up tiles and D down tiles per unit, consumer-ordered with a lag of
// L units: the gate/up tiles of units 0..L-1, then for each unit i the
// gate/up tiles of unit i+L followed by the down tiles of unit i, so a down
// tile is claimed about a grid's worth of tiles after the tiles it needs.
// gu / dn: which GEMMs this queue holds (both when fused).
struct CombineTile {
  bool down;
  int u, nt;
};
constexpr CombineTile combine_tile_of(int j, int U, int G, int D, int L, bool gu, bool dn) {
  if (gu && !dn) return CombineTile{false, j / G, j % G};
  if (!gu) return CombineTile{true, j / D, j % D};
  const int Lc = L < U ? L : U;
  const int head = Lc * G;
  if (j < head) return CombineTile{false, j / G, j % G};
  const int jj = j - head;
  const int nfull = U - L > 0 ? U - L : 0;
  const int GD = G + D;
  if (jj < nfull * GD) {
    const int i = jj / GD, r = jj % GD;
    return r < G ? CombineTile{false, i + L, r} : CombineTile{true, i, r - G};
  }
  const int jj2 = jj - nfull * GD;
  return CombineTile{true, nfull + jj2 / D, jj2 % D};
}

}  // namespace kos
