// Host-side model of the persistent kernels' queue / ready-counter protocol
// -- test infrastructure, CPU only.
//
// One std::thread stands for one workgroup.  The model keeps what the
// kernels' scheduling rests on and nothing else: an arrival ticket that
// assigns the starting role (tickets below the crew communicate first),
// atomic queue heads, the kernels' own entry orders (kos_order.h, the
// header the kernels decode their queues with), ready counters bumped after
// a producer's data is written and polled by consumers with a bounded spin
// (time-out instead of a hang), the one-way and two-way role switches, and
// the last workgroup out returning every counter and head to zero.  Data
// words written by producers and read by consumers after the counter say it
// is there (release / acquire) let ThreadSanitizer check that every read is
// ordered after its write.
//
// Scenarios are read from stdin, one per line:
//   op grid world rank a b c mode crew fault spin
//     op     ag | rs | combine | layer (the expert layer forward in one
//            launch) | bwd (its backward in one launch)
//     a b c  ag: row blocks per shard, slices per row block, column tiles
//            rs: bands per chunk, column tiles, slabs per tile
//            combine: units, gate/up tiles per unit, down tiles per unit
//            layer / bwd: units, first-stage entries per unit (gate/up
//            tiles; dH + SwiGLU recompute), second-stage tiles per unit
//            (down tiles; dX)
//     mode   fused | swapped (fused with the other switching policy: two-way
//            all-gather and reduce-scatter, one-way combine) | fixed
//     crew   workgroups that start communicating (fixed: only communicate)
//     fault  none | drop (one ready bump skipped) | dead (one communicating
//            workgroup stops after its first entry, publishing nothing) |
//            delay (communication 1 ms slower per entry)
//     spin   polls before a wait gives up with a time-out
// and one result line is printed per scenario:
//   status=<ok|timeout> entries=<ok|bad> data=<ok|bad> reset=<ok|bad>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <memory>
#include <numeric>
#include <sstream>
#include <string>
#include <thread>
#include <vector>

#include "../../gemm_collective_persistent_amd/csrc/kos_order.h"

namespace {

constexpr uint32_t kNoEntry = 0xFFFFFFFFu;

struct Workspace {
  std::atomic<uint32_t> ticket{0}, exit_count{0}, status{0}, abort_{0};
  std::atomic<uint32_t> head[8];
  std::vector<std::atomic<uint32_t>> ctr;
  explicit Workspace(size_t n) : ctr(n) {
    for (auto& h : head) h.store(0);
    for (auto& c : ctr) c.store(0);
  }
};

struct Scenario {
  std::string op, mode, fault;
  int grid = 0, world = 0, rank = 0, a = 0, b = 0, c = 0, crew = 0;
  long spin = 0;
};

// the runtime's rules, in host form
uint32_t claim(Workspace& ws, std::atomic<uint32_t>& head) {
  if (ws.abort_.load(std::memory_order_relaxed)) return kNoEntry;
  return head.fetch_add(1, std::memory_order_relaxed);
}

void raise_timeout(Workspace& ws) {
  uint32_t zero = 0;
  ws.status.compare_exchange_strong(zero, 7u);   // KOS_ERR_TIMEOUT
  ws.abort_.store(1);
}

bool observe(Workspace& ws, std::atomic<uint32_t>& c, uint32_t target, long spin) {
  long it = 0;
  while (c.load(std::memory_order_acquire) < target) {
    if (ws.abort_.load(std::memory_order_relaxed)) return false;
    if (++it >= spin) {
      raise_timeout(ws);
      return false;
    }
    std::this_thread::yield();
  }
  return true;
}

void publish(std::atomic<uint32_t>& c) { c.fetch_add(1, std::memory_order_release); }

void depart(Workspace& ws, int grid) {
  if (ws.exit_count.fetch_add(1, std::memory_order_acq_rel) != (uint32_t)grid - 1) return;
  for (auto& c : ws.ctr) c.store(0, std::memory_order_relaxed);
  for (auto& h : ws.head) h.store(0, std::memory_order_relaxed);
  ws.ticket.store(0);
  ws.abort_.store(0);
  ws.exit_count.store(0);
}

struct Faults {
  std::atomic<int> dropped{0}, dead{0};
  bool drop = false, kill = false, delay = false;
  // the first communication entry to ask skips its bump (drop)
  bool skip_bump() { return drop && dropped.exchange(1) == 0; }
  // the first communicating workgroup to ask dies (dead)
  bool die() { return kill && dead.exchange(1) == 0; }
  void pace() const {
    if (delay) std::this_thread::sleep_for(std::chrono::milliseconds(1));
  }
};

struct Result {
  bool timeout = false, entries_ok = true, data_ok = true, reset_ok = true;
};

template <class F>
void run_grid(int grid, F&& body) {
  std::vector<std::thread> t;
  t.reserve(grid);
  for (int g = 0; g < grid; ++g) t.emplace_back(body);
  for (auto& x : t) x.join();
}

bool all_zero(Workspace& ws) {
  for (auto& c : ws.ctr)
    if (c.load()) return false;
  for (auto& h : ws.head)
    if (h.load()) return false;
  return ws.ticket.load() == 0 && ws.exit_count.load() == 0 && ws.abort_.load() == 0;
}

// ---- all-gather + GEMM: movers -> builders (one-way) -----------------------
Result run_ag(const Scenario& s) {
  const int R = s.world, RB = s.a, M = s.b, NT = s.c;
  const int n_move = R * RB * M, n_tile = R * RB * NT;
  Workspace ws(R * RB);
  std::vector<uint32_t> gathered(n_move, 0);                     // one word per slice
  std::unique_ptr<std::atomic<int>[]> moved(new std::atomic<int>[n_move]), built(new std::atomic<int>[n_tile]);
  for (int i = 0; i < n_move; ++i) moved[i] = 0;
  for (int i = 0; i < n_tile; ++i) built[i] = 0;
  std::atomic<int> bad_data{0};
  Faults f;
  f.drop = s.fault == "drop";
  f.kill = s.fault == "dead";
  f.delay = s.fault == "delay";
  const bool fused = s.mode != "fixed", two_way = s.mode == "swapped";
  auto move = [&](uint32_t i) {
    f.pace();
    const kos::AgMove mv = kos::ag_move_of((int)i, R, s.rank, RB, M);
    gathered[(mv.shard * RB + mv.rb) * M + mv.sub] = 1000u * mv.shard + 10u * mv.rb + mv.sub + 1;
    moved[i]++;
    if (!f.skip_bump()) publish(ws.ctr[mv.shard * RB + mv.rb]);
  };
  run_grid(s.grid, [&] {
    const uint32_t ticket = ws.ticket.fetch_add(1);
    if (ticket < (uint32_t)s.crew) {
      for (bool first = true;; first = false) {
        const uint32_t i = claim(ws, ws.head[0]);
        if (i >= (uint32_t)n_move) break;
        if (first && f.die()) {   // claimed, never delivered, never departs normally
          depart(ws, s.grid);
          return;
        }
        move(i);
      }
      if (!fused) {
        depart(ws, s.grid);
        return;
      }
    }
    for (;;) {
      if (two_way && ws.head[0].load(std::memory_order_relaxed) < (uint32_t)n_move) {
        const uint32_t i = claim(ws, ws.head[0]);   // builders take move entries while any is left
        if (i < (uint32_t)n_move) {
          move(i);
          continue;
        }
      }
      const uint32_t j = claim(ws, ws.head[1]);
      if (j >= (uint32_t)n_tile) break;
      const kos::AgTile t = kos::ag_tile_of((int)j, R, s.rank, RB, NT);
      if (t.q > 0) {
        if (!observe(ws, ws.ctr[t.shard * RB + t.rb], (uint32_t)M, s.spin)) break;
        for (int sub = 0; sub < M; ++sub)
          if (gathered[(t.shard * RB + t.rb) * M + sub] != 1000u * t.shard + 10u * t.rb + sub + 1) bad_data++;
      }
      built[j]++;
    }
    depart(ws, s.grid);
  });
  Result r;
  r.timeout = ws.status.load() != 0;
  for (int i = 0; i < n_tile && !r.timeout; ++i) r.entries_ok &= built[i] == 1;
  for (int i = 0; i < n_move && !r.timeout; ++i) r.entries_ok &= moved[i] == 1;
  r.data_ok = bad_data == 0;
  r.reset_ok = all_zero(ws);
  return r;
}

// ---- GEMM + reduce-scatter: builders -> reducers (one-way) -----------------
Result run_rs(const Scenario& s) {
  const int R = s.world, B = s.a, NT = s.b, SL = s.c;
  const int n_tile = R * B * NT, n_red = B * NT * SL;
  Workspace ws(B * NT);
  std::vector<uint32_t> partial(n_tile, 0);   // one word per tile
  std::unique_ptr<std::atomic<int>[]> built(new std::atomic<int>[n_tile]), reduced(new std::atomic<int>[n_red]);
  for (int i = 0; i < n_tile; ++i) built[i] = 0;
  for (int i = 0; i < n_red; ++i) reduced[i] = 0;
  std::atomic<int> bad_data{0};
  Faults f;
  f.drop = s.fault == "drop";
  f.kill = s.fault == "dead";
  f.delay = s.fault == "delay";
  const bool fused = s.mode != "fixed", two_way = s.mode == "swapped";
  auto reduce = [&](uint32_t i) {
    f.pace();
    const kos::RsReduce re = kos::rs_reduce_of((int)i, NT, SL);
    if (partial[(s.rank * B + re.band) * NT + re.col] != 100u * s.rank + 10u * re.band + re.col + 1) bad_data++;
    reduced[i]++;
  };
  run_grid(s.grid, [&] {
    const uint32_t ticket = ws.ticket.fetch_add(1);
    const bool reducer_first = ticket < (uint32_t)s.crew;
    if (!reducer_first) {
      for (bool first = true;; first = false) {
        while (two_way) {   // builders reduce while the reduce queue's head is ready
          uint32_t hd = ws.head[2].load(std::memory_order_relaxed);
          if (hd >= (uint32_t)n_red) break;
          const kos::RsReduce re = kos::rs_reduce_of((int)hd, NT, SL);
          if (ws.ctr[re.band * NT + re.col].load(std::memory_order_acquire) < 1u) break;
          if (ws.head[2].compare_exchange_strong(hd, hd + 1, std::memory_order_relaxed)) reduce(hd);
        }
        const uint32_t j = claim(ws, ws.head[1]);
        if (j >= (uint32_t)n_tile) break;
        if (first && f.die()) {
          depart(ws, s.grid);
          return;
        }
        const kos::RsTile t = kos::rs_tile_of((int)j, false, R, B, NT);
        partial[(t.chunk * B + t.band) * NT + t.col] = 100u * t.chunk + 10u * t.band + t.col + 1;
        built[j]++;
        if (t.chunk == s.rank && !f.skip_bump()) publish(ws.ctr[t.band * NT + t.col]);
      }
      if (!fused) {
        depart(ws, s.grid);
        return;
      }
    }
    for (;;) {
      const uint32_t i = claim(ws, ws.head[2]);
      if (i >= (uint32_t)n_red) break;
      const kos::RsReduce re = kos::rs_reduce_of((int)i, NT, SL);
      if (!observe(ws, ws.ctr[re.band * NT + re.col], 1u, s.spin)) break;
      reduce(i);
    }
    depart(ws, s.grid);
  });
  Result r;
  r.timeout = ws.status.load() != 0;
  for (int i = 0; i < n_tile && !r.timeout; ++i) r.entries_ok &= built[i] == 1;
  for (int i = 0; i < n_red && !r.timeout; ++i) r.entries_ok &= reduced[i] == 1;
  r.data_ok = bad_data == 0;
  r.reset_ok = all_zero(ws);
  return r;
}

// ---- expert combine: builders <-> pushers (two-way), then folders ----------
Result run_combine(const Scenario& s) {
  const int U = s.a, G = s.b, D = s.c;
  const int L = (s.grid + G - 1) / G;
  const int n_tile = U * (G + D), n_push = U, n_fold = U;   // one push slab and one fold block per unit
  Workspace ws(2 * U);
  std::atomic<uint32_t>* gu = &ws.ctr[0];
  std::atomic<uint32_t>* dn = &ws.ctr[U];
  std::vector<uint32_t> h(U * G, 0), y(U * D, 0);
  std::unique_ptr<std::atomic<int>[]> done(new std::atomic<int>[n_tile]), pushed(new std::atomic<int>[n_push]),
      folded(new std::atomic<int>[n_fold]);
  for (int i = 0; i < n_tile; ++i) done[i] = 0;
  for (int i = 0; i < n_push; ++i) pushed[i] = 0;
  for (int i = 0; i < n_fold; ++i) folded[i] = 0;
  std::atomic<int> bad_data{0};
  Faults f;
  f.drop = s.fault == "drop";
  f.kill = s.fault == "dead";
  f.delay = s.fault == "delay";
  const bool fused = s.mode != "fixed", two_way = s.mode == "fused";
  auto push = [&](int u) {
    f.pace();
    for (int nt = 0; nt < D; ++nt)
      if (y[u * D + nt] != 10u * u + nt + 1) bad_data++;
    pushed[u]++;
  };
  run_grid(s.grid, [&] {
    const uint32_t ticket = ws.ticket.fetch_add(1);
    const bool crew = !fused && ticket < (uint32_t)s.crew;
    bool ok = true;
    if (!crew) {
      for (bool first = true;; first = false) {
        if (two_way) {   // take the push queue's head while it is ready
          for (;;) {
            uint32_t hd = ws.head[2].load(std::memory_order_relaxed);
            if (hd >= (uint32_t)n_push || dn[hd].load(std::memory_order_acquire) < (uint32_t)D) break;
            if (!ws.head[2].compare_exchange_strong(hd, hd + 1, std::memory_order_relaxed)) continue;
            push((int)hd);
          }
        }
        const uint32_t j = claim(ws, ws.head[1]);
        if (j >= (uint32_t)n_tile) break;
        if (first && f.die()) {
          depart(ws, s.grid);
          return;
        }
        const kos::CombineTile t = kos::combine_tile_of((int)j, U, G, D, L, true, true);
        if (!t.down) {
          h[t.u * G + t.nt] = 100u * t.u + t.nt + 1;
          done[j]++;
          if (!f.skip_bump()) publish(gu[t.u]);
        } else {
          if (!observe(ws, gu[t.u], (uint32_t)G, s.spin)) {
            ok = false;
            break;
          }
          for (int g = 0; g < G; ++g)
            if (h[t.u * G + g] != 100u * t.u + g + 1) bad_data++;
          y[t.u * D + t.nt] = 10u * t.u + t.nt + 1;
          done[j]++;
          publish(dn[t.u]);
        }
      }
      if (!fused) {
        depart(ws, s.grid);
        return;
      }
    }
    for (; ok;) {   // pushes left over, in unit order
      const uint32_t i = claim(ws, ws.head[2]);
      if (i >= (uint32_t)n_push) break;
      if (!observe(ws, dn[i], (uint32_t)D, s.spin)) {
        ok = false;
        break;
      }
      push((int)i);
    }
    for (; ok;) {   // fold blocks: block b needs units b and U-1-b
      const uint32_t i = claim(ws, ws.head[3]);
      if (i >= (uint32_t)n_fold) break;
      if (!observe(ws, dn[i], (uint32_t)D, s.spin) || !observe(ws, dn[U - 1 - i], (uint32_t)D, s.spin)) break;
      if (y[i * D] != 10u * i + 1 || y[(U - 1 - i) * D] != 10u * (U - 1 - i) + 1) bad_data++;
      folded[i]++;
    }
    depart(ws, s.grid);
  });
  Result r;
  r.timeout = ws.status.load() != 0;
  for (int i = 0; i < n_tile && !r.timeout; ++i) r.entries_ok &= done[i] == 1;
  for (int i = 0; i < n_push && !r.timeout; ++i) r.entries_ok &= pushed[i] == 1;
  for (int i = 0; i < n_fold && !r.timeout; ++i) r.entries_ok &= folded[i] == 1;
  r.data_ok = bad_data == 0;
  r.reset_ok = all_zero(ws);
  return r;
}

// ---- the expert layer in one launch (forward, and backward) ----------------
// Movers deliver every unit's rows (two mover entries per unit, in an
// order that completes the units out of order; in the forward, the first
// `own` entries stand for our own tokens' entries, whose packed positions
// the fold reads); a unit's first-stage entries wait for its rows, its
// second-stage tiles for its first-stage entries; pushes are taken between
// tiles when ready (two-way), the rest after the tiles; a fold block waits
// for two units' second stage (and, forward, for every own-token mover
// entry).  The forward starts with the router (R entries, counted) and the
// per-expert scan (3 entries, each after every router entry), then a
// barrier of every workgroup on the scan count before any mover entry.
Result run_expert(const Scenario& s, bool layer) {
  const int U = s.a, G = s.b, D = s.c;
  const int L = (s.grid + G - 1) / G;
  const int n_mv = 2 * U, n_own = layer ? U / 2 : 0, n_route = layer ? 5 : 0, n_scan = layer ? 3 : 0;
  const int n_tile = U * (G + D), n_push = U, n_fold = U;
  // counters: route, scan, own moved, rows_in[U], st1[U], st2[U]
  Workspace ws(3 + 3 * U);
  std::atomic<uint32_t>& c_route = ws.ctr[0];
  std::atomic<uint32_t>& c_scan = ws.ctr[1];
  std::atomic<uint32_t>& c_own = ws.ctr[2];
  std::atomic<uint32_t>* rows_in = &ws.ctr[3];
  std::atomic<uint32_t>* st1 = &ws.ctr[3 + U];
  std::atomic<uint32_t>* st2 = &ws.ctr[3 + 2 * U];
  std::vector<uint32_t> rows(2 * U, 0), h(U * G, 0), y(U * D, 0), scanned(n_scan, 0);
  std::unique_ptr<std::atomic<int>[]> moved(new std::atomic<int>[n_mv]), done(new std::atomic<int>[n_tile]),
      pushed(new std::atomic<int>[n_push]), folded(new std::atomic<int>[n_fold]);
  for (int i = 0; i < n_mv; ++i) moved[i] = 0;
  for (int i = 0; i < n_tile; ++i) done[i] = 0;
  for (int i = 0; i < n_push; ++i) pushed[i] = 0;
  for (int i = 0; i < n_fold; ++i) folded[i] = 0;
  std::atomic<int> bad_data{0};
  Faults f;
  f.drop = s.fault == "drop";
  f.kill = s.fault == "dead";
  f.delay = s.fault == "delay";
  int stride = 7;   // mover entry i fills row slot (i * stride) % n_mv: a permutation (stride coprime to n_mv)
  while (std::gcd(stride, n_mv) != 1) stride += 2;
  auto mv_slot = [&](int i) { return (int)(((long)i * stride) % n_mv); };
  auto push = [&](int u) {
    f.pace();
    for (int nt = 0; nt < D; ++nt)
      if (y[u * D + nt] != 10u * u + nt + 1) bad_data++;
    pushed[u]++;
  };
  run_grid(s.grid, [&] {
    ws.ticket.fetch_add(1);
    bool ok = true;
    if (layer) {
      for (;;) {   // router entries
        const uint32_t i = claim(ws, ws.head[0]);
        if (i >= (uint32_t)n_route) break;
        publish(c_route);
      }
      for (;;) {   // scan entries, each after every router entry
        const uint32_t e = claim(ws, ws.head[1]);
        if (e >= (uint32_t)n_scan) break;
        if (!(ok = observe(ws, c_route, (uint32_t)n_route, s.spin))) break;
        scanned[e] = 1;
        publish(c_scan);
      }
      if (ok) ok = observe(ws, c_scan, (uint32_t)n_scan, s.spin);   // every workgroup: the layer's bookkeeping
      for (int e = 0; e < n_scan && ok; ++e)
        if (scanned[e] != 1) bad_data++;
    }
    for (bool first = true; ok; first = false) {   // movers
      const uint32_t i = claim(ws, ws.head[2]);
      if (i >= (uint32_t)n_mv) break;
      if (first && f.die()) {   // claimed, never delivered, never departs normally
        depart(ws, s.grid);
        return;
      }
      f.pace();
      const int slot = mv_slot((int)i), u = slot / 2;
      rows[slot] = 1000u * u + slot % 2 + 1;
      moved[i]++;
      if (!f.skip_bump()) publish(rows_in[u]);
      if ((int)i < n_own) publish(c_own);
    }
    for (; ok;) {   // tiles, two-way with pushes
      for (;;) {
        uint32_t hd = ws.head[4].load(std::memory_order_relaxed);
        if (hd >= (uint32_t)n_push || st2[hd].load(std::memory_order_acquire) < (uint32_t)D) break;
        if (!ws.head[4].compare_exchange_strong(hd, hd + 1, std::memory_order_relaxed)) continue;
        push((int)hd);
      }
      const uint32_t j = claim(ws, ws.head[3]);
      if (j >= (uint32_t)n_tile) break;
      const kos::CombineTile t = kos::combine_tile_of((int)j, U, G, D, L, true, true);
      if (!t.down) {
        if (!(ok = observe(ws, rows_in[t.u], 2u, s.spin))) break;
        for (int k = 0; k < 2; ++k)
          if (rows[2 * t.u + k] != 1000u * t.u + k + 1) bad_data++;
        h[t.u * G + t.nt] = 100u * t.u + t.nt + 1;
        done[j]++;
        publish(st1[t.u]);
      } else {
        if (!(ok = observe(ws, st1[t.u], (uint32_t)G, s.spin))) break;
        for (int g = 0; g < G; ++g)
          if (h[t.u * G + g] != 100u * t.u + g + 1) bad_data++;
        y[t.u * D + t.nt] = 10u * t.u + t.nt + 1;
        done[j]++;
        publish(st2[t.u]);
      }
    }
    for (; ok;) {   // pushes left over
      const uint32_t i = claim(ws, ws.head[4]);
      if (i >= (uint32_t)n_push) break;
      if (!(ok = observe(ws, st2[i], (uint32_t)D, s.spin))) break;
      push((int)i);
    }
    if (ok && layer) ok = observe(ws, c_own, (uint32_t)n_own, s.spin);
    for (; ok;) {   // fold blocks: block b needs units b and U-1-b
      const uint32_t i = claim(ws, ws.head[5]);
      if (i >= (uint32_t)n_fold) break;
      if (!observe(ws, st2[i], (uint32_t)D, s.spin) || !observe(ws, st2[U - 1 - i], (uint32_t)D, s.spin)) break;
      if (y[i * D] != 10u * i + 1 || y[(U - 1 - i) * D] != 10u * (U - 1 - i) + 1) bad_data++;
      folded[i]++;
    }
    depart(ws, s.grid);
  });
  Result r;
  r.timeout = ws.status.load() != 0;
  for (int i = 0; i < n_mv && !r.timeout; ++i) r.entries_ok &= moved[i] == 1;
  for (int i = 0; i < n_tile && !r.timeout; ++i) r.entries_ok &= done[i] == 1;
  for (int i = 0; i < n_push && !r.timeout; ++i) r.entries_ok &= pushed[i] == 1;
  for (int i = 0; i < n_fold && !r.timeout; ++i) r.entries_ok &= folded[i] == 1;
  r.data_ok = bad_data == 0;
  r.reset_ok = all_zero(ws);
  return r;
}

// "order <op> ..." lines print a queue's decoded entries, one per line, so
// the tests can check the orders themselves:
//   order ag W R RB M NT     moves "m shard rb sub", then tiles "t q shard rb nt"
//   order rs W B NT ROW      tiles "t band chunk col"
//   order combine U G D L    tiles "t down u nt"
void print_order(std::istringstream& in) {
  std::string op;
  in >> op;
  if (op == "ag") {
    int W, R, RB, M, NT;
    in >> W >> R >> RB >> M >> NT;
    for (int i = 0; i < W * RB * M; ++i) {
      const kos::AgMove m = kos::ag_move_of(i, W, R, RB, M);
      std::printf("m %d %d %d\n", m.shard, m.rb, m.sub);
    }
    for (int j = 0; j < W * RB * NT; ++j) {
      const kos::AgTile t = kos::ag_tile_of(j, W, R, RB, NT);
      std::printf("t %d %d %d %d\n", t.q, t.shard, t.rb, t.nt);
    }
  } else if (op == "rs") {
    int W, B, NT, row;
    in >> W >> B >> NT >> row;
    for (int j = 0; j < W * B * NT; ++j) {
      const kos::RsTile t = kos::rs_tile_of(j, row != 0, W, B, NT);
      std::printf("t %d %d %d\n", t.band, t.chunk, t.col);
    }
  } else {
    int U, G, D, L;
    in >> U >> G >> D >> L;
    for (int j = 0; j < U * (G + D); ++j) {
      const kos::CombineTile t = kos::combine_tile_of(j, U, G, D, L, true, true);
      std::printf("t %d %d %d\n", t.down ? 1 : 0, t.u, t.nt);
    }
  }
  std::printf("end\n");
  std::fflush(stdout);
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    if (line.empty() || line[0] == '#') continue;
    std::istringstream in(line);
    if (line.compare(0, 6, "order ") == 0) {
      std::string w;
      in >> w;
      print_order(in);
      continue;
    }
    Scenario s;
    in >> s.op >> s.grid >> s.world >> s.rank >> s.a >> s.b >> s.c >> s.mode >> s.crew >> s.fault >> s.spin;
    if (!in || s.grid < 1 || s.world < 1 || s.rank < 0 || s.rank >= s.world || s.a < 1 || s.b < 1 || s.c < 1) {
      std::printf("bad scenario: %s\n", line.c_str());
      return 2;
    }
    Result r = s.op == "ag"      ? run_ag(s)
               : s.op == "rs"    ? run_rs(s)
               : s.op == "layer" ? run_expert(s, true)
               : s.op == "bwd"   ? run_expert(s, false)
                                 : run_combine(s);
    std::printf("status=%s entries=%s data=%s reset=%s\n", r.timeout ? "timeout" : "ok",
                r.entries_ok ? "ok" : "bad", r.data_ok ? "ok" : "bad", r.reset_ok ? "ok" : "bad");
    std::fflush(stdout);
  }
  return 0;
}
