"""The queue / ready-counter protocol, modelled on the CPU with one thread per
workgroup (tests/protocol_model/kos_protocol_model.cpp, built here with
ThreadSanitizer): the kernels' own entry orders and role rules, every crew
size, and forced faults; the expert layer's one-launch forward and
backward protocols too.  Checks: no deadlock for any crew of one or more
(every entry done exactly once, every read ordered after its write, the
last workgroup out leaves the counters at zero), and a time-out -- not a
hang -- when the protocol is broken (no mover at all, a dropped ready bump,
a workgroup that dies holding an entry)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol_model", "kos_protocol_model.cpp")

OK = "status=ok entries=ok data=ok reset=ok"
TIMEOUT = "status=timeout entries=ok data=ok reset=ok"


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("kpm") / "kos_protocol_model")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", SRC, "-o", exe], check=True,
                   capture_output=True, text=True)
    return exe


def run(model, lines, timeout=180):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([model], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=timeout,
                       env=env)
    assert r.returncode == 0, f"model exit {r.returncode} (66 = data race):\n{r.stderr[-3000:]}"
    out = r.stdout.strip().splitlines()
    assert len(out) == len(lines), r.stdout
    return out


def test_every_crew_completes(model):
    """Fused (both switching policies) and fixed, every crew from 1 to
    grid-1 (reduce-scatter fused also 0: its builders switch), several grids
    and worlds."""
    lines = []
    for grid in (2, 3, 5, 8):
        for world, rank in ((1, 0), (2, 1), (4, 3)):
            for crew in range(0, grid):
                for mode in ("fused", "swapped", "fixed"):
                    if crew >= 1 or mode != "fixed":
                        if crew >= 1:
                            lines.append(f"ag {grid} {world} {rank} 2 3 4 {mode} {crew} none 10000000")
                        lines.append(f"rs {grid} {world} {rank} 2 3 2 {mode} {crew} none 10000000")
            lines.append(f"combine {grid} 1 0 7 2 3 fused 0 none 10000000")
            lines.append(f"combine {grid} 1 0 7 2 3 swapped 0 none 10000000")
            for crew in range(1, grid):
                lines.append(f"combine {grid} 1 0 7 2 3 fixed {crew} none 10000000")
    out = run(model, lines)
    bad = [(l, o) for l, o in zip(lines, out) if o != OK]
    assert not bad, bad[:5]


def test_expert_layer_one_launch_completes(model):
    """The expert layer forward in one launch (router, scan, barrier,
    movers, two-way tiles and pushes, fold) and its backward (movers,
    first-stage entries, second-stage tiles, pushes, fold): every grid and
    shape completes with every entry done once and every read after its
    write."""
    lines = []
    for grid in (2, 3, 5, 8):
        for op in ("layer", "bwd"):
            for u, g, d in ((1, 1, 1), (5, 2, 3), (9, 3, 2), (14, 4, 5)):
                lines.append(f"{op} {grid} 1 0 {u} {g} {d} fused 0 none 10000000")
            lines.append(f"{op} {grid} 1 0 6 2 2 fused 0 delay 100000000")
    assert run(model, lines) == [OK] * len(lines)


def test_expert_layer_broken_protocol_times_out(model):
    lines = ["layer 6 1 0 9 2 3 fused 0 drop 20000",   # one unit's row bump lost
             "bwd 6 1 0 9 2 3 fused 0 drop 20000",
             "layer 6 1 0 9 2 3 fused 0 dead 20000",   # a mover dies holding an entry
             "bwd 6 1 0 9 2 3 fused 0 dead 20000"]
    assert run(model, lines, timeout=120) == [TIMEOUT] * len(lines)


def test_slow_communication_still_completes(model):
    lines = ["ag 6 4 1 2 2 3 fused 1 delay 100000000", "rs 6 4 2 2 2 2 fused 0 delay 100000000",
             "combine 6 1 0 6 2 2 fused 0 delay 100000000", "ag 6 4 0 1 4 2 fixed 2 delay 100000000"]
    assert run(model, lines) == [OK] * len(lines)


def test_broken_protocol_times_out_instead_of_hanging(model):
    lines = [
        "ag 8 4 1 2 3 4 fused 0 none 20000",         # no mover: remote tiles never become ready
        "ag 8 4 1 2 3 4 fused 3 drop 20000",         # one slice's ready bump lost
        "ag 8 4 1 2 3 4 fixed 2 dead 20000",         # a mover dies holding an entry
        "rs 6 4 0 2 3 2 fused 0 drop 20000",         # one of our tiles never flagged
        "rs 6 4 0 2 3 2 fixed 2 dead 20000",         # the builder of our first tile dies
        "combine 6 1 0 9 2 3 fused 0 drop 20000",    # a gate/up tile never flagged
        "combine 6 1 0 9 2 3 fixed 2 dead 20000",    # a builder dies holding a gate/up tile
        "ag 8 4 1 2 3 4 swapped 0 none 20000",       # two-way builders take the moves: completes
        "rs 6 4 0 2 3 2 swapped 0 drop 20000",
        "combine 6 1 0 9 2 3 swapped 0 drop 20000",
    ]
    assert run(model, lines, timeout=120) == [TIMEOUT] * 7 + [OK] + [TIMEOUT] * 2


def _order(model, spec):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([model], input=f"order {spec}\n", capture_output=True, text=True, timeout=60, env=env)
    assert r.returncode == 0, r.stderr
    rows = r.stdout.strip().splitlines()
    assert rows[-1] == "end"
    return [tuple([x[0]] + [int(v) for v in x.split()[1:]]) for x in rows[:-1]]


def test_queue_orders_follow_the_pages(model):
    """The orders the kernels decode their queues with (kos_order.h):
    all-gather -- movers copy remote shards in tile-consumption order
    (rank+1, rank+2, ...), whole row blocks at a time, then the
    local copy; tiles of the local shard come first, then the remote shards
    in the movers' order ("Role switching only works if ...": local shard
    first, remote shards in consumption order).  Reduce-scatter band order
    -- every chunk's band b before any band b+1 (the same paragraph's
    consumer order for the reducers); row order -- one chunk after another.
    Combine -- every
    down tile after all gate/up tiles of its unit, by about L units."""
    W, R, RB, M, NT = 4, 1, 2, 3, 5
    o = _order(model, f"ag {W} {R} {RB} {M} {NT}")
    moves = [x[1:] for x in o if x[0] == "m"]
    tiles = [x[1:] for x in o if x[0] == "t"]
    assert sorted(moves) == sorted((s, b, u) for s in range(W) for b in range(RB) for u in range(M))
    shard_seq = [m[0] for m in moves]
    expect = [(R + 1 + i) % W for i in range(W - 1)] + [R]
    assert [shard_seq[i * RB * M] for i in range(W)] == expect, "remote shards in consumption order, local last"
    assert moves == sorted(moves, key=lambda m: (expect.index(m[0]), m[1], m[2]))
    assert sorted(t[1:] for t in tiles) == sorted((s, b, n) for s in range(W) for b in range(RB) for n in range(NT))
    assert [t[1] for t in tiles[:RB * NT]] == [R] * (RB * NT) and all(t[0] == 0 for t in tiles[:RB * NT])
    assert [t[1] for t in tiles] == [expect[(t[0] - 1) % W] if t[0] else R for t in tiles]
    assert [t[1] for t in tiles][RB * NT::RB * NT] == expect[:-1], "remote tiles follow the movers"

    W, B, NT = 4, 3, 2
    band = [x[1:] for x in _order(model, f"rs {W} {B} {NT} 0")]
    row = [x[1:] for x in _order(model, f"rs {W} {B} {NT} 1")]
    full = sorted((b, c, n) for b in range(B) for c in range(W) for n in range(NT))
    assert sorted(band) == full and sorted(row) == full
    assert [t[0] for t in band] == sorted(t[0] for t in band), "band by band"
    assert {t[1] for t in band[:W * NT]} == set(range(W)), "the first band covers every chunk"
    assert [t[1] for t in row] == sorted(t[1] for t in row), "row order: chunk after chunk"

    U, G, D, L = 7, 2, 3, 2
    comb = [x[1:] for x in _order(model, f"combine {U} {G} {D} {L}")]
    assert sorted(comb) == sorted([(0, u, n) for u in range(U) for n in range(G)] +
                                  [(1, u, n) for u in range(U) for n in range(D)])
    pos = {t: i for i, t in enumerate(comb)}
    for u in range(U):
        last_gu = max(pos[(0, u, n)] for n in range(G))
        first_dn = min(pos[(1, u, n)] for n in range(D))
        assert first_dn > last_gu
        if u + L - 1 < U:
            assert first_dn > max(pos[(0, u + L - 1, n)] for n in range(G)), "down tiles lag by L units"
