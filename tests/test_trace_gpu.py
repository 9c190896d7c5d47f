"""Per-workgroup timelines (kos_opts.trace) on the GPU: a traced call still
matches the oracle, and its timeline is consistent with the queues it ran."""
import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


def test_ag_trace_covers_every_entry(kos):
    from gemm_collective_persistent_amd.timeline import summarize
    say("[trace ag tiny]")
    ws = kos.Workspace("cuda")
    s, rank = KI.AG_TINY, 1
    grid = kos.lib.kos_device_cu_count()
    inp = KI.ag_inputs(s, rank, "cuda", integer=True)
    g = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws, kos.opts(trace=True))
    ws.status()
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    gref, cref = O.ag_gemm(KI.bf16_bits(inp["a_local"]), peers, KI.bf16_bits(inp["w"]), rank, out_dtype="f32")
    assert np.array_equal(KI.bf16_bits(g), gref) and np.array_equal(c.cpu().numpy(), cref)

    tl = ws.trace(grid)
    assert sorted(t for t, _, _, _ in tl) == list(range(grid)), "every workgroup took one ticket"
    tiles, moves = [], []
    for _, b, e, recs in tl:
        assert e >= b
        for kind, entry, t0, t1 in recs:
            assert b - 1e-3 <= t0 <= t1 <= e + 1e-3, "records lie inside their workgroup's lifetime"
            (tiles if kind == "tile" else moves if kind == "move" else []).append(entry)
    # 4 shards of 64 rows, 64 x 64 tiles: 16 tiles; one 64-row move per shard
    assert sorted(tiles) == list(range(16))
    assert sorted(moves) == list(range(4))
    sm = summarize(tl)
    assert 0.0 <= sm["wait_frac"] <= sm["idle_frac"] <= 1.0
    assert sm["kinds"]["tile"]["n"] == 16
    # clock record: every workgroup ran between 100 MHz and the 2.4 GHz peak
    assert len(ws.trace_clock_mhz) == grid
    assert all(100.0 <= f <= 2500.0 for f in ws.trace_clock_mhz), ws.trace_clock_mhz[:8]


def test_trace_off_leaves_header_untouched(kos):
    """Without the option nothing is written to the trace region."""
    say("[trace off]")
    ws = kos.Workspace("cuda")
    s, rank = KI.AG_TINY, 0
    inp = KI.ag_inputs(s, rank, "cuda", integer=True)
    g = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    region = 4 * 256 * 512 * 16            # KOS_TRACE_LAUNCHES slots at the end of the workspace
    ws.buf[-region:].fill_(0)
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws, kos.opts())
    ws.status()
    assert int(ws.buf[-region:].count_nonzero()) == 0


def test_unfused_trace_holds_every_launch(kos):
    """An unfused call's two launches record into two slots of the trace
    region: the moves in the first, the tiles in the second, the second
    starting after the first ended; the summary over both counts the gap
    between them as idle."""
    from gemm_collective_persistent_amd.timeline import summarize
    say("[trace ag unfused]")
    ws = kos.Workspace("cuda")
    s, rank = KI.AG_TINY, 2
    grid = kos.lib.kos_device_cu_count()
    inp = KI.ag_inputs(s, rank, "cuda", integer=True)
    g = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws, kos.opts(mode=2, trace=True))
    ws.status()
    tl = ws.trace(grid, launches=2)
    assert len(tl) == 2 * grid
    first, second = tl[:grid], tl[grid:]
    moves = sorted(e for _, _, _, recs in first for k, e, _, _ in recs if k == "move")
    tiles = sorted(e for _, _, _, recs in second for k, e, _, _ in recs if k == "tile")
    assert moves == list(range(4)) and tiles == list(range(16))
    assert not any(k == "tile" for _, _, _, recs in first for k, _, _, _ in recs)
    end_first = max(e for _, _, e, _ in first)
    assert min(b for _, b, _, _ in second) >= end_first - 1e-3
    sm = summarize(tl, workgroups=grid)
    work = sum(t1 - t0 for _, _, _, recs in tl for k, _, t0, t1 in recs if k != "wait")
    assert sm["idle_frac"] == pytest.approx(1.0 - work / (grid * sm["span_us"]), abs=2e-4)
