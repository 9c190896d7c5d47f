"""Seeded random shapes for the MXFP8 and transposed-weight variants of both
collectives on the GPU against the oracle: world sizes 1-8, ranks, modes and
(for the transposed weights) tile-ragged sizes drawn from a fixed seed.
Integer-valued inputs: every fp32 sum is exact, outputs compared bit for
bit."""
import random

import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu

_rng = random.Random(20261203)


def _cases():
    ag_mx, rs_mx, ag_wt, rs_wt = [], [], [], []
    for i in range(4):
        world = _rng.randint(1, 8)
        s = KI.AgShape(f"ag_mx_rand{i}", 100 + i, world, _rng.choice([256, 512]), _rng.choice([256, 512, 768]),
                       _rng.choice([256, 512, 768]))
        ag_mx.append((s, _rng.randrange(world), _rng.choice([0, 1, 2])))
    for i in range(4):
        world = _rng.randint(1, 8)
        s = KI.RsShape(f"rs_mx_rand{i}", 110 + i, world, world * _rng.choice([256, 512]),
                       _rng.choice([256, 512, 768]), _rng.choice([256, 512]))
        rs_mx.append((s, _rng.randrange(world), _rng.choice([0, 1, 2]), _rng.choice([0, 1])))
    for i in range(4):
        world = _rng.randint(1, 8)
        s = KI.AgShape(f"ag_wt_rand{i}", 120 + i, world, _rng.choice([64, 128, 192, 256]),
                       _rng.choice([64, 192, 320, 512]), _rng.choice([64, 128, 192, 384]))
        ag_wt.append((s, _rng.randrange(world), _rng.choice([0, 1, 2])))
    for i in range(4):
        world = _rng.randint(1, 8)
        s = KI.RsShape(f"rs_wt_rand{i}", 130 + i, world, world * _rng.choice([64, 128, 256]),
                       _rng.choice([64, 192, 320]), _rng.choice([64, 128, 256, 384]))
        rs_wt.append((s, _rng.randrange(world), _rng.choice([0, 1, 2]), _rng.choice([0, 1])))
    return ag_mx, rs_mx, ag_wt, rs_wt


AG_MX, RS_MX, AG_WT, RS_WT = _cases()


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


@pytest.fixture(scope="module")
def ws(kos):
    return kos.Workspace("cuda")


def _np(t):
    return None if t is None else t.cpu().numpy()


def _nat(t):
    return None if t is None else O.scales_from_slabs(_np(t))


def _crew(kos, mode):
    return kos.opts(mode=mode, n_movers=-1 if mode == 0 else 2)


@pytest.mark.parametrize("case", range(len(AG_MX)))
def test_random_ag_mx(kos, ws, case):
    s, rank, mode = AG_MX[case]
    say(f"[random ag mx] {s} rank={rank} mode={mode}")
    inp = KI.ag_mx_inputs(s, rank, "cuda", integer=True)
    g = torch.empty((s.m, s.k), dtype=torch.uint8, device="cuda")
    gs = torch.empty((s.k // 64, s.m, 2), dtype=torch.uint8, device="cuda")
    c = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    kos.ag_gemm_mx(inp["a_local"], inp["s_local"], inp["a_peers"], inp["s_peers"], inp["w"], inp["w_scales"],
                   g, gs, c, rank, ws, _crew(kos, mode))
    ws.status()
    gref, gsref, cref = O.ag_gemm_mx(_np(inp["a_local"]), _nat(inp["s_local"]), [_np(t) for t in inp["a_peers"]],
                                     [_nat(t) for t in inp["s_peers"]], _np(inp["w"]), _nat(inp["w_scales"]), rank,
                                     "f32")
    assert np.array_equal(_np(g), gref) and np.array_equal(_nat(gs), gsref)
    assert np.array_equal(_np(c), cref)


@pytest.mark.parametrize("case", range(len(RS_MX)))
def test_random_rs_mx(kos, ws, case):
    s, rank, mode, order = RS_MX[case]
    say(f"[random rs mx] {s} rank={rank} mode={mode} order={order}")
    inp = KI.rs_mx_inputs(s, rank, "cuda", integer=True)
    partial = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device="cuda")
    o = kos.opts(mode=mode, n_movers=0 if mode == 0 else 2, rs_order=order)
    kos.gemm_rs_mx(inp["a"], inp["a_scales"], inp["w"], inp["w_scales"], inp["peer_slices"], partial, y, rank, ws, o)
    ws.status()
    pref, yref = O.gemm_rs_mx(_np(inp["a"]), _nat(inp["a_scales"]), _np(inp["w"]), _nat(inp["w_scales"]),
                              [_np(t) for t in inp["peer_slices"]], rank)
    assert np.array_equal(_np(partial), pref) and np.array_equal(_np(y), yref)


@pytest.mark.parametrize("case", range(len(AG_WT)))
def test_random_ag_wt(kos, ws, case):
    s, rank, mode = AG_WT[case]
    say(f"[random ag wt] {s} rank={rank} mode={mode}")
    inp = KI.ag_inputs(s, rank, "cuda", integer=True, wt=True)
    g = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws, _crew(kos, mode),
                w_transposed=True)
    ws.status()
    bits = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    gref, cref = O.ag_gemm_wt(KI.bf16_bits(inp["a_local"]), bits, KI.bf16_bits(inp["w"]), rank, "f32")
    assert np.array_equal(KI.bf16_bits(g), gref) and np.array_equal(_np(c), cref)


@pytest.mark.parametrize("case", range(len(RS_WT)))
def test_random_rs_wt(kos, ws, case):
    s, rank, mode, order = RS_WT[case]
    say(f"[random rs wt] {s} rank={rank} mode={mode} order={order}")
    inp = KI.rs_inputs(s, rank, "cuda", integer=True, wt=True)
    partial = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device="cuda")
    o = kos.opts(mode=mode, n_movers=0 if mode == 0 else 2, rs_order=order)
    kos.gemm_rs(inp["a"], inp["w"], inp["peer_slices"], partial, y, rank, ws, o, w_transposed=True)
    ws.status()
    pref, yref = O.gemm_rs_wt(KI.bf16_bits(inp["a"]), KI.bf16_bits(inp["w"]), [_np(t) for t in inp["peer_slices"]],
                              rank)
    assert np.array_equal(_np(partial), pref) and np.array_equal(_np(y), yref)
