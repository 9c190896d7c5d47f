"""Seeded random shapes for every op on the GPU against the oracle: world
sizes 1-8, ranks, tile-ragged sizes and modes drawn from a fixed seed, so a
run checks the same cases every time.  AG and RS use integer-valued inputs
(exact in fp32, compared bit for bit); the expert layer checks routing,
permutation and movement bit for bit and the float outputs within the
tolerance."""
import random

import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import assert_close, say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu

_rng = random.Random(20261202)


def _ag_cases(n):
    out = []
    for i in range(n):
        world = _rng.randint(1, 8)
        s = KI.AgShape(f"ag_rand{i}", 70 + i, world, _rng.choice([64, 128, 192, 256, 320]),
                       _rng.choice([64, 128, 192, 320, 512]), _rng.choice([64, 128, 192, 256, 384, 640]))
        out.append((s, _rng.randrange(world), _rng.choice([0, 1, 2])))
    return out


def _rs_cases(n):
    out = []
    for i in range(n):
        world = _rng.randint(1, 8)
        s = KI.RsShape(f"rs_rand{i}", 80 + i, world, world * _rng.choice([64, 128, 256, 320]),
                       _rng.choice([64, 128, 192, 320, 512]), _rng.choice([64, 128, 192, 256, 384]))
        out.append((s, _rng.randrange(world), _rng.choice([0, 1, 2]), _rng.choice([0, 1])))
    return out


def _moe_cases(n):
    out = []
    for i in range(n):
        world = _rng.randint(1, 4)
        experts = world * _rng.randint(1, 5)
        s = KI.MoeShape(f"moe_rand{i}", 90 + i, world, _rng.randint(1, 150), _rng.choice([128, 256, 384, 512]),
                        experts, _rng.randint(1, min(experts, 6)), _rng.choice([64, 128, 192, 256]))
        out.append((s, _rng.randrange(world), _rng.choice([0, 2])))
    return out


AG_CASES, RS_CASES, MOE_CASES = _ag_cases(6), _rs_cases(6), _moe_cases(6)


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


@pytest.fixture(scope="module")
def ws(kos):
    return kos.Workspace("cuda")


def _crew(mode, grid):
    return -1 if mode != 1 else min(4, grid - 1)


@pytest.mark.parametrize("s,rank,mode", AG_CASES, ids=[f"{c[0].world}r_{c[0].m_local}x{c[0].k}x{c[0].n}_r{c[1]}_m{c[2]}"
                                                        for c in AG_CASES])
def test_ag_random(kos, ws, s, rank, mode):
    say(f"[ag rand] {s} rank={rank} mode={mode}")
    dev = "cuda"
    inp = KI.ag_inputs(s, rank, dev, integer=True)
    g = torch.full((s.m, s.k), float("nan"), dtype=torch.bfloat16, device=dev)
    c = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device=dev)
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws,
                kos.opts(mode=mode, n_movers=_crew(mode, kos.lib.kos_device_cu_count())))
    ws.status()
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    gref, cref = O.ag_gemm(KI.bf16_bits(inp["a_local"]), peers, KI.bf16_bits(inp["w"]), rank, out_dtype="f32")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert np.array_equal(c.cpu().numpy(), cref)


@pytest.mark.parametrize("s,rank,mode,order", RS_CASES,
                         ids=[f"{c[0].world}r_{c[0].m}x{c[0].k}x{c[0].n}_r{c[1]}_m{c[2]}_o{c[3]}" for c in RS_CASES])
def test_rs_random(kos, ws, s, rank, mode, order):
    say(f"[rs rand] {s} rank={rank} mode={mode} order={order}")
    dev = "cuda"
    inp = KI.rs_inputs(s, rank, dev, integer=True)
    part = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device=dev)
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device=dev)
    crew = -1 if mode != 1 else 3
    kos.gemm_rs(inp["a"], inp["w"], inp["peer_slices"], part, y, rank, ws,
                kos.opts(mode=mode, n_movers=crew, rs_order=order))
    ws.status()
    peers = [None if t is None else t.cpu().numpy() for t in inp["peer_slices"]]
    pref, yref = O.gemm_rs(KI.bf16_bits(inp["a"]), KI.bf16_bits(inp["w"]), peers, rank)
    assert np.array_equal(y.cpu().numpy(), yref)
    pgpu = part.cpu().numpy()
    for c in range(s.world):   # outbound rows (every chunk but ours) are the exact partial product
        if c != rank:
            rows = slice(c * s.m_chunk, (c + 1) * s.m_chunk)
            assert np.array_equal(pgpu[rows], pref[rows])


@pytest.mark.parametrize("s,rank,mode", MOE_CASES,
                         ids=[f"{c[0].world}r_t{c[0].tokens}_h{c[0].hidden}_e{c[0].experts}_k{c[0].topk}_f{c[0].ffn}"
                              f"_r{c[1]}_m{c[2]}" for c in MOE_CASES])
def test_moe_random(kos, ws, s, rank, mode):
    from gemm_collective_persistent_amd.api import moe_shape
    say(f"[moe rand] {s} rank={rank} mode={mode}")
    dev = "cuda"
    inp = KI.moe_inputs(s, rank, dev)
    T, k, E, H, F = s.tokens, s.topk, s.experts, s.hidden, s.ffn
    pc = inp["peer_counts"].cpu().numpy()
    cap = max(int(pc.sum()) + T * min(k, s.e_local), 1)
    shp = moe_shape(s.world, rank, T, H, E, k, F)
    o = kos.opts(mode=mode)
    idx = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev)
    counts = torch.full((E,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    send = [None if p == rank else torch.zeros((max(s.peer_cap, 1), H), dtype=torch.bfloat16, device=dev)
            for p in range(s.world)]
    grouped = torch.zeros((cap, H), dtype=torch.bfloat16, device=dev)
    goff = torch.full((s.e_local + 1,), -1, dtype=torch.int32, device=dev)
    row_src = torch.full((cap, 2), -1, dtype=torch.int32, device=dev)
    kos.moe_dispatch(shp, inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"], idx, w, counts, perm,
                     send, grouped, goff, row_src, ws, o)
    ws.status()
    peer_send = [None if t is None else KI.bf16_bits(t) for t in inp["peer_send"]]
    d = O.dispatch(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), peer_send, pc, s.world, rank, k)
    n = int(d["grouped_offsets"][-1])
    assert np.array_equal(idx.cpu().numpy(), d["idx"])
    assert np.array_equal(perm.cpu().numpy(), d["perm"])
    assert np.array_equal(counts.cpu().numpy(), d["counts"])
    assert np.array_equal(goff.cpu().numpy(), d["grouped_offsets"])
    assert np.array_equal(row_src[:n].cpu().numpy(), d["row_src"])
    assert np.array_equal(KI.bf16_bits(grouped[:n]), d["grouped"])
    assert_close(w.cpu().numpy(), d["w"], "topk weights")
    for q in range(s.world):
        if q != rank:
            nq = d["send"][q].shape[0]
            assert np.array_equal(KI.bf16_bits(send[q][:nq]), d["send"][q])

    h = torch.full((cap, F), float("nan"), dtype=torch.bfloat16, device=dev)
    yg = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    ret = [None if q == rank else torch.full((max(int(pc[q].sum()), 1), H), float("nan"), dtype=torch.bfloat16,
                                             device=dev) for q in range(s.world)]
    kos.moe_combine(shp, grouped, goff, row_src, inp["wg"], inp["wu"], inp["wd"], idx, w, counts, perm,
                    inp["peer_counts"], inp["peer_return"], h, yg, ret, y, ws, o)
    ws.status()
    wg, wu, wd = (KI.bf16_bits(inp[x]) for x in ("wg", "wu", "wd"))
    yg_ref = O.grouped_ffn(d["grouped"], d["grouped_offsets"], wg, wu, wd)
    if n:
        assert_close(O.bf16_to_f64(KI.bf16_bits(yg[:n])), O.bf16_to_f64(yg_ref), "y_grouped")
        ygpu = KI.bf16_bits(yg[:n])
        for r_, (q, i) in enumerate(d["row_src"]):
            if q != rank:
                assert np.array_equal(KI.bf16_bits(ret[q][i]), ygpu[r_]), "pushed rows are bit copies"
    pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
    yref = O.fold(d["idx"], d["w"], d["perm"], d["offsets"], yg_ref, d["grouped_offsets"], pc, pret, s.world, rank)
    assert_close(O.bf16_to_f64(KI.bf16_bits(y)), O.bf16_to_f64(yref), "y")
