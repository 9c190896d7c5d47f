"""The single-launch expert layer (kos_moe_layer: router -> fold in one
persistent launch) on the GPU against the oracle, through the C ABI.

Small shapes: every output against the oracle's whole layer -- routing,
counts, permutation, offsets, provenance, grouped and send rows bit-exact;
pushed rows bit copies of the expert outputs at the oracle's provenance;
expert outputs and folded tokens within the floating-point bar.  Full
shapes: the dispatch outputs bit-exact against the oracle, every expert
output and every folded token bit-identical to the two-launch path
(dispatch then combine, itself checked against the oracle), whole first
and last units of every expert and 512 tokens end to end against the
oracle."""
import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import assert_close, say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


@pytest.fixture(scope="module")
def ws(kos):
    return kos.Workspace("cuda")


def _shape(s, rank):
    from gemm_collective_persistent_amd.api import moe_shape
    return moe_shape(s.world, rank, s.tokens, s.hidden, s.experts, s.topk, s.ffn)


def _buffers(s, rank, pc):
    dev = "cuda"
    T, k, E, H, F = s.tokens, s.topk, s.experts, s.hidden, s.ffn
    cap = max(int(pc.sum()) + T * min(k, s.e_local), 1)
    nan = float("nan")
    return dict(
        idx=torch.full((max(T, 1), k), -1, dtype=torch.int32, device=dev)[:T] if T else
        torch.empty((0, k), dtype=torch.int32, device=dev),
        w=torch.full((T, k), nan, dtype=torch.float32, device=dev),
        counts=torch.full((E,), -1, dtype=torch.int32, device=dev),
        perm=torch.full((T * k,), -1, dtype=torch.int32, device=dev),
        send=[None if p == rank else torch.zeros((max(s.peer_cap, 1), H), dtype=torch.bfloat16, device=dev)
              for p in range(s.world)],
        grouped=torch.zeros((cap, H), dtype=torch.bfloat16, device=dev),
        goff=torch.full((s.e_local + 1,), -1, dtype=torch.int32, device=dev),
        row_src=torch.full((cap, 2), -1, dtype=torch.int32, device=dev),
        h=torch.full((cap, F), nan, dtype=torch.bfloat16, device=dev),
        gs=torch.full((cap, F), nan, dtype=torch.bfloat16, device=dev),
        us=torch.full((cap, F), nan, dtype=torch.bfloat16, device=dev),
        yg=torch.full((cap, H), nan, dtype=torch.bfloat16, device=dev),
        ret=[None if p == rank else torch.full((max(int(pc[p].sum()), 1), H), nan, dtype=torch.bfloat16,
                                               device=dev) for p in range(s.world)],
        y=torch.full((T, H), nan, dtype=torch.bfloat16, device=dev),
    )


def run_layer(kos, ws, s, rank, inp, o=None, save=False):
    """save: the layer also keeps bf16 g and u (b["gs"], b["us"])."""
    pc = inp["peer_counts"].cpu().numpy()
    b = _buffers(s, rank, pc)
    kos.moe_layer(_shape(s, rank), inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"], inp["wg"],
                  inp["wu"], inp["wd"], inp["peer_return"], b["idx"], b["w"], b["counts"], b["perm"], b["send"],
                  b["grouped"], b["goff"], b["row_src"], b["h"], b["yg"], b["ret"], b["y"], ws, o,
                  gate_save=b["gs"] if save else None, up_save=b["us"] if save else None)
    ws.status()
    torch.cuda.synchronize()
    return b


def run_two_launch(kos, ws, s, rank, inp, save=False):
    pc = inp["peer_counts"].cpu().numpy()
    b = _buffers(s, rank, pc)
    shp = _shape(s, rank)
    kos.moe_dispatch(shp, inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"], b["idx"], b["w"],
                     b["counts"], b["perm"], b["send"], b["grouped"], b["goff"], b["row_src"], ws)
    kos.moe_combine(shp, b["grouped"], b["goff"], b["row_src"], inp["wg"], inp["wu"], inp["wd"], b["idx"], b["w"],
                    b["counts"], b["perm"], inp["peer_counts"], inp["peer_return"], b["h"], b["yg"], b["ret"],
                    b["y"], ws, gate_save=b["gs"] if save else None, up_save=b["us"] if save else None)
    ws.status()
    torch.cuda.synchronize()
    return b


def _check_dispatch_part(s, rank, b, ref):
    n = int(ref["grouped_offsets"][-1])
    T = s.tokens
    assert np.array_equal(b["idx"][:T].cpu().numpy(), ref["idx"])
    assert np.array_equal(b["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(b["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(b["goff"].cpu().numpy(), ref["grouped_offsets"])
    assert np.array_equal(b["row_src"][:n].cpu().numpy(), ref["row_src"])
    assert np.array_equal(KI.bf16_bits(b["grouped"][:n]), ref["grouped"])
    if T:
        w = b["w"].cpu().numpy()
        assert_close(w, ref["w"], "topk weights")
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-5)
    for d in range(s.world):
        if d != rank:
            nd = ref["send"][d].shape[0]
            assert np.array_equal(KI.bf16_bits(b["send"][d][:nd]), ref["send"][d])


def _check_pushes(s, rank, b, ref, ygpu):
    rs = ref["row_src"]
    for p in range(s.world):
        if p == rank:
            continue
        sel = np.where(rs[:, 0] == p)[0]
        if sel.size:
            assert np.array_equal(KI.bf16_bits(b["ret"][p])[rs[sel, 1]], ygpu[sel]), f"pushed rows to rank {p}"


EDGE = [
    KI.MoeShape("moe_edge_2r_t70_h384_e6_k1_f64", 40, 2, 70, 384, 6, 1, 64),
    KI.MoeShape("moe_edge_1r_t33_h256_e8_k3_f128", 41, 1, 33, 256, 8, 3, 128),
    KI.MoeShape("moe_edge_2r_t40_h128_e4_k4_f192", 42, 2, 40, 128, 4, 4, 192),
    KI.MoeShape("moe_edge_3r_t0_h256_e6_k2_f128", 43, 3, 0, 256, 6, 2, 128),
]
SMALL = [(KI.MOE_TINY, 0), (KI.MOE_TINY, 3), (KI.MOE_TINY_SKEW, 0), (KI.MOE_TINY_SKEW, 2)] + \
    [(e, e.world - 1) for e in EDGE]


@pytest.mark.parametrize("s,rank", SMALL, ids=[f"{s.name}-r{r}" for s, r in SMALL])
def test_layer_small_vs_oracle(kos, ws, s, rank):
    """With the bf16 g and u kept as well (checked against the oracle)."""
    say(f"[moe layer] {s.name} rank={rank}")
    inp = KI.moe_inputs(s, rank, "cuda")
    b = run_layer(kos, ws, s, rank, inp, save=True)
    pc = inp["peer_counts"].cpu().numpy()
    wg, wu, wd = (KI.bf16_bits(inp[k]) for k in ("wg", "wu", "wd"))
    peer_send = [None if t is None else KI.bf16_bits(t) for t in inp["peer_send"]]
    pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
    ref = O.moe_layer(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), wg, wu, wd, peer_send, pc, pret,
                      s.world, rank, s.topk)
    _check_dispatch_part(s, rank, b, ref)
    n = int(ref["grouped_offsets"][-1])
    if n:
        href = np.zeros((n, s.ffn), np.uint16)
        go = ref["grouped_offsets"]
        for e in range(s.e_local):
            lo, hi = int(go[e]), int(go[e + 1])
            if hi > lo:
                href[lo:hi] = O.expert_hidden(ref["grouped"][lo:hi], wg[e], wu[e])
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["h"][:n])), O.bf16_to_f64(href), "h")
        gref, uref = O.grouped_gate_up(ref["grouped"], go, wg, wu)
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["gs"][:n])), O.bf16_to_f64(gref), "kept g")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["us"][:n])), O.bf16_to_f64(uref), "kept u")
        ygpu = KI.bf16_bits(b["yg"][:n])
        assert_close(O.bf16_to_f64(ygpu), O.bf16_to_f64(ref["y_grouped"]), "y_grouped")
        _check_pushes(s, rank, b, ref, ygpu)
    if s.tokens:
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["y"])), O.bf16_to_f64(ref["y"]), "y")


def test_layer_repeated_calls_and_trace(kos, ws):
    """Two calls in a row on one workspace give identical outputs (the last
    workgroup out leaves the workspace clean); a traced call's timeline holds
    every kind of work the layer runs."""
    from gemm_collective_persistent_amd.timeline import summarize
    s, rank = KI.MOE_TINY_SKEW, 1
    say("[moe layer repeated + trace]")
    inp = KI.moe_inputs(s, rank, "cuda")
    b1 = run_layer(kos, ws, s, rank, inp)
    b2 = run_layer(kos, ws, s, rank, inp, kos.opts(trace=True))
    for key in ("idx", "perm", "goff", "row_src"):
        assert torch.equal(b1[key], b2[key])
    n = int(b1["goff"][-1].item())
    assert torch.equal(b1["yg"][:n].view(torch.int16), b2["yg"][:n].view(torch.int16))
    assert torch.equal(b1["y"].view(torch.int16), b2["y"].view(torch.int16))
    grid = int(kos.lib.kos_device_cu_count())
    sm = summarize(ws.trace(grid), workgroups=grid)
    for kind in ("route", "scan", "move", "tile", "tile_down", "fold"):
        assert sm["kinds"][kind]["n"] > 0, kind
    assert sm["kinds"]["push"]["n"] > 0


def test_layer_rejects_other_modes(kos, ws):
    s, rank = KI.MOE_TINY, 0
    inp = KI.moe_inputs(s, rank, "cuda")
    with pytest.raises(kos.KosError) as e:
        run_layer(kos, ws, s, rank, inp, kos.opts(mode=2))
    assert "UNSUPPORTED" in str(e.value)


UNIT_ROWS = 256


@pytest.mark.parametrize("shape,save", [(KI.MOE_DSV3, True), (KI.MOE_QWEN3, False)])
def test_layer_full_size(kos, ws, shape, save):
    """save: the kept g and u as well -- bit-identical between the two
    paths, the sampled units' against the oracle."""
    rank = 0
    say(f"[moe layer full] {shape.name} save={save}")
    inp = KI.moe_inputs(shape, rank, "cuda")
    b = run_layer(kos, ws, shape, rank, inp, save=save)
    peer_send = [None if t is None else KI.bf16_bits(t) for t in inp["peer_send"]]
    pc = inp["peer_counts"].cpu().numpy()
    ref = O.dispatch(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), peer_send, pc, shape.world, rank,
                     shape.topk)
    _check_dispatch_part(shape, rank, b, ref)
    go = ref["grouped_offsets"]
    n = int(go[-1])
    ygpu = KI.bf16_bits(b["yg"][:n])
    _check_pushes(shape, rank, b, ref, ygpu)
    say(f"[moe layer full] {shape.name}: dispatch part bit-exact; two-launch path")
    two = run_two_launch(kos, ws, shape, rank, inp, save=save)
    assert np.array_equal(KI.bf16_bits(two["yg"][:n]), ygpu), "expert outputs differ from the two-launch path"
    assert np.array_equal(KI.bf16_bits(two["y"]), KI.bf16_bits(b["y"])), "folded tokens differ from the two-launch path"
    if save:
        for key in ("gs", "us"):
            assert torch.equal(two[key][:n].view(torch.int16), b[key][:n].view(torch.int16)), key
    del two
    El = shape.e_local
    for e in range(El):
        lo, hi = int(go[e]), int(go[e + 1])
        if hi == lo:
            continue
        last = lo + ((hi - lo - 1) // UNIT_ROWS) * UNIT_ROWS
        rows = np.unique(np.concatenate([np.arange(lo, min(lo + UNIT_ROWS, hi)), np.arange(last, hi)]))
        yref = O.expert_ffn(ref["grouped"][rows], KI.bf16_bits(inp["wg"][e]), KI.bf16_bits(inp["wu"][e]),
                            KI.bf16_bits(inp["wd"][e]))
        assert_close(O.bf16_to_f64(ygpu[rows]), O.bf16_to_f64(yref), f"expert {e} first/last units")
        if save:
            gref, uref = O.expert_gate_up(ref["grouped"][rows], KI.bf16_bits(inp["wg"][e]),
                                          KI.bf16_bits(inp["wu"][e]))
            idx = torch.as_tensor(rows, device="cuda")
            assert_close(O.bf16_to_f64(KI.bf16_bits(b["gs"][idx])), O.bf16_to_f64(gref), f"expert {e} kept g")
            assert_close(O.bf16_to_f64(KI.bf16_bits(b["us"][idx])), O.bf16_to_f64(uref), f"expert {e} kept u")
    say(f"[moe layer full] {shape.name}: units checked; 512 tokens end to end")
    pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
    rng = np.random.default_rng(9)
    toks = np.sort(rng.choice(shape.tokens, 512, replace=False))
    need = {}
    for t in toks:
        for j in range(shape.topk):
            e = int(ref["idx"][t, j])
            if e // El == rank:
                r_ = O.local_row(e, int(ref["perm"][t * shape.topk + j]), rank, El, ref["offsets"], go, pc)
                need.setdefault(e - rank * El, []).append(r_)
    yg_sparse = np.zeros((n, shape.hidden), np.uint16)
    for el, rows in need.items():
        rows = np.unique(rows)
        yg_sparse[rows] = O.expert_ffn(ref["grouped"][rows], KI.bf16_bits(inp["wg"][el]),
                                       KI.bf16_bits(inp["wu"][el]), KI.bf16_bits(inp["wd"][el]))
    yref = O.fold(ref["idx"], ref["w"], ref["perm"], ref["offsets"], yg_sparse, go, pc, pret, shape.world, rank,
                  tokens=toks)
    assert_close(O.bf16_to_f64(KI.bf16_bits(b["y"])[toks]), O.bf16_to_f64(yref), "512 folded tokens end to end")


def test_kept_activations_in_every_mode(kos, ws):
    """The combine keeps the same bf16 g and u whichever way it runs: fused,
    with a fixed crew and as separate launches -- bit-identical, and against
    the oracle."""
    s, rank = KI.MOE_TINY_SKEW, 2
    say(f"[moe kept g/u, modes] {s.name} rank={rank}")
    inp = KI.moe_inputs(s, rank, "cuda")
    pc = inp["peer_counts"].cpu().numpy()
    shp = _shape(s, rank)
    got = {}
    for label, o in (("fused", None), ("fixed", kos.opts(mode=1, n_movers=3)), ("unfused", kos.opts(mode=2))):
        b = _buffers(s, rank, pc)
        kos.moe_dispatch(shp, inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"], b["idx"], b["w"],
                         b["counts"], b["perm"], b["send"], b["grouped"], b["goff"], b["row_src"], ws)
        kos.moe_combine(shp, b["grouped"], b["goff"], b["row_src"], inp["wg"], inp["wu"], inp["wd"], b["idx"],
                        b["w"], b["counts"], b["perm"], inp["peer_counts"], inp["peer_return"], b["h"], b["yg"],
                        b["ret"], b["y"], ws, o, gate_save=b["gs"], up_save=b["us"])
        ws.status()
        torch.cuda.synchronize()
        n = int(b["goff"][-1].item())
        got[label] = (b["grouped"][:n].clone(), b["goff"].cpu().numpy(), b["gs"][:n].clone(), b["us"][:n].clone(),
                      b["yg"][:n].clone())
    for label in ("fixed", "unfused"):
        for i, what in ((2, "g"), (3, "u"), (4, "y_grouped")):
            assert torch.equal(got[label][i].view(torch.int16), got["fused"][i].view(torch.int16)), (label, what)
    grouped, go = KI.bf16_bits(got["fused"][0]), got["fused"][1]
    wg, wu = KI.bf16_bits(inp["wg"]), KI.bf16_bits(inp["wu"])
    gref, uref = O.grouped_gate_up(grouped, go, wg, wu)
    assert_close(O.bf16_to_f64(KI.bf16_bits(got["fused"][2])), O.bf16_to_f64(gref), "kept g")
    assert_close(O.bf16_to_f64(KI.bf16_bits(got["fused"][3])), O.bf16_to_f64(uref), "kept u")
