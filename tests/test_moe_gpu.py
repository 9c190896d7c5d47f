"""Expert layer (dispatch, combine) on the GPU against the oracle (through the
C ABI).  The combine is fed the oracle's dispatch results, never the GPU's."""
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


def _shape(kos, s, rank):
    from gemm_collective_persistent_amd.api import moe_shape
    return moe_shape(s.world, rank, s.tokens, s.hidden, s.experts, s.topk, s.ffn)


def _grouped_cap(s, pc):
    return int(pc.sum()) + s.tokens * min(s.topk, s.e_local)


def _oracle_dispatch(s, rank, inp):
    peer_send = [None if t is None else KI.bf16_bits(t) for t in inp["peer_send"]]
    return O.dispatch(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), peer_send,
                      inp["peer_counts"].cpu().numpy(), s.world, rank, s.topk)


def _run_dispatch(kos, ws, s, rank, inp, mode=0):
    dev = "cuda"
    T, k, E, H = s.tokens, s.topk, s.experts, s.hidden
    pc = inp["peer_counts"].cpu().numpy()
    cap = _grouped_cap(s, pc)
    out = dict(
        idx=torch.full((T, k), -1, dtype=torch.int32, device=dev),
        w=torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
        counts=torch.full((E,), -1, dtype=torch.int32, device=dev),
        perm=torch.full((T * k,), -1, dtype=torch.int32, device=dev),
        send=[None if p == rank else torch.zeros((s.peer_cap, H), dtype=torch.bfloat16, device=dev)
              for p in range(s.world)],
        grouped=torch.zeros((cap, H), dtype=torch.bfloat16, device=dev),
        goff=torch.full((s.e_local + 1,), -1, dtype=torch.int32, device=dev),
        row_src=torch.full((cap, 2), -1, dtype=torch.int32, device=dev),
    )
    kos.moe_dispatch(_shape(kos, s, rank), inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"],
                     out["idx"], out["w"], out["counts"], out["perm"], out["send"], out["grouped"],
                     out["goff"], out["row_src"], ws, kos.opts(mode=mode))
    ws.status()
    torch.cuda.synchronize()
    return out


def _check_dispatch(s, rank, out, ref, rows=None):
    assert np.array_equal(out["idx"].cpu().numpy(), ref["idx"])
    w = out["w"].cpu().numpy()
    assert_close(w, ref["w"], "topk weights")
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-5)
    assert np.array_equal(out["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(out["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(out["goff"].cpu().numpy(), ref["grouped_offsets"])
    n = int(ref["grouped_offsets"][-1])
    assert np.array_equal(out["row_src"][:n].cpu().numpy(), ref["row_src"])
    g = out["grouped"][:n]
    if rows is None:
        assert np.array_equal(KI.bf16_bits(g), ref["grouped"])
    else:
        rows = rows[rows < n]
        assert np.array_equal(KI.bf16_bits(g[torch.as_tensor(rows, device=g.device)]), ref["grouped"][rows])
    for d in range(s.world):
        if d == rank:
            continue
        nd = ref["send"][d].shape[0]
        got = out["send"][d][:nd]
        if rows is None:
            assert np.array_equal(KI.bf16_bits(got), ref["send"][d])
        else:
            rr = rows[rows < nd]
            assert np.array_equal(KI.bf16_bits(got[torch.as_tensor(rr, device=got.device)]), ref["send"][d][rr])


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("shape,rank", [(KI.MOE_TINY, 0), (KI.MOE_TINY, 3), (KI.MOE_TINY_SKEW, 0),
                                        (KI.MOE_TINY_SKEW, 2)])
def test_dispatch_tiny(kos, ws, shape, rank, mode):
    say(f"[moe dispatch] {shape.name} rank={rank} mode={mode}")
    inp = KI.moe_inputs(shape, rank, "cuda", with_weights=False)
    out = _run_dispatch(kos, ws, shape, rank, inp, mode)
    _check_dispatch(shape, rank, out, _oracle_dispatch(shape, rank, inp))


def test_dispatch_ties_lowest_index(kos, ws):
    """Logits with exact ties (and +0/-0): the lower expert index wins."""
    s = KI.MOE_TINY
    say("[moe dispatch ties]")
    inp = KI.moe_inputs(s, 1, "cuda", with_weights=False)
    lg = inp["logits"].clone()
    lg[:8] = 0.0                      # whole rows tied
    lg[8, 3] = lg[8, 11] = lg[8].max() + 1.0
    lg[9, 5] = -0.0
    lg[9, 2] = 0.0
    lg[9, [0, 1, 3, 4, 6]] = 5.0
    inp["logits"] = lg
    out = _run_dispatch(kos, ws, s, 1, inp)
    ref = _oracle_dispatch(s, 1, inp)
    _check_dispatch(s, 1, out, ref)
    assert out["idx"][0].tolist() == list(range(s.topk))


def _run_combine(kos, ws, s, rank, inp, dref, mode=0, n_movers=-1):
    dev = "cuda"
    T, H, F = s.tokens, s.hidden, s.ffn
    pc = inp["peer_counts"].cpu().numpy()
    cap = _grouped_cap(s, pc)
    n = int(dref["grouped_offsets"][-1])
    grouped = torch.zeros((cap, H), dtype=torch.bfloat16, device=dev)
    grouped[:n] = KI.from_bf16_bits(dref["grouped"], dev)
    row_src = torch.zeros((cap, 2), dtype=torch.int32, device=dev)
    row_src[:n] = torch.as_tensor(dref["row_src"], device=dev)
    goff = torch.as_tensor(dref["grouped_offsets"], device=dev)
    idx = torch.as_tensor(dref["idx"], device=dev)
    w = torch.as_tensor(dref["w"], device=dev)
    counts = torch.as_tensor(dref["counts"], device=dev)
    perm = torch.as_tensor(dref["perm"], device=dev)
    h = torch.full((cap, F), float("nan"), dtype=torch.bfloat16, device=dev)
    yg = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    out_ret = [None if p == rank else torch.full((max(int(pc[p].sum()), 1), H), float("nan"),
                                                 dtype=torch.bfloat16, device=dev) for p in range(s.world)]
    kos.moe_combine(_shape(kos, s, rank), grouped, goff, row_src, inp["wg"], inp["wu"], inp["wd"], idx, w, counts,
                    perm, inp["peer_counts"], inp["peer_return"], h, yg, out_ret, y, ws,
                    kos.opts(mode=mode, n_movers=n_movers))
    ws.status()
    torch.cuda.synchronize()
    return dict(h=h[:n], yg=yg[:n], y=y, out_return=out_ret)


@pytest.mark.parametrize("mode,crew", [(0, -1), (1, 4), (2, -1)])
@pytest.mark.parametrize("shape,rank", [(KI.MOE_TINY, 0), (KI.MOE_TINY_SKEW, 0), (KI.MOE_TINY_SKEW, 3)])
def test_combine_tiny(kos, ws, shape, rank, mode, crew):
    say(f"[moe combine] {shape.name} rank={rank} mode={mode}")
    inp = KI.moe_inputs(shape, rank, "cuda")
    dref = _oracle_dispatch(shape, rank, inp)
    out = _run_combine(kos, ws, shape, rank, inp, dref, mode, crew)
    wg, wu, wd = (KI.bf16_bits(inp[k]) for k in ("wg", "wu", "wd"))
    go = dref["grouped_offsets"]
    href = np.zeros((int(go[-1]), shape.ffn), np.uint16)
    for e in range(shape.e_local):
        lo, hi = int(go[e]), int(go[e + 1])
        if hi > lo:
            href[lo:hi] = O.expert_hidden(dref["grouped"][lo:hi], wg[e], wu[e])
    assert_close(O.bf16_to_f64(KI.bf16_bits(out["h"])), O.bf16_to_f64(href), "h")
    yg_ref = O.grouped_ffn(dref["grouped"], go, wg, wu, wd)
    assert_close(O.bf16_to_f64(KI.bf16_bits(out["yg"])), O.bf16_to_f64(yg_ref), "y_grouped")
    pc = inp["peer_counts"].cpu().numpy()
    # pushed rows are bit copies of the GPU's own expert outputs
    ygpu = KI.bf16_bits(out["yg"])
    for r_, (p, i) in enumerate(dref["row_src"]):
        if p != rank:
            assert np.array_equal(KI.bf16_bits(out["out_return"][p][i]), ygpu[r_])
    pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
    yref = O.fold(dref["idx"], dref["w"], dref["perm"], dref["offsets"], yg_ref, go, pc, pret, shape.world, rank)
    assert_close(O.bf16_to_f64(KI.bf16_bits(out["y"])), O.bf16_to_f64(yref), "y")


# Rows per local expert straddling the combine's tile heights (64-, 128- and
# 256-row tiles): one row, one short of / exactly / one past each height, and
# a second 256-row unit holding a single row.
TAIL_COUNTS = [1, 63, 64, 65, 127, 128, 129, 257]
MOE_TAILS = KI.MoeShape("moe_tails_1r_t417_h256_e8_k2_f128", 44, 1, sum(TAIL_COUNTS) // 2, 256,
                        len(TAIL_COUNTS), 2, 128)


def _tail_logits(s, counts):
    """Logits whose top-2 routing gives expert e exactly counts[e] pairs:
    the pair list sorted by expert, token t taking entries t and t + T (two
    different experts, as no count exceeds T), the first one ranked higher."""
    T = s.tokens
    ids = np.repeat(np.arange(len(counts)), counts)
    assert ids.size == 2 * T and max(counts) <= T
    g = torch.Generator().manual_seed(44)
    lg = 0.1 * torch.randn((T, s.experts), generator=g)
    for t in range(T):
        lg[t, int(ids[t])] = 10.0
        lg[t, int(ids[t + T])] = 9.0
    return lg


@pytest.mark.parametrize("mode", [0, 2])
def test_combine_tile_boundaries(kos, ws, mode):
    """Expert row counts at and around every tile height: h, the expert
    outputs and the folded tokens against the oracle."""
    s, rank = MOE_TAILS, 0
    say(f"[moe combine tails] mode={mode}")
    inp = KI.moe_inputs(s, rank, "cuda")
    inp["logits"] = _tail_logits(s, TAIL_COUNTS).to("cuda")
    dref = _oracle_dispatch(s, rank, inp)
    assert dref["counts"].tolist() == TAIL_COUNTS
    out = _run_combine(kos, ws, s, rank, inp, dref, mode)
    wg, wu, wd = (KI.bf16_bits(inp[k]) for k in ("wg", "wu", "wd"))
    go = dref["grouped_offsets"]
    href = np.zeros((int(go[-1]), s.ffn), np.uint16)
    for e in range(s.e_local):
        lo, hi = int(go[e]), int(go[e + 1])
        href[lo:hi] = O.expert_hidden(dref["grouped"][lo:hi], wg[e], wu[e])
    assert_close(O.bf16_to_f64(KI.bf16_bits(out["h"])), O.bf16_to_f64(href), "h")
    yg_ref = O.grouped_ffn(dref["grouped"], go, wg, wu, wd)
    assert_close(O.bf16_to_f64(KI.bf16_bits(out["yg"])), O.bf16_to_f64(yg_ref), "y_grouped")
    pc = inp["peer_counts"].cpu().numpy()
    yref = O.fold(dref["idx"], dref["w"], dref["perm"], dref["offsets"], yg_ref, go, pc, [None], s.world, rank)
    assert_close(O.bf16_to_f64(KI.bf16_bits(out["y"])), O.bf16_to_f64(yref), "y")


UNIT_ROWS = 256   # the combine's work unit: 256 grouped rows of one expert


@pytest.mark.parametrize("shape", [KI.MOE_DSV3, KI.MOE_QWEN3])
def test_moe_full_size(kos, ws, shape):
    """Full expert-layer shapes, rank 0, at full concurrency:
    - dispatch: routing, counts, permutation, offsets, provenance, every
      grouped row and every send row bit-exact;
    - combine (fed the oracle's dispatch): every pushed row a bit copy of the
      expert output at the oracle's provenance; the whole first and last
      256-row unit of every local expert (tail units included, all columns)
      against the oracle's expert FFN; every folded token against the
      oracle's fold of the GPU's expert outputs (the fold and push step
      alone); and 512 tokens end to end against the oracle (every local
      result they need recomputed by the oracle)."""
    rank = 0
    say(f"[moe full] {shape.name}")
    inp = KI.moe_inputs(shape, rank, "cuda")
    dref = _oracle_dispatch(shape, rank, inp)
    out = _run_dispatch(kos, ws, shape, rank, inp)
    _check_dispatch(shape, rank, out, dref)
    del out
    say(f"[moe full] {shape.name}: dispatch bit-exact; combine")
    c = _run_combine(kos, ws, shape, rank, inp, dref)
    go = dref["grouped_offsets"]
    n = int(go[-1])
    El, H = shape.e_local, shape.hidden
    ygpu = KI.bf16_bits(c["yg"])
    # pushes: out_return[p][i] == y_grouped[r] for row_src[r] == (p, i)
    rs = dref["row_src"]
    pc = inp["peer_counts"].cpu().numpy()
    for p in range(shape.world):
        if p == rank:
            continue
        sel = np.where(rs[:, 0] == p)[0]
        assert sel.size == int(pc[p].sum())
        got = KI.bf16_bits(c["out_return"][p])[rs[sel, 1]]
        assert np.array_equal(got, ygpu[sel]), f"pushed rows to rank {p}"
    # whole first and last unit of every local expert
    for e in range(El):
        lo, hi = int(go[e]), int(go[e + 1])
        if hi == lo:
            continue
        last = lo + ((hi - lo - 1) // UNIT_ROWS) * UNIT_ROWS
        rows = np.unique(np.concatenate([np.arange(lo, min(lo + UNIT_ROWS, hi)), np.arange(last, hi)]))
        ref = O.expert_ffn(dref["grouped"][rows], KI.bf16_bits(inp["wg"][e]), KI.bf16_bits(inp["wu"][e]),
                           KI.bf16_bits(inp["wd"][e]))
        assert_close(O.bf16_to_f64(ygpu[rows]), O.bf16_to_f64(ref), f"expert {e} first/last units")
    say(f"[moe full] {shape.name}: units checked; fold")
    pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
    ygot = KI.bf16_bits(c["y"])
    # every token: the fold of the GPU's own expert outputs
    yfold = O.fold(dref["idx"], dref["w"], dref["perm"], dref["offsets"], ygpu, go, pc, pret, shape.world, rank)
    assert_close(O.bf16_to_f64(ygot), O.bf16_to_f64(yfold), "every folded token (GPU expert outputs)")
    # 512 tokens end to end
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(shape.tokens, 512, replace=False))
    need = {}
    for t in toks:
        for j in range(shape.topk):
            e = int(dref["idx"][t, j])
            if e // El == rank:
                r_ = O.local_row(e, int(dref["perm"][t * shape.topk + j]), rank, El, dref["offsets"], go, pc)
                need.setdefault(e - rank * El, []).append(r_)
    yg_sparse = np.zeros((n, H), np.uint16)
    for el, rows in need.items():
        rows = np.unique(rows)
        yg_sparse[rows] = O.expert_ffn(dref["grouped"][rows], KI.bf16_bits(inp["wg"][el]),
                                       KI.bf16_bits(inp["wu"][el]), KI.bf16_bits(inp["wd"][el]))
    yref = O.fold(dref["idx"], dref["w"], dref["perm"], dref["offsets"], yg_sparse, go, pc, pret, shape.world,
                  rank, tokens=toks)
    assert_close(O.bf16_to_f64(ygot[toks]), O.bf16_to_f64(yref), "512 folded tokens end to end")
