"""Expert layer edge cases on the GPU against the oracle: a ragged token
count, top-1 routing, widths that take the small (128 x 128) tile, expert
counts that are not multiples of 64, a single rank (no peers), top-k = all
experts, one and 64 local experts per rank, and an empty batch."""
import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import assert_close, say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu

# name, workload id, world, tokens, hidden, experts, topk, ffn
EDGE = [
    KI.MoeShape("moe_edge_2r_t70_h384_e6_k1_f64", 40, 2, 70, 384, 6, 1, 64),
    KI.MoeShape("moe_edge_1r_t33_h256_e8_k3_f128", 41, 1, 33, 256, 8, 3, 128),
    KI.MoeShape("moe_edge_2r_t40_h128_e4_k4_f192", 42, 2, 40, 128, 4, 4, 192),
    KI.MoeShape("moe_edge_3r_t0_h256_e6_k2_f128", 43, 3, 0, 256, 6, 2, 128),
    # one local expert per rank, and the most a rank may hold (64: every lane
    # of the wave that sums the grouped offsets)
    KI.MoeShape("moe_edge_4r_t48_h128_e4_k2_f64", 46, 4, 48, 128, 4, 2, 64),
    KI.MoeShape("moe_edge_2r_t80_h128_e128_k6_f64", 47, 2, 80, 128, 128, 6, 64),
]


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


@pytest.fixture(scope="module")
def ws(kos):
    return kos.Workspace("cuda")


def _dev(a, dtype=None):
    return torch.as_tensor(np.ascontiguousarray(a), device="cuda", dtype=dtype)


@pytest.mark.parametrize("s", EDGE, ids=[e.name for e in EDGE])
def test_moe_edge_layer(kos, ws, s):
    from gemm_collective_persistent_amd.api import moe_shape
    rank = s.world - 1
    say(f"[moe edge] {s.name} rank={rank}")
    dev = "cuda"
    inp = KI.moe_inputs(s, rank, dev)
    T, k, E, H, F = s.tokens, s.topk, s.experts, s.hidden, s.ffn
    pc = inp["peer_counts"].cpu().numpy()
    cap = max(int(pc.sum()) + T * min(k, s.e_local), 1)
    shp = moe_shape(s.world, rank, T, H, E, k, F)
    idx = torch.full((max(T, 1), k), -1, dtype=torch.int32, device=dev)
    w = torch.full((max(T, 1), k), float("nan"), dtype=torch.float32, device=dev)
    counts = torch.full((E,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((max(T * k, 1),), -1, dtype=torch.int32, device=dev)
    send = [None if p == rank else torch.zeros((max(s.peer_cap, 1), H), dtype=torch.bfloat16, device=dev)
            for p in range(s.world)]
    grouped = torch.zeros((cap, H), dtype=torch.bfloat16, device=dev)
    goff = torch.full((s.e_local + 1,), -1, dtype=torch.int32, device=dev)
    row_src = torch.full((cap, 2), -1, dtype=torch.int32, device=dev)
    kos.moe_dispatch(shp, inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"], idx, w, counts, perm,
                     send, grouped, goff, row_src, ws)
    ws.status()
    peer_send = [None if t is None else KI.bf16_bits(t) for t in inp["peer_send"]]
    d = O.dispatch(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), peer_send, pc, s.world, rank, k)
    n = int(d["grouped_offsets"][-1])
    assert np.array_equal(idx[:T].cpu().numpy(), d["idx"])
    assert np.array_equal(perm[:T * k].cpu().numpy(), d["perm"])
    assert np.array_equal(counts.cpu().numpy(), d["counts"])
    assert np.array_equal(goff.cpu().numpy(), d["grouped_offsets"])
    assert np.array_equal(row_src[:n].cpu().numpy(), d["row_src"])
    assert np.array_equal(KI.bf16_bits(grouped[:n]), d["grouped"])
    if T:
        ww = w[:T].cpu().numpy()
        assert_close(ww, d["w"], "topk weights")
        assert np.all(np.abs(ww.astype(np.float64).sum(1) - 1.0) <= 1e-5)
        if k == 1:
            assert np.all(ww == 1.0), "top-1: weight exactly 1"
    for q in range(s.world):
        if q != rank:
            nq = d["send"][q].shape[0]
            assert np.array_equal(KI.bf16_bits(send[q][:nq]), d["send"][q])

    # combine, fed the GPU's dispatch outputs (checked bit-exact above)
    h = torch.full((cap, F), float("nan"), dtype=torch.bfloat16, device=dev)
    yg = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((max(T, 1), H), float("nan"), dtype=torch.bfloat16, device=dev)
    ret = [None if q == rank else torch.full((max(int(pc[q].sum()), 1), H), float("nan"), dtype=torch.bfloat16,
                                             device=dev) for q in range(s.world)]
    kos.moe_combine(shp, grouped, goff, row_src, inp["wg"], inp["wu"], inp["wd"], idx, w, counts, perm,
                    inp["peer_counts"], inp["peer_return"], h, yg, ret, y, ws)
    ws.status()
    wg, wu, wd = (KI.bf16_bits(inp[x]) for x in ("wg", "wu", "wd"))
    yg_ref = O.grouped_ffn(d["grouped"], d["grouped_offsets"], wg, wu, wd)
    if n:
        assert_close(O.bf16_to_f64(KI.bf16_bits(yg[:n])), O.bf16_to_f64(yg_ref), "y_grouped")
        ygpu = KI.bf16_bits(yg[:n])
        for r_, (q, i) in enumerate(d["row_src"]):
            if q != rank:
                assert np.array_equal(KI.bf16_bits(ret[q][i]), ygpu[r_]), "pushed rows are bit copies"
    if T:
        pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
        yref = O.fold(d["idx"], d["w"], d["perm"], d["offsets"], yg_ref, d["grouped_offsets"], pc, pret,
                      s.world, rank)
        assert_close(O.bf16_to_f64(KI.bf16_bits(y[:T])), O.bf16_to_f64(yref), "y")


def test_null_peer_buffer_with_rows_is_reported(kos, ws):
    """A peer send buffer passed as NULL although its counts say it sends
    rows: the dispatch skips that source (never reads the NULL buffer) and
    reports KOS_ERR_ARG through the workspace status; the next call on the
    same workspace works."""
    from gemm_collective_persistent_amd._binding import KOS_ERR_ARG, KosError
    s, rank = KI.MOE_TINY, 0
    say("[moe null peer buffer]")
    inp = KI.moe_inputs(s, rank, "cuda", with_weights=False)
    assert int(inp["peer_counts"][1].sum()) > 0
    bad = list(inp["peer_send"])
    bad[1] = None
    from test_moe_gpu import _run_dispatch  # noqa: E402  (same directory)
    inp_bad = dict(inp, peer_send=bad)
    with pytest.raises(KosError) as ei:
        _run_dispatch(kos, ws, s, rank, inp_bad)
    assert ei.value.status == KOS_ERR_ARG
    out = _run_dispatch(kos, ws, s, rank, inp)     # workspace usable again
    peer_send = [None if t is None else KI.bf16_bits(t) for t in inp["peer_send"]]
    d = O.dispatch(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), peer_send,
                   inp["peer_counts"].cpu().numpy(), s.world, rank, s.topk)
    assert np.array_equal(out["perm"].cpu().numpy(), d["perm"])


def test_capacity_overflows_are_reported_not_written(kos, ws):
    """Buffers too small for what the routing needs: an out_send buffer
    shorter than the rows routed to its rank (dispatch), grouped offsets
    describing more rows than the grouped capacity, and a return buffer
    shorter than the rows its rank sent (combine).  Each call reports
    KOS_ERR_CAPACITY through the workspace status and writes nothing past
    the buffers it was given (guard rows keep their fill); the workspace
    works again afterwards."""
    from gemm_collective_persistent_amd._binding import KOS_ERR_CAPACITY, KosError
    from test_moe_gpu import _oracle_dispatch, _run_combine, _shape
    s, rank = KI.MOE_TINY, 0
    say("[moe capacity overflows]")
    inp = KI.moe_inputs(s, rank, "cuda")
    dref = _oracle_dispatch(s, rank, inp)
    dev, T, k, E, H, F = "cuda", s.tokens, s.topk, s.experts, s.hidden, s.ffn
    pc = inp["peer_counts"].cpu().numpy()
    cap = int(pc.sum()) + T * min(k, s.e_local)
    sent = [0 if d == rank else dref["send"][d].shape[0] for d in range(s.world)]
    assert sent[2] > 1
    guard = 0x4242
    full = [None if p == rank else torch.full((max(sent[p], 1) + 8, H), 0, dtype=torch.int16, device=dev)
            for p in range(s.world)]
    for p in range(s.world):
        if p != rank:
            full[p].fill_(guard)
    views = [None if t is None else t.view(torch.bfloat16)[:(sent[p] - 1 if p == 2 else sent[p] + 8)]
             for p, t in enumerate(full)]
    grouped = torch.zeros((cap, H), dtype=torch.bfloat16, device=dev)
    out = dict(idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               w=torch.empty((T, k), dtype=torch.float32, device=dev),
               counts=torch.empty((E,), dtype=torch.int32, device=dev),
               perm=torch.empty((T * k,), dtype=torch.int32, device=dev),
               goff=torch.full((s.e_local + 1,), -7, dtype=torch.int32, device=dev),
               row_src=torch.empty((cap, 2), dtype=torch.int32, device=dev))
    kos.moe_dispatch(_shape(kos, s, rank), inp["x"], inp["logits"], inp["peer_send"], inp["peer_counts"],
                     out["idx"], out["w"], out["counts"], out["perm"], views, grouped, out["goff"],
                     out["row_src"], ws)
    with pytest.raises(KosError) as ei:
        ws.status()
    assert ei.value.status == KOS_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int((full[2][sent[2] - 1:] != guard).sum()) == 0, "rows past out_send[2]'s capacity were written"
    assert out["goff"].tolist() == [-7] * (s.e_local + 1), "grouped offsets written after an overflow"

    # combine: offsets describing more rows than the capacity
    n = int(dref["grouped_offsets"][-1])
    small = n - 3
    with pytest.raises(KosError) as ei:
        grouped_s = torch.zeros((small, H), dtype=torch.bfloat16, device=dev)
        grouped_s[:] = KI.from_bf16_bits(dref["grouped"][:small], dev)
        row_src = torch.as_tensor(dref["row_src"][:small], device=dev)
        goff = torch.as_tensor(dref["grouped_offsets"], device=dev)
        hh = torch.full((small + 8, F), float("nan"), dtype=torch.bfloat16, device=dev)
        yg = torch.full((small + 8, H), float("nan"), dtype=torch.bfloat16, device=dev)
        y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
        ret = [None if p == rank else torch.full((max(int(pc[p].sum()), 1), H), float("nan"), dtype=torch.bfloat16,
                                                 device=dev) for p in range(s.world)]
        kos.moe_combine(_shape(kos, s, rank), grouped_s, goff, row_src, inp["wg"], inp["wu"], inp["wd"],
                        torch.as_tensor(dref["idx"], device=dev), torch.as_tensor(dref["w"], device=dev),
                        torch.as_tensor(dref["counts"], device=dev), torch.as_tensor(dref["perm"], device=dev),
                        inp["peer_counts"], inp["peer_return"], hh, yg, ret, y, ws)
        ws.status()
    assert ei.value.status == KOS_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool(torch.isnan(hh.float()).all()) and bool(torch.isnan(yg.float()).all()) and bool(
        torch.isnan(y.float()).all()), "the combine wrote after a capacity error"

    # combine: a return buffer shorter than the rows its rank sent us
    q = int(np.argmax(pc.sum(axis=1)))
    assert pc[q].sum() > 1
    with pytest.raises(KosError) as ei:
        _run_combine_short(kos, ws, s, rank, inp, dref, q)
    assert ei.value.status == KOS_ERR_CAPACITY
    # the workspace is clean again: a correct call passes
    c = _run_combine(kos, ws, s, rank, inp, dref)
    assert bool(torch.isfinite(c["y"].float()).all())


def _run_combine_short(kos, ws, s, rank, inp, dref, q):
    """The combine with out_return[q] one row shorter than the rows q sent."""
    dev, T, H, F = "cuda", s.tokens, s.hidden, s.ffn
    pc = inp["peer_counts"].cpu().numpy()
    cap = int(pc.sum()) + T * min(s.topk, s.e_local)
    n = int(dref["grouped_offsets"][-1])
    grouped = torch.zeros((cap, H), dtype=torch.bfloat16, device=dev)
    grouped[:n] = KI.from_bf16_bits(dref["grouped"], dev)
    row_src = torch.zeros((cap, 2), dtype=torch.int32, device=dev)
    row_src[:n] = torch.as_tensor(dref["row_src"], device=dev)
    ret_full = torch.full((int(pc[q].sum()) + 4, H), 0, dtype=torch.int16, device=dev).fill_(0x4242)
    ret = [None if p == rank else (ret_full.view(torch.bfloat16)[:int(pc[q].sum()) - 1] if p == q else
                                   torch.empty((max(int(pc[p].sum()), 1), H), dtype=torch.bfloat16, device=dev))
           for p in range(s.world)]
    from test_moe_gpu import _shape
    try:
        kos.moe_combine(_shape(kos, s, rank), grouped, torch.as_tensor(dref["grouped_offsets"], device=dev),
                        row_src, inp["wg"], inp["wu"], inp["wd"], torch.as_tensor(dref["idx"], device=dev),
                        torch.as_tensor(dref["w"], device=dev), torch.as_tensor(dref["counts"], device=dev),
                        torch.as_tensor(dref["perm"], device=dev), inp["peer_counts"], inp["peer_return"],
                        torch.empty((cap, F), dtype=torch.bfloat16, device=dev),
                        torch.empty((cap, H), dtype=torch.bfloat16, device=dev), ret,
                        torch.empty((T, H), dtype=torch.bfloat16, device=dev), ws)
        ws.status()
    finally:
        torch.cuda.synchronize()
        assert int((ret_full != 0x4242).sum()) == 0, "the combine wrote into a return buffer too short for it"
