"""Expert layer edge cases on the GPU against the oracle: a ragged token
count, top-1 routing, widths that take the small (128 x 128) tile, expert
counts that are not multiples of 64, a single rank (no peers), top-k = all
experts, and an empty batch."""
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
