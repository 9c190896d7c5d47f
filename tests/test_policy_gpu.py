"""The other role-switching policy (kos_opts.policy = SWAPPED: two-way
all-gather and reduce-scatter, one-way combine) gives the same results as
the pages' default, against the oracle, through the C ABI."""
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


AG_MID = KI.AgShape("ag_policy_mid_4r_1024x512x384", 31, 4, 256, 512, 384)


@pytest.mark.parametrize("crew", [-1, 1])
@pytest.mark.parametrize("s,rank", [(KI.AG_TINY, 0), (KI.AG_TINY, 3), (AG_MID, 2)])
def test_ag_two_way_integer_exact(kos, ws, s, rank, crew):
    say(f"[ag two-way] {s.name} rank={rank} crew={crew}")
    inp = KI.ag_inputs(s, rank, "cuda", integer=True)
    g = torch.full((s.m, s.k), float("nan"), dtype=torch.bfloat16, device="cuda")
    c = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws,
                kos.opts(policy=kos._binding.POLICY_SWAPPED, n_movers=crew))
    ws.status()
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    gref, cref = O.ag_gemm(KI.bf16_bits(inp["a_local"]), peers, KI.bf16_bits(inp["w"]), rank, out_dtype="f32")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert np.array_equal(c.cpu().numpy(), cref)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("s,rank", [(KI.RS_TINY, 0), (KI.RS_TINY, 3), (KI.RS_MID, 1)])
def test_rs_two_way_integer_exact(kos, ws, s, rank, order):
    say(f"[rs two-way] {s.name} rank={rank} order={order}")
    inp = KI.rs_inputs(s, rank, "cuda", integer=True)
    part = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device="cuda")
    kos.gemm_rs(inp["a"], inp["w"], inp["peer_slices"], part, y, rank, ws,
                kos.opts(policy=kos._binding.POLICY_SWAPPED, rs_order=order))
    ws.status()
    pref, yref = O.gemm_rs(KI.bf16_bits(inp["a"]), KI.bf16_bits(inp["w"]),
                           [None if t is None else t.cpu().numpy() for t in inp["peer_slices"]], rank)
    assert np.array_equal(part.cpu().numpy(), pref)
    assert np.array_equal(y.cpu().numpy(), yref)


def test_rs_two_way_full_size_equals_one_way(kos, ws):
    """MLP-down at full size, rank 7: the two-way builders reduce the same
    slabs in the same per-element order, so y is bit-identical."""
    s, rank = KI.RS_MLP, 7
    say("[rs two-way full]")
    inp = KI.rs_inputs(s, rank, "cuda")
    ys = []
    for pol in (0, 1):
        part = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
        y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device="cuda")
        kos.gemm_rs(inp["a"], inp["w"], inp["peer_slices"], part, y, rank, ws, kos.opts(policy=pol))
        ws.status()
        ys.append(y)
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("s,rank", [(KI.MOE_TINY, 0), (KI.MOE_TINY_SKEW, 2)])
def test_combine_one_way_matches_oracle(kos, ws, s, rank):
    from test_moe_gpu import _oracle_dispatch, _shape
    say(f"[combine one-way] {s.name} rank={rank}")
    inp = KI.moe_inputs(s, rank, "cuda")
    dref = _oracle_dispatch(s, rank, inp)
    pc = inp["peer_counts"].cpu().numpy()
    n = int(dref["grouped_offsets"][-1])
    cap = int(pc.sum()) + s.tokens * min(s.topk, s.e_local)
    dev = "cuda"
    grouped = torch.zeros((cap, s.hidden), dtype=torch.bfloat16, device=dev)
    grouped[:n] = KI.from_bf16_bits(dref["grouped"], dev)
    row_src = torch.zeros((cap, 2), dtype=torch.int32, device=dev)
    row_src[:n] = torch.as_tensor(dref["row_src"], device=dev)
    h = torch.empty((cap, s.ffn), dtype=torch.bfloat16, device=dev)
    yg = torch.empty((cap, s.hidden), dtype=torch.bfloat16, device=dev)
    y = torch.full((s.tokens, s.hidden), float("nan"), dtype=torch.bfloat16, device=dev)
    ret = [None if p == rank else torch.full((max(int(pc[p].sum()), 1), s.hidden), float("nan"),
                                             dtype=torch.bfloat16, device=dev) for p in range(s.world)]
    kos.moe_combine(_shape(kos, s, rank), grouped, torch.as_tensor(dref["grouped_offsets"], device=dev), row_src,
                    inp["wg"], inp["wu"], inp["wd"], torch.as_tensor(dref["idx"], device=dev),
                    torch.as_tensor(dref["w"], device=dev), torch.as_tensor(dref["counts"], device=dev),
                    torch.as_tensor(dref["perm"], device=dev), inp["peer_counts"], inp["peer_return"], h, yg, ret, y,
                    ws, kos.opts(policy=kos._binding.POLICY_SWAPPED))
    ws.status()
    wg, wu, wd = (KI.bf16_bits(inp[k]) for k in ("wg", "wu", "wd"))
    yg_ref = O.grouped_ffn(dref["grouped"], dref["grouped_offsets"], wg, wu, wd)
    ygpu = KI.bf16_bits(yg[:n])
    assert_close(O.bf16_to_f64(ygpu), O.bf16_to_f64(yg_ref), "y_grouped")
    for r_, (p, i) in enumerate(dref["row_src"]):
        if p != rank:
            assert np.array_equal(KI.bf16_bits(ret[p][i]), ygpu[r_])
    pret = [None if t is None else KI.bf16_bits(t) for t in inp["peer_return"]]
    yref = O.fold(dref["idx"], dref["w"], dref["perm"], dref["offsets"], yg_ref, dref["grouped_offsets"], pc, pret,
                  s.world, rank)
    assert_close(O.bf16_to_f64(KI.bf16_bits(y)), O.bf16_to_f64(yref), "y")
