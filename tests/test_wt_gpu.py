"""The two collectives with the weight stored transposed (the backward pass's
data-gradient products) on the GPU against the oracle (through the C ABI).

Integer-valued small cases must match bit for bit on every rank and mode;
the backward shapes of the layer (QKV's GEMM+reduce-scatter, MLP-down's
all-gather+GEMM, 8 ranks) are compared on sampled rows, and y entirely.
"""
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


def _bits(t):
    return None if t is None else KI.bf16_bits(t)


def _run_ag(kos, ws, s, rank, integer, c_dtype, o):
    inp = KI.ag_inputs(s, rank, "cuda", integer=integer, wt=True)
    g = torch.full((s.m, s.k), float("nan"), dtype=torch.bfloat16, device="cuda")
    c = torch.full((s.m, s.n), float("nan"), dtype=c_dtype, device="cuda")
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws, o, w_transposed=True)
    ws.status()
    torch.cuda.synchronize()
    return inp, g, c


def _run_rs(kos, ws, s, rank, integer, o):
    inp = KI.rs_inputs(s, rank, "cuda", integer=integer, wt=True)
    partial = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device="cuda")
    kos.gemm_rs(inp["a"], inp["w"], inp["peer_slices"], partial, y, rank, ws, o, w_transposed=True)
    ws.status()
    torch.cuda.synchronize()
    return inp, partial, y


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rank", [0, 3])
def test_ag_wt_tiny_integer_exact(kos, ws, rank, mode):
    say(f"[ag wt tiny int] rank={rank} mode={mode}")
    inp, g, c = _run_ag(kos, ws, KI.AG_TINY, rank, True, torch.float32, kos.opts(mode=mode, n_movers=2))
    gref, cref = O.ag_gemm_wt(_bits(inp["a_local"]), [_bits(t) for t in inp["a_peers"]], _bits(inp["w"]), rank, "f32")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert np.array_equal(c.cpu().numpy(), cref)


def test_ag_wt_ragged_shapes(kos, ws):
    s = KI.AgShape("ag_wt_odd", 20, 3, 192, 320, 192)   # three 64-row tiles per shard
    say("[ag wt odd shapes]")
    for rank in range(3):
        inp, g, c = _run_ag(kos, ws, s, rank, True, torch.float32, kos.opts(n_movers=3))
        gref, cref = O.ag_gemm_wt(_bits(inp["a_local"]), [_bits(t) for t in inp["a_peers"]], _bits(inp["w"]),
                                  rank, "f32")
        assert np.array_equal(c.cpu().numpy(), cref)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rank", [0, 3])
def test_rs_wt_tiny_integer_exact(kos, ws, rank, mode, order):
    say(f"[rs wt tiny int] rank={rank} mode={mode} order={order}")
    o = kos.opts(mode=mode, n_movers=0 if mode == 0 else 2, rs_order=order)
    inp, partial, y = _run_rs(kos, ws, KI.RS_TINY, rank, True, o)
    pref, yref = O.gemm_rs_wt(_bits(inp["a"]), _bits(inp["w"]), [None if t is None else t.cpu().numpy()
                                                                for t in inp["peer_slices"]], rank)
    assert np.array_equal(partial.cpu().numpy(), pref)
    assert np.array_equal(y.cpu().numpy(), yref)


def test_rs_wt_mid_shape(kos, ws):
    s = KI.RS_MID   # 2048 x 192 . 192 x 384 on 4 ranks: 64-row tiles, several bands
    say("[rs wt mid]")
    inp, partial, y = _run_rs(kos, ws, s, 2, True, kos.opts())
    pref, yref = O.gemm_rs_wt(_bits(inp["a"]), _bits(inp["w"]), [None if t is None else t.cpu().numpy()
                                                                for t in inp["peer_slices"]], 2)
    assert np.array_equal(y.cpu().numpy(), yref)


@pytest.mark.parametrize("rank", [0, 7])
def test_rs_wt_qkv_backward_full_size(kos, ws, rank):
    """dX of the QKV projection: GEMM+RS of dY [4096, 3072] with W_qkv^T
    (8192 output columns), 8 ranks; y (512 x 8192) entirely."""
    s = KI.RS_QKV_BWD
    say(f"[rs wt qkv bwd full] rank={rank}")
    inp, partial, y = _run_rs(kos, ws, s, rank, False, kos.opts())
    mc = s.m_chunk
    own = O.gemm(_bits(inp["a"])[rank * mc:(rank + 1) * mc], _bits(inp["w"]).T).astype(np.float32)
    yref = np.zeros(own.shape)
    for p in range(s.world):
        yref += own if p == rank else inp["peer_slices"][p].cpu().numpy().astype(np.float64)
    assert_close(y.cpu().numpy(), yref, "y")


def test_ag_wt_mlp_backward_full_size_sampled(kos, ws):
    """dX of the MLP down projection: all-gather of dY shards [512, 8192] and
    . W_down^T (3584 output columns), 8 ranks; gathered bit-exact, sampled
    rows of C."""
    s = KI.AG_MLP_BWD
    say("[ag wt mlp bwd full]")
    inp, g, c = _run_ag(kos, ws, s, 6, False, torch.bfloat16, kos.opts())
    shards = [_bits(inp["a_local"]) if p == 6 else _bits(inp["a_peers"][p]) for p in range(s.world)]
    gref = O.gather(shards)
    assert np.array_equal(KI.bf16_bits(g), gref)
    rows = np.sort(np.random.default_rng(6).choice(s.m, 64, replace=False))
    cref = O.round_bf16(O.gemm(gref[rows], _bits(inp["w"]).T))
    assert_close(O.bf16_to_f64(KI.bf16_bits(c)[rows]), O.bf16_to_f64(cref), "C rows")
