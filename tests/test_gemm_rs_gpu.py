"""GEMM + reduce-scatter on the GPU against the oracle (through the C ABI)."""
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


def _run(kos, ws, s, rank, integer, o, inp=None):
    dev = "cuda"
    inp = inp or KI.rs_inputs(s, rank, dev, integer=integer)
    part = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device=dev)
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device=dev)
    kos.gemm_rs(inp["a"], inp["w"], inp["peer_slices"], part, y, rank, ws, o)
    ws.status()
    torch.cuda.synchronize()
    return inp, part, y


def _oracle(inp, rank):
    peers = [None if t is None else t.cpu().numpy() for t in inp["peer_slices"]]
    return O.gemm_rs(KI.bf16_bits(inp["a"]), KI.bf16_bits(inp["w"]), peers, rank)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rank", [0, 1, 3])
def test_rs_tiny_integer_exact(kos, ws, rank, mode, order):
    say(f"[rs tiny int] rank={rank} mode={mode} order={order}")
    inp, part, y = _run(kos, ws, KI.RS_TINY, rank, True, kos.opts(mode=mode, n_movers=3, rs_order=order))
    pref, yref = _oracle(inp, rank)
    assert np.array_equal(part.cpu().numpy(), pref)
    assert np.array_equal(y.cpu().numpy(), yref)


@pytest.mark.parametrize("rank", [0, 3])
def test_rs_mid_several_bands(kos, ws, rank):
    say(f"[rs mid int] rank={rank}")
    for order in (0, 1):
        inp, part, y = _run(kos, ws, KI.RS_MID, rank, True, kos.opts(rs_order=order))
        pref, yref = _oracle(inp, rank)
        assert np.array_equal(part.cpu().numpy(), pref)
        assert np.array_equal(y.cpu().numpy(), yref)


def test_rs_tiny_normal(kos, ws):
    say("[rs tiny normal]")
    inp, part, y = _run(kos, ws, KI.RS_TINY, 2, False, kos.opts())
    pref, yref = _oracle(inp, 2)
    assert_close(part.cpu().numpy(), pref, "partial")
    assert_close(y.cpu().numpy(), yref, "y")


def test_rs_single_rank_is_gemm(kos, ws):
    s = KI.RsShape("rs_r1", 13, 1, 128, 128, 192)
    say("[rs world=1]")
    inp, part, y = _run(kos, ws, s, 0, True, kos.opts(n_movers=1))
    pref, yref = _oracle(inp, 0)
    assert np.array_equal(y.cpu().numpy(), pref)


@pytest.mark.parametrize("rank", [7, 0])
def test_rs_mlp_full_size(kos, ws, rank):
    """Full 8-rank MLP-down shape: band and row order give bit-identical
    chunks; the whole reduced chunk y and our own partial rows against the
    oracle, sampled outbound partial rows, within tolerance."""
    s = KI.RS_MLP
    say(f"[rs mlp full] rank={rank}")
    inp, part_b, y_band = _run(kos, ws, s, rank, False, kos.opts(rs_order=0))
    _, part_r, y_row = _run(kos, ws, s, rank, False, kos.opts(rs_order=1), inp=inp)
    assert torch.equal(y_band, y_row)
    assert torch.equal(part_b, part_r)
    _, _, y_unf = _run(kos, ws, s, rank, False, kos.opts(mode=2), inp=inp)
    assert torch.equal(y_band, y_unf)
    rng = np.random.default_rng(rank)
    a = KI.bf16_bits(inp["a"])
    w = KI.bf16_bits(inp["w"])
    # the whole reduced chunk: our own partial of chunk `rank` (every row)
    # plus every peer's slice, against the oracle
    own_rows = np.arange(rank * s.m_chunk, (rank + 1) * s.m_chunk)
    p_own = O.gemm(a[own_rows], w)
    assert_close(part_b[own_rows].cpu().numpy(), p_own, "own partial rows")
    peers = [None if t is None else t.cpu().numpy() for t in inp["peer_slices"]]
    full = np.zeros((s.m, s.n), np.float32)
    full[own_rows] = p_own.astype(np.float32)
    yref = O.reduce_chunk(full, peers, rank)
    assert_close(y_band.cpu().numpy(), yref, "y (whole chunk)")
    other = np.sort(rng.choice(s.m, 64, replace=False))
    assert_close(part_b[other].cpu().numpy(), O.gemm(a[other], w), "outbound partial rows")


def test_rs_outproj_full_size(kos, ws):
    """Attention output-projection shape (8 ranks, 4096 x 1024 . 1024 x 8192,
    rank 7): band and row order bit-identical; the whole reduced chunk within
    tolerance."""
    s, rank = KI.RS_OUTPROJ, 7
    say("[rs out-proj full]")
    inp, part_b, y_band = _run(kos, ws, s, rank, False, kos.opts(rs_order=0))
    _, part_r, y_row = _run(kos, ws, s, rank, False, kos.opts(rs_order=1), inp=inp)
    assert torch.equal(y_band, y_row) and torch.equal(part_b, part_r)
    a = KI.bf16_bits(inp["a"])
    w = KI.bf16_bits(inp["w"])
    own_rows = np.arange(rank * s.m_chunk, (rank + 1) * s.m_chunk)
    full = np.zeros((s.m, s.n), np.float32)
    full[own_rows] = O.gemm(a[own_rows], w).astype(np.float32)
    peers = [None if t is None else t.cpu().numpy() for t in inp["peer_slices"]]
    assert_close(y_band.cpu().numpy(), O.reduce_chunk(full, peers, rank), "y (whole chunk)")
