"""All-gather + GEMM on the GPU against the oracle (through the C ABI)."""
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


def _run(kos, ws, shape, rank, integer, c_dtype, o, peers_on_host=False):
    dev = "cuda"
    inp = KI.ag_inputs(shape, rank, dev, integer=integer)
    peers = inp["a_peers"]
    if peers_on_host:
        peers = [None if t is None else t.cpu().pin_memory() for t in peers]
    g = torch.empty((shape.m, shape.k), dtype=torch.bfloat16, device=dev)
    c = torch.empty((shape.m, shape.n), dtype=c_dtype, device=dev)
    g.fill_(float("nan"))
    c.fill_(float("nan"))
    kos.ag_gemm(inp["a_local"], peers, inp["w"], g, c, rank, ws, o)
    ws.status()
    torch.cuda.synchronize()
    return inp, g, c


def _oracle(inp, rank, out):
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    return O.ag_gemm(KI.bf16_bits(inp["a_local"]), peers, KI.bf16_bits(inp["w"]), rank, out_dtype=out)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_ag_tiny_integer_exact(kos, ws, rank, mode):
    say(f"[ag tiny int] rank={rank} mode={mode}")
    o = kos.opts(mode=mode, n_movers=2)
    inp, g, c = _run(kos, ws, KI.AG_TINY, rank, True, torch.float32, o)
    gref, cref = _oracle(inp, rank, "f32")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert np.array_equal(c.cpu().numpy(), cref)


@pytest.mark.parametrize("rank", [0, 3])
def test_ag_tiny_normal_bf16(kos, ws, rank):
    say(f"[ag tiny bf16] rank={rank}")
    inp, g, c = _run(kos, ws, KI.AG_TINY, rank, False, torch.bfloat16, kos.opts())
    gref, cref = _oracle(inp, rank, "bf16")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert_close(O.bf16_to_f64(KI.bf16_bits(c)), O.bf16_to_f64(cref), "C")


def test_ag_ragged_shapes_several_tiles(kos, ws):
    # 3 ranks, 192-row shards (three 64-row tiles), k=320, n=192
    s = KI.AgShape("ag_odd", 11, 3, 192, 320, 192)
    say("[ag odd shapes]")
    for rank in range(3):
        inp, g, c = _run(kos, ws, s, rank, True, torch.float32, kos.opts(n_movers=3))
        gref, cref = _oracle(inp, rank, "f32")
        assert np.array_equal(KI.bf16_bits(g), gref)
        assert np.array_equal(c.cpu().numpy(), cref)


def test_ag_single_rank(kos, ws):
    s = KI.AgShape("ag_r1", 12, 1, 128, 128, 128)
    say("[ag world=1]")
    inp, g, c = _run(kos, ws, s, 0, True, torch.float32, kos.opts(n_movers=1))
    gref, cref = _oracle(inp, 0, "f32")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert np.array_equal(c.cpu().numpy(), cref)


def test_ag_pinned_host_peers(kos, ws):
    say("[ag tiny pinned-host peers]")
    inp, g, c = _run(kos, ws, KI.AG_TINY, 1, True, torch.float32, kos.opts(peer_link=1), peers_on_host=True)
    gref, cref = _oracle(inp, 1, "f32")
    assert np.array_equal(KI.bf16_bits(g), gref)
    assert np.array_equal(c.cpu().numpy(), cref)


def test_ag_timeout_is_reported_not_hung(kos, ws):
    # a one-poll spin limit: a builder that finds a remote row block not yet
    # landed records KOS_ERR_TIMEOUT and every workgroup drains
    say("[ag forced timeout]")
    o = kos.opts(mode=1, n_movers=1, spin_limit=1)
    inp = KI.ag_inputs(KI.AG_QKV, 0, "cuda")
    g = torch.empty((KI.AG_QKV.m, KI.AG_QKV.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((KI.AG_QKV.m, KI.AG_QKV.n), dtype=torch.bfloat16, device="cuda")
    kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, 0, ws, o)
    with pytest.raises(kos.KosError) as e:
        ws.status()
    assert "TIMEOUT" in str(e.value)
    # the workspace is usable again
    inp, g, c = _run(kos, ws, KI.AG_TINY, 0, True, torch.float32, kos.opts())
    assert np.array_equal(c.cpu().numpy(), _oracle(inp, 0, "f32")[1])


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_ag_qkv_full_size_sampled(kos, ws, mode):
    """Full 8-rank QKV shape: gathered matrix bit-exact, sampled rows of C
    within tolerance (the oracle computes those rows alone)."""
    s = KI.AG_QKV
    say(f"[ag qkv full] mode={mode}")
    inp, g, c = _run(kos, ws, s, 0, False, torch.bfloat16, kos.opts(mode=mode))
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    shards = [KI.bf16_bits(inp["a_local"]) if p == 0 else peers[p] for p in range(s.world)]
    gref = O.gather(shards)
    assert np.array_equal(KI.bf16_bits(g), gref)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(s.m, 96, replace=False))
    cref = O.round_bf16(O.gemm(gref[rows], KI.bf16_bits(inp["w"])))
    assert_close(O.bf16_to_f64(KI.bf16_bits(c)[rows]), O.bf16_to_f64(cref), "C rows")


def test_ag_mlpup_full_size_sampled(kos, ws):
    """MLP-up shape (8 ranks, 4096 x 8192 . 8192 x 7168, 256 x 256 tiles):
    gathered matrix bit-exact, sampled rows of C within tolerance."""
    s = KI.AG_MLPUP
    say("[ag mlp-up full]")
    inp, g, c = _run(kos, ws, s, 3, False, torch.bfloat16, kos.opts())
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    shards = [KI.bf16_bits(inp["a_local"]) if p == 3 else peers[p] for p in range(s.world)]
    gref = O.gather(shards)
    assert np.array_equal(KI.bf16_bits(g), gref)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(s.m, 64, replace=False))
    cref = O.round_bf16(O.gemm(gref[rows], KI.bf16_bits(inp["w"])))
    assert_close(O.bf16_to_f64(KI.bf16_bits(c)[rows]), O.bf16_to_f64(cref), "C rows")
