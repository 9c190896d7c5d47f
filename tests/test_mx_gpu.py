"""MXFP8 all-gather + GEMM and GEMM + reduce-scatter on the GPU against the
oracle (through the C ABI).

Small cases use integer-valued codes with scales near 1, where every fp32
sum is exact: the outputs must equal the oracle bit for bit.  The full-size
cases (8 ranks, QKV and MLP-down shapes) compare the gathered codes and
scales bit for bit and sampled output rows within the floating-point bar.
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


def _np(t):
    return None if t is None else t.cpu().numpy()


def _nat(slabs):
    return O.scales_from_slabs(_np(slabs))


def _run_ag(kos, ws, s, rank, integer, c_dtype, o, edge=False):
    inp = KI.ag_mx_inputs(s, rank, "cuda", integer=integer, edge=edge)
    g = torch.full((s.m, s.k), 0xFF, dtype=torch.uint8, device="cuda")
    gs = torch.full((s.k // 64, s.m, 2), 0xFF, dtype=torch.uint8, device="cuda")
    c = torch.full((s.m, s.n), float("nan"), dtype=c_dtype, device="cuda")
    kos.ag_gemm_mx(inp["a_local"], inp["s_local"], inp["a_peers"], inp["s_peers"], inp["w"], inp["w_scales"],
                   g, gs, c, rank, ws, o)
    ws.status()
    torch.cuda.synchronize()
    return inp, g, gs, c


def _ag_oracle(inp, rank, out, rows=None):
    """(gathered codes, gathered scales row-major, C or C[rows])."""
    world = len(inp["a_peers"])
    shards = [_np(inp["a_local"]) if p == rank else _np(inp["a_peers"][p]) for p in range(world)]
    scales = [_nat(inp["s_local"]) if p == rank else _nat(inp["s_peers"][p]) for p in range(world)]
    w, wsc = _np(inp["w"]), _nat(inp["w_scales"])
    if rows is None:
        return O.ag_gemm_mx(shards[rank], scales[rank], shards, scales, w, wsc, rank, out)
    g, gs = np.concatenate(shards), np.concatenate(scales)
    c = O.gemm_mx(g[rows], gs[rows], w, wsc)
    return g, gs, (O.round_bf16(c) if out == "bf16" else c.astype(np.float32))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rank", [0, 3])
def test_ag_mx_tiny_integer_exact(kos, ws, rank, mode):
    say(f"[ag mx tiny int] rank={rank} mode={mode}")
    inp, g, gs, c = _run_ag(kos, ws, KI.AG_TINY_MX, rank, True, torch.float32, kos.opts(mode=mode, n_movers=2))
    gref, gsref, cref = _ag_oracle(inp, rank, "f32")
    assert np.array_equal(_np(g), gref)
    assert np.array_equal(_nat(gs), gsref)
    assert np.array_equal(_np(c), cref)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_ag_mx_192_column_tiles_integer_exact(kos, ws, mode):
    """n = 768 on four ranks: 256 x 192 MX tiles fill more compute units than
    256 x 256 ones (16 tiles against 12), so they are the ones that run."""
    s = KI.AgShape("ag_mx_4r_1024x512x768", 18, 4, 256, 512, 768)
    say(f"[ag mx 192-column tiles] mode={mode}")
    inp, g, gs, c = _run_ag(kos, ws, s, 2, True, torch.float32, kos.opts(mode=mode, n_movers=2))
    gref, gsref, cref = _ag_oracle(inp, 2, "f32")
    assert np.array_equal(_np(g), gref)
    assert np.array_equal(_nat(gs), gsref)
    assert np.array_equal(_np(c), cref)


def test_ag_mx_tiny_bf16_out(kos, ws):
    say("[ag mx tiny bf16 out]")
    inp, g, gs, c = _run_ag(kos, ws, KI.AG_TINY_MX, 1, False, torch.bfloat16, kos.opts())
    gref, gsref, cref = _ag_oracle(inp, 1, "bf16")
    assert np.array_equal(_np(g), gref)
    assert_close(O.bf16_to_f64(KI.bf16_bits(c)), O.bf16_to_f64(cref), "C")


def test_ag_mx_single_rank(kos, ws):
    s = KI.AgShape("ag_mx_r1", 16, 1, 512, 256, 768)
    say("[ag mx world=1]")
    inp, g, gs, c = _run_ag(kos, ws, s, 0, True, torch.float32, kos.opts(n_movers=1))
    gref, gsref, cref = _ag_oracle(inp, 0, "f32")
    assert np.array_equal(_np(g), gref) and np.array_equal(_nat(gs), gsref)
    assert np.array_equal(_np(c), cref)


@pytest.mark.parametrize("mode", [0, 2])
def test_ag_mx_qkv_full_size_sampled(kos, ws, mode):
    s = KI.AG_QKV_MX
    say(f"[ag mx qkv full] mode={mode}")
    inp, g, gs, c = _run_ag(kos, ws, s, 5, False, torch.bfloat16, kos.opts(mode=mode))
    rows = np.sort(np.random.default_rng(1).choice(s.m, 64, replace=False))
    gref, gsref, cref = _ag_oracle(inp, 5, "bf16", rows)
    assert np.array_equal(_np(g), gref)
    assert np.array_equal(_nat(gs), gsref)
    assert_close(O.bf16_to_f64(KI.bf16_bits(c)[rows]), O.bf16_to_f64(cref), "C rows")


def test_ag_mx_rejects_untiled_shapes(kos, ws):
    s = KI.AgShape("ag_mx_bad", 17, 2, 128, 256, 256)   # m_local not a multiple of 256
    inp = KI.ag_mx_inputs(s, 0, "cuda")
    g = torch.empty((s.m, s.k), dtype=torch.uint8, device="cuda")
    gs = torch.empty((s.k // 64, s.m, 2), dtype=torch.uint8, device="cuda")
    c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    with pytest.raises(kos.KosError) as e:
        kos.ag_gemm_mx(inp["a_local"], inp["s_local"], inp["a_peers"], inp["s_peers"], inp["w"],
                       inp["w_scales"], g, gs, c, 0, ws)
    assert "SHAPE" in str(e.value)


def _run_rs(kos, ws, s, rank, integer, o, edge=False):
    inp = KI.rs_mx_inputs(s, rank, "cuda", integer=integer, edge=edge)
    partial = torch.full((s.m, s.n), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((s.m_chunk, s.n), float("nan"), dtype=torch.float32, device="cuda")
    kos.gemm_rs_mx(inp["a"], inp["a_scales"], inp["w"], inp["w_scales"], inp["peer_slices"], partial, y, rank,
                   ws, o)
    ws.status()
    torch.cuda.synchronize()
    return inp, partial, y


def _rs_oracle(inp, rank):
    return O.gemm_rs_mx(_np(inp["a"]), _nat(inp["a_scales"]), _np(inp["w"]), _nat(inp["w_scales"]),
                        [_np(t) for t in inp["peer_slices"]], rank)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rank", [0, 3])
def test_rs_mx_tiny_integer_exact(kos, ws, rank, mode, order):
    say(f"[rs mx tiny int] rank={rank} mode={mode} order={order}")
    o = kos.opts(mode=mode, n_movers=0 if mode == 0 else 2, rs_order=order)
    inp, partial, y = _run_rs(kos, ws, KI.RS_TINY_MX, rank, True, o)
    pref, yref = _rs_oracle(inp, rank)
    assert np.array_equal(_np(partial), pref)
    assert np.array_equal(_np(y), yref)


@pytest.mark.parametrize("rank", [0, 7])
def test_rs_mx_mlp_full_size(kos, ws, rank):
    """Full 8-rank MLP-down shape: y (512 x 8192) entirely, against the oracle's
    MX product of chunk `rank` plus the peers' slices."""
    s = KI.RS_MLP_MX
    say(f"[rs mx mlp full] rank={rank}")
    inp, partial, y = _run_rs(kos, ws, s, rank, False, kos.opts())
    mc = s.m_chunk
    a, sa = _np(inp["a"]), _nat(inp["a_scales"])
    own = O.gemm_mx(a[rank * mc:(rank + 1) * mc], sa[rank * mc:(rank + 1) * mc], _np(inp["w"]),
                    _nat(inp["w_scales"])).astype(np.float32)
    yref = np.zeros_like(own, dtype=np.float64)
    for p in range(s.world):
        yref += own if p == rank else _np(inp["peer_slices"][p]).astype(np.float64)
    assert_close(_np(y), yref, "y")
    assert_close(_np(partial)[rank * mc:(rank + 1) * mc], own, "own chunk of the partial")


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("rank", [0, 3])
def test_mx_edge_values(kos, ws, rank, mode):
    """Codes and scales at the format's edges -- subnormal E4M3 codes, zeros,
    codes up to +-448, scales 2^-27 .. 2^27 -- through both collectives:
    the gathered codes and scales bit-exact, C, the partial and y within
    the floating-point bar against the oracle's exact decode."""
    say(f"[mx edge] rank={rank} mode={mode}")
    o = kos.opts(mode=mode)
    inp, g, gs, c = _run_ag(kos, ws, KI.AG_TINY_MX, rank, False, torch.float32, o, edge=True)
    gref, gsref, cref = _ag_oracle(inp, rank, "f32")
    codes = _np(g)
    assert ((codes & 0x78) == 0).mean() > 0.2 and np.abs(O.e4m3_to_f64(codes)).max() == 448.0
    assert np.array_equal(codes, gref) and np.array_equal(_nat(gs), gsref)
    assert np.all(np.isfinite(cref)) and np.abs(cref).max() > 1e15
    assert_close(_np(c), cref, "C (edge values)")
    inp, partial, y = _run_rs(kos, ws, KI.RS_TINY_MX, rank, False, o, edge=True)
    pref, yref = _rs_oracle(inp, rank)
    assert_close(_np(partial), pref, "partial (edge values)")
    assert_close(_np(y), yref, "y (edge values)")
