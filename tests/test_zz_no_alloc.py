"""The allocation-free all-gather + GEMM (kos_ag_gemm_noalloc: no workspace,
the library's static scratch) against the workspace entry point
(kos_ag_gemm) on the same inputs, through the C ABI: two calls in a row on
one device, the second with smaller inputs, and the oracle beside both."""
import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import assert_close, say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu

# a larger call first (several 256-row blocks per shard, ragged column
# tiles), then a smaller one on the same static scratch
MID = KI.AgShape("ag_noalloc_mid_4r_1024x512x384", 30, 4, 256, 512, 384)


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


def _pair(kos, ws, s, rank, integer, c_dtype, mode):
    inp = KI.ag_inputs(s, rank, "cuda", integer=integer)
    out = {}
    for name in ("ws", "noalloc"):
        g = torch.full((s.m, s.k), float("nan"), dtype=torch.bfloat16, device="cuda")
        c = torch.full((s.m, s.n), float("nan"), dtype=c_dtype, device="cuda")
        o = kos.opts(mode=mode)
        if name == "ws":
            kos.ag_gemm(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, ws, o)
            ws.status()
            st = None
        else:
            st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            kos.ag_gemm_noalloc(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, st, o)
        torch.cuda.synchronize()
        out[name] = (g, c, st)
    return inp, out


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_noalloc_matches_workspace_entry_point(kos, mode):
    ws = kos.Workspace("cuda")
    for s, rank, integer, c_dtype in ((MID, 1, False, torch.bfloat16), (KI.AG_TINY, 2, True, torch.float32)):
        say(f"[ag noalloc] {s.name} rank={rank} mode={mode}")
        inp, out = _pair(kos, ws, s, rank, integer, c_dtype, mode)
        g_ws, c_ws, _ = out["ws"]
        g_na, c_na, st = out["noalloc"]
        assert int(st.item()) == 0, "device-side status of the allocation-free call"
        # the same kernels on the same inputs: identical bits
        assert torch.equal(g_na.view(torch.int16), g_ws.view(torch.int16))
        assert torch.equal(c_na.view(torch.int16) if c_dtype == torch.bfloat16 else c_na.view(torch.int32),
                           c_ws.view(torch.int16) if c_dtype == torch.bfloat16 else c_ws.view(torch.int32))
        # and both against the oracle
        peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
        gref, cref = O.ag_gemm(KI.bf16_bits(inp["a_local"]), peers, KI.bf16_bits(inp["w"]), rank,
                               out_dtype="f32" if integer else "bf16")
        assert np.array_equal(KI.bf16_bits(g_na), gref)
        if integer:
            assert np.array_equal(c_na.cpu().numpy(), cref)
        else:
            assert_close(O.bf16_to_f64(KI.bf16_bits(c_na)), O.bf16_to_f64(cref), "C")


def test_noalloc_status_may_be_omitted_and_rejects_oversize(kos):
    s, rank = KI.AG_TINY, 0
    say("[ag noalloc] no status buffer; oversize and traced calls rejected")
    inp = KI.ag_inputs(s, rank, "cuda", integer=True)
    g = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    kos.ag_gemm_noalloc(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank)
    torch.cuda.synchronize()
    peers = [None if t is None else KI.bf16_bits(t) for t in inp["a_peers"]]
    _, cref = O.ag_gemm(KI.bf16_bits(inp["a_local"]), peers, KI.bf16_bits(inp["w"]), rank, out_dtype="f32")
    assert np.array_equal(c.cpu().numpy(), cref)
    with pytest.raises(kos.KosError) as e:
        kos.ag_gemm_noalloc(inp["a_local"], inp["a_peers"], inp["w"], g, c, rank, o=kos.opts(trace=True))
    assert "ARG" in str(e.value)
    # more row blocks than the static scratch's 16384 ready counters (checked
    # on the host before anything is launched or read)
    big = torch.empty((2, 64), dtype=torch.bfloat16, device="cuda")
    lib = kos.lib
    from gemm_collective_persistent_amd._binding import KOS_ERR_SHAPE, ptr_array
    st = lib.kos_ag_gemm_noalloc(8, 0, 64 * 4096, 64, 64, big.data_ptr(),
                                 ptr_array([None] + [big.data_ptr()] * 7), big.data_ptr(), big.data_ptr(),
                                 big.data_ptr(), 0, None, None, None)
    assert st == KOS_ERR_SHAPE
