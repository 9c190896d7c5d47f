"""The C-ABI library: loads, exports every declared symbol, validates
arguments before touching a device (CPU only: no compute calls)."""
import ctypes
import os

import pytest

from kos_testutil import header_symbols

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kos.h")


def test_library_exports_every_declared_symbol():
    import gemm_collective_persistent_amd as kos
    declared = header_symbols(HEADER)
    assert declared, "no declarations parsed"
    missing = [s for s in declared if not hasattr(kos.lib, s)]
    assert not missing, f"declared in kos.h but not exported: {missing}"
    assert sorted(kos.EXPORTS) == declared


def test_opts_defaults_and_workspace_size():
    import gemm_collective_persistent_amd as kos
    o = kos.opts()
    assert (o.mode, o.n_movers, o.rs_order, o.grid, o.spin_limit, o.peer_link) == (0, -1, 0, 0, 0, 0)
    assert kos.lib.kos_workspace_bytes() >= 16 << 20


def _ag(kos, **over):
    lib = kos.lib
    fake = ctypes.c_void_p(0x10000)           # never dereferenced: validation fails first
    peers = kos._binding.ptr_array([None, 0x10000, 0x10000, 0x10000])
    args = dict(world=4, rank=0, m=64, k=256, n=256, a=fake, peers=peers, w=fake, g=fake, c=fake,
                dt=0, ws=fake, wsb=lib.kos_workspace_bytes())
    args.update(over)
    o = kos.opts()
    return lib.kos_ag_gemm(args["world"], args["rank"], args["m"], args["k"], args["n"], args["a"],
                           args["peers"], args["w"], args["g"], args["c"], args["dt"], ctypes.byref(o),
                           args["ws"], args["wsb"], None)


def test_ag_gemm_argument_validation():
    import gemm_collective_persistent_amd as kos
    from gemm_collective_persistent_amd._binding import (KOS_ERR_ALIGN, KOS_ERR_ARG, KOS_ERR_SHAPE,
                                                         KOS_ERR_WORKSPACE)
    assert _ag(kos, world=9) == KOS_ERR_ARG
    assert _ag(kos, rank=4) == KOS_ERR_ARG
    assert _ag(kos, dt=7) == KOS_ERR_ARG
    assert _ag(kos, a=None) == KOS_ERR_ARG
    assert _ag(kos, peers=kos._binding.ptr_array([None, None, 0x10000, 0x10000])) == KOS_ERR_ARG
    assert _ag(kos, k=100) == KOS_ERR_SHAPE
    assert _ag(kos, m=0) == KOS_ERR_SHAPE
    assert _ag(kos, a=ctypes.c_void_p(0x10008)) == KOS_ERR_ALIGN
    assert _ag(kos, wsb=1024) == KOS_ERR_WORKSPACE
    assert b"workspace" in kos.lib.kos_last_error()


def test_trace_reader_validation():
    import gemm_collective_persistent_amd as kos
    from gemm_collective_persistent_amd._binding import KOS_ERR_ARG, TRACE_LAUNCHES, TRACE_MAX_WG, TRACE_RECORDS
    lib = kos.lib
    fake = ctypes.c_void_p(0x10000)            # never dereferenced: validation fails first
    assert lib.kos_workspace_trace(None, fake, 1, None) == KOS_ERR_ARG
    assert lib.kos_workspace_trace(fake, None, 1, None) == KOS_ERR_ARG
    assert lib.kos_workspace_trace(fake, fake, TRACE_LAUNCHES * TRACE_MAX_WG * TRACE_RECORDS + 1, None) == KOS_ERR_ARG
    assert ctypes.sizeof(kos._binding.TraceRec) == 16
    assert ctypes.sizeof(kos.Opts) == 32


def _ag_mx(kos, **over):
    lib = kos.lib
    fake = ctypes.c_void_p(0x10000)           # never dereferenced: validation fails first
    peers = kos._binding.ptr_array([None, 0x10000])
    args = dict(world=2, rank=0, m=256, k=256, n=256, a=fake, sa=fake, peers=peers, speers=peers, w=fake,
                sw=fake, g=fake, sg=fake, c=fake, dt=0, ws=fake, wsb=lib.kos_workspace_bytes())
    args.update(over)
    o = kos.opts()
    return lib.kos_ag_gemm_mx(args["world"], args["rank"], args["m"], args["k"], args["n"], args["a"], args["sa"],
                              args["peers"], args["speers"], args["w"], args["sw"], args["g"], args["sg"],
                              args["c"], args["dt"], ctypes.byref(o), args["ws"], args["wsb"], None)


def _rs(kos, fn, **over):
    lib = kos.lib
    fake = ctypes.c_void_p(0x10000)
    peers = kos._binding.ptr_array([None, 0x10000])
    args = dict(world=2, rank=0, m=512, k=256, n=256, a=fake, sa=fake, w=fake, sw=fake, peers=peers, p=fake,
                y=fake, ws=fake, wsb=lib.kos_workspace_bytes())
    args.update(over)
    o = kos.opts()
    if fn == "mx":
        return lib.kos_gemm_rs_mx(args["world"], args["rank"], args["m"], args["k"], args["n"], args["a"],
                                  args["sa"], args["w"], args["sw"], args["peers"], args["p"], args["y"],
                                  ctypes.byref(o), args["ws"], args["wsb"], None)
    return lib.kos_gemm_rs_wt(args["world"], args["rank"], args["m"], args["k"], args["n"], args["a"], args["w"],
                              args["peers"], args["p"], args["y"], ctypes.byref(o), args["ws"], args["wsb"], None)


def test_mx_and_wt_argument_validation():
    import gemm_collective_persistent_amd as kos
    from gemm_collective_persistent_amd._binding import KOS_ERR_ALIGN, KOS_ERR_ARG, KOS_ERR_SHAPE
    # MX: whole 256 x 256 tiles and whole 256-wide K trips only
    assert _ag_mx(kos, m=128) == KOS_ERR_SHAPE
    assert _ag_mx(kos, k=320) == KOS_ERR_SHAPE
    assert _ag_mx(kos, n=192) == KOS_ERR_SHAPE
    assert _ag_mx(kos, sa=None) == KOS_ERR_ARG
    assert _ag_mx(kos, speers=kos._binding.ptr_array([None, None])) == KOS_ERR_ARG
    assert _ag_mx(kos, sg=ctypes.c_void_p(0x10004)) == KOS_ERR_ALIGN
    assert _rs(kos, "mx", m=256) == KOS_ERR_SHAPE       # m/world = 128
    assert _rs(kos, "mx", sw=None) == KOS_ERR_ARG
    # transposed weights: the bf16 rules
    assert _rs(kos, "wt", k=100) == KOS_ERR_SHAPE
    assert _rs(kos, "wt", w=None) == KOS_ERR_ARG


def _moe_call(kos, name, **over):
    """kos_moe_layer / kos_moe_combine / kos_moe_layer_bwd with one world-1
    rank and fake (never dereferenced) pointers: only the host checks run."""
    lib = kos.lib
    from gemm_collective_persistent_amd._binding import MoeShape
    s = MoeShape(1, 0, 64, 256, 8, 2, 256, 0)
    f = 0x10000
    a = dict(g=None, u=None, dh=f, gate=None, up=None)
    a.update(over)
    P = ctypes.c_void_p
    o = kos.opts()
    ws, wsb = P(f), lib.kos_workspace_bytes()
    one = kos._binding.ptr_array([None])
    caps = (ctypes.c_int64 * 1)(0)
    if name == "layer":
        return lib.kos_moe_layer(ctypes.byref(s), P(f), P(f), one, P(f), P(f), P(f), P(f), one, P(f), P(f), P(f),
                                 P(f), one, caps, P(f), 1024, P(f), P(f), P(f), P(a["g"]), P(a["u"]), P(f), one,
                                 caps, P(f), ctypes.byref(o), ws, wsb, None)
    if name == "combine":
        return lib.kos_moe_combine(ctypes.byref(s), P(f), P(f), P(f), 1024, P(f), P(f), P(f), P(f), P(f), P(f),
                                   P(f), P(f), one, P(f), P(a["g"]), P(a["u"]), P(f), one, caps, P(f),
                                   ctypes.byref(o), ws, wsb, None)
    return lib.kos_moe_layer_bwd(ctypes.byref(s), P(f), P(f), P(f), P(f), P(f), P(f), P(f), 1024, P(f), P(f), P(f),
                                 one, P(f), P(f), P(f), P(a["gate"]), P(a["up"]), one, one, caps, P(f), P(f), P(f),
                                 P(a["dh"]), P(f), one, one, caps, P(f), P(f), ctypes.byref(o), ws, wsb, None)


def test_kept_activation_argument_validation():
    """The optional kept g and u: both or neither, 16-byte aligned; the
    backward needs dh only when it recomputes them."""
    import gemm_collective_persistent_amd as kos
    from gemm_collective_persistent_amd._binding import KOS_ERR_ALIGN, KOS_ERR_ARG
    for name in ("layer", "combine"):
        assert _moe_call(kos, name, g=0x20000) == KOS_ERR_ARG, name
        assert _moe_call(kos, name, u=0x20000) == KOS_ERR_ARG, name
        assert b"together" in kos.lib.kos_last_error(), name
        assert _moe_call(kos, name, g=0x20008, u=0x20000) == KOS_ERR_ALIGN, name
    assert _moe_call(kos, "bwd", dh=None) == KOS_ERR_ARG
    assert _moe_call(kos, "bwd", gate=0x20000) == KOS_ERR_ARG
    assert b"together" in kos.lib.kos_last_error()
    assert _moe_call(kos, "bwd", gate=0x20000, up=0x20004) == KOS_ERR_ALIGN
