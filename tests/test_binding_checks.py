"""The Python binding's argument checks (CPU only: tensors stay on the host,
the library's entry points are replaced by a recorder, so nothing reaches a
device).  Every buffer's shape is checked against the sizes the call implies
before the C ABI is called, and each send / return buffer's own row count is
passed as its capacity."""
import ctypes

import pytest
import torch

import kos_inputs as KI


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append((name, args))
            return 0
        return fn


class _Ws:
    ptr, nbytes = 0x1000, 1 << 20


@pytest.fixture()
def api(monkeypatch):
    from gemm_collective_persistent_amd import api as A
    rec = _Recorder()
    monkeypatch.setattr(A, "lib", rec)
    monkeypatch.setattr(A, "_placed", lambda t, host_ok: True)
    monkeypatch.setattr(A, "_stream", lambda s=None: None)
    A._rec = rec
    return A


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def test_ag_gemm_shapes(api):
    w, m, k, n = 4, 64, 256, 128
    peers = [None] + [bf(m, k) for _ in range(w - 1)]
    good = dict(a_local=bf(m, k), a_peers=peers, w=bf(k, n), a_gathered=bf(w * m, k), c=bf(w * m, n))
    api.ag_gemm(**good, rank=0, ws=_Ws())
    assert api._rec.calls[-1][0] == "kos_ag_gemm"
    for key, bad in (("a_gathered", bf(w * m - 64, k)), ("c", bf(w * m, n + 64)), ("w", bf(k + 64, n)),
                     ("c", f32(w * m - 1, n))):
        with pytest.raises(ValueError, match=key):
            api.ag_gemm(**{**good, key: bad}, rank=0, ws=_Ws())
    with pytest.raises(ValueError, match=r"a_peers\[2\]"):
        api.ag_gemm(**{**good, "a_peers": [None, bf(m, k), bf(m - 64, k), bf(m, k)]}, rank=0, ws=_Ws())
    # transposed weight: [n, k]
    api.ag_gemm(**{**good, "w": bf(n, k)}, rank=0, ws=_Ws(), w_transposed=True)
    assert api._rec.calls[-1][0] == "kos_ag_gemm_wt"


def test_gemm_rs_shapes(api):
    w, m, k, n = 4, 256, 128, 192
    peers = [None] + [f32(m // w, n) for _ in range(w - 1)]
    good = dict(a=bf(m, k), w=bf(k, n), peer_slices=peers, partial=f32(m, n), y=f32(m // w, n))
    api.gemm_rs(**good, rank=0, ws=_Ws())
    for key, bad in (("partial", f32(m, n - 64)), ("y", f32(m, n)), ("w", bf(n, k))):
        with pytest.raises(ValueError, match=key):
            api.gemm_rs(**{**good, key: bad}, rank=0, ws=_Ws())
    with pytest.raises(ValueError, match=r"peer_slices\[1\]"):
        api.gemm_rs(**{**good, "peer_slices": [None, f32(m // w + 1, n)] + peers[2:]}, rank=0, ws=_Ws())


def _moe_buffers(s, rank, send_rows, ret_rows):
    T, H, E, k, El, F = s.tokens, s.hidden, s.experts, s.topk, s.e_local, s.ffn
    cap = 4 * T
    return dict(
        x=bf(T, H), logits=f32(T, E), peer_counts=i32(s.world, El), topk_idx=i32(T, k), topk_w=f32(T, k),
        counts=i32(E), perm=i32(T * k), x_grouped=bf(cap, H), grouped_offsets=i32(El + 1), row_src=i32(cap, 2),
        out_send=[None if p == rank else bf(send_rows[p], H) for p in range(s.world)],
        peer_send=[None if p == rank else bf(3, H) for p in range(s.world)],
        wg=bf(El, H, F), wu=bf(El, H, F), wd=bf(El, F, H), h=bf(cap, F), yg=bf(cap, H), y=bf(T, H),
        peer_return=[None if p == rank else bf(5, H) for p in range(s.world)],
        out_return=[None if p == rank else bf(ret_rows[p], H) for p in range(s.world)])


def test_dispatch_passes_each_destination_its_own_capacity(api):
    s, rank = KI.MOE_TINY, 1
    shp = api.moe_shape(s.world, rank, s.tokens, s.hidden, s.experts, s.topk, s.ffn)
    b = _moe_buffers(s, rank, [17, 0, 5, 300], [1, 0, 1, 1])
    api.moe_dispatch(shp, b["x"], b["logits"], b["peer_send"], b["peer_counts"], b["topk_idx"], b["topk_w"],
                     b["counts"], b["perm"], b["out_send"], b["x_grouped"], b["grouped_offsets"], b["row_src"],
                     _Ws())
    name, args = api._rec.calls[-1]
    assert name == "kos_moe_dispatch"
    caps = args[10]
    assert [caps[p] for p in range(s.world)] == [17, 0, 5, 300]
    assert args[12] == b["x_grouped"].shape[0]
    with pytest.raises(ValueError, match="row_src"):
        api.moe_dispatch(shp, b["x"], b["logits"], b["peer_send"], b["peer_counts"], b["topk_idx"], b["topk_w"],
                         b["counts"], b["perm"], b["out_send"], b["x_grouped"], b["grouped_offsets"],
                         i32(b["x_grouped"].shape[0] - 1, 2), _Ws())
    with pytest.raises(ValueError, match=r"out_send\[2\]"):
        bad = list(b["out_send"])
        bad[2] = bf(5, s.hidden + 64)
        api.moe_dispatch(shp, b["x"], b["logits"], b["peer_send"], b["peer_counts"], b["topk_idx"], b["topk_w"],
                         b["counts"], b["perm"], bad, b["x_grouped"], b["grouped_offsets"], b["row_src"], _Ws())
    with pytest.raises(ValueError, match="logits"):
        api.moe_dispatch(shp, b["x"], f32(s.tokens, s.experts - 1), b["peer_send"], b["peer_counts"],
                         b["topk_idx"], b["topk_w"], b["counts"], b["perm"], b["out_send"], b["x_grouped"],
                         b["grouped_offsets"], b["row_src"], _Ws())


def test_combine_checks_and_return_capacities(api):
    s, rank = KI.MOE_TINY, 0
    shp = api.moe_shape(s.world, rank, s.tokens, s.hidden, s.experts, s.topk, s.ffn)
    b = _moe_buffers(s, rank, [0, 1, 1, 1], [0, 9, 2, 40])

    def call(**over):
        a = {**b, "gate_save": None, "up_save": None, **over}
        api.moe_combine(shp, a["x_grouped"], a["grouped_offsets"], a["row_src"], a["wg"], a["wu"], a["wd"],
                        a["topk_idx"], a["topk_w"], a["counts"], a["perm"], a["peer_counts"], a["peer_return"],
                        a["h"], a["yg"], a["out_return"], a["y"], _Ws(), gate_save=a["gate_save"],
                        up_save=a["up_save"])

    call()
    name, args = api._rec.calls[-1]
    assert name == "kos_moe_combine"
    caps = args[19]
    assert [caps[p] for p in range(1, s.world)] == [9, 2, 40]
    assert args[15] is None and args[16] is None
    cap = b["x_grouped"].shape[0]
    g, u = bf(cap, s.ffn), bf(cap + 3, s.ffn)
    call(gate_save=g, up_save=u)
    args = api._rec.calls[-1][1]
    assert args[14] == b["h"].data_ptr() and args[15] == g.data_ptr() and args[16] == u.data_ptr()
    assert args[17] == b["yg"].data_ptr()
    for key, bad in (("h", bf(cap - 1, s.ffn)), ("yg", bf(cap - 1, s.hidden)), ("wd", bf(s.e_local, s.hidden, s.ffn)),
                     ("y", bf(s.tokens + 1, s.hidden)), ("h", bf(cap, s.ffn + 64))):
        with pytest.raises(ValueError):
            call(**{key: bad})
    with pytest.raises(ValueError, match="topk_w"):
        call(topk_w=f32(s.tokens, s.topk + 1))
    with pytest.raises(ValueError, match="together"):
        call(gate_save=g)
    for bad in (bf(cap - 1, s.ffn), bf(cap, s.ffn + 64), f32(cap, s.ffn)):
        with pytest.raises((ValueError, TypeError)):
            call(gate_save=g, up_save=bad)


def test_layer_and_backward_pass_the_saved_activations(api):
    s, rank = KI.MOE_TINY, 0
    shp = api.moe_shape(s.world, rank, s.tokens, s.hidden, s.experts, s.topk, s.ffn)
    b = _moe_buffers(s, rank, [0, 1, 1, 1], [0, 9, 2, 40])
    cap = b["x_grouped"].shape[0]
    g, u = bf(cap, s.ffn), bf(cap, s.ffn)
    api.moe_layer(shp, b["x"], b["logits"], b["peer_send"], b["peer_counts"], b["wg"], b["wu"], b["wd"],
                  b["peer_return"], b["topk_idx"], b["topk_w"], b["counts"], b["perm"], b["out_send"],
                  b["x_grouped"], b["grouped_offsets"], b["row_src"], b["h"], b["yg"], b["out_return"], b["y"],
                  _Ws(), gate_save=g, up_save=u)
    name, args = api._rec.calls[-1]
    assert name == "kos_moe_layer"
    assert args[19] == b["h"].data_ptr() and args[20] == g.data_ptr() and args[21] == u.data_ptr()
    assert args[22] == b["yg"].data_ptr()
    T, H, F = s.tokens, s.hidden, s.ffn
    grads = dict(dy=bf(T, H), dres=bf(cap, H), dg=bf(cap, F), du=bf(cap, F), dh=f32(cap, F), dxg=bf(cap, H),
                 dx=bf(T, H), dl=f32(T, s.experts),
                 psg=[None if p == rank else bf(3, H) for p in range(s.world)],
                 osg=[None if p == rank else bf(7, H) for p in range(s.world)],
                 prg=[None if p == rank else bf(5, H) for p in range(s.world)],
                 org=[None if p == rank else bf(9, H) for p in range(s.world)])

    def bwd(dh, **kw):
        api.moe_layer_bwd(shp, grads["dy"], b["topk_idx"], b["topk_w"], b["perm"], b["counts"], b["peer_counts"],
                          b["x_grouped"], b["grouped_offsets"], b["row_src"], b["yg"], b["peer_return"], b["wg"],
                          b["wu"], b["wd"], grads["psg"], grads["osg"], grads["dres"], grads["dg"], grads["du"], dh,
                          grads["dxg"], grads["prg"], grads["org"], grads["dx"], grads["dl"], _Ws(), **kw)
        return api._rec.calls[-1][1]

    args = bwd(grads["dh"])
    assert args[16] is None and args[17] is None and args[24] == grads["dh"].data_ptr()
    args = bwd(None, gate_saved=g, up_saved=u)
    assert args[15] == b["wd"].data_ptr() and args[16] == g.data_ptr() and args[17] == u.data_ptr()
    assert args[24] is None
    with pytest.raises(ValueError, match="dh"):
        bwd(None)
    with pytest.raises(ValueError, match="together"):
        bwd(grads["dh"], up_saved=u)
    with pytest.raises(ValueError):
        bwd(grads["dh"], gate_saved=g, up_saved=bf(cap, F + 64))


def test_kos_error_carries_the_status():
    from gemm_collective_persistent_amd._binding import KOS_ERR_CAPACITY, KosError
    e = KosError(KOS_ERR_CAPACITY, "too many rows")
    assert e.status == KOS_ERR_CAPACITY and "KOS_ERR_CAPACITY" in str(e)
    assert ctypes.sizeof(__import__("gemm_collective_persistent_amd")._binding.DeviceError) == 8
