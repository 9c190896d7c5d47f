"""torch-tensor front end of the C ABI (argument marshalling only)."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from ._binding import (KOS_BF16, KOS_ERR_ARG, KOS_F32, DeviceError, KosError, MoeShape, Opts, check, lib,
                       opts as make_opts, ptr_array)


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str, ndim: int, shape=None, host_ok: bool = False):
    """dtype, rank, contiguity, shape (None entries are free) and placement:
    on the GPU, or (host_ok: an emulated peer's buffer) in pinned host memory
    the device can map."""
    if t is None:
        raise ValueError(f"{name}: missing")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {ndim}-d tensor")
    if shape is not None and any(w is not None and g != w for g, w in zip(t.shape, shape)):
        want = tuple("*" if w is None else w for w in shape)
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    if not _placed(t, host_ok):
        raise ValueError(f"{name}: must be a GPU tensor" + (" or pinned host memory" if host_ok else ""))


def _placed(t: torch.Tensor, host_ok: bool) -> bool:
    return t.is_cuda or (host_ok and t.is_pinned())


def _min_rows(t: torch.Tensor, rows: int, name: str):
    if t.shape[0] < rows:
        raise ValueError(f"{name}: {t.shape[0]} rows, needs at least {rows}")


def _check_saved(g, u, cap: int, F: int):
    """The optional saved gate/up activations: both or neither, bf16 [>= cap, F]."""
    if (g is None) != (u is None):
        raise ValueError("the saved gate and up activations are given together or not at all")
    for name, t in (("gate", g), ("up", u)):
        if t is not None:
            _need(t, torch.bfloat16, name, 2, (None, F))
            _min_rows(t, cap, name)


class Workspace:
    """Device workspace of kos_workspace_bytes() bytes, zeroed once."""

    def __init__(self, device="cuda", stream=None):
        self.nbytes = int(lib.kos_workspace_bytes())
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        check(lib.kos_workspace_init(self.ptr, self.nbytes, _stream(stream)))

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    def status(self, stream=None) -> None:
        """Synchronizes and raises KosError if a device-side error was
        recorded (``self.last_error`` then holds (status, entry))."""
        err = DeviceError()
        st = lib.kos_workspace_status(self.ptr, _stream(stream), ctypes.byref(err))
        self.last_error = (int(err.status), int(err.entry))
        check(st)

    def trace(self, grid: int, stream=None, launches: int = 1):
        """Timeline of the last call made with ``opts(trace=True)`` on a grid of
        `grid` workgroups that made `launches` kernel launches (1 for a fused
        call; the unfused baselines make 2, or 4 for the expert combine): a
        list, per workgroup and launch, of (ticket, t_begin, t_end, [(kind,
        entry, t0, t1), ...]) with times in microseconds from the earliest
        workgroup start of the call (kos_workspace_trace; every launch reads
        the same constant-rate clock).  ``self.trace_xcd`` then holds each
        entry's XCD and ``self.trace_clock_mhz`` the shader clock it ran at
        (its clock record)."""
        from ._binding import TRACE_CLOCK, TRACE_KINDS, TRACE_LAUNCHES, TRACE_MAX_WG, TRACE_RECORDS, TraceRec
        if not 0 < grid <= TRACE_MAX_WG:
            raise ValueError(f"grid {grid} outside [1, {TRACE_MAX_WG}]")
        if not 0 < launches <= TRACE_LAUNCHES:
            raise ValueError(f"launches {launches} outside [1, {TRACE_LAUNCHES}]")
        slot = TRACE_MAX_WG * TRACE_RECORDS
        n = (launches - 1) * slot + grid * TRACE_RECORDS
        buf = (TraceRec * n)()
        check(lib.kos_workspace_trace(self.ptr, ctypes.cast(buf, ctypes.c_void_p), n, _stream(stream)))
        tick_us = 0.01                      # 100 MHz constant-rate counter
        rows = [l * slot + g * TRACE_RECORDS for l in range(launches) for g in range(grid)]
        heads = [buf[r] for r in rows]
        t_ref = min(h.t0 for h in heads)
        out = []
        self.trace_xcd = [(h.tag >> 12) & 15 for h in heads]
        self.trace_clock_mhz = []
        for r0, h in zip(rows, heads):
            clk = buf[r0 + 1]
            if clk.tag >> 24 != TRACE_CLOCK:
                raise KosError(KOS_ERR_ARG, f"trace row {r0 // TRACE_RECORDS}: record 1 is not a clock record")
            self.trace_clock_mhz.append(100.0 * clk.t0 / clk.dt if clk.dt else 0.0)
            used = h.tag & 0xFFF
            recs = []
            for i in range(2, min(used, TRACE_RECORDS)):
                r = buf[r0 + i]
                t0 = (r.t0 - t_ref) * tick_us
                recs.append((TRACE_KINDS.get(r.tag >> 24, str(r.tag >> 24)), r.tag & 0xFFFFFF, t0,
                             t0 + r.dt * tick_us))
            tb = (h.t0 - t_ref) * tick_us
            out.append((h.tag >> 16, tb, tb + h.dt * tick_us, recs))
        return out


def ag_gemm(a_local: torch.Tensor, a_peers: Sequence[Optional[torch.Tensor]], w: torch.Tensor,
            a_gathered: torch.Tensor, c: torch.Tensor, rank: int, ws: Workspace,
            o: Optional[Opts] = None, stream=None, w_transposed: bool = False) -> None:
    """kos_ag_gemm: a_gathered = concat(shards); c = a_gathered @ w (w [k, n]).
    w_transposed (kos_ag_gemm_wt): w is W^T [n, k] and c = a_gathered @ w.T."""
    world = len(a_peers)
    _need(a_local, torch.bfloat16, "a_local", 2)
    m_local, k = a_local.shape
    _need(w, torch.bfloat16, "w", 2)
    n = w.shape[0] if w_transposed else w.shape[1]
    _need(w, torch.bfloat16, "w", 2, (n, k) if w_transposed else (k, n))
    _need(a_gathered, torch.bfloat16, "a_gathered", 2, (world * m_local, k))
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("c must be bf16 or fp32")
    _need(c, c.dtype, "c", 2, (world * m_local, n))
    for p, t in enumerate(a_peers):
        if p != rank:
            _need(t, torch.bfloat16, f"a_peers[{p}]", 2, (m_local, k), host_ok=True)
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(a_peers)])
    o = o if o is not None else make_opts()
    fn = lib.kos_ag_gemm_wt if w_transposed else lib.kos_ag_gemm
    check(fn(world, rank, m_local, k, n, _p(a_local), peers, _p(w), _p(a_gathered),
             _p(c), KOS_BF16 if c.dtype == torch.bfloat16 else KOS_F32,
             ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def ag_gemm_noalloc(a_local: torch.Tensor, a_peers: Sequence[Optional[torch.Tensor]], w: torch.Tensor,
                    a_gathered: torch.Tensor, c: torch.Tensor, rank: int, status: Optional[torch.Tensor] = None,
                    o: Optional[Opts] = None, stream=None) -> None:
    """kos_ag_gemm_noalloc: as ag_gemm (w [k, n]) with no workspace -- the
    library's static scratch holds the queues.  `status` (optional int32 [1]
    on the GPU) receives the call's device-side status when it finishes."""
    world = len(a_peers)
    _need(a_local, torch.bfloat16, "a_local", 2)
    m_local, k = a_local.shape
    _need(w, torch.bfloat16, "w", 2, (k, None))
    n = w.shape[1]
    _need(a_gathered, torch.bfloat16, "a_gathered", 2, (world * m_local, k))
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("c must be bf16 or fp32")
    _need(c, c.dtype, "c", 2, (world * m_local, n))
    for p, t in enumerate(a_peers):
        if p != rank:
            _need(t, torch.bfloat16, f"a_peers[{p}]", 2, (m_local, k), host_ok=True)
    if status is not None:
        _need(status, torch.int32, "status", 1, (1,))
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(a_peers)])
    o = o if o is not None else make_opts()
    check(lib.kos_ag_gemm_noalloc(world, rank, m_local, k, n, _p(a_local), peers, _p(w), _p(a_gathered), _p(c),
                                  KOS_BF16 if c.dtype == torch.bfloat16 else KOS_F32, ctypes.byref(o),
                                  _p(status), _stream(stream)))


def gemm_rs(a: torch.Tensor, w: torch.Tensor, peer_slices: Sequence[Optional[torch.Tensor]],
            partial: torch.Tensor, y: torch.Tensor, rank: int, ws: Workspace,
            o: Optional[Opts] = None, stream=None, w_transposed: bool = False) -> None:
    """kos_gemm_rs: partial = a @ w (fp32, w [k, n]); y = reduce of chunk
    `rank`.  w_transposed (kos_gemm_rs_wt): w is W^T [n, k], partial = a @ w.T."""
    world = len(peer_slices)
    _need(a, torch.bfloat16, "a", 2)
    m, k = a.shape
    _need(w, torch.bfloat16, "w", 2)
    n = w.shape[0] if w_transposed else w.shape[1]
    _need(w, torch.bfloat16, "w", 2, (n, k) if w_transposed else (k, n))
    mc = m // world
    _need(partial, torch.float32, "partial", 2, (m, n))
    _need(y, torch.float32, "y", 2, (mc, n))
    for p, t in enumerate(peer_slices):
        if p != rank:
            _need(t, torch.float32, f"peer_slices[{p}]", 2, (mc, n), host_ok=True)
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(peer_slices)])
    o = o if o is not None else make_opts()
    fn = lib.kos_gemm_rs_wt if w_transposed else lib.kos_gemm_rs
    check(fn(world, rank, m, k, n, _p(a), _p(w), peers, _p(partial), _p(y),
             ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def _need_scales(t: torch.Tensor, rows: int, k: int, what: str, host_ok: bool = False) -> None:
    """MX scales in the slab layout: uint8 [k/64, rows, 2]."""
    _need(t, torch.uint8, what, 3, (k // 64, rows, 2), host_ok=host_ok)


def ag_gemm_mx(a_local: torch.Tensor, a_local_scales: torch.Tensor,
               a_peers: Sequence[Optional[torch.Tensor]], a_peer_scales: Sequence[Optional[torch.Tensor]],
               w: torch.Tensor, w_scales: torch.Tensor, a_gathered: torch.Tensor,
               a_gathered_scales: torch.Tensor, c: torch.Tensor, rank: int, ws: Workspace,
               o: Optional[Opts] = None, stream=None) -> None:
    """kos_ag_gemm_mx: gathers E4M3 shards and their scales (uint8 codes;
    scales uint8 [k/64, rows, 2]); c = gathered . w^T with w E4M3 [n, k]."""
    world = len(a_peers)
    if len(a_peer_scales) != world:
        raise ValueError("a_peer_scales must have one entry per rank")
    _need(a_local, torch.uint8, "a_local", 2)
    m_local, k = a_local.shape
    _need_scales(a_local_scales, m_local, k, "a_local_scales")
    _need(w, torch.uint8, "w", 2, (None, k))
    n = w.shape[0]
    _need_scales(w_scales, n, k, "w_scales")
    _need(a_gathered, torch.uint8, "a_gathered", 2, (world * m_local, k))
    _need_scales(a_gathered_scales, world * m_local, k, "a_gathered_scales")
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("c must be bf16 or fp32")
    _need(c, c.dtype, "c", 2, (world * m_local, n))
    for p in range(world):
        if p != rank:
            _need(a_peers[p], torch.uint8, f"a_peers[{p}]", 2, (m_local, k), host_ok=True)
            _need_scales(a_peer_scales[p], m_local, k, f"a_peer_scales[{p}]", host_ok=True)
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(a_peers)])
    speers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(a_peer_scales)])
    o = o if o is not None else make_opts()
    check(lib.kos_ag_gemm_mx(world, rank, m_local, k, n, _p(a_local), _p(a_local_scales), peers, speers,
                             _p(w), _p(w_scales), _p(a_gathered), _p(a_gathered_scales), _p(c),
                             KOS_BF16 if c.dtype == torch.bfloat16 else KOS_F32,
                             ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def gemm_rs_mx(a: torch.Tensor, a_scales: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor,
               peer_slices: Sequence[Optional[torch.Tensor]], partial: torch.Tensor, y: torch.Tensor,
               rank: int, ws: Workspace, o: Optional[Opts] = None, stream=None) -> None:
    """kos_gemm_rs_mx: partial = a . w^T (E4M3 codes, slab-layout scales,
    fp32 result); y = reduce of chunk `rank`."""
    world = len(peer_slices)
    _need(a, torch.uint8, "a", 2)
    m, k = a.shape
    _need_scales(a_scales, m, k, "a_scales")
    _need(w, torch.uint8, "w", 2, (None, k))
    n = w.shape[0]
    _need_scales(w_scales, n, k, "w_scales")
    mc = m // world
    _need(partial, torch.float32, "partial", 2, (m, n))
    _need(y, torch.float32, "y", 2, (mc, n))
    for p, t in enumerate(peer_slices):
        if p != rank:
            _need(t, torch.float32, f"peer_slices[{p}]", 2, (mc, n), host_ok=True)
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(peer_slices)])
    o = o if o is not None else make_opts()
    check(lib.kos_gemm_rs_mx(world, rank, m, k, n, _p(a), _p(a_scales), _p(w), _p(w_scales), peers,
                             _p(partial), _p(y), ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def moe_shape(world, rank, tokens, hidden, experts, topk, ffn) -> MoeShape:
    return MoeShape(world, rank, tokens, hidden, experts, topk, ffn, 0)


def _check_tokens(s: MoeShape, topk_idx, topk_w, perm, counts):
    T, k, E = s.tokens, s.topk, s.experts
    if T > 0:
        _need(topk_idx, torch.int32, "topk_idx", 2, (T, k))
        _need(topk_w, torch.float32, "topk_w", 2, (T, k))
        _need(perm, torch.int32, "perm", 1, (T * k,))
    _need(counts, torch.int32, "counts", 1, (E,))


def moe_dispatch(s: MoeShape, x, logits, peer_send, peer_counts, topk_idx, topk_w, counts, perm,
                 out_send, x_grouped, grouped_offsets, row_src, ws: Workspace,
                 o: Optional[Opts] = None, stream=None) -> None:
    """kos_moe_dispatch (see include/kos.h for every buffer's layout).  Each
    out_send[d] buffer's row count is passed as its own capacity; the rows in
    peer_send[p] must cover what peer_counts says p sends."""
    T, H, E, R = s.tokens, s.hidden, s.experts, s.world
    E_loc = E // R
    if len(peer_send) != R or len(out_send) != R:
        raise ValueError("peer_send and out_send need one entry per rank")
    if T > 0:
        _need(x, torch.bfloat16, "x", 2, (T, H))
        _need(logits, torch.float32, "logits", 2, (T, E))
    _need(peer_counts, torch.int32, "peer_counts", 2, (R, E_loc))
    _check_tokens(s, topk_idx, topk_w, perm, counts)
    _need(x_grouped, torch.bfloat16, "x_grouped", 2, (None, H))
    cap = x_grouped.shape[0]
    _need(grouped_offsets, torch.int32, "grouped_offsets", 1, (E_loc + 1,))
    _need(row_src, torch.int32, "row_src", 2, (None, 2))
    _min_rows(row_src, cap, "row_src")
    for p in range(R):
        if p == s.rank:
            continue
        if peer_send[p] is not None:
            _need(peer_send[p], torch.bfloat16, f"peer_send[{p}]", 2, (None, H), host_ok=True)
        if out_send[p] is not None:
            _need(out_send[p], torch.bfloat16, f"out_send[{p}]", 2, (None, H))
    send = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(peer_send)])
    osend = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(out_send)])
    caps = (ctypes.c_int64 * R)(*[0 if p == s.rank or t is None else t.shape[0] for p, t in enumerate(out_send)])
    o = o if o is not None else make_opts()
    check(lib.kos_moe_dispatch(ctypes.byref(s), _p(x), _p(logits), send, _p(peer_counts),
                               _p(topk_idx), _p(topk_w), _p(counts), _p(perm), osend, caps,
                               _p(x_grouped), cap, _p(grouped_offsets), _p(row_src),
                               ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def moe_combine(s: MoeShape, x_grouped, grouped_offsets, row_src, w_gate, w_up, w_down,
                topk_idx, topk_w, counts, perm, peer_counts, peer_return, h, y_grouped,
                out_return, y, ws: Workspace, o: Optional[Opts] = None, stream=None, *,
                gate_save=None, up_save=None) -> None:
    """kos_moe_combine (see include/kos.h for every buffer's layout).  h and
    y_grouped must hold at least x_grouped's rows (the capacity); each
    out_return[p] must hold the rows p sent us, and peer_return[d] the rows
    we sent d.  gate_save / up_save (optional, together): bf16 [cap, F]
    outputs for moe_layer_bwd."""
    T, H, E, R, F = s.tokens, s.hidden, s.experts, s.world, s.ffn
    E_loc = E // R
    if len(peer_return) != R or len(out_return) != R:
        raise ValueError("peer_return and out_return need one entry per rank")
    _need(x_grouped, torch.bfloat16, "x_grouped", 2, (None, H))
    cap = x_grouped.shape[0]
    _need(grouped_offsets, torch.int32, "grouped_offsets", 1, (E_loc + 1,))
    _need(row_src, torch.int32, "row_src", 2, (None, 2))
    _min_rows(row_src, cap, "row_src")
    _need(w_gate, torch.bfloat16, "w_gate", 3, (E_loc, H, F))
    _need(w_up, torch.bfloat16, "w_up", 3, (E_loc, H, F))
    _need(w_down, torch.bfloat16, "w_down", 3, (E_loc, F, H))
    _check_tokens(s, topk_idx, topk_w, perm, counts)
    _need(peer_counts, torch.int32, "peer_counts", 2, (R, E_loc))
    _need(h, torch.bfloat16, "h", 2, (None, F))
    _min_rows(h, cap, "h")
    _need(y_grouped, torch.bfloat16, "y_grouped", 2, (None, H))
    _min_rows(y_grouped, cap, "y_grouped")
    _check_saved(gate_save, up_save, cap, F)
    if T > 0:
        _need(y, torch.bfloat16, "y", 2, (T, H))
    for p in range(R):
        if p == s.rank:
            continue
        if peer_return[p] is not None:
            _need(peer_return[p], torch.bfloat16, f"peer_return[{p}]", 2, (None, H), host_ok=True)
        if out_return[p] is not None:
            _need(out_return[p], torch.bfloat16, f"out_return[{p}]", 2, (None, H))
    pret = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(peer_return)])
    oret = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(out_return)])
    rcaps = (ctypes.c_int64 * R)(*[0 if p == s.rank or t is None else t.shape[0] for p, t in enumerate(out_return)])
    o = o if o is not None else make_opts()
    check(lib.kos_moe_combine(ctypes.byref(s), _p(x_grouped), _p(grouped_offsets), _p(row_src),
                              cap, _p(w_gate), _p(w_up), _p(w_down), _p(topk_idx),
                              _p(topk_w), _p(counts), _p(perm), _p(peer_counts), pret, _p(h),
                              _p(gate_save), _p(up_save), _p(y_grouped), oret, rcaps, _p(y),
                              ctypes.byref(o), ws.ptr, ws.nbytes,
                              _stream(stream)))


def moe_layer(s: MoeShape, x, logits, peer_send, peer_counts, w_gate, w_up, w_down, peer_return,
              topk_idx, topk_w, counts, perm, out_send, x_grouped, grouped_offsets, row_src, h, y_grouped,
              out_return, y, ws: Workspace, o: Optional[Opts] = None, stream=None, *,
              gate_save=None, up_save=None) -> None:
    """kos_moe_layer: the whole expert layer in one launch -- what moe_dispatch
    followed by moe_combine computes, with the same buffers (see include/kos.h)."""
    T, H, E, R, F = s.tokens, s.hidden, s.experts, s.world, s.ffn
    E_loc = E // R
    for name, lst in (("peer_send", peer_send), ("out_send", out_send), ("peer_return", peer_return),
                      ("out_return", out_return)):
        if len(lst) != R:
            raise ValueError(f"{name} needs one entry per rank")
    if T > 0:
        _need(x, torch.bfloat16, "x", 2, (T, H))
        _need(logits, torch.float32, "logits", 2, (T, E))
        _need(y, torch.bfloat16, "y", 2, (T, H))
    _need(peer_counts, torch.int32, "peer_counts", 2, (R, E_loc))
    _check_tokens(s, topk_idx, topk_w, perm, counts)
    _need(w_gate, torch.bfloat16, "w_gate", 3, (E_loc, H, F))
    _need(w_up, torch.bfloat16, "w_up", 3, (E_loc, H, F))
    _need(w_down, torch.bfloat16, "w_down", 3, (E_loc, F, H))
    _need(x_grouped, torch.bfloat16, "x_grouped", 2, (None, H))
    cap = x_grouped.shape[0]
    _need(grouped_offsets, torch.int32, "grouped_offsets", 1, (E_loc + 1,))
    _need(row_src, torch.int32, "row_src", 2, (None, 2))
    _min_rows(row_src, cap, "row_src")
    _need(h, torch.bfloat16, "h", 2, (None, F))
    _min_rows(h, cap, "h")
    _need(y_grouped, torch.bfloat16, "y_grouped", 2, (None, H))
    _min_rows(y_grouped, cap, "y_grouped")
    _check_saved(gate_save, up_save, cap, F)
    for p in range(R):
        if p == s.rank:
            continue
        for name, lst, host_ok in (("peer_send", peer_send, True), ("out_send", out_send, False),
                                   ("peer_return", peer_return, True), ("out_return", out_return, False)):
            if lst[p] is not None:
                _need(lst[p], torch.bfloat16, f"{name}[{p}]", 2, (None, H), host_ok=host_ok)
    arr = {n: ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(lst)])
           for n, lst in (("ps", peer_send), ("os", out_send), ("pr", peer_return), ("or", out_return))}
    scaps = (ctypes.c_int64 * R)(*[0 if p == s.rank or t is None else t.shape[0] for p, t in enumerate(out_send)])
    rcaps = (ctypes.c_int64 * R)(*[0 if p == s.rank or t is None else t.shape[0] for p, t in enumerate(out_return)])
    o = o if o is not None else make_opts()
    check(lib.kos_moe_layer(ctypes.byref(s), _p(x), _p(logits), arr["ps"], _p(peer_counts), _p(w_gate), _p(w_up),
                            _p(w_down), arr["pr"], _p(topk_idx), _p(topk_w), _p(counts), _p(perm), arr["os"], scaps,
                            _p(x_grouped), cap, _p(grouped_offsets), _p(row_src), _p(h), _p(gate_save),
                            _p(up_save), _p(y_grouped), arr["or"],
                            rcaps, _p(y), ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def moe_layer_bwd(s: MoeShape, dy, topk_idx, topk_w, perm, counts, peer_counts, x_grouped, grouped_offsets,
                  row_src, y_grouped, peer_return, w_gate, w_up, w_down, peer_send_grad, out_send_grad,
                  dres_grouped, dg, du, dh, dx_grouped, peer_return_grad, out_return_grad, dx, dlogits,
                  ws: Workspace, o: Optional[Opts] = None, stream=None, *,
                  gate_saved=None, up_saved=None) -> None:
    """kos_moe_layer_bwd: the expert layer's data and router gradients in one
    launch (see include/kos.h).  The forward's routing and grouped buffers
    come in unchanged; grouped_cap is x_grouped's row count, and each
    out_send_grad[d] / out_return_grad[p] buffer's row count is its
    capacity.  gate_saved / up_saved (optional, together): the forward's
    gate_save / up_save, used instead of recomputing g and u; dh may then be
    None."""
    T, H, E, R, F = s.tokens, s.hidden, s.experts, s.world, s.ffn
    E_loc = E // R
    for name, lst in (("peer_return", peer_return), ("peer_send_grad", peer_send_grad),
                      ("out_send_grad", out_send_grad), ("peer_return_grad", peer_return_grad),
                      ("out_return_grad", out_return_grad)):
        if len(lst) != R:
            raise ValueError(f"{name} needs one entry per rank")
    if T > 0:
        _need(dy, torch.bfloat16, "dy", 2, (T, H))
        _need(dx, torch.bfloat16, "dx", 2, (T, H))
        _need(dlogits, torch.float32, "dlogits", 2, (T, E))
    _need(peer_counts, torch.int32, "peer_counts", 2, (R, E_loc))
    _check_tokens(s, topk_idx, topk_w, perm, counts)
    _need(w_gate, torch.bfloat16, "w_gate", 3, (E_loc, H, F))
    _need(w_up, torch.bfloat16, "w_up", 3, (E_loc, H, F))
    _need(w_down, torch.bfloat16, "w_down", 3, (E_loc, F, H))
    _need(x_grouped, torch.bfloat16, "x_grouped", 2, (None, H))
    cap = x_grouped.shape[0]
    _need(grouped_offsets, torch.int32, "grouped_offsets", 1, (E_loc + 1,))
    _need(row_src, torch.int32, "row_src", 2, (None, 2))
    _min_rows(row_src, cap, "row_src")
    for name, t, width in (("y_grouped", y_grouped, H), ("dres_grouped", dres_grouped, H), ("dg", dg, F),
                           ("du", du, F), ("dx_grouped", dx_grouped, H)):
        _need(t, torch.bfloat16, name, 2, (None, width))
        _min_rows(t, cap, name)
    _check_saved(gate_saved, up_saved, cap, F)
    if dh is None and gate_saved is None:
        raise ValueError("dh is needed unless the saved gate and up activations are given")
    if dh is not None:
        _need(dh, torch.float32, "dh", 2, (None, F))
        _min_rows(dh, cap, "dh")
    lists = (("peer_return", peer_return, True), ("peer_send_grad", peer_send_grad, True),
             ("out_send_grad", out_send_grad, False), ("peer_return_grad", peer_return_grad, True),
             ("out_return_grad", out_return_grad, False))
    for p in range(R):
        if p == s.rank:
            continue
        for name, lst, host_ok in lists:
            if lst[p] is not None:
                _need(lst[p], torch.bfloat16, f"{name}[{p}]", 2, (None, H), host_ok=host_ok)
    arr = {n: ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(lst)]) for n, lst, _ in lists}
    scaps = (ctypes.c_int64 * R)(*[0 if p == s.rank or t is None else t.shape[0] for p, t in enumerate(out_send_grad)])
    rcaps = (ctypes.c_int64 * R)(*[0 if p == s.rank or t is None else t.shape[0]
                                   for p, t in enumerate(out_return_grad)])
    o = o if o is not None else make_opts()
    check(lib.kos_moe_layer_bwd(ctypes.byref(s), _p(dy), _p(topk_idx), _p(topk_w), _p(perm), _p(counts),
                                _p(peer_counts), _p(x_grouped), cap, _p(grouped_offsets), _p(row_src), _p(y_grouped),
                                arr["peer_return"], _p(w_gate), _p(w_up), _p(w_down), _p(gate_saved),
                                _p(up_saved), arr["peer_send_grad"],
                                arr["out_send_grad"], scaps, _p(dres_grouped), _p(dg), _p(du), _p(dh), _p(dx_grouped),
                                arr["peer_return_grad"], arr["out_return_grad"], rcaps, _p(dx), _p(dlogits),
                                ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))
