"""torch-tensor front end of the C ABI (argument marshalling only)."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from ._binding import KOS_BF16, KOS_F32, KosError, MoeShape, Opts, check, lib, opts as make_opts, ptr_array


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str, ndim: int):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {ndim}-d tensor")


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
        """Synchronizes and raises KosError if a device-side error was recorded."""
        check(lib.kos_workspace_status(self.ptr, _stream(stream)))

    def trace(self, grid: int, stream=None):
        """Timeline of the last call made with ``opts(trace=True)`` on a grid of
        `grid` workgroups: a list, per workgroup, of (ticket, t_begin, t_end,
        [(kind, entry, t0, t1), ...]) with times in microseconds from the
        earliest workgroup start (kos_workspace_trace).  ``self.trace_xcd``
        then holds each workgroup's XCD and ``self.trace_clock_mhz`` the
        shader clock it ran at (its clock record)."""
        from ._binding import TRACE_CLOCK, TRACE_KINDS, TRACE_MAX_WG, TRACE_RECORDS, TraceRec
        if not 0 < grid <= TRACE_MAX_WG:
            raise ValueError(f"grid {grid} outside [1, {TRACE_MAX_WG}]")
        n = grid * TRACE_RECORDS
        buf = (TraceRec * n)()
        check(lib.kos_workspace_trace(self.ptr, ctypes.cast(buf, ctypes.c_void_p), n, _stream(stream)))
        tick_us = 0.01                      # 100 MHz constant-rate counter
        heads = [buf[g * TRACE_RECORDS] for g in range(grid)]
        t_ref = min(h.t0 for h in heads)
        out = []
        self.trace_xcd = [(h.tag >> 12) & 15 for h in heads]
        self.trace_clock_mhz = []
        for g, h in enumerate(heads):
            clk = buf[g * TRACE_RECORDS + 1]
            if clk.tag >> 24 != TRACE_CLOCK:
                raise KosError(f"workgroup {g}: record 1 is not a clock record")
            self.trace_clock_mhz.append(100.0 * clk.t0 / clk.dt if clk.dt else 0.0)
            used = h.tag & 0xFFF
            recs = []
            for i in range(2, min(used, TRACE_RECORDS)):
                r = buf[g * TRACE_RECORDS + i]
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
    _need(w, torch.bfloat16, "w", 2)
    _need(a_gathered, torch.bfloat16, "a_gathered", 2)
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("c must be bf16 or fp32")
    _need(c, c.dtype, "c", 2)
    for p, t in enumerate(a_peers):
        if p != rank:
            _need(t, torch.bfloat16, f"a_peers[{p}]", 2)
    m_local, k = a_local.shape
    n = w.shape[0] if w_transposed else w.shape[1]
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(a_peers)])
    o = o if o is not None else make_opts()
    fn = lib.kos_ag_gemm_wt if w_transposed else lib.kos_ag_gemm
    check(fn(world, rank, m_local, k, n, _p(a_local), peers, _p(w), _p(a_gathered),
             _p(c), KOS_BF16 if c.dtype == torch.bfloat16 else KOS_F32,
             ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def gemm_rs(a: torch.Tensor, w: torch.Tensor, peer_slices: Sequence[Optional[torch.Tensor]],
            partial: torch.Tensor, y: torch.Tensor, rank: int, ws: Workspace,
            o: Optional[Opts] = None, stream=None, w_transposed: bool = False) -> None:
    """kos_gemm_rs: partial = a @ w (fp32, w [k, n]); y = reduce of chunk
    `rank`.  w_transposed (kos_gemm_rs_wt): w is W^T [n, k], partial = a @ w.T."""
    world = len(peer_slices)
    _need(a, torch.bfloat16, "a", 2)
    _need(w, torch.bfloat16, "w", 2)
    _need(partial, torch.float32, "partial", 2)
    _need(y, torch.float32, "y", 2)
    for p, t in enumerate(peer_slices):
        if p != rank:
            _need(t, torch.float32, f"peer_slices[{p}]", 2)
    m, k = a.shape
    n = w.shape[0] if w_transposed else w.shape[1]
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(peer_slices)])
    o = o if o is not None else make_opts()
    fn = lib.kos_gemm_rs_wt if w_transposed else lib.kos_gemm_rs
    check(fn(world, rank, m, k, n, _p(a), _p(w), peers, _p(partial), _p(y),
             ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def _need_scales(t: torch.Tensor, rows: int, k: int, what: str) -> None:
    """MX scales in the slab layout: uint8 [k/64, rows, 2]."""
    _need(t, torch.uint8, what, 3)
    if tuple(t.shape) != (k // 64, rows, 2):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {(k // 64, rows, 2)}")


def ag_gemm_mx(a_local: torch.Tensor, a_local_scales: torch.Tensor,
               a_peers: Sequence[Optional[torch.Tensor]], a_peer_scales: Sequence[Optional[torch.Tensor]],
               w: torch.Tensor, w_scales: torch.Tensor, a_gathered: torch.Tensor,
               a_gathered_scales: torch.Tensor, c: torch.Tensor, rank: int, ws: Workspace,
               o: Optional[Opts] = None, stream=None) -> None:
    """kos_ag_gemm_mx: gathers E4M3 shards and their scales (uint8 codes;
    scales uint8 [k/64, rows, 2]); c = gathered . w^T with w E4M3 [n, k]."""
    world = len(a_peers)
    _need(a_local, torch.uint8, "a_local", 2)
    m_local, k = a_local.shape
    _need_scales(a_local_scales, m_local, k, "a_local_scales")
    _need(w, torch.uint8, "w", 2)
    n = w.shape[0]
    _need_scales(w_scales, n, k, "w_scales")
    _need(a_gathered, torch.uint8, "a_gathered", 2)
    _need_scales(a_gathered_scales, world * m_local, k, "a_gathered_scales")
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("c must be bf16 or fp32")
    _need(c, c.dtype, "c", 2)
    for p in range(world):
        if p != rank:
            _need(a_peers[p], torch.uint8, f"a_peers[{p}]", 2)
            _need_scales(a_peer_scales[p], m_local, k, f"a_peer_scales[{p}]")
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
    _need(w, torch.uint8, "w", 2)
    n = w.shape[0]
    _need_scales(w_scales, n, k, "w_scales")
    _need(partial, torch.float32, "partial", 2)
    _need(y, torch.float32, "y", 2)
    for p, t in enumerate(peer_slices):
        if p != rank:
            _need(t, torch.float32, f"peer_slices[{p}]", 2)
    peers = ptr_array([None if p == rank else _p(t) for p, t in enumerate(peer_slices)])
    o = o if o is not None else make_opts()
    check(lib.kos_gemm_rs_mx(world, rank, m, k, n, _p(a), _p(a_scales), _p(w), _p(w_scales), peers,
                             _p(partial), _p(y), ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def moe_shape(world, rank, tokens, hidden, experts, topk, ffn) -> MoeShape:
    return MoeShape(world, rank, tokens, hidden, experts, topk, ffn, 0)


def moe_dispatch(s: MoeShape, x, logits, peer_send, peer_counts, topk_idx, topk_w, counts, perm,
                 out_send, x_grouped, grouped_offsets, row_src, ws: Workspace,
                 o: Optional[Opts] = None, stream=None) -> None:
    """kos_moe_dispatch (see include/kos.h for every buffer's layout)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(logits, torch.float32, "logits", 2)
    _need(peer_counts, torch.int32, "peer_counts", 2)
    _need(x_grouped, torch.bfloat16, "x_grouped", 2)
    send = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(peer_send)])
    osend = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(out_send)])
    send_cap = max((t.shape[0] for p, t in enumerate(out_send) if p != s.rank), default=0)
    o = o if o is not None else make_opts()
    check(lib.kos_moe_dispatch(ctypes.byref(s), _p(x), _p(logits), send, _p(peer_counts),
                               _p(topk_idx), _p(topk_w), _p(counts), _p(perm), osend, send_cap,
                               _p(x_grouped), x_grouped.shape[0], _p(grouped_offsets), _p(row_src),
                               ctypes.byref(o), ws.ptr, ws.nbytes, _stream(stream)))


def moe_combine(s: MoeShape, x_grouped, grouped_offsets, row_src, w_gate, w_up, w_down,
                topk_idx, topk_w, counts, perm, peer_counts, peer_return, h, y_grouped,
                out_return, y, ws: Workspace, o: Optional[Opts] = None, stream=None) -> None:
    """kos_moe_combine (see include/kos.h for every buffer's layout)."""
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, torch.bfloat16, name, 3)
    _need(h, torch.bfloat16, "h", 2)
    _need(y_grouped, torch.bfloat16, "y_grouped", 2)
    _need(y, torch.bfloat16, "y", 2)
    pret = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(peer_return)])
    oret = ptr_array([None if p == s.rank else _p(t) for p, t in enumerate(out_return)])
    o = o if o is not None else make_opts()
    check(lib.kos_moe_combine(ctypes.byref(s), _p(x_grouped), _p(grouped_offsets), _p(row_src),
                              x_grouped.shape[0], _p(w_gate), _p(w_up), _p(w_down), _p(topk_idx),
                              _p(topk_w), _p(counts), _p(perm), _p(peer_counts), pret, _p(h),
                              _p(y_grouped), oret, _p(y), ctypes.byref(o), ws.ptr, ws.nbytes,
                              _stream(stream)))
