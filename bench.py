#!/usr/bin/env python
"""Benchmark of the fused GEMM+collective persistent kernels on one MI355X.

One step = one pass of the whole hot path on one rank's share of an
8-rank job, peers emulated in HBM:
  1. all-gather + GEMM   (QKV column-parallel: 8 x 512x8192 shards, W 8192x3072)
  2. GEMM + reduce-scatter (MLP down: A 4096x3584, W 3584x8192 -> 512x8192 chunk)
  3. expert layer, DeepSeek-V3 shape (4096 tokens, H 7168, 256 experts top-8,
     32 local SwiGLU experts 7168->2048->7168): dispatch, then combine.
Each op is one persistent launch (fused mode).  `value` is the step's
algorithmic GEMM FLOPs (AG + RS + expert FFN) / step time, in TFLOP/s; the
MoE layer's tokens/s and each op's own TFLOP/s are reported beside it.

Also reported: the same-GPU baselines (unfused launches, best fixed crew),
the GEMM's throughput with 224 of the 256 compute units building, the roofline of the
dominant kernel, and the CPU oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused GEMM+collective TFLOP/s (% bf16 MFMA peak); MoE layer tokens/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 / MXFP8 MFMA, published
PEAK_CLOCK_MHZ = 2400.0        # MI355X peak engine clock (the published peaks assume it)


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def build_moe_inputs(torch, KI, s, rank=0):
    """One rank's expert-layer inputs (seeded) and output buffers, resident on
    the GPU: the send buffers hold every row a rank can send one peer, the
    grouped buffers every row this rank can receive."""
    dev = "cuda"
    m = KI.moe_inputs(s, rank, dev)
    pc = m["peer_counts"].cpu()
    cap = int(pc.sum()) + s.tokens * min(s.topk, s.e_local)
    m.update(
        idx=torch.empty((s.tokens, s.topk), dtype=torch.int32, device=dev),
        w=torch.empty((s.tokens, s.topk), dtype=torch.float32, device=dev),
        counts=torch.empty((s.experts,), dtype=torch.int32, device=dev),
        perm=torch.empty((s.tokens * s.topk,), dtype=torch.int32, device=dev),
        send=[None if p == rank else torch.empty((s.peer_cap, s.hidden), dtype=torch.bfloat16, device=dev)
              for p in range(s.world)],
        grouped=torch.empty((cap, s.hidden), dtype=torch.bfloat16, device=dev),
        goff=torch.empty((s.e_local + 1,), dtype=torch.int32, device=dev),
        row_src=torch.empty((cap, 2), dtype=torch.int32, device=dev),
        h=torch.empty((cap, s.ffn), dtype=torch.bfloat16, device=dev),
        yg=torch.empty((cap, s.hidden), dtype=torch.bfloat16, device=dev),
        y=torch.empty((s.tokens, s.hidden), dtype=torch.bfloat16, device=dev),
        ret=[None if p == rank else torch.empty((max(int(pc[p].sum()), 1), s.hidden), dtype=torch.bfloat16,
                                                device=dev) for p in range(s.world)],
    )
    return m


def build_inputs(torch, KI, kos, moe_shape):
    dev = "cuda"
    inp = {}
    ag = KI.ag_inputs(KI.AG_QKV, 0, dev)
    s = KI.AG_QKV
    ag["g"] = torch.empty((s.m, s.k), dtype=torch.bfloat16, device=dev)
    ag["c"] = torch.empty((s.m, s.n), dtype=torch.bfloat16, device=dev)
    inp["ag"] = ag
    rs = KI.rs_inputs(KI.RS_MLP, 7, dev)
    s = KI.RS_MLP
    rs["partial"] = torch.empty((s.m, s.n), dtype=torch.float32, device=dev)
    rs["y"] = torch.empty((s.m_chunk, s.n), dtype=torch.float32, device=dev)
    inp["rs"] = rs
    inp["moe"] = build_moe_inputs(torch, KI, moe_shape)
    return inp


def make_ops(kos, KI, inp, ws, moe_shape, mode=0, n_movers=-1, grid=0, trace=False, rank_moe=0, policy=0):
    """The step's ops as closures over resident inputs (the AG and RS ones
    only when `inp` holds their inputs).  FIXED mode runs the dispatch fused:
    it has no compute role to split a crew from."""
    from gemm_collective_persistent_amd.api import moe_shape as mk_shape
    o = kos.opts(mode=mode, n_movers=n_movers, grid=grid, trace=trace, policy=policy)
    ag, rs, m = inp.get("ag"), inp.get("rs"), inp["moe"]
    s = moe_shape
    shp = mk_shape(s.world, rank_moe, s.tokens, s.hidden, s.experts, s.topk, s.ffn)

    def op_ag():
        kos.ag_gemm(ag["a_local"], ag["a_peers"], ag["w"], ag["g"], ag["c"], 0, ws, o)

    def op_rs():
        kos.gemm_rs(rs["a"], rs["w"], rs["peer_slices"], rs["partial"], rs["y"], 7, ws, o)

    def op_dispatch():
        od = o if mode != 1 else kos.opts(mode=0, grid=grid, trace=trace)
        kos.moe_dispatch(shp, m["x"], m["logits"], m["peer_send"], m["peer_counts"], m["idx"], m["w"],
                         m["counts"], m["perm"], m["send"], m["grouped"], m["goff"], m["row_src"], ws, od)

    def op_combine():
        kos.moe_combine(shp, m["grouped"], m["goff"], m["row_src"], m["wg"], m["wu"], m["wd"], m["idx"], m["w"],
                        m["counts"], m["perm"], m["peer_counts"], m["peer_return"], m["h"], m["yg"], m["ret"],
                        m["y"], ws, o)

    ops = [("moe_dispatch", op_dispatch), ("moe_combine", op_combine)]
    if rs is not None:
        ops.insert(0, ("gemm_rs", op_rs))
    if ag is not None:
        ops.insert(0, ("ag_gemm", op_ag))
    return ops


def moe_block(torch, kos, KI, ws, flush, reps, shape, rank=0):
    """A whole expert layer (dispatch, then combine) of one rank on its own:
    fused times, tokens/s and the combine's TFLOP/s, the same-GPU baselines
    (unfused; the combine's FIXED crew sweep, the planned crew included), and
    per mode the idle-CU fraction and the communication-phase rates."""
    m = build_moe_inputs(torch, KI, shape, rank)
    inp = {"moe": m}
    names = ["moe_dispatch", "moe_combine"]
    ops = make_ops(kos, KI, inp, ws, shape, rank_moe=rank)
    for _ in range(2):
        for _, fn in ops:
            fn()
    ws.status()
    per, _ = time_ops(torch, ops, reps, ws, flush)
    rows = int(m["goff"][-1].item())
    fl = rows * shape.flops_per_row
    ops_u = make_ops(kos, KI, inp, ws, shape, mode=2, rank_moe=rank)
    for _, fn in ops_u:
        fn()
    pu, _ = time_ops(torch, ops_u, reps, ws, flush)
    grid = int(kos.lib.kos_device_cu_count())
    planned = planned_crews(KI, shape, rows, grid)["moe_combine"]
    make_ops(kos, KI, inp, ws, shape, rank_moe=rank)[0][1]()   # dispatch outputs for the combine runs
    sweep = crew_sweep_moe(torch, kos, KI, inp, ws, shape, flush, reps, planned, rank)
    best = min(sweep, key=sweep.get)
    peer_rows = int(m["peer_counts"].sum().item())
    pb = phase_bytes(KI, shape, rows, peer_rows)
    idle, rates = idle_fractions(torch, kos, KI, inp, ws, shape, flush, {"moe_combine": best}, pb, names,
                                 rank_moe=rank)
    t_layer = per[0] + per[1]
    one = single_launch(torch, kos, KI, m, ws, flush, reps, shape, t_layer, rank)
    bwd = moe_backward(torch, kos, KI, m, ws, flush, reps, shape, one["ms"], rank)
    return {
        "single_launch": one, "backward": bwd,
        "workload": shape.name, "rank": rank, "grouped_rows": rows,
        "ms": {"moe_dispatch": round(per[0], 4), "moe_combine": round(per[1], 4), "layer": round(t_layer, 4)},
        "tokens_per_s": round(shape.tokens / (t_layer * 1e-3), 1),
        "combine_tflops": round(fl / (per[1] * 1e-3) / 1e12, 1),
        "combine_pct_bf16_peak": round(100 * fl / (per[1] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
        "unfused_ms": {"moe_dispatch": round(pu[0], 4), "moe_combine": round(pu[1], 4)},
        "speedup_vs_unfused": {"moe_dispatch": round(pu[0] / per[0], 3), "moe_combine": round(pu[1] / per[1], 3),
                               "layer": round((pu[0] + pu[1]) / t_layer, 3)},
        "combine_fixed_crew_sweep_ms": {str(c): t for c, t in sweep.items()},
        "combine_best_fixed": {"crew": best, "ms": sweep[best], "speedup": round(sweep[best] / per[1], 3)},
        "combine_planned_split": {"crew": planned, "ms": sweep[planned], "speedup": round(sweep[planned] / per[1], 3)},
        "idle_cu_fraction": idle,
        "phase_rate_gb_s": {lab: {n: {k: v["gb_s"] for k, v in d.items()} for n, d in r.items()}
                            for lab, r in rates.items()},
    }


def crew_sweep_moe(torch, kos, KI, inp, ws, shape, flush, reps, planned, rank):
    """The combine's FIXED crew over CREW_SWEEP and the planned crew."""
    out = {}
    for c in sorted(set(CREW_SWEEP) | {planned}):
        fn = dict(make_ops(kos, KI, inp, ws, shape, mode=1, n_movers=c, rank_moe=rank))["moe_combine"]
        fn()
        out[c] = round(time_ops(torch, [("moe_combine", fn)], reps, ws, flush)[0][0], 4)
    return out


def layer_op(kos, m, ws, shape, rank=0, trace=False, save=False):
    """The whole expert layer in one launch (kos_moe_layer) on resident inputs
    (save: also keeping bf16 g and u in m["gs"], m["us"])."""
    from gemm_collective_persistent_amd.api import moe_shape as mk_shape
    shp = mk_shape(shape.world, rank, shape.tokens, shape.hidden, shape.experts, shape.topk, shape.ffn)
    o = kos.opts(trace=trace)
    kw = dict(gate_save=m["gs"], up_save=m["us"]) if save else {}
    return lambda: kos.moe_layer(shp, m["x"], m["logits"], m["peer_send"], m["peer_counts"], m["wg"], m["wu"],
                                 m["wd"], m["peer_return"], m["idx"], m["w"], m["counts"], m["perm"], m["send"],
                                 m["grouped"], m["goff"], m["row_src"], m["h"], m["yg"], m["ret"], m["y"], ws, o,
                                 **kw)


def single_launch(torch, kos, KI, m, ws, flush, reps, shape, two_ms, rank=0, baseline=True):
    """The expert layer in one launch, router to fold (kos_moe_layer), against
    the two launches (dispatch, then combine) on the same inputs, and (with
    `baseline`) against the same forward composed of PyTorch operations."""
    fn = layer_op(kos, m, ws, shape, rank)
    fn()
    t = time_ops(torch, [("moe_layer", fn)], reps, ws, flush)[0][0]
    d = {"ms": round(t, 4), "two_launch_ms": round(two_ms, 4), "speedup_vs_two_launch": round(two_ms / t, 3),
         "tokens_per_s": round(shape.tokens / (t * 1e-3), 1)}
    if baseline:
        fn()
        ws.status()
        run, out = torch_fwd_baseline(torch, m, shape, rank)
        run()
        torch.cuda.synchronize()
        tb = time_ops(torch, [("torch_fwd", run)], reps, ws, flush)[0][0]
        d["torch_composed"] = {"ms": round(tb, 4), "speedup_two_launch": round(tb / two_ms, 3),
                               "speedup_one_launch": round(tb / t, 3),
                               "y_rel_diff": float(f"{_rel(out['y'], m['y']):.3g}")}
    return d


def build_moe_grad(torch, KI, shape, m, rank=0):
    """The backward's inputs (seeded: dy, the gradients peers send us and the
    data gradients they return) and its output buffers, resident."""
    dev = "cuda"
    g = KI.moe_grad_inputs(shape, rank, dev)
    cap = m["grouped"].shape[0]
    H, F, T, E = shape.hidden, shape.ffn, shape.tokens, shape.experts
    pc = m["peer_counts"].cpu()
    g.update(
        send=[None if p == rank else torch.empty((shape.peer_cap, H), dtype=torch.bfloat16, device=dev)
              for p in range(shape.world)],
        dres=torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
        dg=torch.empty((cap, F), dtype=torch.bfloat16, device=dev),
        du=torch.empty((cap, F), dtype=torch.bfloat16, device=dev),
        dh=torch.empty((cap, F), dtype=torch.float32, device=dev),
        dxg=torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
        ret=[None if p == rank else torch.empty((max(int(pc[p].sum()), 1), H), dtype=torch.bfloat16, device=dev)
             for p in range(shape.world)],
        dx=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        dl=torch.empty((T, E), dtype=torch.float32, device=dev))
    return g


def bwd_op(kos, m, g, ws, shape, rank=0, trace=False, saved=False):
    """The expert layer's backward in one launch (kos_moe_layer_bwd), reading
    the forward's buffers in `m` (kept from a forward call; saved: with the
    g and u it kept, and no dH written)."""
    from gemm_collective_persistent_amd.api import moe_shape as mk_shape
    shp = mk_shape(shape.world, rank, shape.tokens, shape.hidden, shape.experts, shape.topk, shape.ffn)
    o = kos.opts(trace=trace)
    kw = dict(gate_saved=m["gs"], up_saved=m["us"]) if saved else {}
    return lambda: kos.moe_layer_bwd(shp, g["dy"], m["idx"], m["w"], m["perm"], m["counts"], m["peer_counts"],
                                     m["grouped"], m["goff"], m["row_src"], m["yg"], m["peer_return"], m["wg"],
                                     m["wu"], m["wd"], g["peer_send_grad"], g["send"], g["dres"], g["dg"], g["du"],
                                     None if saved else g["dh"], g["dxg"], g["peer_return_grad"], g["ret"], g["dx"],
                                     g["dl"], ws, o, **kw)


def _rel(a, b):
    """||a - b|| / ||b|| in fp32."""
    a, b = a.float(), b.float()
    return float((a - b).norm() / b.norm().clamp_min(1e-30))


def _moe_maps(torch, m, shape, rank=0):
    """Index maps of one forward's routing, for the PyTorch-composed
    baselines (built once, untimed): grouped row -> row of cat(our own local
    pairs' rows in packed order, each peer's rows); the rows to push back per
    peer; every pair -> its local grouped row or (rank, row) of what that rank
    returns."""
    import numpy as np
    T, k, E, H, R = shape.tokens, shape.topk, shape.experts, shape.hidden, shape.world
    el = shape.e_local
    dev = m["grouped"].device
    idx = m["idx"].long()
    perm = m["perm"].long()
    counts = m["counts"].cpu().numpy().astype(np.int64)
    off = np.concatenate([[0], np.cumsum(counts)])
    so = [int(off[d * el]) for d in range(R + 1)]
    go = m["goff"].cpu().numpy().astype(np.int64)
    rs = m["row_src"][:int(go[-1])].cpu().numpy().astype(np.int64)
    pc = m["peer_counts"].cpu().numpy().astype(np.int64)
    # grouped row -> row of cat(our own local pairs' rows, each peer's rows)
    base = {rank: 0}
    acc = so[rank + 1] - so[rank]
    for p in range(R):
        if p != rank:
            base[p] = acc
            acc += int(pc[p].sum())
    gidx = torch.as_tensor(np.array([base[p] + i for p, i in rs], dtype=np.int64), device=dev)
    push = {p: (torch.as_tensor(np.where(rs[:, 0] == p)[0], device=dev),
                torch.as_tensor(rs[rs[:, 0] == p, 1], device=dev)) for p in range(R) if p != rank}
    # every pair (t, j) -> local grouped row, or (rank d, row)
    perm_np = m["perm"].cpu().numpy().astype(np.int64)
    idx_np = m["idx"].cpu().numpy().astype(np.int64).reshape(-1)
    dst = idx_np // el
    before = pc[:rank].sum(axis=0)
    loc = np.where(dst == rank)[0]
    e_l = idx_np[loc] - rank * el
    loc_rows = go[e_l] + before[e_l] + (perm_np[loc] - off[idx_np[loc]])
    pairs_loc = (torch.as_tensor(loc, device=dev), torch.as_tensor(loc_rows, device=dev))
    pairs_rem = {}
    for d in range(R):
        sel = np.where(dst == d)[0]
        if d != rank and sel.size:
            pairs_rem[d] = (torch.as_tensor(sel, device=dev), torch.as_tensor(perm_np[sel] - so[d], device=dev))
    bounds = [(int(go[e]), int(go[e + 1])) for e in range(el)]
    return dict(idx=idx, perm=perm, so=so, gidx=gidx, push=push, pairs_loc=pairs_loc, pairs_rem=pairs_rem,
                bounds=bounds)


def torch_fwd_baseline(torch, m, shape, rank=0):
    """The same forward (router to fold) composed of PyTorch operations on
    the same GPU (hipBLASLt GEMMs per expert, elementwise and indexing
    kernels): a same-GPU library baseline.  The routing (top-k and softmax)
    is computed in the timed closure; the index maps of the permutation are
    built once, untimed, from the routing the kernels produced (the same
    routing, top-k being deterministic on these logits).  Returns the closure
    and a dict that receives y."""
    T, k, H, R = shape.tokens, shape.topk, shape.hidden, shape.world
    mp = _moe_maps(torch, m, shape, rank)
    perm, so, gidx = mp["perm"], mp["so"], mp["gidx"]
    push, pairs_loc, pairs_rem, bounds = mp["push"], mp["pairs_loc"], mp["pairs_rem"], mp["bounds"]
    dev = m["grouped"].device
    wg, wu, wd, x = m["wg"], m["wu"], m["wd"], m["x"]
    rows = int(m["goff"][-1].item())
    yg = torch.empty((max(rows, 1), H), dtype=torch.bfloat16, device=dev)
    packed = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    res = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    send = {d: torch.empty((max(so[d + 1] - so[d], 1), H), dtype=torch.bfloat16, device=dev)
            for d in range(R) if d != rank}
    ret = {p: torch.empty((max(int(r.numel()), 1), H), dtype=torch.bfloat16, device=dev) for p, (r, _) in push.items()}
    pair_tok = torch.arange(T * k, device=dev) // k
    out = {}

    def run():
        vals = torch.topk(m["logits"], k, dim=1).values
        w = torch.softmax(vals, dim=1)
        # every pair's row in packed (expert-major) order, sent or kept
        packed[perm] = x[pair_tok]
        for d in send:
            if so[d + 1] > so[d]:
                send[d][:so[d + 1] - so[d]].copy_(packed[so[d]:so[d + 1]])
        src = torch.cat([packed[so[rank]:so[rank + 1]]] + [m["peer_send"][p] for p in range(R) if p != rank])
        xg = src[gidx]
        for e, (lo, hi) in enumerate(bounds):
            if hi == lo:
                continue
            xe = xg[lo:hi]
            h = (torch.nn.functional.silu((xe @ wg[e]).float()) * (xe @ wu[e]).float()).to(torch.bfloat16)
            torch.matmul(h, wd[e], out=yg[lo:hi])
        for p, (rws, dst_rows) in push.items():
            ret[p].index_copy_(0, dst_rows, yg[rws])
        # per token: the weighted sum of its pairs' results
        res[pairs_loc[0]] = yg[pairs_loc[1]]
        for d, (sel, rws) in pairs_rem.items():
            res[sel] = m["peer_return"][d][rws]
        out["y"] = (res.view(T, k, H).float() * w[:, :, None]).sum(1).to(torch.bfloat16)

    return run, out


def torch_bwd_baseline(torch, m, g, shape, rank=0, saved=False):
    """The same backward composed of PyTorch operations on the same GPU
    (hipBLASLt GEMMs per expert, elementwise and indexing kernels): a
    same-GPU library baseline.  Index maps are built once, untimed, from the
    forward's routing; the returned closure computes dx and dlogits (and the
    rows sent and returned) from the resident inputs.  saved: g and u are the
    forward's kept copies (m["gs"], m["us"]) rather than two more GEMMs."""
    T, k, E, H, R = shape.tokens, shape.topk, shape.experts, shape.hidden, shape.world
    mp = _moe_maps(torch, m, shape, rank)
    idx, perm, so, gidx = mp["idx"], mp["perm"], mp["so"], mp["gidx"]
    push, pairs_loc, pairs_rem, bounds = mp["push"], mp["pairs_loc"], mp["pairs_rem"], mp["bounds"]
    dev = m["grouped"].device
    wg, wu, wd = m["wg"], m["wu"], m["wd"]
    dy, w = g["dy"], m["w"]
    xg, yg = m["grouped"], m["yg"]
    dxg, dxp = g["dxg"], torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    res = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    packed = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    out = {}

    def run():
        # the pairs' gradients in packed order, sent and grouped
        packed[perm] = (w.reshape(-1, 1) * dy.float().repeat_interleave(k, 0)).to(torch.bfloat16)
        for d in range(R):
            if d != rank and so[d + 1] > so[d]:
                g["send"][d][:so[d + 1] - so[d]].copy_(packed[so[d]:so[d + 1]])
        src = torch.cat([packed[so[rank]:so[rank + 1]]] + [g["peer_send_grad"][p] for p in range(R) if p != rank])
        dres = src[gidx]
        for e, (lo, hi) in enumerate(bounds):
            if hi == lo:
                continue
            if saved:
                gg, uu = m["gs"][lo:hi].float(), m["us"][lo:hi].float()
            else:
                x = xg[lo:hi]
                gg = (x @ wg[e]).float()
                uu = (x @ wu[e]).float()
            dh = (dres[lo:hi] @ wd[e].t()).float()
            sg = torch.sigmoid(gg)
            du = (dh * gg * sg).to(torch.bfloat16)
            dgr = (dh * uu * sg * (1 + gg * (1 - sg))).to(torch.bfloat16)
            torch.matmul(dgr, wg[e].t(), out=dxg[lo:hi])
            dxg[lo:hi].addmm_(du, wu[e].t())
        for p, (rows, dst_rows) in push.items():
            g["ret"][p].index_copy_(0, dst_rows, dxg[rows])
        # per token: the sum of its pairs' gradients and the router gradient
        dxp[pairs_loc[0]] = dxg[pairs_loc[1]]
        res[pairs_loc[0]] = yg[pairs_loc[1]]
        for d, (sel, rows) in pairs_rem.items():
            dxp[sel] = g["peer_return_grad"][d][rows]
            res[sel] = m["peer_return"][d][rows]
        out["dx"] = dxp.view(T, k, H).float().sum(1).to(torch.bfloat16)
        dw = (res.view(T, k, H).float() * dy.float()[:, None, :]).sum(-1)
        gl = w * (dw - (w * dw).sum(1, keepdim=True))
        out["dl"] = torch.zeros((T, E), dtype=torch.float32, device=dev).scatter_(1, idx, gl)

    return run, out


def moe_backward(torch, kos, KI, m, ws, flush, reps, shape, fwd_ms, rank=0, baseline=True):
    """The expert layer's backward direction in one launch on the forward's
    buffers: time, executed and algorithmic TFLOP/s, the clock it ran at,
    the idle-CU fraction, tokens/s of forward + backward, and the
    PyTorch-composed baseline on the same inputs (with how closely its dx
    and router gradient agree with the kernel's)."""
    from gemm_collective_persistent_amd.timeline import summarize
    g = build_moe_grad(torch, KI, shape, m, rank)
    fn = bwd_op(kos, m, g, ws, shape, rank)
    fn()
    ws.status()
    t = time_ops(torch, [("moe_layer_bwd", fn)], reps, ws, flush)[0][0]
    rows = int(m["goff"][-1].item())
    fl_exec = rows * 10.0 * shape.hidden * shape.ffn   # g, u recomputed; dH; dX
    fl_alg = rows * 6.0 * shape.hidden * shape.ffn     # dH; dX
    grid = int(kos.lib.kos_device_cu_count())
    tl = traced_call(kos, ws, bwd_op(kos, m, g, ws, shape, rank, trace=True), grid, 1, flush)
    clk = sum(ws.trace_clock_mhz) / len(ws.trace_clock_mhz)
    summ = summarize(tl, workgroups=grid)
    tf = fl_exec / (t * 1e-3) / 1e12
    d = {"workload": shape.name, "rank": rank, "grouped_rows": rows, "ms": round(t, 4),
         "tflops_executed": round(tf, 1), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1),
         "tflops_algorithmic_no_recompute": round(fl_alg / (t * 1e-3) / 1e12, 1),
         "clock_mhz": round(clk, 1), "pct_bf16_peak_at_clock": round(100 * tf / (PEAK_BF16_TFLOPS * clk / PEAK_CLOCK_MHZ), 1),
         "idle_cu_fraction": summ["idle_frac"], "wait_fraction": summ["wait_frac"],
         "tokens_per_s": round(shape.tokens / (t * 1e-3), 1),
         "forward_ms": round(fwd_ms, 4),
         "fwd_plus_bwd_tokens_per_s": round(shape.tokens / ((t + fwd_ms) * 1e-3), 1),
         "traffic": measured_traffic("moe_layer_bwd", shape.name)}
    if baseline:
        run, out = torch_bwd_baseline(torch, m, g, shape, rank)
        run()
        torch.cuda.synchronize()
        tb = time_ops(torch, [("torch_bwd", run)], reps, ws, flush)[0][0]
        d["torch_composed"] = {"ms": round(tb, 4), "speedup": round(tb / t, 3),
                               "dx_rel_diff": float(f"{_rel(out['dx'], g['dx']):.3g}"),
                               "dlogits_rel_diff": float(f"{_rel(out['dl'], g['dl']):.3g}"),
                               "dlogits_norm": float(f"{float(g['dl'].norm()):.4g}")}
    d["saved_activations"] = saved_backward(torch, kos, m, g, ws, flush, reps, shape, fwd_ms, t, rows, rank,
                                            baseline)
    return d


def saved_backward(torch, kos, m, g, ws, flush, reps, shape, fwd_ms, bwd_ms, rows, rank=0, baseline=True):
    """The forward keeps bf16 g and u (two more [rows, F] outputs) and the
    backward reads them instead of recomputing them, writing no dH: the
    forward's extra time, the backward's time and TFLOP/s (6 H F per row,
    all of it algorithmic), forward + backward tokens/s, and the PyTorch
    composition on the same kept values."""
    cap, F = m["grouped"].shape[0], shape.ffn
    m["gs"] = torch.empty((cap, F), dtype=torch.bfloat16, device="cuda")
    m["us"] = torch.empty((cap, F), dtype=torch.bfloat16, device="cuda")
    fs = layer_op(kos, m, ws, shape, rank, save=True)
    fs()
    ws.status()
    tf = time_ops(torch, [("moe_layer_save", fs)], reps, ws, flush)[0][0]
    fb = bwd_op(kos, m, g, ws, shape, rank, saved=True)
    fb()
    ws.status()
    tb = time_ops(torch, [("moe_layer_bwd_saved", fb)], reps, ws, flush)[0][0]
    fl = rows * 6.0 * shape.hidden * shape.ffn
    tfl = fl / (tb * 1e-3) / 1e12
    d = {"forward_ms": round(tf, 4), "forward_extra_ms": round(tf - fwd_ms, 4), "ms": round(tb, 4),
         "tflops": round(tfl, 1), "pct_bf16_peak": round(100 * tfl / PEAK_BF16_TFLOPS, 1),
         "speedup_vs_recompute": round(bwd_ms / tb, 3),
         "kept_bytes": 2 * rows * F * 2,
         "fwd_plus_bwd_tokens_per_s": round(shape.tokens / ((tf + tb) * 1e-3), 1),
         "fwd_plus_bwd_speedup_vs_recompute": round((fwd_ms + bwd_ms) / (tf + tb), 3),
         "traffic": measured_traffic("moe_layer_bwd_saved", shape.name)}
    if baseline:
        run, out = torch_bwd_baseline(torch, m, g, shape, rank, saved=True)
        run()
        torch.cuda.synchronize()
        tt = time_ops(torch, [("torch_bwd_saved", run)], reps, ws, flush)[0][0]
        d["torch_composed"] = {"ms": round(tt, 4), "speedup": round(tt / tb, 3),
                               "dx_rel_diff": float(f"{_rel(out['dx'], g['dx']):.3g}"),
                               "dlogits_rel_diff": float(f"{_rel(out['dl'], g['dl']):.3g}")}
    del m["gs"], m["us"]
    return d


def policy_comparison(torch, kos, KI, inp, ws, moe_shape, flush, reps, fused_ms, unfused_ms, sweep, planned):
    """The role-switching policies side by side, per op with a compute role
    (the explainer's "How do the policies compare?": each against a fixed
    communication crew): the pages' policy (one-way all-gather and
    reduce-scatter, two-way combine), the other one (kos_opts.policy =
    SWAPPED), the best fixed crew of the sweep, the planned crew and the
    unfused launches; speed-ups over the best fixed crew."""
    out = {}
    for n in ("ag_gemm", "gemm_rs", "moe_combine"):
        fn = dict(make_ops(kos, KI, inp, ws, moe_shape, policy=1))[n]
        fn()
        sw = time_ops(torch, [(n, fn)], reps, ws, flush)[0][0]
        best = min(sweep[n].values())
        d = {"default": round(fused_ms[n], 4), "swapped": round(sw, 4), "best_fixed": best,
             "planned": sweep[n][planned[n]], "unfused": unfused_ms[n]}
        d["speedup_vs_best_fixed"] = {k: round(best / d[k], 3) for k in ("default", "swapped")}
        d["policy"] = {"default": "two-way" if n == "moe_combine" else "one-way",
                       "swapped": "one-way" if n == "moe_combine" else "two-way"}
        out[n] = d
    return out


def tiny_ag(torch, kos, KI, ws, flush, reps=50):
    """The tiny all-gather+GEMM (4 emulated ranks, 64x256 shards, 256x256
    weight; rank 0): latency-bound, reported in microseconds -- fused,
    unfused and a FIXED crew of 4 (one workgroup per remote shard)."""
    s = KI.AG_TINY
    a = KI.ag_inputs(s, 0, "cuda")
    g = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((s.m, s.n), dtype=torch.bfloat16, device="cuda")
    t = {}
    for label, mode, crew in (("fused", 0, -1), ("unfused", 2, -1), ("fixed_crew4", 1, 4)):
        o = kos.opts(mode=mode, n_movers=crew)
        fn = lambda o=o: kos.ag_gemm(a["a_local"], a["a_peers"], a["w"], g, c, 0, ws, o)  # noqa: E731
        fn()
        t[label] = time_ops(torch, [("ag_tiny", fn)], reps, ws, flush)[0][0] * 1e3
    return {"workload": s.name, "us": {k: round(v, 2) for k, v in t.items()},
            "speedup_vs_unfused": round(t["unfused"] / t["fused"], 3),
            "speedup_vs_fixed": round(t["fixed_crew4"] / t["fused"], 3)}


def source_digest() -> str:
    """Digest of the kernel sources with comments and whitespace removed:
    ties a stored counter reading to the kernels it was taken on (an edit to
    a comment does not change the kernels)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "gemm_collective_persistent_amd", "csrc"), os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h")):
                with open(os.path.join(d, name)) as f:
                    text = f.read()
                text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
                text = re.sub(r"//[^\n]*", "", text)
                h.update(name.encode())
                h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(op: str, workload: str):
    """HBM bytes per launch of `op` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or
    None when there is none for this workload or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"{op}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#")):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _summary(path: str) -> dict:
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#")):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def measured_counters():
    """What the committed rocprofv3 summaries of the current kernel sources
    say: per kernel the matrix cores' busy share and the counted bf16 FLOPs
    over the algorithmic ones (``*_mfma.txt``), and per communication-only
    launch of the unfused baselines the bytes moved per second against the
    HBM peak (``*_rates.txt``).  Summaries taken on other kernel sources are
    left out."""
    import glob
    dig = source_digest()
    out = {"mfma": {}, "unfused_comm_launches": {}}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_mfma.txt"))):
        kv = _summary(path)
        if kv.get("source_digest") != dig:
            continue
        base = os.path.basename(path)
        op = next((o for o in ("ag_gemm", "gemm_rs", "moe_dispatch", "moe_combine", "moe_layer_bwd_saved",
                               "moe_layer_bwd", "moe_layer_save", "moe_layer")
                   if base.startswith(o + "_")), base)
        out["mfma"][op] = {"busy_fraction": float(kv["mfma_busy_fraction"]),
                           "counted_over_algorithmic_flops": float(kv["counted_over_algorithmic"]),
                           "clock_mhz_counter_run": float(kv["clock_mhz"]), "file": os.path.basename(path)}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_rates.txt"))):
        kv = _summary(path)
        if kv.get("source_digest") != dig:
            continue
        out["unfused_comm_launches"][os.path.basename(path)[:-len("_rates.txt")]] = {
            "gb_s": float(kv["algorithmic_gb_s"]), "frac_hbm_peak": float(kv["fraction_of_hbm_peak_8tb_s"]),
            "duration_us": float(kv["duration_us"])}
    return out


def copy_calibration(torch):
    """Three plain elementwise passes over 1 GiB of bf16 (dst = -src: 1 GiB
    read, 1 GiB written, 16-byte vector accesses like the kernels'): the
    reference that scales the HBM byte counters (FETCH_SIZE, WRITE_SIZE) read
    under rocprofv3."""
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"copy_bytes": 1 << 30, "copies": 3, "kernel": "neg"}


class CacheFlush:
    """Writes a buffer twice the size of the 256 MB Infinity Cache, so that the
    next op reads its inputs from HBM rather than from a cache."""

    def __init__(self, torch, enabled=True):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if enabled else None

    def __call__(self):
        if self.buf is not None:
            self.buf.fill_(1)


def time_ops(torch, ops, reps, ws, flush):
    """Runs `reps` steps, each op preceded by a cache flush outside its timed
    interval; returns (per-op mean ms from events on the launch stream, wall
    ms/step including the flushes)."""
    n = len(ops)
    ev = [_events(torch, 2 * n) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(reps):
        for i, (_, fn) in enumerate(ops):
            flush()
            ev[r][2 * i].record()
            fn()
            ev[r][2 * i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / reps
    ws.status()
    per = [sum(ev[r][2 * i].elapsed_time(ev[r][2 * i + 1]) for r in range(reps)) / reps for i in range(n)]
    return per, wall


# launches an unfused call makes (its trace fills one slot per launch)
UNFUSED_LAUNCHES = {"ag_gemm": 2, "gemm_rs": 2, "moe_dispatch": 2, "moe_combine": 4}
# the fixed-crew sweep: every crew size from 8 to 128 in steps of 8 (plus the
# planned crew), the best of which is the "best fixed split"
CREW_SWEEP = tuple(range(8, 129, 8))


def phase_bytes(KI, moe_shape, rows, peer_rows):
    """Algorithmic bytes of each op's communication phase (read + written):
    AG the gather (every shard read and written into the gathered matrix);
    RS the reduction (the peers' slices and our staged rows read, the chunk
    written); dispatch the token movement (our tokens read, one row per
    (token, expert) pair written, the peers' rows read and written into the
    grouped input); combine the pushes (rows returned to peers, read and
    written) and the fold (k results read per token, the token written)."""
    ag, rs, m = KI.AG_QKV, KI.RS_MLP, moe_shape
    row = m.hidden * 2
    return {"ag_gemm": {"move": 2.0 * ag.m * ag.k * 2},
            "gemm_rs": {"reduce": (rs.world + 1) * rs.m_chunk * rs.n * 4.0},
            "moe_dispatch": {"move": (m.tokens + m.tokens * m.topk + 2.0 * peer_rows) * row},
            "moe_combine": {"push": 2.0 * peer_rows * row, "fold": m.tokens * (m.topk + 1.0) * row}}


def traced_call(kos, ws, fn, grid, launches, flush):
    """One traced, untimed call; its timeline (every launch)."""
    flush()
    fn()
    ws.status()
    return ws.trace(grid, launches=launches)


def idle_fractions(torch, kos, KI, inp, ws, moe_shape, flush, best_crew, pbytes, names, rank_moe=0):
    """Per op and mode: the idle-CU fraction (share of compute-unit time, over
    the call's span, that no piece of work covers; the unfused baselines'
    gaps between launches count as idle) and the rate of each communication
    phase (its algorithmic bytes over the span of its pieces of work), from
    one traced call each (kos_opts.trace).  FIXED is traced at its best crew."""
    from gemm_collective_persistent_amd.timeline import phase_rate, summarize
    grid = int(kos.lib.kos_device_cu_count())
    idle, rates = {}, {}
    for label in ("fused", "unfused", "fixed_best"):
        idle[label], rates[label] = {}, {}
        for n in names:
            if label == "fixed_best" and n not in best_crew:
                continue
            mode = {"fused": 0, "unfused": 2, "fixed_best": 1}[label]
            crew = best_crew.get(n, -1) if label == "fixed_best" else -1
            fn = dict(make_ops(kos, KI, inp, ws, moe_shape, mode=mode, n_movers=crew, trace=True,
                               rank_moe=rank_moe))[n]
            L = UNFUSED_LAUNCHES[n] if mode == 2 else 1
            tl = traced_call(kos, ws, fn, grid, L, flush)
            idle[label][n] = summarize(tl, workgroups=grid)["idle_frac"]
            rates[label][n] = {k: phase_rate(tl, k, b) for k, b in pbytes[n].items()}
    return idle, rates


def crew_sweep(torch, kos, KI, inp, ws, moe_shape, flush, reps, names, extra):
    """FIXED mode of each op with a compute role at every crew of CREW_SWEEP
    and the crews in `extra` (op -> crew): {op: {crew: ms}}.  The dispatch
    has no compute role to split from (no FIXED mode)."""
    out = {}
    for n in names:
        if n == "moe_dispatch":
            continue
        out[n] = {}
        for c in sorted(set(CREW_SWEEP) | ({extra[n]} if n in extra else set())):
            fn = dict(make_ops(kos, KI, inp, ws, moe_shape, mode=1, n_movers=c))[n]
            fn()
            out[n][c] = round(time_ops(torch, [(n, fn)], reps, ws, flush)[0][0], 4)
    return out


def measured_clocks(torch, kos, KI, inp, ws, moe_shape, flush, reps=3):
    """Shader clock (MHz) each fused op runs at: `reps` traced steps, run
    like the timed ones (each op after a cache flush), averaging every
    workgroup's clock record (s_memtime cycles over its lifetime)."""
    grid = int(kos.lib.kos_device_cu_count())
    ops = make_ops(kos, KI, inp, ws, moe_shape, trace=True)
    acc = {n: [] for n, _ in ops}
    for _ in range(reps):
        for n, fn in ops:
            flush()
            fn()
            ws.trace(grid)
            acc[n].extend(ws.trace_clock_mhz)
    ws.status()
    return {n: round(sum(v) / len(v), 1) for n, v in acc.items()}


def cu_subset_gemm(torch, kos, inp, ws, reps, flush):
    """Plain GEMM throughput on 224 of the 256 compute units relative to all
    256, on the QKV GEMM (4096 x 8192 x 3072: exactly 256 tiles, so 224
    workgroups need a second round) and on a large square GEMM (8192^3:
    1024 tiles) -- the explainer's worked example reports about 93%.  Beside
    it, the vendor library's GEMM on the same operands (torch.matmul, i.e.
    hipBLASLt): a reference for the tile itself."""
    res = {}
    ag = inp["ag"]
    big = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    rs = inp["rs"]
    cases = {"qkv_4096x8192x3072": (ag["g"], ag["w"], True), "square_8192": (big, big, True),
             "mlp_down_4096x3584x8192": (rs["a"], rs["w"], False)}
    for name, (a, w, subset) in cases.items():
        c = torch.empty((a.shape[0], w.shape[1]), dtype=torch.bfloat16, device="cuda")
        t = {}
        for grid in (256, 224) if subset else (256,):
            o = kos.opts(mode=2, grid=grid)
            fn = lambda: kos.ag_gemm(a, [None], w, a, c, 0, ws, o)  # noqa: E731
            fn()
            t[grid] = time_ops(torch, [("gemm", fn)], reps, ws, flush)[0][0]
        vend = lambda: torch.matmul(a, w, out=c)  # noqa: E731
        for _ in range(3):   # the library picks and loads its kernel on the first calls
            vend()
        tv = time_ops(torch, [("hipblaslt", vend)], reps, ws, flush)[0][0]
        fl = 2.0 * a.shape[0] * a.shape[1] * w.shape[1]
        d = {"ms_256": round(t[256], 4), "tflops": round(fl / (t[256] * 1e-3) / 1e12, 1),
             "hipblaslt_ms": round(tv, 4), "hipblaslt_tflops": round(fl / (tv * 1e-3) / 1e12, 1),
             "vs_hipblaslt": round(tv / t[256], 3)}
        if subset:
            d.update(ms_224=round(t[224], 4), throughput_224_vs_256=round(t[256] / t[224], 3))
        res[name] = d
    del big
    return res


def ag_pinned(torch, kos, KI, inp, ws, reps, flush):
    """The QKV all-gather+GEMM with the 7 peer shards in pinned,
    device-mapped host memory (a PCIe link instead of HBM): fused, unfused
    and fixed-crew times, the link rate implied by the unfused copy, and the
    overlap (t_unfused - t_fused) / min(t_copy, t_gemm)."""
    ag = inp["ag"]
    peers = [None if t is None else t.cpu().pin_memory() for t in ag["a_peers"]]
    gemm_only = lambda: kos.ag_gemm(ag["g"], [None], ag["w"], ag["g"], ag["c"], 0, ws,  # noqa: E731
                                    kos.opts(mode=2))
    gemm_only()
    t_gemm = time_ops(torch, [("gemm", gemm_only)], reps, ws, flush)[0][0]
    t = {}
    runs = [("fused", 0, -1), ("unfused", 2, -1)] + [(f"fixed_crew{c}", 1, c) for c in (8, 16, 24, 32, 48, 64)]
    for label, mode, crew in runs:
        o = kos.opts(mode=mode, n_movers=crew, peer_link=1)
        fn = lambda: kos.ag_gemm(ag["a_local"], peers, ag["w"], ag["g"], ag["c"], 0, ws, o)  # noqa: E731
        fn()
        t[label] = time_ops(torch, [("ag", fn)], max(2, reps // 2), ws, flush)[0][0]
    t_copy = max(t["unfused"] - t_gemm, 1e-6)
    moved = sum(p.numel() * 2 for p in peers if p is not None)
    best = min((k for k in t if k.startswith("fixed")), key=t.get)
    return {"ms": {k: round(v, 4) for k, v in t.items()}, "gemm_alone_ms": round(t_gemm, 4),
            "link_gb_s": round(moved / (t_copy * 1e-3) / 1e9, 1),
            "overlap": round((t["unfused"] - t["fused"]) / min(t_copy, t_gemm), 3),
            "best_fixed": best, "speedup_vs_best_fixed": round(t[best] / t["fused"], 3),
            "speedup_vs_unfused": round(t["unfused"] / t["fused"], 3)}


def planned_crews(KI, moe_shape, rows, grid):
    """The split a per-call cost model would plan (the explainer's kitchen
    paragraph: a split predicted before each call, which did worse than an
    untuned fixed crew in the paper's measurements): the crew that finishes its bytes at the
    published HBM rate when the builders finish their FLOPs at the published
    MFMA rate, M = grid * t_bytes / (t_bytes + t_flops).  Bytes per op: AG
    the gather (peer shards read + written, local shard copied); RS the
    reduction (7 peer slices + own staging read, reduced chunk written);
    combine the pushes (rows returned to peers, read + written) and the fold
    (k results read per token, the token written)."""
    ag, rs, m = KI.AG_QKV, KI.RS_MLP, moe_shape
    b = {"ag_gemm": 2.0 * ag.world * ag.m_local * ag.k * 2,
         "gemm_rs": (rs.world + 1) * rs.m_chunk * rs.n * 4.0,
         "moe_combine": 2.0 * rows * m.hidden * 2 * (m.world - 1) / m.world
                        + m.tokens * (m.topk + 1) * m.hidden * 2.0}
    f = {"ag_gemm": ag.flops, "gemm_rs": rs.flops, "moe_combine": rows * m.flops_per_row}
    out = {}
    for n in b:
        tb, tf = b[n] / (PEAK_HBM_GBS * 1e9), f[n] / (PEAK_BF16_TFLOPS * 1e12)
        out[n] = max(1, min(grid - 1, round(grid * tb / (tb + tf))))
    return out


def rest_of_layer(torch, kos, KI, inp, ws, reps, flush):
    """The other two fused GEMM+collectives of a TP+SP transformer layer at
    the QKV shape's width -- MLP-up all-gather+GEMM (rank 0) and the
    attention output projection GEMM+reduce-scatter (rank 7) -- fused and
    unfused, and the four fused collectives of the layer together (QKV and
    MLP-down taken from the timed step)."""
    res = {}
    ag, rs = KI.AG_MLPUP, KI.RS_OUTPROJ
    a = KI.ag_inputs(ag, 0, "cuda")
    g = torch.empty((ag.m, ag.k), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((ag.m, ag.n), dtype=torch.bfloat16, device="cuda")
    r = KI.rs_inputs(rs, 7, "cuda")
    part = torch.empty((rs.m, rs.n), dtype=torch.float32, device="cuda")
    y = torch.empty((rs.m_chunk, rs.n), dtype=torch.float32, device="cuda")
    for name, shape, call in (
            ("ag_mlpup", ag, lambda o: kos.ag_gemm(a["a_local"], a["a_peers"], a["w"], g, c, 0, ws, o)),
            ("rs_outproj", rs, lambda o: kos.gemm_rs(r["a"], r["w"], r["peer_slices"], part, y, 7, ws, o))):
        t = {}
        for label, mode in (("fused", 0), ("unfused", 2)):
            o = kos.opts(mode=mode)
            fn = lambda o=o, call=call: call(o)  # noqa: E731
            fn()
            t[label] = time_ops(torch, [(name, fn)], reps, ws, flush)[0][0]
        res[name] = {"workload": shape.name, "ms": round(t["fused"], 4),
                     "tflops": round(shape.flops / (t["fused"] * 1e-3) / 1e12, 1),
                     "unfused_ms": round(t["unfused"], 4), "speedup_vs_unfused": round(t["unfused"] / t["fused"], 3)}
    del a, g, c, r, part, y
    return res


def mxfp8(torch, kos, KI, ws, reps, flush, bf16_ms, baselines=True):
    """The TP+SP layer's four fused collectives with MXFP8 operands -- QKV and
    MLP-up all-gather+GEMM (rank 0), MLP-down and output-projection
    GEMM+reduce-scatter (rank 7): fused (and, with `baselines`, unfused and
    FIXED crews of 16 and 32), TFLOP/s against the dense fp8 peak, HBM bytes
    per launch from the committed counter summary, the speed-up over the bf16
    op, and the four together.  Without `baselines` only the QKV and MLP-down
    ops."""
    res = {}

    def ag_call(shape):
        a = KI.ag_mx_inputs(shape, 0, "cuda")
        g = torch.empty((shape.m, shape.k), dtype=torch.uint8, device="cuda")
        gs = torch.empty((shape.k // 64, shape.m, 2), dtype=torch.uint8, device="cuda")
        c = torch.empty((shape.m, shape.n), dtype=torch.bfloat16, device="cuda")
        return lambda o: kos.ag_gemm_mx(a["a_local"], a["s_local"], a["a_peers"], a["s_peers"], a["w"],
                                        a["w_scales"], g, gs, c, 0, ws, o)

    def rs_call(shape):
        r = KI.rs_mx_inputs(shape, 7, "cuda")
        part = torch.empty((shape.m, shape.n), dtype=torch.float32, device="cuda")
        y = torch.empty((shape.m_chunk, shape.n), dtype=torch.float32, device="cuda")
        return lambda o: kos.gemm_rs_mx(r["a"], r["a_scales"], r["w"], r["w_scales"], r["peer_slices"], part, y, 7,
                                        ws, o)

    ops = [("ag_gemm_mx", "ag_gemm", KI.AG_QKV_MX, ag_call), ("gemm_rs_mx", "gemm_rs", KI.RS_MLP_MX, rs_call),
           ("ag_mlpup_mx", "ag_mlpup", KI.AG_MLPUP_MX, ag_call),
           ("rs_outproj_mx", "rs_outproj", KI.RS_OUTPROJ_MX, rs_call)]
    # without baselines (the profiling runs): one shape per kernel, so the
    # counters of a kernel belong to one workload
    if not baselines:
        ops = ops[:2]
    tot_ms = tot_fl = 0.0
    for name, bf16_name, shape, mk in ops:
        call = mk(shape)
        t = {}
        runs = (("fused", 0, -1), ("unfused", 2, -1), ("fixed16", 1, 16), ("fixed32", 1, 32))
        for label, mode, crew in runs if baselines else runs[:1]:
            o = kos.opts(mode=mode, n_movers=crew)
            fn = lambda o=o, call=call: call(o)  # noqa: E731
            fn()
            t[label] = time_ops(torch, [(name, fn)], reps, ws, flush)[0][0]
        tf = shape.flops / (t["fused"] * 1e-3) / 1e12
        d = {"workload": shape.name, "ms": round(t["fused"], 4), "tflops": round(tf, 1),
             "pct_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 1),
             "traffic": measured_traffic(name, shape.name)}
        if bf16_name in bf16_ms:
            d["speedup_vs_bf16"] = round(bf16_ms[bf16_name] / t["fused"], 3)
        if baselines:
            fixed = min(t["fixed16"], t["fixed32"])
            d.update(unfused_ms=round(t["unfused"], 4), speedup_vs_unfused=round(t["unfused"] / t["fused"], 3),
                     best_fixed_ms=round(fixed, 4), speedup_vs_best_fixed=round(fixed / t["fused"], 3))
        res[name] = d
        tot_ms += t["fused"]
        tot_fl += shape.flops
        del call
    ws.status()
    if baselines:
        res["tp_sp_layer_mx"] = {"ms": round(tot_ms, 4), "tflops": round(tot_fl / (tot_ms * 1e-3) / 1e12, 1)}
    return res


def backward_collectives(torch, kos, KI, ws, reps, flush):
    """The data-gradient collectives of the same TP+SP layer's backward pass
    (weights read transposed): the QKV and MLP-up all-gathers become
    GEMM+reduce-scatters of dY . W^T (rank 7), the MLP-down and output
    projection reduce-scatters become all-gather+GEMMs of dY with W^T (rank 0);
    fused and unfused, and the four together."""
    res = {}
    tot_ms = tot_fl = 0.0
    for name, shape in (("rs_qkv_bwd", KI.RS_QKV_BWD), ("rs_mlpup_bwd", KI.RS_MLPUP_BWD),
                        ("ag_mlpdown_bwd", KI.AG_MLP_BWD), ("ag_outproj_bwd", KI.AG_OUTPROJ_BWD)):
        if name.startswith("rs"):
            r = KI.rs_inputs(shape, 7, "cuda", wt=True)
            part = torch.empty((shape.m, shape.n), dtype=torch.float32, device="cuda")
            y = torch.empty((shape.m_chunk, shape.n), dtype=torch.float32, device="cuda")
            call = lambda o, r=r, part=part, y=y: kos.gemm_rs(r["a"], r["w"], r["peer_slices"], part, y, 7, ws, o,  # noqa: E731
                                                              w_transposed=True)
        else:
            a = KI.ag_inputs(shape, 0, "cuda", wt=True)
            g = torch.empty((shape.m, shape.k), dtype=torch.bfloat16, device="cuda")
            c = torch.empty((shape.m, shape.n), dtype=torch.bfloat16, device="cuda")
            call = lambda o, a=a, g=g, c=c: kos.ag_gemm(a["a_local"], a["a_peers"], a["w"], g, c, 0, ws, o,  # noqa: E731
                                                        w_transposed=True)
        t = {}
        for label, mode in (("fused", 0), ("unfused", 2)):
            o = kos.opts(mode=mode)
            fn = lambda o=o, call=call: call(o)  # noqa: E731
            fn()
            t[label] = time_ops(torch, [(name, fn)], reps, ws, flush)[0][0]
        res[name] = {"workload": shape.name, "ms": round(t["fused"], 4),
                     "tflops": round(shape.flops / (t["fused"] * 1e-3) / 1e12, 1),
                     "unfused_ms": round(t["unfused"], 4), "speedup_vs_unfused": round(t["unfused"] / t["fused"], 3)}
        tot_ms += t["fused"]
        tot_fl += shape.flops
    ws.status()
    res["layer_backward_data"] = {"ms": round(tot_ms, 4), "tflops": round(tot_fl / (tot_ms * 1e-3) / 1e12, 1)}
    return res


def rs_order_ablation(torch, kos, KI, inp, ws, reps, flush):
    """GEMM+reduce-scatter in band order (the design) and row order (the
    slower ablation the explainer compares it with), fused, at rank 7 (whose
    chunk comes last in row order: the reduction waits for the whole GEMM)
    and at rank 0."""
    s = KI.RS_MLP
    res = {}
    for rank, rs in ((7, inp["rs"]), (0, None)):
        if rs is None:
            rs = KI.rs_inputs(s, rank, "cuda")
            rs["partial"], rs["y"] = inp["rs"]["partial"], inp["rs"]["y"]
        t = {}
        for label, order in (("band", kos.RS_BAND), ("row", kos.RS_ROW)):
            o = kos.opts(rs_order=order)
            fn = lambda: kos.gemm_rs(rs["a"], rs["w"], rs["peer_slices"], rs["partial"], rs["y"], rank, ws, o)  # noqa: E731
            fn()
            t[label] = time_ops(torch, [("rs", fn)], reps, ws, flush)[0][0]
        res[f"rank{rank}"] = {"band_ms": round(t["band"], 4), "row_ms": round(t["row"], 4),
                              "row_over_band": round(t["row"] / t["band"], 3)}
        del rs
    return res


def cpu_baseline(inp, moe_shape, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same step: the
    all-gather+GEMM of 8 rows of each of the 8 shards, the GEMM+reduce-scatter
    of 8 rows of each of the 8 chunks, and the whole expert layer for the
    first 128 tokens (no rows from peers).  FLOPs of the sample / time,
    repeated until `budget_s` has elapsed."""
    import numpy as np
    import kos_inputs as KI
    from oracle import kos_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    ag, rs, m = inp["ag"], inp["rs"], inp["moe"]
    s2, s3, s4 = KI.AG_QKV, KI.RS_MLP, moe_shape
    r = 8
    ag_local = KI.bf16_bits(ag["a_local"][:r])
    ag_peers = [None if t is None else KI.bf16_bits(t[:r]) for t in ag["a_peers"]]
    w_ag = KI.bf16_bits(ag["w"])
    a_rs = np.concatenate([KI.bf16_bits(rs["a"][c * s3.m_chunk:c * s3.m_chunk + r]) for c in range(s3.world)])
    w_rs = KI.bf16_bits(rs["w"])
    rs_peers = [None if t is None else t[:r].cpu().numpy() for t in rs["peer_slices"]]
    ts = 128
    x = KI.bf16_bits(m["x"][:ts])
    lg = m["logits"][:ts].cpu().numpy()
    wg, wu, wd = (KI.bf16_bits(m[k]) for k in ("wg", "wu", "wd"))
    no_counts = np.zeros((s4.world, s4.e_local), np.int32)
    no_rows = [np.zeros((0, s4.hidden), np.uint16)] * s4.world
    cap = ts * min(s4.topk, s4.e_local)
    pret = [None if t is None else KI.bf16_bits(t[:cap]) for t in m["peer_return"]]
    flops, done, t0 = 0.0, 0, time.perf_counter()
    while True:
        O.ag_gemm(ag_local, ag_peers, w_ag, 0)
        O.gemm_rs(a_rs, w_rs, rs_peers, 7)
        out = O.moe_layer(x, lg, wg, wu, wd, no_rows, no_counts, pret, s4.world, 0, s4.topk)
        flops += 2.0 * (8 * r) * s2.n * s2.k + 2.0 * (8 * r) * s3.n * s3.k
        flops += int(out["grouped_offsets"][-1]) * s4.flops_per_row
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"{done} x [AG+GEMM: 8 rows of each of 8 shards (64x{s2.k} . {s2.k}x{s2.n}); "
                       f"GEMM+RS: 8 rows of each of 8 chunks (64x{s3.k} . {s3.k}x{s3.n}) + 8 partials; "
                       f"expert layer on the first {ts} tokens ({s4.name}, no peer rows)], float64 NumPy, "
                       f"{dt:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--moe", choices=["dsv3", "qwen3"], default="dsv3")
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--mode", choices=["fused", "fixed", "unfused"], default="fused",
                    help="fused: the persistent kernels (the measured product); fixed / unfused: the same-GPU "
                         "baselines timed as the step (for per-launch profiles)")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between ops")
    ap.add_argument("--mxfp8", action="store_true",
                    help="with --no-baselines: still time the MXFP8 ops (fused only; for their profiles)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three plain 1 GiB device copies (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs one GPU's share only (emulated peers); --gpus {args.gpus} is not supported: "
              "the library runs one GPU's share; there is no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import kos_inputs as KI
    import gemm_collective_persistent_amd as kos

    moe_shape = KI.MOE_DSV3 if args.moe == "dsv3" else KI.MOE_QWEN3
    torch.cuda.set_device(0)
    ws = kos.Workspace("cuda")
    inp = build_inputs(torch, KI, kos, moe_shape)
    mode = {"fused": 0, "fixed": 1, "unfused": 2}[args.mode]
    ops = make_ops(kos, KI, inp, ws, moe_shape, mode=mode)
    for _ in range(args.warmup):
        for _, fn in ops:
            fn()
    torch.cuda.synchronize()
    ws.status()
    flush = CacheFlush(torch, not args.no_flush)
    per, wall = time_ops(torch, ops, args.steps, ws, flush)
    ms_step = sum(per)
    names = [n for n, _ in ops]
    rows = int(inp["moe"]["goff"][-1].item())
    fl = {"ag_gemm": KI.AG_QKV.flops, "gemm_rs": KI.RS_MLP.flops, "moe_dispatch": 0.0,
          "moe_combine": rows * moe_shape.flops_per_row}
    total_flops = sum(fl.values())
    value = total_flops / (ms_step * 1e-3) / 1e12
    per_op = {}
    for n, t in zip(names, per):
        d = {"ms": round(t, 4)}
        if fl[n] > 0:
            tf = fl[n] / (t * 1e-3) / 1e12
            d.update(tflops=round(tf, 1), pct_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
        per_op[n] = d
    t_moe = per[names.index("moe_dispatch")] + per[names.index("moe_combine")]
    moe_tok_s = moe_shape.tokens / (t_moe * 1e-3)
    dom = max(range(len(per)), key=lambda i: per[i] if fl[names[i]] > 0 else -1)
    ach = fl[names[dom]] / (per[dom] * 1e-3) / 1e12
    traffic = measured_traffic(names[dom], moe_shape.name if names[dom].startswith("moe") else "")
    roofline = {"kernel": names[dom], "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    # the published peak assumes the 2.4 GHz peak clock; under sustained MFMA
    # load the clock is lower: the same peak at the clock the kernel ran at
    clocks = measured_clocks(torch, kos, KI, inp, ws, moe_shape, flush)
    peak_clk = PEAK_BF16_TFLOPS * clocks[names[dom]] / PEAK_CLOCK_MHZ
    roofline.update(clock_mhz=clocks[names[dom]], peak_at_clock=round(peak_clk, 1),
                    frac_at_clock=round(ach / peak_clk, 4))

    for n in names:
        per_op[n]["clock_mhz"] = clocks[n]
    extra = {"per_op": per_op, "moe_tokens_per_s": round(moe_tok_s, 1), "moe_grouped_rows": rows,
             "counters": measured_counters(),
             "wall_ms_per_step": round(wall, 3), "caches_flushed": not args.no_flush,
             "source_digest": source_digest()}
    if args.copy_calibration:
        extra["copy_calibration"] = copy_calibration(torch)
    # the expert layer in one launch, router to fold, beside the two launches
    t_two = per[names.index("moe_dispatch")] + per[names.index("moe_combine")]
    extra["moe_single_launch"] = single_launch(torch, kos, KI, inp["moe"], ws, flush, max(3, args.steps // 4),
                                               moe_shape, t_two, baseline=not args.no_baselines)
    # the expert layer's backward direction in one launch, on the forward
    # buffers the single launch just left (the forward's routing and rows)
    extra["moe_backward"] = moe_backward(torch, kos, KI, inp["moe"], ws, flush, max(3, args.steps // 4), moe_shape,
                                         extra["moe_single_launch"]["ms"], baseline=not args.no_baselines)
    if not args.no_baselines:
        reps = max(3, args.steps // 4)
        ops_u = make_ops(kos, KI, inp, ws, moe_shape, mode=2)
        for _, fn in ops_u:
            fn()
        pu, _ = time_ops(torch, ops_u, reps, ws, flush)
        unfused = {n: round(t, 4) for n, t in zip(names, pu)}
        # the planned split: a FIXED crew sized per op by the cost model; the
        # best fixed split: the fastest crew of the sweep (planned crew included)
        grid = int(kos.lib.kos_device_cu_count())
        crews = planned_crews(KI, moe_shape, rows, grid)
        sweep = crew_sweep(torch, kos, KI, inp, ws, moe_shape, flush, reps, names, crews)
        best = {n: min(v, key=v.get) for n, v in sweep.items()}
        extra["baselines_ms"] = {"unfused": unfused,
                                 "fixed_crew_sweep": {n: {str(c): t for c, t in v.items()} for n, v in sweep.items()},
                                 "moe_dispatch_fixed": "n/a (no compute role to split from)"}
        extra["best_fixed_split"] = {n: {"crew": best[n], "ms": sweep[n][best[n]]} for n in sweep}
        extra["planned_split"] = {n: {"crew": c, "ms": sweep[n][c]} for n, c in crews.items()}
        extra["speedup_vs_unfused"] = {n: round(unfused[n] / t, 3) for n, t in zip(names, per)}
        extra["speedup_vs_best_fixed"] = {n: round(sweep[n][best[n]] / per[names.index(n)], 3) for n in sweep}
        extra["speedup_vs_planned_split"] = {n: round(sweep[n][c] / per[names.index(n)], 3) for n, c in crews.items()}
        # idle-CU fraction and communication-phase rates of each op in each
        # mode (one traced, untimed call each)
        peer_rows = int(inp["moe"]["peer_counts"].sum().item())
        pb = phase_bytes(KI, moe_shape, rows, peer_rows)
        idle, rates = idle_fractions(torch, kos, KI, inp, ws, moe_shape, flush, best, pb, names)
        extra["idle_cu_fraction"] = idle
        extra["phase_rate_gb_s"] = {lab: {n: {k: v["gb_s"] for k, v in d.items()} for n, d in r.items()}
                                    for lab, r in rates.items()}
        extra["phase_bytes"] = {n: {k: round(v) for k, v in d.items()} for n, d in pb.items()}
        # the two switching policies against the fixed crews
        extra["policy_comparison"] = policy_comparison(torch, kos, KI, inp, ws, moe_shape, flush, reps,
                                                       {n: t for n, t in zip(names, per)}, unfused, sweep, crews)
        # the tiny all-gather+GEMM (latency-bound; microseconds)
        extra["ag_tiny"] = tiny_ag(torch, kos, KI, ws, flush)
        # the other expert-layer shape, as a block of its own (the Qwen3-235B
        # shape's skewed routing exercises the combine's two-way switching)
        other = KI.MOE_QWEN3 if moe_shape is KI.MOE_DSV3 else KI.MOE_DSV3
        extra["moe_qwen3" if other is KI.MOE_QWEN3 else "moe_dsv3"] = moe_block(torch, kos, KI, ws, flush, reps,
                                                                                 other)
        # GEMM throughput on 224 of 256 CUs: the explainer's worked example
        # (plain GEMM = the unfused GEMM launch at world 1)
        extra["gemm_224_of_256_cus"] = cu_subset_gemm(torch, kos, inp, ws, reps, flush)
        # all-gather+GEMM with the peers' shards in pinned host memory (PCIe)
        extra["ag_gemm_pinned_host_peers"] = ag_pinned(torch, kos, KI, inp, ws, reps, flush)
        # reduce-scatter band order vs row order
        extra["gemm_rs_band_vs_row"] = rs_order_ablation(torch, kos, KI, inp, ws, reps, flush)
        # the rest of the TP+SP layer, and the layer's four fused collectives
        rest = rest_of_layer(torch, kos, KI, inp, ws, reps, flush)
        t4 = per[names.index("ag_gemm")] + per[names.index("gemm_rs")] + rest["ag_mlpup"]["ms"] + \
            rest["rs_outproj"]["ms"]
        f4 = KI.AG_QKV.flops + KI.RS_MLP.flops + KI.AG_MLPUP.flops + KI.RS_OUTPROJ.flops
        rest["tp_sp_layer"] = {"ms": round(t4, 4), "tflops": round(f4 / (t4 * 1e-3) / 1e12, 1)}
        extra["tp_sp_layer"] = rest
        # the backward pass's data-gradient collectives of the layer
        extra["tp_sp_backward"] = backward_collectives(torch, kos, KI, ws, reps, flush)
        # the same two collectives with MXFP8 operands
        bf16_ms = {n: per[names.index(n)] for n in ("ag_gemm", "gemm_rs")}
        bf16_ms.update(ag_mlpup=rest["ag_mlpup"]["ms"], rs_outproj=rest["rs_outproj"]["ms"])
        extra["mxfp8"] = mxfp8(torch, kos, KI, ws, reps, flush, bf16_ms)
    elif args.mxfp8:
        extra["mxfp8"] = mxfp8(torch, kos, KI, ws, max(3, args.steps // 4), flush,
                               {n: per[names.index(n)] for n in ("ag_gemm", "gemm_rs")}, baselines=False)
    if not args.no_cpu:
        cpu = cpu_baseline(inp, moe_shape)
    else:
        cpu = None

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"kosmos layer pass: ag_gemm {KI.AG_QKV.name} + gemm_rs {KI.RS_MLP.name} + "
                               f"moe {moe_shape.name}", "emulated_ranks": 8, "mode": args.mode,
                   "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 1)},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
