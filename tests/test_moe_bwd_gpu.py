"""The expert layer's backward direction in one launch (kos_moe_layer_bwd)
on the GPU against the oracle, through the C ABI.

Small shapes: the forward's buffers come from the oracle's forward, and
every output is compared with the oracle's backward -- the pairs'
gradients sent and grouped, dG, dU, dX, the token gradients and the
router gradient within the floating-point bar (zero exactly where an
expert was not selected), the pushed rows bit copies of dX at the
forward's provenance.  One small case chains the GPU forward into the
backward.  The saved-activation variant (the forward's bf16 g and u read
instead of recomputed, dh optional) against the oracle's variant, on the
small cases, chained, and at full size.  Full DeepSeek-V3 shape: the GPU forward feeds the backward;
sampled grouped rows, tokens and sent rows against the oracle evaluated
row by row, every pushed row against the grouped dX.  Bad arguments forced
from the host end in a reported error, with the kernel exiting normally."""
import numpy as np
import pytest
import torch

import kos_inputs as KI
from kos_testutil import assert_close, say
from oracle import kos_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def kos():
    import gemm_collective_persistent_amd as k
    return k


@pytest.fixture(scope="module")
def ws(kos):
    return kos.Workspace(DEV)


def _shape(s, rank):
    from gemm_collective_persistent_amd.api import moe_shape
    return moe_shape(s.world, rank, s.tokens, s.hidden, s.experts, s.topk, s.ffn)


def _bits(lst):
    return [None if t is None else KI.bf16_bits(t) for t in lst]


def _fwd_from_oracle(s, rank, ref, cap):
    """The forward's buffers as the backward reads them, from the oracle."""
    n = int(ref["grouped_offsets"][-1])
    H = s.hidden
    grouped = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
    yg = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
    row_src = torch.zeros((cap, 2), dtype=torch.int32, device=DEV)
    if n:
        grouped[:n] = KI.from_bf16_bits(ref["grouped"], DEV)
        yg[:n] = KI.from_bf16_bits(ref["y_grouped"], DEV)
        row_src[:n] = torch.as_tensor(ref["row_src"], device=DEV)
    return dict(idx=torch.as_tensor(ref["idx"], device=DEV).reshape(s.tokens, s.topk),
                w=torch.as_tensor(ref["w"], device=DEV).reshape(s.tokens, s.topk),
                perm=torch.as_tensor(ref["perm"], device=DEV), counts=torch.as_tensor(ref["counts"], device=DEV),
                goff=torch.as_tensor(ref["grouped_offsets"], device=DEV), row_src=row_src, grouped=grouped, yg=yg)


def _out_buffers(s, rank, pc, cap):
    nan = float("nan")
    T, H, F, E = s.tokens, s.hidden, s.ffn, s.experts
    return dict(
        send=[None if p == rank else torch.full((max(s.peer_cap, 1), H), nan, dtype=torch.bfloat16, device=DEV)
              for p in range(s.world)],
        dres=torch.full((cap, H), nan, dtype=torch.bfloat16, device=DEV),
        dg=torch.full((cap, F), nan, dtype=torch.bfloat16, device=DEV),
        du=torch.full((cap, F), nan, dtype=torch.bfloat16, device=DEV),
        dh=torch.full((cap, F), nan, dtype=torch.float32, device=DEV),
        dxg=torch.full((cap, H), nan, dtype=torch.bfloat16, device=DEV),
        ret=[None if p == rank else torch.full((max(int(pc[p].sum()), 1), H), nan, dtype=torch.bfloat16,
                                               device=DEV) for p in range(s.world)],
        dx=torch.full((T, H), nan, dtype=torch.bfloat16, device=DEV),
        dl=torch.full((T, E), nan, dtype=torch.float32, device=DEV),
    )


def run_bwd(kos, ws, s, rank, inp, gin, f, b, o=None, check=True):
    """f["gs"], f["us"] (optional): the forward's kept g and u, used instead
    of recomputing them."""
    kos.moe_layer_bwd(_shape(s, rank), gin["dy"], f["idx"], f["w"], f["perm"], f["counts"], inp["peer_counts"],
                      f["grouped"], f["goff"], f["row_src"], f["yg"], inp["peer_return"], inp["wg"], inp["wu"],
                      inp["wd"], gin["peer_send_grad"], b["send"], b["dres"], b["dg"], b["du"], b["dh"], b["dxg"],
                      gin["peer_return_grad"], b["ret"], b["dx"], b["dl"], ws, o, gate_saved=f.get("gs"),
                      up_saved=f.get("us"))
    if check:
        ws.status()
    torch.cuda.synchronize()


def _oracle_bwd(s, rank, inp, gin, saved=False):
    pc = inp["peer_counts"].cpu().numpy()
    wg, wu, wd = (KI.bf16_bits(inp[k]) for k in ("wg", "wu", "wd"))
    return O.moe_layer_bwd(KI.bf16_bits(gin["dy"]), KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), wg, wu,
                           wd, _bits(inp["peer_send"]), pc, _bits(inp["peer_return"]), _bits(gin["peer_send_grad"]),
                           _bits(gin["peer_return_grad"]), s.world, rank, s.topk, saved=saved)


def _check_all(s, rank, b, ref):
    n = int(ref["grouped_offsets"][-1])
    for d in range(s.world):
        if d != rank:
            nd = ref["send_grad"][d].shape[0]
            if nd:
                assert_close(O.bf16_to_f64(KI.bf16_bits(b["send"][d][:nd])), O.bf16_to_f64(ref["send_grad"][d]),
                             f"send_grad[{d}]")
    if n:
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["dres"][:n])), O.bf16_to_f64(ref["grouped_grad"]), "dres")
        if b["dh"] is not None:
            assert_close(b["dh"][:n].cpu().numpy(), ref["dh"], "dH")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["dg"][:n])), O.bf16_to_f64(ref["dg"]), "dG")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["du"][:n])), O.bf16_to_f64(ref["du"]), "dU")
        dxg = KI.bf16_bits(b["dxg"][:n])
        assert_close(O.bf16_to_f64(dxg), O.bf16_to_f64(ref["dx_grouped"]), "dX")
        rs = ref["row_src"]
        for p in range(s.world):
            sel = np.where(rs[:, 0] == p)[0] if p != rank else np.zeros(0, int)
            if sel.size:
                assert np.array_equal(KI.bf16_bits(b["ret"][p])[rs[sel, 1]], dxg[sel]), f"pushed rows to {p}"
    if s.tokens:
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["dx"])), O.bf16_to_f64(ref["dx"]), "dx")
        dl = b["dl"].cpu().numpy()
        assert_close(dl, ref["dlogits"], "dlogits")
        sel = np.zeros(dl.shape, dtype=bool)
        np.put_along_axis(sel, ref["idx"].reshape(s.tokens, s.topk).astype(np.int64), True, axis=1)
        assert np.all(dl[~sel] == 0), "router gradient outside the selected experts"


EDGE_T0 = KI.MoeShape("moe_bwd_edge_3r_t0_h256_e6_k2_f128", 44, 3, 0, 256, 6, 2, 128)
SMALL = [(KI.MOE_TINY, 0), (KI.MOE_TINY, 3), (KI.MOE_BWD_MID, 1), (KI.MOE_BWD_K10, 1), (KI.MOE_BWD_1R, 0),
         (KI.MOE_BWD_K1, 2), (EDGE_T0, 2)]


@pytest.mark.parametrize("s,rank", SMALL, ids=[f"{s.name}-r{r}" for s, r in SMALL])
def test_bwd_small_vs_oracle(kos, ws, s, rank):
    say(f"[moe bwd] {s.name} rank={rank}")
    inp = KI.moe_inputs(s, rank, DEV)
    gin = KI.moe_grad_inputs(s, rank, DEV)
    ref = _oracle_bwd(s, rank, inp, gin)
    pc = inp["peer_counts"].cpu().numpy()
    cap = int(pc.sum()) + s.tokens * min(s.topk, s.e_local) + 37   # slack rows past the grouped ones
    f = _fwd_from_oracle(s, rank, ref, cap)
    b = _out_buffers(s, rank, pc, cap)
    run_bwd(kos, ws, s, rank, inp, gin, f, b)
    _check_all(s, rank, b, ref)
    # a second call on the same workspace (counters left at zero)
    b2 = _out_buffers(s, rank, pc, cap)
    run_bwd(kos, ws, s, rank, inp, gin, f, b2)
    n = int(ref["grouped_offsets"][-1])
    for key, m in (("dxg", n), ("dx", s.tokens), ("dl", s.tokens)):
        assert torch.equal(b[key][:m], b2[key][:m]), key


SAVED = [(KI.MOE_TINY, 1, True), (KI.MOE_BWD_MID, 1, False), (KI.MOE_BWD_K10, 1, True), (KI.MOE_BWD_1R, 0, False),
         (KI.MOE_BWD_K1, 2, True), (EDGE_T0, 2, False)]


@pytest.mark.parametrize("s,rank,with_dh", SAVED, ids=[f"{s.name}-r{r}-dh{int(d)}" for s, r, d in SAVED])
def test_bwd_saved_small_vs_oracle(kos, ws, s, rank, with_dh):
    """The forward's kept bf16 g and u (here the oracle's) instead of the
    recomputation, against the oracle's saved-activation backward; dh
    written when given, untouched otherwise."""
    say(f"[moe bwd saved] {s.name} rank={rank} dh={with_dh}")
    inp = KI.moe_inputs(s, rank, DEV)
    gin = KI.moe_grad_inputs(s, rank, DEV)
    ref = _oracle_bwd(s, rank, inp, gin, saved=True)
    pc = inp["peer_counts"].cpu().numpy()
    cap = int(pc.sum()) + s.tokens * min(s.topk, s.e_local) + 37
    f = _fwd_from_oracle(s, rank, ref, cap)
    n = int(ref["grouped_offsets"][-1])
    wg, wu = KI.bf16_bits(inp["wg"]), KI.bf16_bits(inp["wu"])
    g, u = O.grouped_gate_up(ref["grouped"], ref["grouped_offsets"], wg, wu)
    f["gs"] = torch.zeros((cap, s.ffn), dtype=torch.bfloat16, device=DEV)
    f["us"] = torch.zeros((cap, s.ffn), dtype=torch.bfloat16, device=DEV)
    if n:
        f["gs"][:n] = KI.from_bf16_bits(g, DEV)
        f["us"][:n] = KI.from_bf16_bits(u, DEV)
    b = _out_buffers(s, rank, pc, cap)
    if not with_dh:
        b["dh"] = None
    run_bwd(kos, ws, s, rank, inp, gin, f, b)
    _check_all(s, rank, b, ref)
    if n:   # the kept values decide: the recomputing oracle is not what ran
        unsaved = _oracle_bwd(s, rank, inp, gin)
        assert not np.array_equal(unsaved["dg"], ref["dg"])


@pytest.mark.parametrize("saved", [False, True])
def test_forward_then_backward_on_the_gpu(kos, ws, saved):
    """The GPU forward's buffers feed the backward directly (saved: with the
    g and u the forward kept, and no dh)."""
    from test_moe_layer_gpu import run_layer
    s, rank = KI.MOE_BWD_MID, 2
    say(f"[moe fwd+bwd] {s.name} rank={rank} saved={saved}")
    inp = KI.moe_inputs(s, rank, DEV)
    gin = KI.moe_grad_inputs(s, rank, DEV)
    fw = run_layer(kos, ws, s, rank, inp, save=saved)
    pc = inp["peer_counts"].cpu().numpy()
    cap = fw["grouped"].shape[0]
    f = dict(idx=fw["idx"], w=fw["w"], perm=fw["perm"], counts=fw["counts"], goff=fw["goff"], row_src=fw["row_src"],
             grouped=fw["grouped"], yg=fw["yg"])
    if saved:
        f.update(gs=fw["gs"], us=fw["us"])
    b = _out_buffers(s, rank, pc, cap)
    if saved:
        b["dh"] = None
    run_bwd(kos, ws, s, rank, inp, gin, f, b)
    _check_all(s, rank, b, _oracle_bwd(s, rank, inp, gin, saved=saved))


def test_bad_arguments_are_reported(kos, ws):
    """Forced from the host: a send buffer too small for what we send, and
    grouped offsets that disagree with the counts.  The kernel checks
    before it moves anything, records the error and exits normally."""
    s, rank = KI.MOE_TINY, 1
    inp = KI.moe_inputs(s, rank, DEV)
    gin = KI.moe_grad_inputs(s, rank, DEV)
    ref = _oracle_bwd(s, rank, inp, gin)
    pc = inp["peer_counts"].cpu().numpy()
    cap = int(pc.sum()) + s.tokens * min(s.topk, s.e_local)
    f = _fwd_from_oracle(s, rank, ref, cap)
    b = _out_buffers(s, rank, pc, cap)
    d = next(d for d in range(s.world) if d != rank and ref["send_grad"][d].shape[0] > 1)
    b["send"][d] = b["send"][d][:ref["send_grad"][d].shape[0] - 1]
    run_bwd(kos, ws, s, rank, inp, gin, f, b, check=False)
    with pytest.raises(kos.KosError, match="ERR_CAPACITY"):
        ws.status()
    b = _out_buffers(s, rank, pc, cap)
    goff = f["goff"].cpu().clone()
    goff[1] += 1                       # expert 0 claims one row more than arrives
    goff[2] = max(int(goff[2]), int(goff[1]))
    f2 = dict(f, goff=goff.to(DEV))
    run_bwd(kos, ws, s, rank, inp, gin, f2, b, check=False)
    with pytest.raises(kos.KosError, match="ERR_ARG"):
        ws.status()
    # the workspace is usable again
    b = _out_buffers(s, rank, pc, cap)
    run_bwd(kos, ws, s, rank, inp, gin, f, b)
    _check_all(s, rank, b, ref)


FULL = [(KI.MOE_DSV3, 5, False), (KI.MOE_DSV3, 5, True), (KI.MOE_QWEN3, 0, True)]


@pytest.mark.parametrize("s,rank,saved", FULL, ids=[f"{s.name}-r{r}-saved{int(v)}" for s, r, v in FULL])
def test_bwd_full_size_sampled(kos, ws, s, rank, saved):
    """DeepSeek-V3 shape (rank 5) and the Qwen3 shape with skewed routing
    (rank 0, the most loaded): the GPU forward, then the backward; sampled
    outputs against the oracle row by row (saved: the forward keeps g and
    u, the backward reads them and writes no dh)."""
    from test_moe_layer_gpu import run_layer
    say(f"[moe bwd full] {s.name} rank={rank} saved={saved}")
    inp = KI.moe_inputs(s, rank, DEV)
    gin = KI.moe_grad_inputs(s, rank, DEV)
    fw = run_layer(kos, ws, s, rank, inp, save=saved)
    pc = inp["peer_counts"].cpu().numpy()
    cap = fw["grouped"].shape[0]
    f = dict(idx=fw["idx"], w=fw["w"], perm=fw["perm"], counts=fw["counts"], goff=fw["goff"], row_src=fw["row_src"],
             grouped=fw["grouped"], yg=fw["yg"])
    if saved:
        f.update(gs=fw["gs"], us=fw["us"])
    b = _out_buffers(s, rank, pc, cap)
    if saved:
        b["dh"] = None
    run_bwd(kos, ws, s, rank, inp, gin, f, b)
    say("[moe bwd full] kernel done; oracle on samples")
    ref = O.dispatch(KI.bf16_bits(inp["x"]), inp["logits"].cpu().numpy(), _bits(inp["peer_send"]), pc, s.world,
                     rank, s.topk)
    # the forward's routing the backward read is the oracle's
    assert np.array_equal(fw["idx"].cpu().numpy(), ref["idx"])
    assert np.array_equal(fw["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(fw["goff"].cpu().numpy(), ref["grouped_offsets"])
    n = int(ref["grouped_offsets"][-1])
    assert np.array_equal(fw["row_src"][:n].cpu().numpy(), ref["row_src"])
    wg, wu, wd = (KI.bf16_bits(inp[k]) for k in ("wg", "wu", "wd"))
    dy = KI.bf16_bits(gin["dy"])
    w = ref["w"]
    T, k, el = s.tokens, s.topk, s.e_local
    so = ref["send_off"]
    token_of = np.empty(T * k, np.int64)
    slot_of = np.empty(T * k, np.int64)
    token_of[ref["perm"]] = np.arange(T * k) // k
    slot_of[ref["perm"]] = np.arange(T * k) % k
    psg = _bits(gin["peer_send_grad"])
    rs = ref["row_src"]
    go = ref["grouped_offsets"]

    def dres_row(r):
        p, i = int(rs[r, 0]), int(rs[r, 1])
        if p == rank:
            q = so[rank] + i
            return O.pair_grad(dy, w, [token_of[q]], [slot_of[q]])[0]
        return psg[p][i]

    # grouped rows: the first and last rows of a few experts' units
    rng = np.random.default_rng(7)
    exps = rng.choice(el, 6, replace=False)
    dxg_rows = {}
    for e in exps:
        lo, hi = int(go[e]), int(go[e + 1])
        if hi == lo:
            continue
        rows = sorted({lo, min(lo + 255, hi - 1), min(lo + 256, hi - 1), hi - 1})
        dres = np.stack([dres_row(r) for r in rows])
        dg, du, dxr = O.expert_ffn_bwd(ref["grouped"][rows], dres, wg[e], wu[e], wd[e], saved=saved)
        if b["dh"] is not None:
            assert_close(b["dh"][rows].cpu().numpy(), O.expert_dh(dres, wd[e]), f"dH e{e}")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["dres"][rows])), O.bf16_to_f64(dres), f"dres e{e}")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["dg"][rows])), O.bf16_to_f64(dg), f"dG e{e}")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["du"][rows])), O.bf16_to_f64(du), f"dU e{e}")
        assert_close(O.bf16_to_f64(KI.bf16_bits(b["dxg"][rows])), O.bf16_to_f64(dxr), f"dX e{e}")
    say("[moe bwd full] grouped rows ok")
    # every pushed row is the grouped dX row it came from
    dxg_all = KI.bf16_bits(b["dxg"][:n])
    for p in range(s.world):
        sel = np.where(rs[:, 0] == p)[0] if p != rank else np.zeros(0, int)
        if sel.size:
            assert np.array_equal(KI.bf16_bits(b["ret"][p])[rs[sel, 1]], dxg_all[sel]), f"pushed rows to {p}"
    # sent rows: a sample per destination
    for d in range(s.world):
        if d == rank or so[d + 1] == so[d]:
            continue
        qs = np.unique(rng.integers(so[d], so[d + 1], 16))
        want = O.pair_grad(dy, w, token_of[qs], slot_of[qs])
        got = KI.bf16_bits(b["send"][d][torch.as_tensor(qs - so[d])])
        assert_close(O.bf16_to_f64(got), O.bf16_to_f64(want), f"send_grad[{d}]")
    # tokens: dx and the router gradient
    toks = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 14)]))
    need = {}
    for t in toks:
        for j in range(k):
            e = int(ref["idx"][t, j])
            if e // el == rank:
                r = O.local_row(e, int(ref["perm"][t * k + j]), rank, el, ref["offsets"], go, pc)
                need.setdefault(e - rank * el, []).append((r, t, j))
    dxg_s = np.zeros((n, s.hidden), np.uint16)
    yg_s = np.zeros((n, s.hidden), np.uint16)
    for e, lst in need.items():
        rows = [r for r, _, _ in lst]
        xr = ref["grouped"][rows]
        dres = O.pair_grad(dy, w, [t for _, t, _ in lst], [j for _, _, j in lst])
        dxg_s[rows] = O.expert_ffn_bwd(xr, dres, wg[e], wu[e], wd[e], saved=saved)[2]
        yg_s[rows] = O.expert_ffn(xr, wg[e], wu[e], wd[e])
    prg = _bits(gin["peer_return_grad"])
    pr = _bits(inp["peer_return"])
    dx_ref = O.fold(ref["idx"], np.ones_like(w), ref["perm"], ref["offsets"], dxg_s, go, pc, prg, s.world, rank,
                    tokens=toks)
    assert_close(O.bf16_to_f64(KI.bf16_bits(b["dx"][torch.as_tensor(toks)])), O.bf16_to_f64(dx_ref), "dx")
    dl_ref = O.router_grad(dy, ref["idx"], w, ref["perm"], ref["offsets"], yg_s, go, pc, pr, s.world, rank,
                           tokens=toks)
    assert_close(b["dl"][torch.as_tensor(toks)].cpu().numpy(), dl_ref, "dlogits")
