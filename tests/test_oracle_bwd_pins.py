"""Pins of the oracle's expert-layer backward direction (CPU only).

The backward is the chain rule of the forward definition, so the pins are
the derivative itself: central finite differences of an unrounded float64
forward written out here (SwiGLU expert, softmax over the k selected
logits, weighted sum), taken along random directions, against the oracle's
unrounded gradients.  Routing and the ranks' row exchange enter through the
peers' rows, which are rebuilt here from the expert each row belongs to, so
a wrong weight, sign, transposed operand or send/return index fails a
difference.  Special cases (k=1, zero down-projection) and the softmax
invariant (each token's router gradient sums to zero) pin the rounded
version, and rounded vs unrounded stays within bf16 error.
"""
import numpy as np
import pytest

from oracle import kos_oracle as O


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _expert(x, wg, wu, wd):
    """Unrounded SwiGLU expert on float64 rows."""
    return (_silu(x @ wg) * (x @ wu)) @ wd


def _w(rng, shape, scale):
    return O.round_bf16(rng.standard_normal(shape) * scale)


def test_dsilu_is_the_derivative_of_silu():
    z = np.linspace(-12.0, 12.0, 241)
    eps = 1e-6
    fd = (O.silu(z + eps) - O.silu(z - eps)) / (2 * eps)
    assert np.max(np.abs(O.dsilu(z) - fd)) < 1e-8
    assert O.dsilu(np.array([0.0]))[0] == 0.5
    assert abs(O.dsilu(np.array([40.0]))[0] - 1.0) < 1e-12
    assert abs(O.dsilu(np.array([-40.0]))[0]) < 1e-12


def test_expert_ffn_bwd_matches_finite_differences():
    """dX against d<dY, f(X)>/dX; dG and dU through the weight directions
    (dL/dWg = X^T dG, dL/dWu = X^T dU)."""
    rng = np.random.default_rng(101)
    n, H, F = 5, 12, 8
    x = _w(rng, (n, H), 1.0)
    wg, wu, wd = _w(rng, (H, F), 0.4), _w(rng, (H, F), 0.4), _w(rng, (F, H), 0.4)
    dy = rng.standard_normal((n, H))
    dg, du, dx = O.expert_ffn_bwd(x, dy, wg, wu, wd, rounded=False)
    X, Wg, Wu, Wd = (O.bf16_to_f64(a) for a in (x, wg, wu, wd))
    eps = 1e-6
    for _ in range(4):
        v = rng.standard_normal(X.shape)
        fd = (np.sum(dy * _expert(X + eps * v, Wg, Wu, Wd)) - np.sum(dy * _expert(X - eps * v, Wg, Wu, Wd))) / (2 * eps)
        assert abs(fd - np.sum(dx * v)) < 1e-6 * max(1.0, abs(fd))
        V = rng.standard_normal(Wg.shape)
        fd = (np.sum(dy * _expert(X, Wg + eps * V, Wu, Wd)) - np.sum(dy * _expert(X, Wg - eps * V, Wu, Wd))) / (2 * eps)
        assert abs(fd - np.sum((X.T @ dg) * V)) < 1e-6 * max(1.0, abs(fd))
        V = rng.standard_normal(Wu.shape)
        fd = (np.sum(dy * _expert(X, Wg, Wu + eps * V, Wd)) - np.sum(dy * _expert(X, Wg, Wu - eps * V, Wd))) / (2 * eps)
        assert abs(fd - np.sum((X.T @ du) * V)) < 1e-6 * max(1.0, abs(fd))


def test_dh_is_the_gradient_at_the_hidden():
    """dU = dH * silu(g) with g = X.Wg: the unrounded dU over silu(g) is
    expert_dh, and W_down's column scaling shows up in dH's column."""
    rng = np.random.default_rng(102)
    n, H, F = 4, 10, 6
    x = _w(rng, (n, H), 1.0)
    wg, wu, wd = _w(rng, (H, F), 0.4), _w(rng, (H, F), 0.4), _w(rng, (F, H), 0.4)
    dy = rng.standard_normal((n, H))
    _, du, _ = O.expert_ffn_bwd(x, dy, wg, wu, wd, rounded=False)
    dh = O.expert_dh(dy, wd, rounded=False)
    g = O.bf16_to_f64(x) @ O.bf16_to_f64(wg)
    assert np.allclose(du, dh * O.silu(g), rtol=1e-12, atol=1e-12)
    wd2 = wd.copy()
    wd2[2] = O.round_bf16(2.0 * O.bf16_to_f64(wd[2]))
    dh2 = O.expert_dh(dy, wd2, rounded=False)
    assert np.allclose(dh2[:, 2], 2.0 * dh[:, 2]) and np.allclose(np.delete(dh2, 2, 1), np.delete(dh, 2, 1))


def _case(rng, R, rank, T=18, H=8, E=8, k=2, F=6, rounded=False):
    """Our tokens, every rank's expert weights, and peers' rows consistent
    with those weights: rows a peer sends us are random, the rows it
    returns for ours are built from the expert each row was routed to."""
    el = E // R
    x = _w(rng, (T, H), 1.0)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    WG, WU, WD = _w(rng, (E, H, F), 0.4), _w(rng, (E, H, F), 0.4), _w(rng, (E, F, H), 0.4)
    pc = rng.integers(0, 3, (R, el)).astype(np.int32)
    pc[rank] = 0
    ps = [None if p == rank else _w(rng, (int(pc[p].sum()), H), 1.0) for p in range(R)]
    if rounded:
        psg = [None if p == rank else _w(rng, (int(pc[p].sum()), H), 1.0) for p in range(R)]
    else:
        psg = [None if p == rank else rng.standard_normal((int(pc[p].sum()), H)) for p in range(R)]
    dy = _w(rng, (T, H), 1.0)
    loc = slice(rank * el, (rank + 1) * el)
    c = dict(x=x, lg=lg, WG=WG, WU=WU, WD=WD, wg=WG[loc], wu=WU[loc], wd=WD[loc], pc=pc, ps=ps, psg=psg, dy=dy,
             R=R, rank=rank, k=k, el=el, E=E, rounded=rounded)
    # what each peer returns for the rows we send it: the forward result
    # and the data gradient of the expert each row belongs to
    cap = T * k
    zero = [None if p == rank else np.zeros((cap, H), np.uint16) for p in range(R)]
    zf = [None if p == rank else np.zeros((cap, H)) for p in range(R)]
    first = O.moe_layer_bwd(dy, x, lg, c["wg"], c["wu"], c["wd"], ps, pc, zero, psg, zf if not rounded else zero,
                            R, rank, k, rounded)
    offs = first["offsets"]
    so = first["send_off"]
    pr, prg = list(zero), list(zf if not rounded else zero)
    for d in range(R):
        if d == rank:
            continue
        pr[d], prg[d] = pr[d].copy(), prg[d].copy()
        for i in range(so[d + 1] - so[d]):
            e = int(np.searchsorted(offs, so[d] + i, side="right")) - 1
            row = first["send"][d][i:i + 1]
            pr[d][i] = O.expert_ffn(row, WG[e], WU[e], WD[e])[0]
            prg[d][i] = O.expert_ffn_bwd(row, first["send_grad"][d][i:i + 1], WG[e], WU[e], WD[e], rounded)[2][0]
    c["pr"], c["prg"] = pr, prg
    return c


def _bwd(c):
    return O.moe_layer_bwd(c["dy"], c["x"], c["lg"], c["wg"], c["wu"], c["wd"], c["ps"], c["pc"], c["pr"], c["psg"],
                           c["prg"], c["R"], c["rank"], c["k"], c["rounded"])


def _layer_loss(c, X, logits):
    """<dy, y> for the unrounded layer on float64 inputs (every expert here)."""
    dy = O.bf16_to_f64(c["dy"])
    idx, _ = O.router(c["lg"], c["k"])
    tot = 0.0
    for t in range(X.shape[0]):
        sel = logits[t, idx[t]]
        w = np.exp(sel - sel.max())
        w /= w.sum()
        for j in range(c["k"]):
            e = int(idx[t, j])
            y = _expert(X[t:t + 1], O.bf16_to_f64(c["WG"][e]), O.bf16_to_f64(c["WU"][e]), O.bf16_to_f64(c["WD"][e]))
            tot += w[j] * float(np.sum(dy[t] * y[0]))
    return tot


@pytest.mark.parametrize("R,rank", [(1, 0), (2, 1), (4, 2)])
def test_layer_dx_matches_finite_differences(R, rank):
    rng = np.random.default_rng(110 + R + rank)
    c = _case(rng, R, rank)
    out = _bwd(c)
    X = O.bf16_to_f64(c["x"])
    lg = c["lg"].astype(np.float64)
    eps = 1e-6
    for _ in range(3):
        v = rng.standard_normal(X.shape)
        fd = (_layer_loss(c, X + eps * v, lg) - _layer_loss(c, X - eps * v, lg)) / (2 * eps)
        assert abs(fd - np.sum(out["dx"] * v)) < 1e-6 * max(1.0, abs(fd)), (fd, np.sum(out["dx"] * v))


@pytest.mark.parametrize("R,rank", [(1, 0), (2, 0), (4, 3)])
def test_layer_dlogits_matches_finite_differences(R, rank):
    """Through the softmax over the selected logits; the expert results are
    the rounded forward's (the fold weighs rows that are already bf16), so
    the loss here uses those rows too, and a step too small to change the
    selection."""
    rng = np.random.default_rng(120 + R + rank)
    c = _case(rng, R, rank)
    out = _bwd(c)
    dy = O.bf16_to_f64(c["dy"])
    idx, _ = O.router(c["lg"], c["k"])
    T = idx.shape[0]
    res = np.zeros((T, c["k"]))
    for t in range(T):
        for j in range(c["k"]):
            e = int(idx[t, j])
            r = O.expert_ffn(c["x"][t:t + 1], c["WG"][e], c["WU"][e], c["WD"][e])[0]
            res[t, j] = float(dy[t] @ O.bf16_to_f64(r))

    def loss(L):
        tot = 0.0
        for t in range(T):
            sel = L[t, idx[t]]
            w = np.exp(sel - sel.max())
            tot += float((w / w.sum()) @ res[t])
        return tot

    lg = c["lg"].astype(np.float64)
    eps = 1e-7
    for _ in range(3):
        V = rng.standard_normal(lg.shape)
        for s in (1, -1):
            assert np.array_equal(O.router((lg + s * eps * V).astype(np.float32), c["k"])[0], idx)
        fd = (loss(lg + eps * V) - loss(lg - eps * V)) / (2 * eps)
        assert abs(fd - np.sum(out["dlogits"] * V)) < 1e-5 * max(1.0, abs(fd))
    sel = np.zeros_like(out["dlogits"], dtype=bool)
    np.put_along_axis(sel, idx, True, axis=1)
    assert np.all(out["dlogits"][~sel] == 0)


def test_dlogits_rows_sum_to_zero():
    """Shifting all of a token's logits leaves its softmax unchanged, so its
    router gradient sums to zero -- up to the weights' float32 rounding
    (their sum is 1 only to about 1e-7)."""
    rng = np.random.default_rng(130)
    c = _case(rng, 4, 1, k=3, rounded=True)
    out = _bwd(c)
    assert np.abs(out["dlogits"]).max() > 0.01
    assert np.max(np.abs(out["dlogits"].sum(axis=1))) < 1e-6 * np.abs(out["dlogits"]).max()


def test_k1_pair_gradients_are_dy():
    """k=1: every weight is 1, so the gradient a pair carries is dy itself,
    bit for bit, both in our own grouped rows and in what we send."""
    rng = np.random.default_rng(131)
    c = _case(rng, 4, 2, k=1, rounded=True)
    out = _bwd(c)
    assert np.all(out["w"] == 1.0)
    el, rank = c["el"], c["rank"]
    so = out["send_off"]
    for t in range(c["x"].shape[0]):
        e = int(out["idx"][t, 0])
        d = e // el
        pos = int(out["perm"][t])
        if d == rank:
            r = O.local_row(e, pos, rank, el, out["offsets"], out["grouped_offsets"], c["pc"])
            assert np.array_equal(out["grouped_grad"][r], c["dy"][t])
        else:
            assert np.array_equal(out["send_grad"][d][pos - so[d]], c["dy"][t])


def test_zero_down_projection_gives_zero_expert_gradient():
    """W_down = 0: dH = 0, so dG = dU = 0 and our experts contribute no
    data gradient; dx is then the bf16 sum of the peers' returned rows."""
    rng = np.random.default_rng(132)
    c = _case(rng, 2, 0, rounded=True)
    c["wd"] = np.zeros_like(c["wd"])
    out = _bwd(c)
    assert not np.any(O.bf16_to_f64(out["dg"])) and not np.any(O.bf16_to_f64(out["du"]))
    assert not np.any(O.bf16_to_f64(out["dx_grouped"]))
    el, rank = c["el"], c["rank"]
    so = out["send_off"]
    for t in range(c["x"].shape[0]):
        s = np.zeros(c["x"].shape[1])
        for j in range(c["k"]):
            e = int(out["idx"][t, j])
            d = e // el
            if d != rank:
                s += O.bf16_to_f64(c["prg"][d][int(out["perm"][t * c["k"] + j]) - so[d]])
        assert np.array_equal(out["dx"][t], O.round_bf16(s)), t


def test_returned_gradient_rows_through_their_own_expert():
    """Independent of the provenance table: row i that peer p sent us
    belongs to the local expert whose cumulative count range holds i, and
    the row we return at i is that expert's data gradient for that row and
    the gradient p sent with it."""
    rng = np.random.default_rng(133)
    c = _case(rng, 4, 1, rounded=True)
    out = _bwd(c)
    for p in range(c["R"]):
        if p == c["rank"]:
            assert out["out_return_grad"][p] is None
            continue
        bounds = np.cumsum(c["pc"][p])
        for i in range(int(bounds[-1])):
            el = int(np.searchsorted(bounds, i, side="right"))
            want = O.expert_ffn_bwd(c["ps"][p][i:i + 1], c["psg"][p][i:i + 1], c["wg"][el], c["wu"][el],
                                    c["wd"][el])[2][0]
            assert np.array_equal(out["out_return_grad"][p][i], want), (p, i)


def test_rounded_stays_within_bf16_error_of_unrounded():
    rng = np.random.default_rng(134)
    c = _case(rng, 2, 1, rounded=True)
    out = _bwd(c)
    cu = dict(c, rounded=False, prg=[None if a is None else O.bf16_to_f64(a) for a in c["prg"]],
              psg=[None if a is None else O.bf16_to_f64(a) for a in c["psg"]])
    ref = _bwd(cu)
    got = O.bf16_to_f64(out["dx"])
    err = np.linalg.norm(got - ref["dx"]) / np.linalg.norm(ref["dx"])
    assert err < 2e-2


def _ints(rng, shape):
    """bf16 bits of values in {-1, 0, 1}."""
    return O.round_bf16(rng.integers(-1, 2, shape).astype(np.float64))


def test_gate_up_kept_by_the_forward():
    """Rows and weights in {-1, 0, 1}: every X.Wg and X.Wu entry is an
    integer of magnitude <= H = 16, exact in bf16, so the kept copies are the
    brute-force sums themselves -- the gate from Wg, the up from Wu, each
    expert's rows with its own weights."""
    rng = np.random.default_rng(140)
    n, H, F = 5, 16, 6
    x = _ints(rng, (n, H))
    wg, wu = _ints(rng, (2, H, F)), _ints(rng, (2, H, F))
    X, G, U = O.bf16_to_f64(x), O.bf16_to_f64(wg), O.bf16_to_f64(wu)
    g, u = O.grouped_gate_up(x, [0, 2, 5], wg, wu)
    for r in range(n):
        e = 0 if r < 2 else 1
        for c in range(F):
            sg = sum(X[r, h] * G[e, h, c] for h in range(H))
            su = sum(X[r, h] * U[e, h, c] for h in range(H))
            assert O.bf16_to_f64(g[r, c]) == sg and O.bf16_to_f64(u[r, c]) == su, (r, c)
    assert not np.array_equal(g, u)


def test_saved_backward_equals_recompute_when_g_u_are_exact():
    """When X.Wg and X.Wu are exact in bf16 the kept copies are the values
    themselves, so the saved-activation backward is bit-identical to the
    recomputing one -- for one expert and for the whole layer."""
    rng = np.random.default_rng(141)
    n, H, F = 6, 16, 8
    x = _ints(rng, (n, H))
    wg, wu, wd = _ints(rng, (H, F)), _ints(rng, (H, F)), _w(rng, (F, H), 0.4)
    dy = _w(rng, (n, H), 1.0)
    a = O.expert_ffn_bwd(x, dy, wg, wu, wd, saved=False)
    b = O.expert_ffn_bwd(x, dy, wg, wu, wd, saved=True)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    assert np.any(O.bf16_to_f64(a[0])) and np.any(O.bf16_to_f64(a[1]))
    c = _case(rng, 2, 1, H=16, rounded=True)
    c["x"] = _ints(rng, c["x"].shape)
    c["wg"], c["wu"] = _ints(rng, c["wg"].shape), _ints(rng, c["wu"].shape)
    c["ps"] = [None if t is None else _ints(rng, t.shape) for t in c["ps"]]
    full = _bwd(c)
    kept = O.moe_layer_bwd(c["dy"], c["x"], c["lg"], c["wg"], c["wu"], c["wd"], c["ps"], c["pc"], c["pr"],
                           c["psg"], c["prg"], c["R"], c["rank"], c["k"], True, saved=True)
    for key in ("dg", "du", "dx_grouped", "dx", "dlogits"):
        assert np.array_equal(full[key], kept[key]), key


def test_saved_backward_stays_within_bf16_of_recompute():
    """General values: the kept g and u carry one bf16 rounding, which moves
    dG, dU and dX by about that much and no more."""
    rng = np.random.default_rng(142)
    c = _case(rng, 4, 2, rounded=True)
    full = _bwd(c)
    kept = O.moe_layer_bwd(c["dy"], c["x"], c["lg"], c["wg"], c["wu"], c["wd"], c["ps"], c["pc"], c["pr"],
                           c["psg"], c["prg"], c["R"], c["rank"], c["k"], True, saved=True)
    changed = False
    for key in ("dg", "du", "dx_grouped"):
        a, b = O.bf16_to_f64(full[key]), O.bf16_to_f64(kept[key])
        changed |= not np.array_equal(a, b)
        assert np.linalg.norm(a - b) <= 2e-2 * np.linalg.norm(a), key
    assert changed
