"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle function to a brute-force loop written
independently here, a closed form, an invariant of the definition, or a
special case that reduces to a library routine, so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import kos_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals):
    """Exactly representable small values -> bf16 bits (via fp32 top half)."""
    f = np.asarray(vals, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _ints(rng, shape, lo=-4, hi=4):
    return _bf16(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_bf16_golden_cases():
    g = json.load(open(os.path.join(GOLD, "bf16_rne.json")))
    for c in g["cases"]:
        got = int(O.round_bf16(np.array([c["f64"]]))[0])
        assert got == int(c["bf16"], 16), c


def test_bf16_roundtrip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    back = O.round_bf16(O.bf16_to_f64(finite))
    assert np.array_equal(back, finite)


def test_bf16_rounding_is_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))
    got = O.bf16_to_f64(O.round_bf16(x))
    # brute force: the two bf16 neighbours of x by truncating its fp32 bits
    f = x.astype(np.float32)
    lo_bits = (f.view(np.uint32) >> 16).astype(np.uint32)
    cands = np.stack([lo_bits - 1, lo_bits, lo_bits + 1], axis=1).astype(np.uint16)
    cv = O.bf16_to_f64(cands)
    d = np.abs(cv - x[:, None])
    best = cv[np.arange(len(x)), d.argmin(axis=1)]
    assert np.all(np.abs(got - x) <= np.abs(best - x))


# ---------------------------------------------------------------------------
# gather + GEMM
# ---------------------------------------------------------------------------

def test_gather_is_rank_order_concat():
    shards = [np.full((3, 5), p + 1, dtype=np.uint16) for p in range(4)]
    g = O.gather(shards)
    assert g.shape == (12, 5)
    for p in range(4):
        assert np.all(g[3 * p:3 * p + 3] == p + 1)


def test_gemm_golden_hand_example():
    g = json.load(open(os.path.join(GOLD, "gemm_2x3x2.json")))
    c = O.gemm(_bf16(g["a"]), _bf16(g["w"]))
    assert np.array_equal(c, np.array(g["c"], dtype=np.float64))


def test_gemm_vs_triple_loop_integers():
    rng = np.random.default_rng(2)
    a = _ints(rng, (7, 13))
    w = _ints(rng, (13, 5))
    af, wf = O.bf16_to_f64(a).tolist(), O.bf16_to_f64(w).tolist()
    ref = [[sum(af[i][k] * wf[k][j] for k in range(13)) for j in range(5)] for i in range(7)]
    assert np.array_equal(O.gemm(a, w), np.array(ref))


def test_gemm_identity_and_column_select():
    rng = np.random.default_rng(3)
    a = _ints(rng, (16, 8))
    eye = _bf16(np.eye(8))
    assert np.array_equal(O.gemm(a, eye), O.bf16_to_f64(a))
    e3 = np.zeros((8, 4), np.float32)
    e3[3, 1] = 1.0
    c = O.gemm(a, _bf16(e3))
    assert np.array_equal(c[:, 1], O.bf16_to_f64(a)[:, 3])
    assert np.all(c[:, [0, 2, 3]] == 0)


def test_ag_gemm_every_rank_same_result():
    rng = np.random.default_rng(4)
    R, m, K, N = 4, 6, 10, 7
    shards = [_ints(rng, (m, K)) for _ in range(R)]
    w = _ints(rng, (K, N))
    outs = []
    for r in range(R):
        peers = [None if p == r else shards[p] for p in range(R)]
        g, c = O.ag_gemm(shards[r], peers, w, r, out_dtype="f32")
        assert np.array_equal(g, np.concatenate(shards))
        outs.append(c)
    for c in outs[1:]:
        assert np.array_equal(c, outs[0])
    # integer results below 256 are exact in bf16 too
    g, cb = O.ag_gemm(shards[0], [None] + shards[1:], w, 0, out_dtype="bf16")
    cf = outs[0].astype(np.float64)
    small = np.abs(cf) <= 256
    assert np.array_equal(O.bf16_to_f64(cb)[small], cf[small])


# ---------------------------------------------------------------------------
# GEMM + reduce-scatter
# ---------------------------------------------------------------------------

def _rs_brute(a, w, peers, rank):
    af, wf = O.bf16_to_f64(a), O.bf16_to_f64(w)
    M, K = af.shape
    N = wf.shape[1]
    R = len(peers)
    mc = M // R
    y = np.zeros((mc, N))
    for i in range(mc):
        for j in range(N):
            s = 0.0
            for p in range(R):
                if p == rank:
                    s += sum(af[rank * mc + i, kk] * wf[kk, j] for kk in range(K))
                else:
                    s += float(peers[p][i, j])
            y[i, j] = s
    return y


@pytest.mark.parametrize("rank", [0, 2, 3])
def test_gemm_rs_vs_brute_force(rank):
    rng = np.random.default_rng(5 + rank)
    R, M, K, N = 4, 8, 6, 5
    a, w = _ints(rng, (M, K)), _ints(rng, (K, N))
    peers = [None if p == rank else rng.integers(-50, 50, (M // R, N)).astype(np.float32)
             for p in range(R)]
    partial, y = O.gemm_rs(a, w, peers, rank)
    assert np.array_equal(y, _rs_brute(a, w, peers, rank).astype(np.float32))
    assert np.array_equal(partial, O.gemm(a, w).astype(np.float32))


def test_gemm_rs_single_rank_is_gemm():
    rng = np.random.default_rng(6)
    a, w = _ints(rng, (8, 9)), _ints(rng, (9, 4))
    _, y = O.gemm_rs(a, w, [None], 0)
    assert np.array_equal(y, O.gemm(a, w).astype(np.float32))


def test_gemm_rs_zero_partial_sums_peers():
    rng = np.random.default_rng(7)
    R = 4
    a = _bf16(np.zeros((8, 3)))
    w = _ints(rng, (3, 5))
    peers = [None] + [np.full((2, 5), p, np.float32) for p in range(1, R)]
    _, y = O.gemm_rs(a, w, peers, 0)
    assert np.all(y == 1 + 2 + 3)


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def _router_brute(lg, k):
    idx, ws = [], []
    for row in lg.tolist():
        order = sorted(range(len(row)), key=lambda e: (-row[e], e))[:k]
        z = [np.exp(row[e] - row[order[0]]) for e in order]
        idx.append(order)
        ws.append([v / sum(z) for v in z])
    return np.array(idx), np.array(ws)


def test_router_vs_brute_force():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((50, 12)).astype(np.float32)
    lg[3, [2, 7, 9]] = 5.0            # a three-way tie at the top
    lg[4, 5] = lg[4, 1]               # an arbitrary tie
    lg[5, 0], lg[5, 1] = 0.0, -0.0    # +0 / -0 tie
    idx, w = O.router(lg, 4)
    bi, bw = _router_brute(lg, 4)
    assert np.array_equal(idx, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-6)
    assert list(idx[3, :3]) == [2, 7, 9]


def test_router_ties_go_to_lowest_index():
    lg = np.zeros((2, 8), np.float32)
    idx, w = O.router(lg, 3)
    assert idx.tolist() == [[0, 1, 2], [0, 1, 2]]
    np.testing.assert_allclose(w, 1.0 / 3, rtol=1e-7)


def test_router_k1_weight_is_one_and_k_eq_E_is_softmax():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((20, 6)).astype(np.float32)
    idx, w = O.router(lg, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], lg.argmax(axis=1))
    idx, w = O.router(lg, 6)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, idx, 1), rtol=1e-6)


def test_router_weights_sum_to_one_and_decrease():
    rng = np.random.default_rng(10)
    lg = (rng.standard_normal((300, 64)) * 3).astype(np.float32)
    idx, w = O.router(lg, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in idx.tolist())


# ---------------------------------------------------------------------------
# permutation / dispatch
# ---------------------------------------------------------------------------

def test_permute_brute_force_and_invariants():
    rng = np.random.default_rng(11)
    T, E, k = 40, 10, 3
    idx, _ = O.router(rng.standard_normal((T, E)).astype(np.float32), k)
    perm, offs = O.permute(idx, E)
    # brute force: walk experts, then tokens in order
    pos, ref = 0, np.empty(T * k, np.int64)
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    ref[t * k + j] = pos
                    pos += 1
    assert np.array_equal(perm, ref)
    assert np.array_equal(np.sort(perm), np.arange(T * k))       # a permutation
    counts = O.expert_counts(idx, E)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert counts.sum() == T * k and offs[-1] == T * k
    # unpermute(permute(x)) == x
    x = np.arange(T * k)
    packed = np.empty_like(x)
    packed[perm] = x
    assert np.array_equal(packed[perm], x)


def test_dispatch_provenance_by_brute_force():
    rng = np.random.default_rng(12)
    R, rank, T, H, E, k = 4, 1, 30, 8, 8, 3
    el = E // R
    x = _ints(rng, (T, H), -100, 100)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    pc = rng.integers(0, 5, (R, el)).astype(np.int32)
    pc[rank] = 0
    peer_send = [None if p == rank else _ints(rng, (int(pc[p].sum()), H), -100, 100)
                 for p in range(R)]
    d = O.dispatch(x, lg, peer_send, pc, R, rank, k)
    idx = d["idx"]
    # every send buffer row is the token whose (expert, t) comes at that place
    for dst in range(R):
        if dst == rank:
            continue
        want = [x[t] for e in range(dst * el, (dst + 1) * el)
                for t in range(T) if e in idx[t]]
        got = d["send"][dst]
        assert got.shape[0] == len(want)
        if want:
            assert np.array_equal(got, np.stack(want))
    # grouped rows: expert-major, then source rank, then source order
    want, src = [], []
    for e in range(el):
        for p in range(R):
            if p == rank:
                toks = [t for t in range(T) if rank * el + e in idx[t]]
                base = sum(1 for ee in range(rank * el, rank * el + e)
                           for t in range(T) if ee in idx[t])
                for n, t in enumerate(toks):
                    want.append(x[t])
                    src.append((p, base + n))
            else:
                lo = int(pc[p, :e].sum())
                for i in range(lo, lo + int(pc[p, e])):
                    want.append(peer_send[p][i])
                    src.append((p, i))
    assert np.array_equal(d["grouped"], np.stack(want))
    assert d["row_src"].tolist() == [list(s) for s in src]
    assert d["grouped_offsets"][-1] == len(want)


# ---------------------------------------------------------------------------
# expert FFN, push, fold
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    z = np.array([0.0, 40.0, -40.0, 1.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 40.0) < 1e-12 and abs(s[2]) < 1e-15
    assert abs(s[3] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15


def test_ffn_vs_float64_loop():
    rng = np.random.default_rng(13)
    n, H, F = 5, 12, 6
    x = O.round_bf16(rng.standard_normal((n, H)))
    wg = O.round_bf16(rng.standard_normal((H, F)) / np.sqrt(H))
    wu = O.round_bf16(rng.standard_normal((H, F)) / np.sqrt(H))
    wd = O.round_bf16(rng.standard_normal((F, H)) / np.sqrt(F))
    X, G, U, D = (O.bf16_to_f64(v).tolist() for v in (x, wg, wu, wd))
    h = np.zeros((n, F))
    for i in range(n):
        for f in range(F):
            g = sum(X[i][c] * G[c][f] for c in range(H))
            u = sum(X[i][c] * U[c][f] for c in range(H))
            h[i, f] = g / (1 + np.exp(-g)) * u
    hb = O.bf16_to_f64(O.round_bf16(h)).tolist()
    y = [[sum(hb[i][f] * D[f][c] for f in range(F)) for c in range(H)] for i in range(n)]
    got = O.expert_ffn(x, wg, wu, wd)
    assert np.array_equal(got, O.round_bf16(np.array(y)))
    assert np.array_equal(O.expert_hidden(x, wg, wu), O.round_bf16(h))


def test_ffn_selection_closed_form():
    """Selection weights reduce the expert to arithmetic checkable by hand:
    gate column f reads input column a[f] times 40, up column f reads input
    column b[f], down output column c reads hidden column d[c].  With inputs
    of +-1, silu(+40) = 40 to 1e-15 and silu(-40) = 0 to 1e-15, so
    y[t, c] = 40 * x[t, b[d[c]]] where x[t, a[d[c]]] = +1 and ~0 where it is
    -1.  Swapping the gate and up roles, an index or the operand order fails
    this (silu(+-1) * 40 is neither 40 nor ~0)."""
    rng = np.random.default_rng(21)
    n, H, F = 6, 7, 4
    a = [5, 0, 3, 6]          # gate source column of hidden f
    b = [2, 4, 1, 0]          # up source column of hidden f
    d = [3, 1, 0, 2, 2, 1, 3]  # hidden column feeding output column c
    xs = rng.choice([-1.0, 1.0], size=(n, H))
    wg, wu, wd = np.zeros((H, F)), np.zeros((H, F)), np.zeros((F, H))
    for f in range(F):
        wg[a[f], f] = 40.0
        wu[b[f], f] = 1.0
    for c in range(H):
        wd[d[c], c] = 1.0
    x16, wg16, wu16, wd16 = O.round_bf16(xs), O.round_bf16(wg), O.round_bf16(wu), O.round_bf16(wd)
    y = O.bf16_to_f64(O.expert_ffn(x16, wg16, wu16, wd16))
    h = O.bf16_to_f64(O.expert_hidden(x16, wg16, wu16))
    for t in range(n):
        for f in range(F):
            if xs[t, a[f]] > 0:
                assert h[t, f] == 40.0 * xs[t, b[f]], (t, f)
            else:
                assert abs(h[t, f]) < 1e-15, (t, f)
    for t in range(n):
        for c in range(H):
            f = d[c]
            if xs[t, a[f]] > 0:
                assert y[t, c] == 40.0 * xs[t, b[f]], (t, c)
            else:
                assert abs(y[t, c]) < 1e-15, (t, c)


def test_ffn_zero_up_gives_zero():
    rng = np.random.default_rng(14)
    x = O.round_bf16(rng.standard_normal((4, 8)))
    wg = O.round_bf16(rng.standard_normal((8, 4)))
    wu = np.zeros((8, 4), np.uint16)
    wd = O.round_bf16(rng.standard_normal((4, 8)))
    assert np.all(O.bf16_to_f64(O.expert_ffn(x, wg, wu, wd)) == 0)


def _tiny_moe(rng, R=4, rank=2, T=24, H=8, E=8, k=2, F=4):
    el = E // R
    x = _ints(rng, (T, H), -3, 3)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    pc = rng.integers(0, 4, (R, el)).astype(np.int32)
    pc[rank] = 0
    ps = [None if p == rank else _ints(rng, (int(pc[p].sum()), H), -3, 3) for p in range(R)]
    cap = T * min(k, el)
    pr = [None if p == rank else _ints(rng, (cap, H), -3, 3) for p in range(R)]
    wg = np.stack([_ints(rng, (H, F), -1, 1) for _ in range(el)])
    wu = np.stack([_ints(rng, (H, F), -1, 1) for _ in range(el)])
    wd = np.stack([_ints(rng, (F, H), -1, 1) for _ in range(el)])
    return dict(x=x, lg=lg, pc=pc, ps=ps, pr=pr, wg=wg, wu=wu, wd=wd, R=R, rank=rank, k=k)


def test_push_rows_equal_expert_outputs():
    rng = np.random.default_rng(15)
    m = _tiny_moe(rng)
    out = O.moe_layer(m["x"], m["lg"], m["wg"], m["wu"], m["wd"], m["ps"], m["pc"], m["pr"],
                      m["R"], m["rank"], m["k"])
    for r, (p, i) in enumerate(out["row_src"]):
        if p != m["rank"]:
            assert np.array_equal(out["out_return"][p][i], out["y_grouped"][r])
    # push + the sources' own rows cover every grouped row exactly once
    n_peer = sum(o.shape[0] for o in out["out_return"] if o is not None)
    n_own = int((out["row_src"][:, 0] == m["rank"]).sum())
    assert n_peer + n_own == out["grouped"].shape[0]


def test_push_returns_each_peer_row_through_its_own_expert():
    """Independent of the provenance table and of push's own loop: peer p
    sends its rows expert-major over our local experts (peer_counts[p] rows
    per expert, in order), so row i it sent belongs to the local expert
    whose cumulative count range holds i, and the row we return at i must be
    that expert's FFN of exactly that input row."""
    rng = np.random.default_rng(19)
    for rank in (0, 2):
        m = _tiny_moe(rng, rank=rank, T=20, k=2)
        out = O.moe_layer(m["x"], m["lg"], m["wg"], m["wu"], m["wd"], m["ps"], m["pc"], m["pr"],
                          m["R"], m["rank"], m["k"])
        for p in range(m["R"]):
            if p == rank:
                assert out["out_return"][p] is None
                continue
            bounds = np.cumsum(m["pc"][p])
            n_p = int(bounds[-1]) if bounds.size else 0
            assert out["out_return"][p].shape[0] == n_p == m["ps"][p].shape[0]
            for i in range(n_p):
                el = int(np.searchsorted(bounds, i, side="right"))
                want = O.expert_ffn(m["ps"][p][i:i + 1], m["wg"][el], m["wu"][el], m["wd"][el])[0]
                assert np.array_equal(out["out_return"][p][i], want), (rank, p, i)


def test_push_catches_a_swapped_source():
    """A planted provenance mistake (two peer rows of different experts
    swapped in row_src) moves results to the wrong return slots: the
    independent pin above would fail on it."""
    rng = np.random.default_rng(20)
    m = _tiny_moe(rng, rank=1, T=20, k=2)
    m["pc"][0] = [2, 2]
    m["ps"][0] = _ints(rng, (4, 8), -3, 3)
    out = O.moe_layer(m["x"], m["lg"], m["wg"], m["wu"], m["wd"], m["ps"], m["pc"], m["pr"],
                      m["R"], m["rank"], m["k"])
    rs = out["row_src"].copy()
    r0 = int(np.where((rs[:, 0] == 0) & (rs[:, 1] == 0))[0][0])
    r3 = int(np.where((rs[:, 0] == 0) & (rs[:, 1] == 3))[0][0])
    rs[[r0, r3]] = rs[[r3, r0]]
    bad = O.push(out["y_grouped"], rs, m["R"], 1, m["pc"].sum(axis=1))
    want0 = O.expert_ffn(m["ps"][0][0:1], m["wg"][0], m["wu"][0], m["wd"][0])[0]
    assert np.array_equal(out["out_return"][0][0], want0)
    if not np.array_equal(out["y_grouped"][r0], out["y_grouped"][r3]):
        assert not np.array_equal(bad[0][0], want0)


def test_fold_k1_is_the_result_row():
    rng = np.random.default_rng(16)
    m = _tiny_moe(rng, k=1)
    out = O.moe_layer(m["x"], m["lg"], m["wg"], m["wu"], m["wd"], m["ps"], m["pc"], m["pr"],
                      m["R"], m["rank"], 1)
    el = 8 // m["R"]
    so = O.send_offsets(out["offsets"], m["R"], el)
    for t in range(m["x"].shape[0]):
        e = int(out["idx"][t, 0])
        d = e // el
        pos = int(out["perm"][t])
        if d == m["rank"]:
            r = O.local_row(e, pos, m["rank"], el, out["offsets"], out["grouped_offsets"], m["pc"])
            want = out["y_grouped"][r]
        else:
            want = m["pr"][d][pos - so[d]]
        assert np.array_equal(out["y"][t], want)


def test_fold_equal_weights_exact():
    # w = 1/4 for every slot (equal logits) and integer results: exact sums
    rng = np.random.default_rng(17)
    m = _tiny_moe(rng, k=4, E=8)
    m["lg"] = np.zeros_like(m["lg"])
    out = O.moe_layer(m["x"], m["lg"], m["wg"], m["wu"], m["wd"], m["ps"], m["pc"], m["pr"],
                      m["R"], m["rank"], 4)
    assert np.all(out["w"] == 0.25)
    assert out["idx"].tolist() == [[0, 1, 2, 3]] * m["x"].shape[0]
    el = 2
    so = O.send_offsets(out["offsets"], m["R"], el)
    for t in range(m["x"].shape[0]):
        s = np.zeros(m["x"].shape[1])
        for j in range(4):
            e = j
            d = e // el
            pos = int(out["perm"][t * 4 + j])
            if d == m["rank"]:
                r = O.local_row(e, pos, m["rank"], el, out["offsets"], out["grouped_offsets"], m["pc"])
                s += O.bf16_to_f64(out["y_grouped"][r])
            else:
                s += O.bf16_to_f64(m["pr"][d][pos - so[d]])
        assert np.array_equal(O.bf16_to_f64(out["y"][t]), O.bf16_to_f64(O.round_bf16(s / 4)))


def test_moe_layer_vs_independent_loop():
    """Whole layer on a tiny case against a loop that recomputes every
    token's output from scratch (router by sorting, FFN per row)."""
    rng = np.random.default_rng(18)
    m = _tiny_moe(rng, T=16, k=2)
    R, rank, k = m["R"], m["rank"], m["k"]
    E = m["lg"].shape[1]
    el = E // R
    out = O.moe_layer(m["x"], m["lg"], m["wg"], m["wu"], m["wd"], m["ps"], m["pc"], m["pr"],
                      R, rank, k)
    bi, bw = _router_brute(m["lg"], k)
    # our send order to d: (expert, token) ascending; position inside d's rows
    for t in range(16):
        acc = np.zeros(m["x"].shape[1])
        for j in range(k):
            e = int(bi[t, j])
            d = e // el
            if d == rank:
                ee = e - rank * el
                row = O.expert_ffn(m["x"][t:t + 1], m["wg"][ee], m["wu"][ee], m["wd"][ee])[0]
                res = O.bf16_to_f64(row)
            else:
                before = sum(1 for e2 in range(d * el, e) for t2 in range(16) if e2 in bi[t2])
                before += sum(1 for t2 in range(t) if e in bi[t2])
                res = O.bf16_to_f64(m["pr"][d][before])
            acc += bw[t, j] * res
        assert np.array_equal(out["y"][t], O.round_bf16(acc)), t


# ---------------------------------------------------------------------------
# transposed weights (backward data-gradient products)
# ---------------------------------------------------------------------------

def test_ag_gemm_wt_vs_triple_loop():
    rng = np.random.default_rng(21)
    R, m, K, N = 3, 2, 5, 4
    shards = [_ints(rng, (m, K)) for _ in range(R)]
    wt = _ints(rng, (N, K))                      # stored n x k
    g, c = O.ag_gemm_wt(shards[1], [shards[0], None, shards[2]], wt, 1, "f32")
    G = np.vstack([O.bf16_to_f64(x) for x in shards])
    W = O.bf16_to_f64(wt)
    for i in range(R * m):
        for j in range(N):
            assert c[i, j] == sum(G[i, k] * W[j, k] for k in range(K))


def test_gemm_rs_wt_vs_triple_loop():
    rng = np.random.default_rng(22)
    R, M, K, N = 2, 4, 3, 5
    a = _ints(rng, (M, K))
    wt = _ints(rng, (N, K))
    peers = [None, rng.integers(-9, 9, size=(M // R, N)).astype(np.float32)]
    partial, y = O.gemm_rs_wt(a, wt, peers, 0)
    A, W = O.bf16_to_f64(a), O.bf16_to_f64(wt)
    for i in range(M):
        for j in range(N):
            assert partial[i, j] == sum(A[i, k] * W[j, k] for k in range(K))
    assert np.array_equal(y, (partial[:M // R].astype(np.float64) + peers[1]).astype(np.float32))
