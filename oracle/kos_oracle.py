"""CPU oracle for the fused GEMM+collective kernels -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path (the HIP
library and its Python binding) never does, and shares no code with it.

What it computes are the plain definitions of the collectives and products
that the KOSMOS persistent kernels fuse.  The kernels only change *when* and
*by whom* each piece is computed (self-scheduling workgroups, consumer-ordered
queues, ready flags); the values they must produce are those of the unfused
operations, which is what is written out here, one step at a time, in the
order the pages describe them:

* all-gather of sequence shards before a column-parallel GEMM, and scatter and
  add of the partial results after a row-parallel GEMM [KOSMOS explainer,
  "Start with the problem" paragraph];
* the whole expert layer, routing through the final weighted sum: each
  token's row goes to the rank owning its expert and the result comes back
  [same paragraph; KOSMOS arXiv abstract];
* the same two TP+SP collectives with MXFP8 operands [KOSMOS arXiv abstract],
  the format taken from the OCP Microscaling specification v1.0;
* the expert layer's backward direction [KOSMOS arXiv abstract, one launch
  per direction]: the chain rule of the forward definition, written out
  step by step (gradients of the pairs dispatched like the tokens, the
  experts' data gradient, the results pushed back and summed, the router
  gradient through the softmax over the selected logits).

Arithmetic is float64 (NumPy/BLAS), which is exact for every integer-valued
case and more accurate than the kernels' fp32 accumulation otherwise.  bf16
values enter as uint16 bit patterns and are widened exactly; a bf16 result is
the round-to-nearest-even of the float64 value.

Readings where the pages are silent (rank-order gather, K x N weights, top-k
then softmax over the k, ties to the lowest expert index, expert-major
permutation, contiguous expert->rank map, no dedup, SwiGLU rounding points)
are stated at each function.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, invariants).
``expert_ffn`` is pinned by a float64 brute-force loop on random inputs and by
a closed-form case of selection weights (gate and up roles, indices, the
SiLU's asymmetry); the pages print no worked example to pin a value to.
The backward functions are pinned in ``tests/test_oracle_bwd_pins.py`` by
central finite differences of an unrounded forward written out there, and
by special cases and the softmax invariant; the variant that takes the
forward's bf16 copies of g and u (``expert_gate_up``, ``saved=True``) by a
brute-force sum on integer inputs, by equality with the recomputing
backward where those copies are exact, and by bf16-sized distance to it
otherwise.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16 <-> float
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bf16, ties to even; returns uint16.

    The rounding is done on the exact float64 value (no double rounding via
    fp32): x = m * 2^e with 0.5 <= |m| < 1, bf16 keeps 8 significant bits, so
    the quantum is 2^(e-8), or 2^-133 in bf16's subnormal range.  Values past
    the largest finite bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    r = np.rint(x / q) * q          # np.rint rounds half to even
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)    # exact: r has <= 8 significant bits
        big = np.abs(r) > 3.3895313892515355e38   # 0x7F7F, largest finite bf16
    f = np.where(big, np.copysign(np.float32(np.inf), f), f)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# all-gather + GEMM
# ---------------------------------------------------------------------------


def gather(shards) -> np.ndarray:
    """The gathered input: shard p's rows at rows [p*m, (p+1)*m), rank order.

    Sequence-parallel shards split the sequence into contiguous pieces, so
    gathering them is concatenation in rank order [KOSMOS explainer, "Start
    with the problem"].  Bit copy: the result is the input bytes."""
    return np.concatenate([np.asarray(s, dtype=np.uint16) for s in shards], axis=0)


def gemm(a_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """C = A . W in float64 for bf16 A [M,K] and bf16 W [K,N] (row-major,
    weight stored K x N)."""
    return bf16_to_f64(a_bits) @ bf16_to_f64(w_bits)


def ag_gemm(a_local, a_peers, w_bits, rank: int, out_dtype: str = "bf16"):
    """All-gather then GEMM: returns (gathered uint16 [R*m,K], C).

    ``a_peers[p]`` is rank p's shard (entry ``rank`` ignored).  C is bf16 bits
    (nearest even of the exact product) or float32."""
    shards = [a_local if p == rank else a_peers[p] for p in range(len(a_peers))]
    g = gather(shards)
    c = gemm(g, w_bits)
    if out_dtype == "bf16":
        return g, round_bf16(c)
    return g, c.astype(np.float32)


# ---------------------------------------------------------------------------
# GEMM + reduce-scatter
# ---------------------------------------------------------------------------


def gemm_rs(a_bits, w_bits, peer_slices, rank: int):
    """GEMM then reduce-scatter, seen from rank ``rank`` of R.

    P = A . W is this rank's partial sum of the full [M,N] output.  Chunk c is
    rows [c*M/R, (c+1)*M/R); the scatter sends chunk c to rank c, which adds
    the R partials of its chunk [KOSMOS explainer, "Start with the problem"].
    ``peer_slices[p]`` (fp32 [M/R,N]) is rank p's partial for chunk ``rank``.

    Returns (partial fp32 [M,N], y fp32 [M/R,N]) with
    y = sum over p = 0..R-1, ascending, of X_p, X_rank = P[chunk rank]."""
    partial = gemm(a_bits, w_bits).astype(np.float32)   # what the builders store
    return partial, reduce_chunk(partial, peer_slices, rank)


def reduce_chunk(partial, peer_slices, rank: int) -> np.ndarray:
    """This rank's chunk of the reduce-scatter: y = sum over p = 0..R-1,
    ascending, of X_p, with X_rank = rows [rank*M/R, (rank+1)*M/R) of the fp32
    ``partial`` and X_p = ``peer_slices[p]``; summed in float64, returned as
    float32."""
    R = len(peer_slices)
    M = partial.shape[0]
    mc = M // R
    acc = np.zeros((mc, partial.shape[1]), dtype=np.float64)
    for p in range(R):
        if p == rank:
            acc += partial[rank * mc:(rank + 1) * mc].astype(np.float64)
        else:
            acc += np.asarray(peer_slices[p], dtype=np.float32).astype(np.float64)
    return acc.astype(np.float32)


# ---------------------------------------------------------------------------
# the same collectives with the weight stored transposed (backward pass)
# ---------------------------------------------------------------------------
#
# The data-gradient products of the backward pass multiply by the transposed
# forward weight: the backward of Y = AG(X) . W is a reduce-scatter of
# dY . W^T, the backward of Y = RS(X . W) an all-gather of dY followed by
# . W^T [KOSMOS arXiv abstract: every TP+SP collective of the layer is
# fused].  W^T is given as stored, [n, k].


def ag_gemm_wt(a_local, a_peers, w_t_bits, rank: int, out_dtype: str = "bf16"):
    """``ag_gemm`` with C = G . W^T, W^T bf16 [n, k]."""
    return ag_gemm(a_local, a_peers, np.asarray(w_t_bits, dtype=np.uint16).T, rank, out_dtype)


def gemm_rs_wt(a_bits, w_t_bits, peer_slices, rank: int):
    """``gemm_rs`` with P = A . W^T, W^T bf16 [n, k]."""
    return gemm_rs(a_bits, np.asarray(w_t_bits, dtype=np.uint16).T, peer_slices, rank)


# ---------------------------------------------------------------------------
# MXFP8 operands (the same two collectives with microscaled fp8 inputs)
# ---------------------------------------------------------------------------
#
# The pages report MXFP8 speed-ups for the same fused collectives [KOSMOS
# arXiv abstract] and do not restate the format.  Its definition is the OCP
# Microscaling (MX) specification v1.0: a block of 32 consecutive elements
# shares one E8M0 scale (the power of two 2^(s-127), s = 255 is NaN); each
# element is FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; no
# infinities; S.1111.111 is NaN; exponent field 0 holds the subnormals
# m/8 * 2^-6).  The value of element k of a row is its E4M3 value times
# 2^(s_block(k) - 127).  Reading for the products: blocks run along K (the
# reduction dimension) for both operands, so the row of A and the column of
# the weight are both scaled per 32-element piece of K; the weight is stored
# N x K (each output column's K values contiguous, with its scales), the
# layout MX products consume.


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of FP8 E4M3 codes (uint8): (-1)^s * 2^(e-7) * (1 + m/8)
    for exponent field e >= 1, (-1)^s * 2^-6 * m/8 for e = 0; the codes
    0x7F and 0xFF are NaN [OCP MX v1.0, FP8 E4M3]."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale codes (uint8): 2^(s - 127), s = 255 is NaN [OCP MX
    v1.0, E8M0]."""
    s = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(np.ones(s.shape), (s - 127).astype(np.int32))
    return np.where(s == 255, np.nan, v)


MX_BLOCK = 32


def mx_to_f64(data: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Rows of MX elements as float64: data uint8 [R, K] (E4M3 codes), scales
    uint8 [R, K/32] (E8M0, block b covers columns [32b, 32b+32))."""
    d = np.asarray(data, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    R, K = d.shape
    assert K % MX_BLOCK == 0 and s.shape == (R, K // MX_BLOCK)
    return e4m3_to_f64(d) * np.repeat(e8m0_to_f64(s), MX_BLOCK, axis=1)


def scales_from_slabs(slabs: np.ndarray) -> np.ndarray:
    """Row-major scales [R, K/32] from the kernels' slab layout [K/64, R, 2]:
    slab s holds, for row r, blocks 2s and 2s+1 (the layout the MX entry
    points take, chosen so a tile's scales for one 64-wide step of K are one
    contiguous run)."""
    sl = np.asarray(slabs, dtype=np.uint8)
    S, R, two = sl.shape
    assert two == 2
    return np.ascontiguousarray(sl.transpose(1, 0, 2)).reshape(R, 2 * S)


def gemm_mx(a, a_scales, w, w_scales) -> np.ndarray:
    """C = A . W^T in float64: A [M,K] and W [N,K] MX operands (E4M3 codes
    with per-32 E8M0 scales along K)."""
    return mx_to_f64(a, a_scales) @ mx_to_f64(w, w_scales).T


def ag_gemm_mx(a_local, s_local, a_peers, s_peers, w, w_scales, rank: int, out_dtype: str = "bf16"):
    """All-gather of MX shards (codes and their scales, rank order; a bit
    copy), then the MX product.  Returns (gathered codes [R*m,K], gathered
    scales [R*m,K/32], C) with C as in ``ag_gemm``."""
    R = len(a_peers)
    g = np.concatenate([np.asarray(a_local if p == rank else a_peers[p], dtype=np.uint8) for p in range(R)], axis=0)
    gs = np.concatenate([np.asarray(s_local if p == rank else s_peers[p], dtype=np.uint8) for p in range(R)], axis=0)
    c = gemm_mx(g, gs, w, w_scales)
    if out_dtype == "bf16":
        return g, gs, round_bf16(c)
    return g, gs, c.astype(np.float32)


def gemm_rs_mx(a, a_scales, w, w_scales, peer_slices, rank: int):
    """MX product then reduce-scatter, as ``gemm_rs``: returns (partial fp32
    [M,N], y fp32 [M/R,N])."""
    partial = gemm_mx(a, a_scales, w, w_scales).astype(np.float32)
    return partial, reduce_chunk(partial, peer_slices, rank)


# ---------------------------------------------------------------------------
# expert layer: router, permutation, dispatch, FFN, push, fold
# ---------------------------------------------------------------------------


def router(logits: np.ndarray, k: int):
    """Top-k experts per token and their combine weights.

    Selection: experts in order of descending logit, ties to the lowest
    expert index (a stable sort of the negated logits; -0.0 ties +0.0).
    Weights: softmax over the k selected logits, which equals the full
    softmax renormalised over the k, so they sum to 1.  Returns
    (idx int32 [T,k], w float32 [T,k])."""
    lg = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-lg, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(lg, idx, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """counts[e] = number of (token, slot) pairs routed to expert e."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=n_experts).astype(np.int32)


def permute(idx: np.ndarray, n_experts: int):
    """Expert-major packed order of the (token, slot) pairs.

    Pair (t, j) routed to e gets position offset[e] + (number of tokens t' < t
    routed to e), offset the exclusive scan of the counts (a token reaches an
    expert at most once).  Returns (perm int32 [T*k], offsets int32 [E+1]);
    perm[t*k+j] is the pair's position."""
    flat = np.asarray(idx).reshape(-1)
    counts = expert_counts(idx, n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")     # by (expert, t, j)
    perm = np.empty(flat.size, dtype=np.int64)
    perm[order] = np.arange(flat.size)
    return perm.astype(np.int32), offsets.astype(np.int32)


def send_offsets(offsets: np.ndarray, world: int, e_local: int) -> np.ndarray:
    """Destination d holds experts [d*E_loc, (d+1)*E_loc) (contiguous map), so
    its rows are packed positions [offsets[d*E_loc], offsets[(d+1)*E_loc])."""
    return np.array([offsets[d * e_local] for d in range(world + 1)], dtype=np.int64)


def dispatch(x_bits, logits, peer_send, peer_counts, world: int, rank: int, k: int):
    """Router -> permutation -> token movement, for rank ``rank``.

    Returns a dict with idx, w, counts, perm, offsets, send (list: rows for
    each destination d != rank, in our packed order), grouped (rows of our
    local experts, expert-major, then by source rank, then in the source's
    packed order), grouped_offsets [E_loc+1] and row_src [rows, 2] = (source
    rank, row index in what that source sends us)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, E = logits.shape
    el = E // world
    idx, w = router(logits, k)
    counts = expert_counts(idx, E)
    perm, offsets = permute(idx, E)
    token_of = np.empty(T * k, dtype=np.int64)
    token_of[perm] = np.arange(T * k) // k
    packed = x_bits[token_of]
    so = send_offsets(offsets, world, el)
    send = [None if d == rank else packed[so[d]:so[d + 1]] for d in range(world)]
    pc = np.asarray(peer_counts, dtype=np.int64)
    rows, src = [], []
    gofs = [0]
    for e in range(el):
        ge = rank * el + e
        for p in range(world):
            if p == rank:
                lo, hi = offsets[ge], offsets[ge + 1]
                rows.append(packed[lo:hi])
                src += [(p, i - so[rank]) for i in range(lo, hi)]
            else:
                lo = int(pc[p, :e].sum())
                n = int(pc[p, e])
                rows.append(np.asarray(peer_send[p], dtype=np.uint16)[lo:lo + n])
                src += [(p, i) for i in range(lo, lo + n)]
        gofs.append(sum(r.shape[0] for r in rows))
    grouped = np.concatenate(rows, axis=0) if rows else np.zeros((0, x_bits.shape[1]), np.uint16)
    return dict(idx=idx, w=w, counts=counts, perm=perm, offsets=offsets,
                send_off=so, send=send, grouped=grouped,
                grouped_offsets=np.array(gofs, dtype=np.int32),
                row_src=np.array(src, dtype=np.int32).reshape(-1, 2))


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x_bits, wg_bits, wu_bits, wd_bits) -> np.ndarray:
    """SwiGLU expert on rows X (bf16 [n,H]):
    h = bf16(silu(X.Wg) * (X.Wu)), Y = bf16(h.Wd); returns uint16 [n,H].

    Rows are independent, so any subset of rows can be evaluated alone."""
    x = bf16_to_f64(x_bits)
    g = x @ bf16_to_f64(wg_bits)
    u = x @ bf16_to_f64(wu_bits)
    h = round_bf16(silu(g) * u)
    return round_bf16(bf16_to_f64(h) @ bf16_to_f64(wd_bits))


def expert_hidden(x_bits, wg_bits, wu_bits) -> np.ndarray:
    """The rounded SwiGLU hidden h = bf16(silu(X.Wg) * (X.Wu))."""
    x = bf16_to_f64(x_bits)
    return round_bf16(silu(x @ bf16_to_f64(wg_bits)) * (x @ bf16_to_f64(wu_bits)))


def grouped_ffn(grouped, grouped_offsets, wg, wu, wd) -> np.ndarray:
    """Expert FFN over every local expert's rows (expert e: rows
    [grouped_offsets[e], grouped_offsets[e+1]))."""
    out = np.zeros_like(np.asarray(grouped, dtype=np.uint16))
    for e in range(len(grouped_offsets) - 1):
        lo, hi = int(grouped_offsets[e]), int(grouped_offsets[e + 1])
        if hi > lo:
            out[lo:hi] = expert_ffn(grouped[lo:hi], wg[e], wu[e], wd[e])
    return out


def push(y_grouped, row_src, world: int, rank: int, peer_rows):
    """Results travel back: row r of the grouped output whose source is
    (p, i), p != rank, goes to row i of what we return to p.  ``peer_rows[p]``
    is how many rows p sent us.  Returns a list (None at ``rank``)."""
    out = [None if p == rank else np.zeros((int(peer_rows[p]), y_grouped.shape[1]), np.uint16)
           for p in range(world)]
    for r, (p, i) in enumerate(np.asarray(row_src)):
        if p != rank:
            out[p][i] = y_grouped[r]
    return out


def local_row(e, pos, rank, e_local, offsets, grouped_offsets, peer_counts):
    """Grouped row holding our own pair at packed position ``pos`` of expert
    ``e`` (a local expert): after the rows of sources p < rank."""
    el = e - rank * e_local
    before = int(np.asarray(peer_counts)[:rank, el].sum())
    return int(grouped_offsets[el]) + before + int(pos - offsets[e])


def fold(idx, w, perm, offsets, y_grouped, grouped_offsets, peer_counts,
         peer_return, world: int, rank: int, tokens=None):
    """y[t] = bf16(sum_j w[t,j] * res[t,j]), j ascending.

    res[t,j] is the local expert output when expert idx[t,j] lives here,
    otherwise row perm[t*k+j] - send_off[d] of what rank d returned.
    ``tokens`` restricts the evaluation to a subset (rows are independent).
    ``y_grouped`` must hold the local results the chosen tokens need."""
    idx = np.asarray(idx)
    T, k = idx.shape
    E = int(len(offsets) - 1)
    el = E // world
    so = send_offsets(offsets, world, el)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), np.asarray(y_grouped).shape[1]), dtype=np.float64)
    for n, t in enumerate(toks):
        for j in range(k):
            e = int(idx[t, j])
            d = e // el
            pos = int(perm[t * k + j])
            if d == rank:
                r = local_row(e, pos, rank, el, offsets, grouped_offsets, peer_counts)
                res = bf16_to_f64(y_grouped[r])
            else:
                res = bf16_to_f64(peer_return[d][pos - so[d]])
            out[n] += float(w[t, j]) * res
    return round_bf16(out)


def moe_layer(x_bits, logits, wg, wu, wd, peer_send, peer_counts, peer_return,
              world: int, rank: int, k: int):
    """The whole expert layer for one rank: dispatch, expert FFN, push, fold."""
    d = dispatch(x_bits, logits, peer_send, peer_counts, world, rank, k)
    yg = grouped_ffn(d["grouped"], d["grouped_offsets"], wg, wu, wd)
    pc = np.asarray(peer_counts)
    out_return = push(yg, d["row_src"], world, rank, pc.sum(axis=1))
    y = fold(d["idx"], d["w"], d["perm"], d["offsets"], yg, d["grouped_offsets"],
             pc, peer_return, world, rank)
    d.update(y_grouped=yg, out_return=out_return, y=y)
    return d


# ---------------------------------------------------------------------------
# expert layer, backward direction: the gradient of the layer's output with
# respect to its input tokens and router logits [KOSMOS arXiv abstract: one
# launch per direction of the expert layer]
# ---------------------------------------------------------------------------
#
# The pages give no formula for the backward pass; it is the chain rule of
# the forward definition above, read this way.  With dy = dL/dy (bf16 [T,H])
# and y[t] = sum_j w[t,j] * res[t,j]:
#   * each pair's output gradient dres[t,j] = w[t,j] * dy[t] travels to the
#     rank of expert idx[t,j] as a bf16 row, in the forward's packed order;
#   * the expert recomputes g = X.Wg and u = X.Wu from its forward input rows
#     (only the grouped inputs are kept from the forward), then
#     dH = dres . Wd^T, dU = dH * silu(g), dG = dH * u * silu'(g) (the
#     forward's bf16 rounding of h passes the gradient unchanged), each
#     rounded to bf16, and dX = dG . Wg^T + dU . Wu^T, rounded to bf16;
#   * dX rows travel back to their source rank, which sums them:
#     dx[t] = bf16(sum_j dX[t,j]) (the weight is already in dres);
#   * the router gradient: dw[t,j] = <dy[t], res[t,j]> and, through the
#     softmax over the k selected logits,
#     dlogits[t, idx[t,j]] = w[t,j] * (dw[t,j] - sum_i w[t,i] * dw[t,i]),
#     zero for the experts not selected.
# Weight gradients are plain grouped GEMMs with no collective and are not
# part of this path.  ``rounded=False`` keeps every intermediate in float64
# (for the finite-difference pins).


def dsilu(z: np.ndarray) -> np.ndarray:
    """d silu(z) / dz = sigma(z) * (1 + z * (1 - sigma(z)))."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _val(a, rounded):
    return bf16_to_f64(a) if rounded else np.asarray(a, dtype=np.float64)


def expert_gate_up(x_bits, wg_bits, wu_bits):
    """The gate and up projections of rows X as a forward pass keeps them for
    its backward pass: (bf16(X.Wg), bf16(X.Wu)), bf16 bits [n,F] each."""
    x = bf16_to_f64(x_bits)
    return round_bf16(x @ bf16_to_f64(wg_bits)), round_bf16(x @ bf16_to_f64(wu_bits))


def grouped_gate_up(grouped, grouped_offsets, wg, wu):
    """expert_gate_up over every local expert's rows (expert e: rows
    [grouped_offsets[e], grouped_offsets[e+1]))."""
    n = np.asarray(grouped).shape[0]
    F = np.asarray(wg).shape[2]
    g, u = np.zeros((n, F), np.uint16), np.zeros((n, F), np.uint16)
    for e in range(len(grouped_offsets) - 1):
        lo, hi = int(grouped_offsets[e]), int(grouped_offsets[e + 1])
        if hi > lo:
            g[lo:hi], u[lo:hi] = expert_gate_up(grouped[lo:hi], wg[e], wu[e])
    return g, u


def expert_ffn_bwd(x_bits, dy_rows, wg_bits, wu_bits, wd_bits, rounded: bool = True, saved: bool = False):
    """Data gradient of the SwiGLU expert for rows X (bf16 [n,H]) and output
    gradients dY ([n,H]: bf16 bits, or float64 when not rounded): returns
    (dG, dU, dX) -- [n,F], [n,F], [n,H], bf16 bits when `rounded`.
    saved: g and u are the bf16 values the forward kept (expert_gate_up)
    rather than X.Wg and X.Wu themselves."""
    x = bf16_to_f64(x_bits)
    wg, wu, wd = bf16_to_f64(wg_bits), bf16_to_f64(wu_bits), bf16_to_f64(wd_bits)
    dy = _val(dy_rows, rounded)
    if saved:
        g, u = (bf16_to_f64(v) for v in expert_gate_up(x_bits, wg_bits, wu_bits))
    else:
        g = x @ wg
        u = x @ wu
    dh = dy @ wd.T
    du = dh * silu(g)
    dg = dh * u * dsilu(g)
    if rounded:
        du, dg = round_bf16(du), round_bf16(dg)
        dx = round_bf16(bf16_to_f64(dg) @ wg.T + bf16_to_f64(du) @ wu.T)
    else:
        dx = dg @ wg.T + du @ wu.T
    return dg, du, dx


def pair_grad(dy_bits, w, tokens, slots, rounded: bool = True):
    """The output gradient of pairs (tokens[i], slots[i]): w[t,j] * dy[t]
    (bf16 bits when rounded, else float64), one row per pair."""
    t = np.asarray(tokens, dtype=np.int64)
    g = np.asarray(w, dtype=np.float64)[t, np.asarray(slots, dtype=np.int64)][:, None] * bf16_to_f64(
        np.asarray(dy_bits)[t])
    return round_bf16(g) if rounded else g


def expert_dh(dy_rows, wd_bits, rounded: bool = True) -> np.ndarray:
    """dH = dY . Wd^T (float64) for output-gradient rows dY ([n,H]: bf16
    bits, or float64 when not rounded): the gradient at the expert's hidden
    h, before the SwiGLU."""
    return _val(dy_rows, rounded) @ bf16_to_f64(wd_bits).T


def dispatch_grad(dy_bits, w, perm, offsets, peer_send_grad, peer_counts, world: int, rank: int,
                  rounded: bool = True):
    """The pairs' output gradients, placed like the forward dispatch places
    the token rows: dres at packed position perm[t*k+j] is w[t,j] * dy[t]
    (bf16); returns dict(send: rows for each destination d != rank in our
    packed order, grouped: the rows of our local experts -- expert-major,
    then source rank, then the source's packed order, the peers' rows taken
    from ``peer_send_grad``)."""
    w = np.asarray(w, dtype=np.float64)
    T, k = w.shape
    E = len(offsets) - 1
    el = E // world
    token_of = np.empty(T * k, dtype=np.int64)
    slot_of = np.empty(T * k, dtype=np.int64)
    token_of[np.asarray(perm)] = np.arange(T * k) // k
    slot_of[np.asarray(perm)] = np.arange(T * k) % k
    packed = pair_grad(dy_bits, w, token_of, slot_of, rounded)
    so = send_offsets(offsets, world, el)
    send = [None if d == rank else packed[so[d]:so[d + 1]] for d in range(world)]
    pc = np.asarray(peer_counts, dtype=np.int64)
    rows = []
    for e in range(el):
        ge = rank * el + e
        for p in range(world):
            if p == rank:
                rows.append(packed[offsets[ge]:offsets[ge + 1]])
            else:
                lo, n = int(pc[p, :e].sum()), int(pc[p, e])
                rows.append(np.asarray(peer_send_grad[p])[lo:lo + n])
    H = np.asarray(dy_bits).shape[1]
    grouped = np.concatenate(rows, axis=0) if rows else np.zeros((0, H), packed.dtype)
    return dict(send=send, grouped=grouped)


def router_grad(dy_bits, idx, w, perm, offsets, y_grouped, grouped_offsets, peer_counts, peer_return,
                world: int, rank: int, tokens=None):
    """dlogits [len(tokens), E] (float64): through the softmax over the k
    selected logits; res[t,j] is the forward result (our expert's output row
    when the expert is local, else the row its rank returned)."""
    dy = bf16_to_f64(dy_bits)
    idx = np.asarray(idx)
    T, k = idx.shape
    E = len(offsets) - 1
    el = E // world
    so = send_offsets(offsets, world, el)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), E))
    for n, t in enumerate(toks):
        dw = np.zeros(k)
        for j in range(k):
            e = int(idx[t, j])
            d = e // el
            pos = int(perm[t * k + j])
            if d == rank:
                res = bf16_to_f64(y_grouped[local_row(e, pos, rank, el, offsets, grouped_offsets, peer_counts)])
            else:
                res = bf16_to_f64(peer_return[d][pos - so[d]])
            dw[j] = float(dy[t] @ res)
        wt = np.asarray(w[t], dtype=np.float64)
        out[n, idx[t]] = wt * (dw - float(wt @ dw))
    return out


def moe_layer_bwd(dy_bits, x_bits, logits, wg, wu, wd, peer_send, peer_counts, peer_return,
                  peer_send_grad, peer_return_grad, world: int, rank: int, k: int, rounded: bool = True,
                  saved: bool = False):
    """The whole expert layer's backward direction for one rank: the forward
    routing and expert outputs (``moe_layer``), the pairs' gradients
    dispatched, the experts' data gradients, the results pushed back and
    summed per token, and the router gradient.  Returns a dict with the
    forward's fields and send_grad, grouped_grad, dh, dg, du, dx_grouped,
    out_return_grad, dx, dlogits.  saved: the experts' g and u are the
    forward's bf16 copies (expert_ffn_bwd)."""
    f = moe_layer(x_bits, logits, wg, wu, wd, peer_send, peer_counts, peer_return, world, rank, k)
    g = dispatch_grad(dy_bits, f["w"], f["perm"], f["offsets"], peer_send_grad, peer_counts, world, rank,
                      rounded)
    go = f["grouped_offsets"]
    n, H = f["grouped"].shape
    F = np.asarray(wg).shape[2]
    dt = np.uint16 if rounded else np.float64
    dg, du, dxg = np.zeros((n, F), dt), np.zeros((n, F), dt), np.zeros((n, H), dt)
    dh = np.zeros((n, F))
    for e in range(len(go) - 1):
        lo, hi = int(go[e]), int(go[e + 1])
        if hi > lo:
            dg[lo:hi], du[lo:hi], dxg[lo:hi] = expert_ffn_bwd(f["grouped"][lo:hi], g["grouped"][lo:hi], wg[e],
                                                              wu[e], wd[e], rounded, saved)
            dh[lo:hi] = expert_dh(g["grouped"][lo:hi], wd[e], rounded)
    pc = np.asarray(peer_counts)
    out_return = push(dxg, f["row_src"], world, rank, pc.sum(axis=1)) if rounded else None
    ones = np.ones_like(np.asarray(f["w"], dtype=np.float32))
    if rounded:
        dx = fold(f["idx"], ones, f["perm"], f["offsets"], dxg, go, pc, peer_return_grad, world, rank)
    else:
        dx = _sum_pairs(f, dxg, go, pc, peer_return_grad, world, rank)
    dl = router_grad(dy_bits, f["idx"], f["w"], f["perm"], f["offsets"], f["y_grouped"], go, pc, peer_return,
                     world, rank)
    f.update(send_grad=g["send"], grouped_grad=g["grouped"], dh=dh, dg=dg, du=du, dx_grouped=dxg,
             out_return_grad=out_return, dx=dx, dlogits=dl)
    return f


def _sum_pairs(f, dxg, go, pc, peer_return_grad, world, rank):
    """float64 sum over each token's pairs of their data gradients (the
    unrounded fold)."""
    idx = f["idx"]
    T, k = idx.shape
    E = len(f["offsets"]) - 1
    el = E // world
    so = send_offsets(f["offsets"], world, el)
    out = np.zeros((T, dxg.shape[1]))
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            d = e // el
            pos = int(f["perm"][t * k + j])
            if d == rank:
                out[t] += dxg[local_row(e, pos, rank, el, f["offsets"], go, pc)]
            else:
                out[t] += np.asarray(peer_return_grad[d][pos - so[d]], dtype=np.float64)
    return out
