"""Seeded synthetic inputs for the fused GEMM+collective kernels and their oracle.

This module is shared by the tests, the bench and the oracle's callers.  It
holds no arithmetic of the method itself: it only draws seeded random tensors
of the shapes, dtypes and value distributions of the workloads, and emulates
what the *other* ranks would have produced (their shards, partial sums, the
rows they send and return), because only one GPU's share is run.

Workloads (shapes from the KOSMOS pages' problem statement: an all-gather
before a column-parallel GEMM, a reduce-scatter after a row-parallel GEMM, and
an expert layer whose tokens travel to their expert's rank and back):

* ``AG_TINY``  -- 4 ranks, shards 64x256 bf16, weight 256x256.
* ``AG_QKV``   -- 8 ranks, shards 512x8192 bf16, weight 8192x3072 (QKV
  column-parallel projection, sequence 4096, hidden 8192).
* ``RS_MLP``   -- 8 ranks, A 4096x3584 bf16, W 3584x8192, reduce-scattered
  into 512x8192 fp32 chunks (MLP down projection).
* ``MOE_DSV3`` -- DeepSeek-V3-shaped expert layer: 4096 tokens, hidden 7168,
  256 experts, top-8, 32 local experts, SwiGLU 7168->2048->7168.
* ``MOE_QWEN3`` -- Qwen3-235B-shaped: 8192 tokens, hidden 4096, 128 experts,
  top-8, 16 local experts, SwiGLU 4096->1536->4096, router logits N(0,1) plus a
  per-expert Zipf(s=1.1) bias (skewed routing).
* ``AG_QKV_MX``, ``RS_MLP_MX`` -- the QKV and MLP-down shapes with MXFP8
  operands (E4M3 codes with E8M0 scales per 32 along K).

Distributions: N(0, v) means variance v (a fan-in initialiser keeps unit
output variance).  bf16 tensors are drawn in fp32 and rounded to nearest even
by torch's own conversion.  Integer-valued variants draw uniformly from
[-4, 4] so that every fp32 sum of the small cases is exact.

Every tensor is drawn from its own ``torch.Generator`` seeded from
(workload id, tensor id, rank), on the device it is requested for.  CPU and
GPU generators give different streams; a test that compares both sides draws
once and copies.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AgShape:
    name: str
    wid: int          # workload id, part of every seed
    world: int
    m_local: int
    k: int
    n: int

    @property
    def m(self) -> int:
        return self.world * self.m_local

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


@dataclasses.dataclass(frozen=True)
class RsShape:
    name: str
    wid: int
    world: int
    m: int
    k: int
    n: int

    @property
    def m_chunk(self) -> int:
        return self.m // self.world

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


@dataclasses.dataclass(frozen=True)
class MoeShape:
    name: str
    wid: int
    world: int
    tokens: int
    hidden: int
    experts: int
    topk: int
    ffn: int
    zipf_s: Optional[float] = None   # per-expert bias (e+1)^-s added to logits

    @property
    def e_local(self) -> int:
        return self.experts // self.world

    @property
    def peer_cap(self) -> int:
        """Rows one rank can send to one peer: each token reaches a peer's
        experts at most min(topk, e_local) times (one row per pair)."""
        return self.tokens * min(self.topk, self.e_local)

    @property
    def flops_per_row(self) -> float:
        # gate + up (2 GEMMs of H x F) and down (F x H), 2 flops per MAC
        return 6.0 * self.hidden * self.ffn


AG_TINY = AgShape("ag_tiny_4r_256x256x256", 1, 4, 64, 256, 256)
AG_QKV = AgShape("ag_qkv_8r_4096x8192x3072", 2, 8, 512, 8192, 3072)
RS_MLP = RsShape("rs_mlpdown_8r_4096x3584x8192", 3, 8, 4096, 3584, 8192)
MOE_DSV3 = MoeShape("moe_dsv3_8r_t4096_h7168_e256_k8_f2048", 4, 8, 4096, 7168,
                    256, 8, 2048)
MOE_QWEN3 = MoeShape("moe_qwen3_8r_t8192_h4096_e128_k8_f1536_zipf1.1", 5, 8,
                     8192, 4096, 128, 8, 1536, zipf_s=1.1)

# the rest of a TP+SP transformer layer at the QKV shape's model width
# (hidden 8192, 8 ranks): MLP-up (gate and up, 2 x 3584 columns per rank)
# and the attention output projection (1024 columns of attention per rank)
AG_MLPUP = AgShape("ag_mlpup_8r_4096x8192x7168", 10, 8, 512, 8192, 7168)
RS_OUTPROJ = RsShape("rs_outproj_8r_4096x1024x8192", 11, 8, 4096, 1024, 8192)

# MXFP8 operands (E4M3 codes, E8M0 scales) at the QKV and MLP-down shapes,
# and small shapes of whole 256 x 256 tiles with several tiles each way
# the backward pass's data-gradient collectives of the same layer, weights
# stored transposed (n x k): the QKV all-gather+GEMM's backward is a
# GEMM+reduce-scatter of dY [4096, 3072] with W_qkv^T (8192 output columns),
# the MLP-down reduce-scatter's backward an all-gather of dY shards
# [512, 8192] with W_down^T (3584 output columns)
RS_QKV_BWD = RsShape("rs_qkv_bwd_8r_4096x3072x8192", 18, 8, 4096, 3072, 8192)
AG_MLP_BWD = AgShape("ag_mlpdown_bwd_8r_4096x8192x3584", 19, 8, 512, 8192, 3584)
RS_MLPUP_BWD = RsShape("rs_mlpup_bwd_8r_4096x7168x8192", 20, 8, 4096, 7168, 8192)
AG_OUTPROJ_BWD = AgShape("ag_outproj_bwd_8r_4096x8192x1024", 21, 8, 512, 8192, 1024)

AG_QKV_MX = AgShape("ag_qkv_mx_8r_4096x8192x3072", 12, 8, 512, 8192, 3072)
RS_MLP_MX = RsShape("rs_mlpdown_mx_8r_4096x3584x8192", 13, 8, 4096, 3584, 8192)
AG_MLPUP_MX = AgShape("ag_mlpup_mx_8r_4096x8192x7168", 22, 8, 512, 8192, 7168)
RS_OUTPROJ_MX = RsShape("rs_outproj_mx_8r_4096x1024x8192", 23, 8, 4096, 1024, 8192)
AG_TINY_MX = AgShape("ag_tiny_mx_4r_1024x512x512", 14, 4, 256, 512, 512)
RS_TINY_MX = RsShape("rs_tiny_mx_4r_1024x512x512", 15, 4, 1024, 512, 512)

RS_TINY = RsShape("rs_tiny_4r_256x256x256", 8, 4, 256, 256, 256)
RS_MID = RsShape("rs_mid_4r_2048x192x384", 9, 4, 2048, 192, 384)

# small shapes for the CPU oracle tests and the fast GPU parity cases: several
# tiles in each direction and a ragged expert tail
MOE_TINY = MoeShape("moe_tiny_4r_t96_h256_e16_k4_f128", 6, 4, 96, 256, 16, 4,
                    128)
MOE_TINY_SKEW = MoeShape("moe_tiny_skew_4r_t160_h256_e16_k4_f192", 7, 4, 160,
                         256, 16, 4, 192, zipf_s=1.1)

# the expert layer's backward direction (hidden a multiple of 256, ffn of
# 128): several 256-row units per expert with ragged tails, top-10 (more
# than eight pairs per token), one rank, and top-1
MOE_BWD_MID = MoeShape("moe_bwd_mid_4r_t640_h512_e16_k4_f256_zipf1.1", 24, 4, 640, 512, 16, 4, 256,
                       zipf_s=1.1)
MOE_BWD_K10 = MoeShape("moe_bwd_k10_2r_t64_h256_e32_k10_f128", 25, 2, 64, 256, 32, 10, 128)
MOE_BWD_1R = MoeShape("moe_bwd_1r_t96_h256_e8_k2_f128", 26, 1, 96, 256, 8, 2, 128)
MOE_BWD_K1 = MoeShape("moe_bwd_k1_4r_t96_h256_e16_k1_f128", 27, 4, 96, 256, 16, 1, 128)


# ---------------------------------------------------------------------------
# seeded draws
# ---------------------------------------------------------------------------

# tensor ids (stable: part of the seed)
T_A, T_W, T_PEER, T_X, T_LOGITS, T_WG, T_WU, T_WD, T_SEND, T_RET, T_PLOG, T_SA, T_SW = range(13)
T_DY, T_SENDG, T_RETG = 13, 14, 15    # the expert layer's backward direction


def _gen(wid: int, tid: int, rank: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((wid * 97 + tid) * 131 + rank) * 1_000_003 + 12345)
    return g


def normal(shape, var, wid, tid, rank, device, dtype=torch.bfloat16):
    """N(0, var) drawn in fp32 and converted to ``dtype``."""
    g = _gen(wid, tid, rank, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if var != 1.0:
        t.mul_(math.sqrt(var))
    return t.to(dtype)


def integers(shape, lo, hi, wid, tid, rank, device, dtype=torch.bfloat16):
    """Uniform integers in [lo, hi] (exact in bf16 for |v| <= 256)."""
    g = _gen(wid, tid, rank, device)
    t = torch.randint(lo, hi + 1, shape, generator=g, device=device,
                      dtype=torch.int32)
    return t.to(dtype)


# ---------------------------------------------------------------------------
# all-gather + GEMM
# ---------------------------------------------------------------------------

def ag_inputs(s: AgShape, rank: int, device="cpu", integer=False, wt=False):
    """Shards of every rank (shard p is the same whichever rank asks) and the
    column-parallel weight shard (``wt``: stored transposed, n x k).  Returns
    dict(a_local, a_peers, w) with ``a_peers[rank] is None``."""
    shards = []
    for p in range(s.world):
        if integer:
            shards.append(integers((s.m_local, s.k), -4, 4, s.wid, T_A, p, device))
        else:
            shards.append(normal((s.m_local, s.k), 1.0, s.wid, T_A, p, device))
    wshape = (s.n, s.k) if wt else (s.k, s.n)
    if integer:
        w = integers(wshape, -4, 4, s.wid, T_W, 0, device)
    else:
        w = normal(wshape, 1.0 / s.k, s.wid, T_W, 0, device)
    peers = [None if p == rank else shards[p] for p in range(s.world)]
    return dict(a_local=shards[rank], a_peers=peers, w=w)


# ---------------------------------------------------------------------------
# GEMM + reduce-scatter
# ---------------------------------------------------------------------------

def rs_inputs(s: RsShape, rank: int, device="cpu", integer=False, wt=False):
    """A, W (``wt``: stored transposed, n x k) and the fp32 rows of chunk
    ``rank`` that every peer p computed (``peer_slices[rank] is None``).  Same
    law as the local partial's entries: N(0,1) (K * 1 * 1/K)."""
    wshape = (s.n, s.k) if wt else (s.k, s.n)
    if integer:
        a = integers((s.m, s.k), -4, 4, s.wid, T_A, rank, device)
        w = integers(wshape, -4, 4, s.wid, T_W, 0, device)
    else:
        a = normal((s.m, s.k), 1.0, s.wid, T_A, rank, device)
        w = normal(wshape, 1.0 / s.k, s.wid, T_W, 0, device)
    peers = []
    for p in range(s.world):
        if p == rank:
            peers.append(None)
        elif integer:
            peers.append(integers((s.m_chunk, s.n), -4096, 4096, s.wid,
                                  T_PEER, p * 64 + rank, device,
                                  dtype=torch.float32))
        else:
            peers.append(normal((s.m_chunk, s.n), 1.0, s.wid, T_PEER,
                                p * 64 + rank, device, dtype=torch.float32))
    return dict(a=a, w=w, peer_slices=peers)


# ---------------------------------------------------------------------------
# MXFP8 operands
# ---------------------------------------------------------------------------
#
# Codes are drawn directly (no quantisation step): sign uniform, exponent
# field uniform in [3, 9], mantissa uniform -- E4M3 magnitudes 2^-4 .. 7.5,
# never NaN -- and scales uniform in [124, 130], so element values span about
# 2^-7 .. 2^5 around unit size.  Integer-valued variants draw the codes of
# the integers -4..4 (listed below, OCP MX v1.0 E4M3) and scales in
# [126, 128], which keeps every fp32 sum of the small cases exact.  Scales
# are drawn straight into the kernels' slab layout, uint8 [k/64, rows, 2]
# (i.i.d. draws: the layout only fixes where each lands).

MX_INT_CODES = (0xC8, 0xC4, 0xC0, 0xB8, 0x00, 0x38, 0x40, 0x44, 0x48)   # -4 .. 4


def mx_codes(shape, wid, tid, rank, device, integer=False, edge=False):
    g = _gen(wid, tid, rank, device)
    if edge:
        # the format's edges: a quarter subnormals (exponent field 0,
        # mantissa 1..7), a twentieth zeros, a fifth of the largest binade
        # (exponent field 15, mantissa 0..6: 256 .. 448; mantissa 7 is NaN),
        # the rest normal (exponent field 1..14); sign uniform
        cat = torch.rand(shape, generator=g, device=device)
        sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32)
        e_norm = torch.randint(1, 15, shape, generator=g, device=device, dtype=torch.int32)
        m_any = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.int32)
        m_sub = torch.randint(1, 8, shape, generator=g, device=device, dtype=torch.int32)
        m_top = torch.randint(0, 7, shape, generator=g, device=device, dtype=torch.int32)
        e = torch.where(cat < 0.30, 0, torch.where(cat < 0.50, 15, e_norm))
        m = torch.where(cat < 0.25, m_sub, torch.where(cat < 0.30, 0, torch.where(cat < 0.50, m_top, m_any)))
        return ((sign << 7) | (e << 3) | m).to(torch.uint8)
    if integer:
        idx = torch.randint(0, len(MX_INT_CODES), shape, generator=g, device=device)
        return torch.tensor(MX_INT_CODES, dtype=torch.uint8, device=device)[idx]
    sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32)
    e = torch.randint(3, 10, shape, generator=g, device=device, dtype=torch.int32)
    m = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.int32)
    return ((sign << 7) | (e << 3) | m).to(torch.uint8)


def mx_scales(rows, k, wid, tid, rank, device, integer=False, edge=False):
    g = _gen(wid, tid, rank, device)
    # edge: scales 2^-27 .. 2^27 (products of the largest codes at the
    # largest scales stay far below the fp32 range, the smallest above it)
    lo, hi = (126, 128) if integer else (100, 154) if edge else (124, 130)
    return torch.randint(lo, hi + 1, (k // 64, rows, 2), generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)


def ag_mx_inputs(s: AgShape, rank: int, device="cpu", integer=False, edge=False):
    """MX shards of every rank with their scales, and the weight shard stored
    n x k with its scales.  Returns dict(a_local, s_local, a_peers, s_peers,
    w, w_scales); peer entries ``rank`` are None.  ``edge``: codes and scales
    at the format's edges (subnormals, the largest binade, far scales)."""
    shards = [mx_codes((s.m_local, s.k), s.wid, T_A, p, device, integer, edge) for p in range(s.world)]
    scales = [mx_scales(s.m_local, s.k, s.wid, T_SA, p, device, integer, edge) for p in range(s.world)]
    w = mx_codes((s.n, s.k), s.wid, T_W, 0, device, integer, edge)
    ws = mx_scales(s.n, s.k, s.wid, T_SW, 0, device, integer, edge)
    return dict(a_local=shards[rank], s_local=scales[rank],
                a_peers=[None if p == rank else shards[p] for p in range(s.world)],
                s_peers=[None if p == rank else scales[p] for p in range(s.world)],
                w=w, w_scales=ws)


def rs_mx_inputs(s: RsShape, rank: int, device="cpu", integer=False, edge=False):
    """MX A [m, k] and W [n, k] with scales, and the peers' fp32 slices of
    chunk ``rank`` (as ``rs_inputs``)."""
    a = mx_codes((s.m, s.k), s.wid, T_A, rank, device, integer, edge)
    sa = mx_scales(s.m, s.k, s.wid, T_SA, rank, device, integer, edge)
    w = mx_codes((s.n, s.k), s.wid, T_W, 0, device, integer, edge)
    sw = mx_scales(s.n, s.k, s.wid, T_SW, 0, device, integer, edge)
    peers = rs_inputs(s, rank, device, integer)["peer_slices"] if s.world > 1 else [None]
    return dict(a=a, a_scales=sa, w=w, w_scales=sw, peer_slices=peers)


# ---------------------------------------------------------------------------
# expert layer
# ---------------------------------------------------------------------------

def zipf_bias(s: MoeShape, device="cpu") -> torch.Tensor:
    """Unnormalised Zipf weight (e+1)^-s per expert, in fp32."""
    e = torch.arange(s.experts, device=device, dtype=torch.float64)
    return (e + 1.0).pow(-s.zipf_s).to(torch.float32)


def router_logits(s: MoeShape, rank: int, device="cpu", tid=T_LOGITS):
    lg = normal((s.tokens, s.experts), 1.0, s.wid, tid, rank, device,
                dtype=torch.float32)
    if s.zipf_s is not None:
        lg = lg + zipf_bias(s, device)[None, :]
    return lg


def emulated_peer_counts(s: MoeShape, rank: int, device="cpu"):
    """Rows each peer p sends to ``rank``, per local expert of ``rank``.

    A peer's routing is emulated from its own seeded logits of the same law by
    a library top-k: only how many of its tokens land on each of our experts
    matters here (the rows themselves are seeded), so the tie rule is
    irrelevant.  Returns int32 [world, e_local] with row ``rank`` zero."""
    counts = torch.zeros((s.world, s.e_local), dtype=torch.int32)
    lo = rank * s.e_local
    for p in range(s.world):
        if p == rank:
            continue
        lg = router_logits(s, p, "cpu", tid=T_PLOG)
        sel = torch.topk(lg, s.topk, dim=1).indices.reshape(-1)
        hist = torch.bincount(sel, minlength=s.experts)
        counts[p] = hist[lo:lo + s.e_local].to(torch.int32)
    return counts.to(device)


def moe_inputs(s: MoeShape, rank: int, device="cpu", with_weights=True):
    """Everything one rank's expert layer reads.

    x [T,H] bf16 N(0,1); logits [T,E] fp32 N(0,1) (+ Zipf bias);
    local expert weights wg, wu [E_loc,H,F] N(0,1/H), wd [E_loc,F,H] N(0,1/F);
    peer_counts [R,E_loc] int32 (emulated routing of the peers);
    peer_send[p] [n_p,H] bf16 N(0,1): rows p sends us, expert-major;
    peer_return[d] [max(peer_cap,1),H] bf16 N(0,1): results d returns for the rows we
    send it, in our packed order (only the first send-count rows are read)."""
    out = {}
    out["x"] = normal((s.tokens, s.hidden), 1.0, s.wid, T_X, rank, device)
    out["logits"] = router_logits(s, rank, device)
    pc = emulated_peer_counts(s, rank, "cpu")
    out["peer_counts"] = pc.to(device)
    peer_send, peer_ret = [], []
    for p in range(s.world):
        if p == rank:
            peer_send.append(None)
            peer_ret.append(None)
            continue
        n_p = int(pc[p].sum())
        peer_send.append(normal((max(n_p, 1), s.hidden), 1.0, s.wid, T_SEND,
                                p * 64 + rank, device)[:n_p])
        peer_ret.append(normal((max(s.peer_cap, 1), s.hidden), 1.0, s.wid, T_RET,
                               p * 64 + rank, device))
    out["peer_send"] = peer_send
    out["peer_return"] = peer_ret
    if with_weights:
        out.update(moe_weights(s, rank, device))
    return out


def moe_grad_inputs(s: MoeShape, rank: int, device="cpu"):
    """What one rank's expert-layer backward reads besides the forward's
    buffers: dy [T,H] bf16 N(0,1) (the layer output's gradient);
    peer_send_grad[p] [n_p,H] bf16 N(0,1): the gradients of the rows p sent
    us (n_p = what emulated_peer_counts says p sends), in p's order;
    peer_return_grad[d] [max(peer_cap,1),H] bf16 N(0,1): the data gradients
    d returns for the rows we sent it (only the first send-count rows are
    read)."""
    out = {"dy": normal((s.tokens, s.hidden), 1.0, s.wid, T_DY, rank, device)}
    pc = emulated_peer_counts(s, rank, "cpu")
    sg, rg = [], []
    for p in range(s.world):
        if p == rank:
            sg.append(None)
            rg.append(None)
            continue
        n_p = int(pc[p].sum())
        sg.append(normal((max(n_p, 1), s.hidden), 1.0, s.wid, T_SENDG, p * 64 + rank, device)[:n_p])
        rg.append(normal((max(s.peer_cap, 1), s.hidden), 1.0, s.wid, T_RETG, p * 64 + rank, device))
    out["peer_send_grad"] = sg
    out["peer_return_grad"] = rg
    return out


def moe_weights(s: MoeShape, rank: int, device="cpu"):
    H, F, El = s.hidden, s.ffn, s.e_local
    wg = torch.empty((El, H, F), dtype=torch.bfloat16, device=device)
    wu = torch.empty_like(wg)
    wd = torch.empty((El, F, H), dtype=torch.bfloat16, device=device)
    for e in range(El):
        ge = rank * El + e
        wg[e] = normal((H, F), 1.0 / H, s.wid, T_WG, ge, device)
        wu[e] = normal((H, F), 1.0 / H, s.wid, T_WU, ge, device)
        wd[e] = normal((F, H), 1.0 / F, s.wid, T_WD, ge, device)
    return dict(wg=wg, wu=wu, wd=wd)


# ---------------------------------------------------------------------------
# conversions for handing torch tensors to the NumPy oracle
# ---------------------------------------------------------------------------

def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> NumPy uint16 bit patterns (a copy on the host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def from_bf16_bits(a, device="cpu") -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(device)
