"""Pins of the oracle's MXFP8 functions (CPU only).

The format facts come from the OCP Microscaling (MX) specification v1.0
(``golden/mx_formats.json``); the products are tied to exact integer
arithmetic done here block by block, so a wrong block index, a scale applied
to the wrong operand or a transposed weight fails.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kos_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _code(v: int) -> int:
    """E4M3 code of a small integer (|v| <= 8), built from the bit fields."""
    if v == 0:
        return 0
    s = 0x80 if v < 0 else 0
    a = abs(v)
    e = a.bit_length() - 1               # a = 2^e * (1 + m/8)
    m = (a * 8 >> e) - 8
    assert (8 + m) << e == a * 8
    return s | ((e + 7) << 3) | m


def _codes(ints):
    return np.vectorize(_code, otypes=[np.uint8])(ints)


def test_format_golden_values():
    g = json.load(open(os.path.join(GOLD, "mx_formats.json")))
    for c in g["e4m3"]:
        v = O.e4m3_to_f64(np.array([int(c["code"], 16)], dtype=np.uint8))[0]
        assert np.isnan(v) if c["value"] == "nan" else v == c["value"], c
    for c in g["e8m0"]:
        v = O.e8m0_to_f64(np.array([int(c["code"], 16)], dtype=np.uint8))[0]
        assert np.isnan(v) if c["value"] == "nan" else v == c["value"], c


def test_e4m3_exhaustive_by_bit_repacking():
    # normal codes: the same bits placed into a float32 (exponent rebased
    # from 7 to 127, mantissa moved up 20 places); subnormals: m * 2^-9
    codes = np.arange(256, dtype=np.uint32)
    s, e, m = codes >> 7, (codes >> 3) & 15, codes & 7
    f32 = ((s << 31) | ((e + 120) << 23) | (m << 20)).astype(np.uint32).view(np.float32).astype(np.float64)
    sub = np.where(s == 1, -1.0, 1.0) * m * 2.0 ** -9
    want = np.where(e == 0, sub, f32)
    got = O.e4m3_to_f64(codes.astype(np.uint8))
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan], want[~nan])
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes increase"
    assert np.array_equal(got[0x80:0xFF], -pos)


def test_small_integers_are_exact():
    v = np.arange(-8, 9)
    assert np.array_equal(O.e4m3_to_f64(_codes(v)), v.astype(np.float64))


def test_block_scale_mapping():
    rng = np.random.default_rng(5)
    R, K = 3, 96
    ints = rng.integers(-8, 9, size=(R, K))
    sc = rng.integers(120, 135, size=(R, K // 32)).astype(np.uint8)
    got = O.mx_to_f64(_codes(ints), sc)
    for r in range(R):
        for k in range(K):
            assert got[r, k] == ints[r, k] * 2.0 ** (int(sc[r, k // 32]) - 127)


@pytest.mark.parametrize("M,N,K", [(4, 5, 64), (7, 3, 128)])
def test_gemm_mx_vs_exact_block_sums(M, N, K):
    rng = np.random.default_rng(M * 100 + N)
    a = rng.integers(-8, 9, size=(M, K))
    w = rng.integers(-8, 9, size=(N, K))          # stored N x K
    sa = rng.integers(118, 137, size=(M, K // 32)).astype(np.uint8)
    sw = rng.integers(118, 137, size=(N, K // 32)).astype(np.uint8)
    got = O.gemm_mx(_codes(a), sa, _codes(w), sw)
    assert got.shape == (M, N)
    for i in range(M):
        for j in range(N):
            tot = Fraction(0)
            for b in range(K // 32):
                part = sum(int(a[i, k]) * int(w[j, k]) for k in range(32 * b, 32 * b + 32))
                tot += part * Fraction(2) ** (int(sa[i, b]) + int(sw[j, b]) - 254)
            assert Fraction(got[i, j]) == tot


def test_ag_gemm_mx_gather_and_rank_independence():
    rng = np.random.default_rng(9)
    R, m, K, N = 4, 3, 64, 5
    shards = [_codes(rng.integers(-4, 5, size=(m, K))) for _ in range(R)]
    scales = [rng.integers(124, 131, size=(m, K // 32)).astype(np.uint8) for _ in range(R)]
    w = _codes(rng.integers(-4, 5, size=(N, K)))
    ws = rng.integers(124, 131, size=(N, K // 32)).astype(np.uint8)
    outs = []
    for rank in range(R):
        peers = [None if p == rank else shards[p] for p in range(R)]
        speers = [None if p == rank else scales[p] for p in range(R)]
        g, gs, c = O.ag_gemm_mx(shards[rank], scales[rank], peers, speers, w, ws, rank, "f32")
        assert np.array_equal(g, np.vstack(shards)) and np.array_equal(gs, np.vstack(scales))
        outs.append(c)
    for c in outs[1:]:
        assert np.array_equal(c, outs[0])
    # bf16 output is the nearest bf16 of the exact product
    _, _, cb = O.ag_gemm_mx(shards[0], scales[0], [None] + shards[1:], [None] + scales[1:], w, ws, 0, "bf16")
    assert np.array_equal(cb, O.round_bf16(O.gemm_mx(np.vstack(shards), np.vstack(scales), w, ws)))


@pytest.mark.parametrize("rank", [0, 2])
def test_gemm_rs_mx_vs_brute_force(rank):
    rng = np.random.default_rng(17 + rank)
    R, M, K, N = 4, 8, 64, 3
    a = _codes(rng.integers(-4, 5, size=(M, K)))
    sa = rng.integers(124, 131, size=(M, K // 32)).astype(np.uint8)
    w = _codes(rng.integers(-4, 5, size=(N, K)))
    sw = rng.integers(124, 131, size=(N, K // 32)).astype(np.uint8)
    peers = [rng.integers(-50, 50, size=(M // R, N)).astype(np.float32) for _ in range(R)]
    partial, y = O.gemm_rs_mx(a, sa, w, sw, peers, rank)
    full = O.gemm_mx(a, sa, w, sw)
    assert np.array_equal(partial, full.astype(np.float32))
    mc = M // R
    want = sum(peers[p].astype(np.float64) if p != rank else full[rank * mc:(rank + 1) * mc] for p in range(R))
    assert np.array_equal(y, want.astype(np.float32))


def test_scales_from_slabs_index_formula():
    # scale[r][b] sits at byte (b/2)*2R + 2r + (b%2) of the slab array
    rng = np.random.default_rng(3)
    K, R = 256, 5
    flat = rng.integers(0, 256, size=(K // 64) * R * 2).astype(np.uint8)
    nat = O.scales_from_slabs(flat.reshape(K // 64, R, 2))
    assert nat.shape == (R, K // 32)
    for r in range(R):
        for b in range(K // 32):
            assert nat[r, b] == flat[(b // 2) * 2 * R + 2 * r + (b % 2)]


def test_input_integer_codes_decode_to_integers():
    import kos_inputs as KI
    v = O.e4m3_to_f64(np.array(KI.MX_INT_CODES, dtype=np.uint8))
    assert np.array_equal(v, np.arange(-4, 5, dtype=np.float64))
