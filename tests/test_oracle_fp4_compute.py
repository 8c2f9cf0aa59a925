"""Pins of the oracle's FP4 index scores (indexer_scores_fp4): the query heads
quantized to OCP MX FP4 like the keys, products exact.  Checked against a
hand-worked example, a brute-force quantizer that searches the e2m1 grid
(not the oracle's rounding formula), the identity on queries the format
represents exactly, and power-of-two scale invariance."""
import math

import numpy as np
import pytest

from oracle import hybrid as orc
from oracle import numerics as nx
from synth.gen import bf16_bits

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # e2m1 magnitudes, code = index


def brute_mx_fp4(x):
    """MX FP4 round trip of one 32-value block by search: scale 2^(floor(log2
    amax) - 2), each |value| / scale clamped to 6 and sent to the nearest grid
    magnitude, a tie to the one with the even code."""
    amax = max(abs(v) for v in x)
    e = math.frexp(amax)[1] - 1 - 2 if amax > 0 else 0
    e = min(max(e, -127), 127)
    out = []
    for v in x:
        a = min(abs(v) / 2.0 ** e, 6.0)
        d = [abs(a - g) for g in GRID]
        best = min(range(8), key=lambda i: (d[i], i % 2))
        out.append(math.copysign(GRID[best] * 2.0 ** e, v))
    return out


def test_hand_example():
    """One head, block 0 = [7, 3.3, -0.2, 0 ...]: amax 7 -> x = 0; 7 clamps to 6,
    3.3 -> 3, -0.2 -> -0; block 1 zero.  Keys of ones (exact: x = -2, code 4)."""
    q = np.zeros((1, 64))
    q[0, :3] = [7.0, 3.3, -0.2]
    k = np.ones((2, 64))
    k[1, 1] = -1.0
    w = np.array([0.5], dtype=np.float32)
    s = orc.indexer_scores_fp4(bf16_bits(q), w, k)
    # bf16(3.3) = 3.296875 -> 3; (6 + 3) * 0.5 = 4.5; row 1: (6 - 3) * 0.5 = 1.5
    assert s.tolist() == [4.5, 1.5]
    # the bf16 path keeps 7, 3.296875 and bf16(-0.2) = -0.2001953125
    assert orc.indexer_scores(bf16_bits(q), w, k)[0] == 0.5 * (7 + 3.296875 - 0.2001953125)


def test_against_brute_force_quantizer():
    r = np.random.default_rng(11)
    q = r.standard_normal((4, 64)) * np.exp(r.uniform(-6, 6, (4, 1)))
    q[1, 32:] = 0.0                    # a zero block
    q[2, 5] = 1e3                      # a block with one large value
    bits = bf16_bits(q)
    qv = nx.bf16_value(bits)
    q4 = np.array([sum((brute_mx_fp4(list(qv[h, 32 * b: 32 * b + 32])) for b in range(2)), [])
                   for h in range(4)])
    keys = r.standard_normal((50, 64))
    w = r.uniform(0.1, 1.0, 4).astype(np.float32)
    want = np.maximum(keys @ q4.T, 0.0) @ w.astype(np.float64)
    got = orc.indexer_scores_fp4(bits, w, keys)
    assert np.array_equal(got, want)


def test_representable_queries_are_unchanged():
    """Queries already in MX FP4 (each block holds a value of magnitude 4 or 6
    times its scale) score exactly as the bf16 path scores them."""
    r = np.random.default_rng(12)
    codes = r.integers(0, 8, (4, 64))
    q = np.array(GRID)[codes] * np.where(r.random((4, 64)) < 0.5, -1.0, 1.0)
    q[:, 0], q[:, 32] = 6.0, -4.0
    q *= np.repeat(2.0 ** r.integers(-5, 5, (4, 2)), 32, axis=1)
    bits = bf16_bits(q)
    assert np.array_equal(nx.bf16_value(bits), q)
    keys = r.standard_normal((30, 64))
    w = r.uniform(0.1, 1.0, 4).astype(np.float32)
    assert np.array_equal(orc.indexer_scores_fp4(bits, w, keys), orc.indexer_scores(bits, w, keys))


def test_power_of_two_scaling():
    """Scaling the query by 2^s moves every block scale by s: scores scale by 2^s."""
    r = np.random.default_rng(13)
    q = r.standard_normal((4, 64))
    keys = r.standard_normal((40, 64))
    w = r.uniform(0.1, 1.0, 4).astype(np.float32)
    base = orc.indexer_scores_fp4(bf16_bits(q), w, keys)
    for sh in (-7, 3, 20):
        got = orc.indexer_scores_fp4(bf16_bits(q * 2.0 ** sh), w, keys)
        assert np.array_equal(got, base * 2.0 ** sh)
    # and quantizing does change the scores of generic queries
    assert not np.allclose(base, orc.indexer_scores(bf16_bits(q), w, keys), rtol=1e-3)
