"""Pins of the oracle's compression: pooling weights against closed forms,
pooled entries against exact rational arithmetic, the fp8 page format against
a hand-built page."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import hybrid as orc
from oracle import numerics as nx
from synth.gen import bf16_bits


def exact_bf16(fr: Fraction) -> Fraction:
    """Nearest bf16 value of an exact rational, ties to even (rational arithmetic)."""
    if fr == 0:
        return Fraction(0)
    a = abs(fr)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:           # make e exact
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (e - 7)
    n = round(fr / q)                     # Fraction.__round__ ties to even
    return n * q


def test_pooling_weights_closed_forms():
    for m in (1, 4, 128):
        a = orc.pooling_weights(np.zeros((m, 8), np.float32))
        assert np.all(a == np.float32(1.0 / m))
    z = np.full((4, 3), -np.inf, np.float32)
    z[2, :] = 0.3
    a = orc.pooling_weights(z)
    assert np.array_equal(a, np.eye(4, dtype=np.float32)[[2]].T.repeat(3, axis=1))
    r = np.random.default_rng(0)
    z = (0.1 * r.standard_normal((128, 64))).astype(np.float32)
    a = orc.pooling_weights(z)
    assert np.allclose(a.astype(np.float64).sum(axis=0), 1.0, atol=1e-6)
    # larger logits get larger weights, per channel
    assert np.all(np.argsort(a, axis=0, kind="stable") == np.argsort(z, axis=0, kind="stable"))


def test_compress_identity_copy_and_mean():
    r = np.random.default_rng(1)
    x = bf16_bits(r.standard_normal((64, 16)).astype(np.float32))
    # m = 1: softmax over one slot is 1, so every entry is its token
    c = orc.compress(x, np.zeros((1, 16), np.float32), 1)
    assert np.array_equal(c.bits, x)
    # one-hot weights copy that slot
    z = np.full((4, 16), -np.inf, np.float32)
    z[3] = 0
    c = orc.compress(x, z, 4)
    assert np.array_equal(c.bits, x[3::4])
    # zero logits: the block mean, rounded once
    c = orc.compress(x, np.zeros((4, 16), np.float32), 4)
    xv = nx.bf16_value(x)
    for b in range(16):
        for ch in range(16):
            mean = sum(Fraction(float(xv[4 * b + j, ch])) for j in range(4)) / 4
            assert Fraction(float(c.values[b, ch])) == exact_bf16(mean)


def test_compress_matches_exact_rational_weighted_sum():
    r = np.random.default_rng(2)
    for m in (4, 128):
        x = bf16_bits(r.standard_normal((2 * m, 8)).astype(np.float32))
        z = (0.1 * r.standard_normal((m, 8))).astype(np.float32)
        alpha = orc.pooling_weights(z)
        c = orc.compress(x, z, m)
        xv = nx.bf16_value(x)
        for b in range(2):
            for ch in range(8):
                ex = sum(Fraction(float(alpha[j, ch])) * Fraction(float(xv[b * m + j, ch]))
                         for j in range(m))
                assert Fraction(float(c.values[b, ch])) == exact_bf16(ex), (m, b, ch)


def test_compress_drops_incomplete_tail():
    x = bf16_bits(np.ones((10, 4), np.float32))
    c = orc.compress(x, np.zeros((4, 4), np.float32), 4)
    assert len(c) == 2 and np.all(c.values == 1.0)


def test_fp8_page_format():
    # one page: amax 896 -> scale 2; entries are e4m3 codes of value / 2
    c = np.zeros((64, 4))
    c[0, 0] = 896.0
    c[5, 2] = -3.0
    c[7, 1] = 1.0 / 3.0
    codes, scales = orc.store_fp8_pages(c)
    assert scales.tolist() == [2.0]
    assert nx.e4m3_decode(codes[0:1, 0:1])[0, 0] == 448.0
    assert nx.e4m3_decode(codes[5:6, 2:3])[0, 0] == -1.5
    # 1/6 rounds to 0.171875 (1.375 * 2^-3), the nearest e4m3 value
    assert nx.e4m3_decode(codes[7:8, 1:2])[0, 0] == 0.171875
    vals = orc.fp8_values(codes, scales)
    assert vals[0, 0] == 896.0 and vals[5, 2] == -3.0
    # an all-zero page has scale 1; a partial page scales over what it holds
    c2 = np.zeros((64 + 3, 4))
    c2[64:, :] = 0.5
    codes, scales = orc.store_fp8_pages(c2)
    assert scales.tolist() == [1.0, np.float32(0.5 / 448)]
    assert np.all(nx.e4m3_decode(codes[64:]) == 448.0)


def test_fp8_cache_error_bound():
    r = np.random.default_rng(3)
    c = r.standard_normal((256, 32))
    cache = orc.Cache(c, "fp8")
    sc = np.repeat(cache.scales.astype(np.float64), 64)[:, None]
    # relative error of e4m3 is at most 2^-4 of the value (normals), plus the
    # subnormal quantum 2^-10 * scale
    err = np.abs(cache.values - c)
    assert np.all(err <= np.abs(c) * 2.0 ** -4 + sc * 2.0 ** -10 + 1e-300)


def test_mixed_entry_format():
    """A mixed K row (the wiki's §8 entry, RoPE channels in bf16): the first 64
    channels as e4m3 codes with a page scale over those channels only, then the
    64 RoPE channels as bf16, two little-endian bytes each."""
    c = np.zeros((3, 128))
    c[0, 0] = 448 * 2.0 ** -3        # amax of the code channels: scale 2^-3
    c[1, 5] = -(2.0 ** -3)           # -1 in units of the scale: code 1.0111.000
    c[2, 64] = 1.0                   # bf16 0x3F80
    c[2, 65] = 1 + 2.0 ** -8         # a bf16 tie: to the even neighbour, 1.0
    c[1, 127] = 1e6                  # a RoPE channel: must not set the scale
    rows, scales = orc.store_mixed_pages(c)
    assert rows.shape == (3, 192) and rows.dtype == np.uint8
    assert scales.tolist() == [2.0 ** -3]
    assert rows[0, 0] == 0x7E        # 448: 0.1111.110, the largest finite e4m3
    assert rows[1, 5] == 0xB8
    assert rows[2, 64:68].tolist() == [0x80, 0x3F, 0x80, 0x3F]
    v = orc.mixed_values(rows, scales)
    assert v[0, 0] == 56.0 and v[1, 5] == -0.125
    assert v[2, 64] == 1.0 and v[2, 65] == 1.0
    assert v[1, 127] == 999424.0     # 1e6 to 8 significant bits
    assert np.count_nonzero(v) == 5
    # the same entries in an all-fp8 cache: the RoPE channel's 1e6 sets the scale
    _, s8 = orc.store_fp8_pages(c)
    assert s8[0] == np.float32(1e6 / 448)


def test_fp4_mx_key_format():
    """fp4 indexer keys (OCP MX FP4, 32-channel blocks): the block scale is
    2^(floor(log2 amax) - 2), elements round to nearest even on the e2m1 grid
    and clamp to 6, channel 2j sits in the low nibble of byte j."""
    c = np.zeros((3, 64))
    c[0, 0], c[0, 1] = 5.0, -1.25    # block amax 5: x = 0; 5 -> 4 (tie), -1.25 -> -1 (tie)
    c[0, 32] = 7.5                   # block amax 7.5: x = 0; 7.5 clamps to 6
    c[1, 40] = 0.3                   # amax 0.3: x = -4; 0.3 * 16 = 4.8 -> 4 -> 0.25
    codes, sb = orc.store_fp4_mx(c)  # row 2: all zero -> x = 0 in both blocks
    assert codes.shape == (3, 32) and sb.shape == (3, 2)
    assert sb.tolist() == [[127, 127], [127, 123], [127, 127]]
    assert codes[0, 0] == (0x6 | (0xA << 4))          # channel 0: +4 (0110); channel 1: -1 (1010)
    assert codes[0, 16] == 0x7 and codes[1, 20] == 0x6 and np.count_nonzero(codes) == 3
    v = orc.fp4_values(codes, sb)
    assert v[0, 0] == 4.0 and v[0, 1] == -1.0 and v[0, 32] == 6.0 and v[1, 40] == 0.25
    assert np.count_nonzero(v) == 4


def test_fp4_mx_empty_cache():
    """A request with no complete block stores an empty fp4 cache."""
    c = orc.compress(np.zeros((3, 64), dtype=np.uint16), np.zeros((4, 64), dtype=np.float32), 4, "fp4")
    assert len(c) == 0 and c.bits.shape == (0, 32) and c.scales.shape == (0, 2)
