"""Pins of the oracle's positional rotation against closed forms and the
rotation's invariants: exact powers-of-two frequencies give known angles; a
turn by 0 is the identity; rotations compose; q.k depends only on the offset
of the two positions; norms of channel pairs are kept; the channels before
the last 64 never change; one bf16 rounding of the exact result."""
import math

import numpy as np
import pytest

from oracle import hybrid as orc
from oracle import numerics as nx

THETA = 10000.0


def test_inverse_frequencies_closed_form():
    # theta = 2^32: theta^(-2i/64) = 2^-i exactly
    f = orc.rope_inv_freq(2.0 ** 32)
    assert np.array_equal(f, 2.0 ** -np.arange(32))
    f = orc.rope_inv_freq(THETA)
    assert f[0] == 1.0
    # the table is float32: 10000^(-1/2) = 0.01 lands on its float32 neighbour
    assert f[16] == float(np.float32(0.01))
    assert np.all(f.astype(np.float32) == f)
    assert np.all(np.diff(f) < 0)
    # each entry is the float32 rounding of the float64 power
    i = np.arange(32)
    assert np.array_equal(f, np.float32(THETA ** (-i / 32.0)).astype(np.float64))


@pytest.mark.parametrize("i", [0, 1, 5, 31])
def test_pair_turns_by_position_times_frequency(i):
    """Unit vectors of pair i at position p turn counterclockwise by p * 2^-i
    (theta = 2^32): (1, 0) -> (cos a, sin a), (0, 1) -> (-sin a, cos a)."""
    d = 128
    p = 1234567
    a = p * 2.0 ** -i
    x = np.zeros((2, d))
    x[0, 64 + 2 * i] = 1.0
    x[1, 65 + 2 * i] = 1.0
    y = orc.rope_exact(x, [p, p], 2.0 ** 32)
    tol = 1e-15   # the angle is exact; only cos and sin round
    assert abs(y[0, 64 + 2 * i] - math.cos(a)) <= tol
    assert abs(y[0, 65 + 2 * i] - math.sin(a)) <= tol
    assert abs(y[1, 64 + 2 * i] + math.sin(a)) <= tol
    assert abs(y[1, 65 + 2 * i] - math.cos(a)) <= tol
    # no other channel moves
    mask = np.ones(d, bool)
    mask[64 + 2 * i: 66 + 2 * i] = False
    assert np.all(y[:, mask] == 0.0)


def test_position_zero_is_identity_and_front_channels_untouched():
    r = np.random.default_rng(1)
    x = r.standard_normal((7, 3, 128))
    assert np.array_equal(orc.rope_exact(x, np.zeros((7, 3)), THETA), x)
    y = orc.rope_exact(x, r.integers(0, 10 ** 6, (7, 3)), THETA)
    assert np.array_equal(y[..., :64], x[..., :64])
    assert not np.array_equal(y[..., 64:], x[..., 64:])


def test_rotation_keeps_pair_norms_and_composes():
    r = np.random.default_rng(2)
    x = r.standard_normal((50, 128))
    p1 = r.integers(0, 5000, 50)
    p2 = r.integers(0, 5000, 50)
    y = orc.rope_exact(x, p1, THETA)
    n0 = x[:, 64::2] ** 2 + x[:, 65::2] ** 2
    n1 = y[:, 64::2] ** 2 + y[:, 65::2] ** 2
    assert np.max(np.abs(n1 - n0) / n0) < 1e-14
    # R(p2) R(p1) = R(p1 + p2), up to float64 rounding of the angles
    z = orc.rope_exact(y, p2, THETA)
    w = orc.rope_exact(x, p1 + p2, THETA)
    assert np.max(np.abs(z - w)) < 1e-11


def test_scores_depend_only_on_relative_position():
    """q rotated at t and k at u: q'.k' is the same for (t + s, u + s)."""
    r = np.random.default_rng(3)
    q = r.standard_normal((20, 128))
    k = r.standard_normal((20, 128))
    t = r.integers(0, 2000, 20)
    u = r.integers(0, 2000, 20)
    s = r.integers(1, 200000, 20)
    a = np.sum(orc.rope_exact(q, t, THETA) * orc.rope_exact(k, u, THETA), axis=1)
    b = np.sum(orc.rope_exact(q, t + s, THETA) * orc.rope_exact(k, u + s, THETA), axis=1)
    assert np.max(np.abs(a - b)) < 1e-9
    # and it does depend on the offset
    c = np.sum(orc.rope_exact(q, t + 1, THETA) * orc.rope_exact(k, u, THETA), axis=1)
    assert np.max(np.abs(a - c)) > 1e-3


def test_bf16_rotation_is_one_rounding_of_the_exact_value():
    r = np.random.default_rng(4)
    bits = nx.bf16_bits_from_f64(r.standard_normal((64, 2, 128)))
    pos = r.integers(0, 1 << 20, (64, 1))
    got = orc.rope(bits, pos, THETA)
    want = nx.bf16_bits_from_f64(orc.rope_exact(nx.bf16_value(bits), pos, THETA))
    assert np.array_equal(got, want)
    assert np.array_equal(got[..., :64], bits[..., :64])


def test_rotate_tokens_positions():
    r = np.random.default_rng(5)
    T = 40
    inp = {"k": nx.bf16_bits_from_f64(r.standard_normal((T, 128))),
           "q": nx.bf16_bits_from_f64(r.standard_normal((T, 4, 128))),
           "v": nx.bf16_bits_from_f64(r.standard_normal((T, 128)))}
    out = orc.rotate_tokens(inp, THETA)
    assert out["v"] is inp["v"]
    for t in (0, 1, 17, T - 1):
        assert np.array_equal(out["k"][t], orc.rope(inp["k"][t], t, THETA))
        assert np.array_equal(out["q"][t], orc.rope(inp["q"][t], t, THETA))
    assert np.array_equal(out["k"][0], inp["k"][0])
