"""Pins of the oracle's storage formats (bf16, fp8 e4m3fn) against torch's
converters and hand-built halfway cases."""
import numpy as np
import pytest
import torch

from oracle import numerics as nx


def torch_bf16_bits(x32):
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_float32_inputs():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000) * 10 ** r.uniform(-30, 30, 100000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-38, 1e-40]]).astype(np.float32)
    got = nx.bf16_bits_from_f64(x.astype(np.float64))
    assert np.array_equal(got, torch_bf16_bits(x))


def test_bf16_ties_to_even_and_single_rounding():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert nx.bf16_round_value(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6
    assert nx.bf16_round_value(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above the halfway point, below float32 resolution: a detour through
    # float32 would land on the tie and round down; one rounding rounds up.
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(x) == np.float32(1 + 2.0 ** -8)
    assert nx.bf16_round_value(np.array([x]))[0] == 1 + 2.0 ** -7
    assert nx.bf16_round_value(np.array([-x]))[0] == -(1 + 2.0 ** -7)


def test_bf16_value_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = nx.bf16_value(bits)
    finite = np.isfinite(v)
    back = nx.bf16_bits_from_f64(v[finite])
    # every finite pattern but -0 maps back to itself (-0 -> -0 too)
    assert np.array_equal(back, bits[finite])


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nx.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                       # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0 and nx.e4m3_decode(np.array([1], np.uint8))[0] == 2.0 ** -9


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(nx.e4m3_encode(nx.e4m3_decode(codes)), codes)


def test_e4m3_encode_matches_torch_in_range():
    r = np.random.default_rng(1)
    x = np.concatenate([r.uniform(-448, 448, 50000), r.standard_normal(50000) * 2.0 ** r.uniform(-12, 8, 50000),
                        r.uniform(-2.0 ** -8, 2.0 ** -8, 20000)]).astype(np.float32)
    x = np.clip(x, -448, 448)                   # torch does not saturate; compare in range
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = nx.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_saturates_and_ties():
    assert nx.e4m3_decode(nx.e4m3_encode(np.array([1e6, -1e6, 460.0])))[0] == 448.0
    assert nx.e4m3_decode(nx.e4m3_encode(np.array([-1e6])))[0] == -448.0
    # 1 + 1/16 is halfway between 1 and 1 + 1/8 -> even (1); 1 + 3/16 -> 1 + 1/4
    assert nx.e4m3_decode(nx.e4m3_encode(np.array([1 + 1 / 16])))[0] == 1.0
    assert nx.e4m3_decode(nx.e4m3_encode(np.array([1 + 3 / 16])))[0] == 1.25
    # half the smallest subnormal ties to 0; a little more rounds up
    assert nx.e4m3_decode(nx.e4m3_encode(np.array([2.0 ** -10])))[0] == 0.0
    assert nx.e4m3_decode(nx.e4m3_encode(np.array([2.0 ** -10 * 1.001])))[0] == 2.0 ** -9
    assert nx.e4m3_encode(np.array([-1e-9]))[0] == 0x80


def test_e2m1_grid_ties_and_clamp():
    """Every e2m1 code decodes to the OCP MX FP4 grid and encodes back; the
    midpoints between neighbours go to the even code; magnitudes clamp to 6."""
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    codes = np.arange(16, dtype=np.uint8)
    vals = nx.e2m1_decode(codes)
    assert vals[:8].tolist() == grid and (-vals[8:]).tolist() == grid
    assert np.array_equal(nx.e2m1_encode(vals[1:8]), codes[1:8])
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert nx.e2m1_decode(nx.e2m1_encode(np.array(mids))).tolist() == [0, 1, 1, 2, 2, 4, 4]
    assert nx.e2m1_decode(nx.e2m1_encode(np.array([7.0, -100.0, 5.99, 0.26]))).tolist() == \
        [6, -6, 6, 0.5]
