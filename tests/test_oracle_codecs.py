"""Pins for the oracle's scalar codecs (CPU only).

Each codec is checked against something other than itself: torch's bfloat16
and float8_e4m3fn dtypes (library routines), exact rational rounding, and the
E2M1 value list printed on the FP4 page.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16_to_f64(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_decode_all_patterns_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_double(bits)
    ref = _torch_bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _float32_cases(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    raw = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    ties = (g.integers(0, 1 << 16, size=n // 4, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near_ties = ties ^ g.integers(1, 4, size=ties.size, dtype=np.uint64).astype(np.uint32)
    big = np.array([0x7F7F0000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x7F7F8001,
                    0x00000001, 0x00008000, 0x00018000, 0x80008000], dtype=np.uint32)
    words = np.concatenate([raw, ties, near_ties, big])
    f = words.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_round_matches_torch_for_binary32_inputs():
    # For inputs that are binary32 values, one-step rounding from binary64 and
    # torch's float32 -> bfloat16 cast (round to nearest even) must agree.
    f = _float32_cases(200_000, 11)
    ours = oracle.bf16_from_double(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_is_single_step_from_double():
    # Values between binary32 neighbours: rounding through binary32 first would
    # land on a tie and go to even; the direct rounding must not.
    cases = {
        1 + 2.0 ** -8: 0x3F80,                 # exact tie -> even (1.0)
        1 + 3 * 2.0 ** -8: 0x3F82,             # exact tie -> even (1 + 2^-6)
        1 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,    # just above the tie -> up
        1 + 2.0 ** -8 - 2.0 ** -40: 0x3F80,    # just below the tie -> down
        2 - 2.0 ** -8: 0x4000,                 # tie carries into the exponent
        -(1 + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** -133: 0x0001,                   # smallest subnormal
        2.0 ** -134: 0x0000,                   # half the smallest subnormal: tie -> 0
        3 * 2.0 ** -134: 0x0002,               # 1.5 quanta: tie -> even (2)
        2.0 ** 128 * (1 - 2.0 ** -9): 0x7F80,  # rounds up past the largest finite
        2.0 ** 128 * (1 - 2.0 ** -8): 0x7F7F,  # largest finite BF16
    }
    xs = np.array(list(cases.keys()), dtype=np.float64)
    got = oracle.bf16_from_double(xs)
    for x, g in zip(xs, got):
        assert int(g) == cases[float(x)], (x, hex(int(g)))
        assert int(g) == exact.rne_bf16(Fraction(float(x)))


def test_bf16_round_random_doubles_against_exact_rounding():
    g = np.random.Generator(np.random.PCG64(5))
    mant = g.uniform(1.0, 2.0, size=3000)
    expo = g.integers(-140, 128, size=3000)
    sign = np.where(g.random(3000) < 0.5, -1.0, 1.0)
    xs = sign * np.ldexp(mant, expo)
    got = oracle.bf16_from_double(xs)
    for x, b in zip(xs, got):
        assert int(b) == exact.rne_bf16(Fraction(float(x))), x


def _golden_e2m1():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    return vals


def test_e2m1_values_are_the_pages_set():
    page = _golden_e2m1()
    ours = [oracle.e2m1_to_double(c) for c in range(16)]
    assert sorted(ours) == sorted(page)
    # and the signed-zero pair is there
    assert sum(1 for v in ours if v == 0 and np.signbit(v)) == 1


def test_e2m1_bit_layout():
    # Reading: bit 3 is the sign, codes 0..7 ascend through the magnitudes.
    mags = [oracle.e2m1_to_double(c) for c in range(8)]
    assert mags == sorted(mags) and len(set(mags)) == 8
    for c in range(8):
        assert oracle.e2m1_to_double(c | 8) == -oracle.e2m1_to_double(c)
        assert oracle.e2m1_to_double(c) == float(exact.e2m1_fraction(c))


def test_e4m3_all_bytes_match_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_to_double(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("u", range(-4, 5))
def test_scale_recipe_bytes(u):
    for m in range(8):
        byte = ((u + 7) << 3) | m
        assert oracle.e4m3_to_double(byte) == 2.0 ** u * (1 + m / 8)
