"""Pins of the oracle's bf16 rounding (nearest, ties to even)."""
from fractions import Fraction

import numpy as np
import torch

import oracle


def _exact_nearest_bf16(v):
    """Brute force: enumerate the two bf16 neighbours with Fractions."""
    f32 = np.float32(v)
    # candidates: all bf16 patterns around the fp32 truncation
    b = int(np.array(f32, dtype=np.float32).view(np.uint32)) >> 16
    best = None
    fv = Fraction(float(v))
    for cand in (b - 1, b, b + 1, b + 2):
        cand &= 0xFFFF
        val = Fraction(float(oracle.bf16_bits_to_f32(np.uint16(cand))))
        d = abs(val - fv)
        key = (d, cand & 1)          # ties: prefer even significand
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_fp32_inputs_match_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-40, 40, 200_000))).astype(np.float32)
    ties = (rng.integers(0, 1 << 16, 5000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)


def test_fp64_values_brute_force():
    rng = np.random.default_rng(8)
    v = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    got = oracle.round_to_bf16_bits(v)
    for vi, gi in zip(v, got):
        assert int(gi) == _exact_nearest_bf16(vi)


def test_fp64_ties_and_subnormals():
    # exact midpoint between 1.0 and the next bf16 (1 + 2^-7): ties to even -> 1.0
    assert oracle.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # just above the midpoint (not representable in fp32) rounds up: a single rounding from fp64
    assert oracle.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    # midpoint between 1+2^-7 (odd) and 1+2^-6 (even) -> up to even
    assert oracle.round_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # smallest bf16 subnormal 2^-133 and half of it (tie to even -> 0)
    assert oracle.round_to_bf16_bits(np.array([2.0 ** -133]))[0] == 0x0001
    assert oracle.round_to_bf16_bits(np.array([2.0 ** -134]))[0] == 0x0000
    assert oracle.round_to_bf16_bits(np.array([-3 * 2.0 ** -134]))[0] == 0x8002
