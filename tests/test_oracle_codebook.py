"""Pins of the oracle's NF4 codebook (construction from N(0,1) quantiles,
"QLoRA 原理精讲" section 2.1; "从LoRA到QLoRA" section 2.3)."""
import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.codebook import tail_offset


def test_invariants():
    q = oracle.nf4_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q) > 0), "strictly ascending"
    assert q[0] == -1.0 and q[15] == 1.0 and q[7] == 0.0
    assert not np.signbit(q[7])
    assert np.all(np.abs(q) <= 1.0)
    assert (q > 0).sum() == 8 and (q < 0).sum() == 7


def test_equal_probability_spacing():
    """Each half of the codebook sits at evenly spaced probabilities of N(0,1):
    Phi(z q) - 1/2 steps by (d - 1/2)/8 on the positive side and (d - 1/2)/7 on
    the negative side.  Checked with scipy's normal CDF (independent of the
    stdlib quantile the oracle uses)."""
    q = oracle.nf4_codebook_f64()
    d = tail_offset()
    z = stats.norm.ppf(d)
    p_pos = stats.norm.cdf(z * q[8:]) - 0.5
    p_neg = 0.5 - stats.norm.cdf(z * q[:7][::-1])
    np.testing.assert_allclose(p_pos, (d - 0.5) * np.arange(1, 9) / 8, rtol=0, atol=1e-12)
    np.testing.assert_allclose(p_neg, (d - 0.5) * np.arange(1, 8) / 7, rtol=0, atol=1e-12)


def test_scipy_quantiles_give_same_fp32():
    d = tail_offset()
    z = stats.norm.ppf(d)
    pos = stats.norm.ppf(0.5 + np.arange(1, 9) * (d - 0.5) / 8) / z
    neg = -stats.norm.ppf(0.5 + np.arange(1, 8) * (d - 0.5) / 7) / z
    ref = np.concatenate([np.sort(neg), [0.0], pos]).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def _bin_masses():
    q = oracle.nf4_codebook().astype(np.float64)
    m = (q[:-1] + q[1:]) / 2
    z = stats.norm.ppf(tail_offset())
    edges = np.concatenate([[-np.inf], m * z, [np.inf]])
    return np.diff(stats.norm.cdf(edges))


def test_bins_near_equiprobable_closed_form():
    mass = _bin_masses()
    assert abs(mass.sum() - 1) < 1e-12
    assert mass.min() >= 0.05 and mass.max() <= 0.075, mass


def test_bins_near_equiprobable_sampled():
    """Nearest-codeword frequencies of N(0,1)/z samples match the bin masses to 4 sigma."""
    rng = np.random.default_rng(1234)
    z = stats.norm.ppf(tail_offset())
    x = rng.standard_normal(1_000_000) / z
    mids = oracle.nf4_midpoints()
    codes = (x[:, None] > mids[None, :]).sum(axis=1)
    freq = np.bincount(codes, minlength=16) / x.size
    mass = _bin_masses()
    sigma = np.sqrt(mass * (1 - mass) / x.size)
    assert np.all(np.abs(freq - mass) <= 4 * sigma), (freq, mass)


def test_midpoints_exact():
    q = oracle.nf4_codebook()
    m = oracle.nf4_midpoints()
    # the midpoint of two fp32 numbers is exact in fp64: doubling it gives back the sum exactly
    assert np.array_equal(2 * m, q[:-1].astype(np.float64) + q[1:].astype(np.float64))
