"""The 16-entry NF4 codebook, built from N(0,1) quantiles.

Pages: "从LoRA到QLoRA", section 2.3 and "QLoRA 原理精讲", section 2.1: the codewords
are quantiles of the standard normal taken at evenly spaced probabilities, so
each bin carries (about) equal probability mass, then normalised to [-1, 1].
The Volcengine article, section 3.1, says the same but lost the count and the
formula in extraction.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * exact zero with 16 values forces an asymmetric set: 8 positive codewords,
    7 negative ones and 0;
  * the positive half uses probabilities 1/2 + j(d - 1/2)/8, j = 1..8, the
    negative half 1/2 + j(d - 1/2)/7, j = 1..7 (mirrored), with the tail
    offset d = ((1 - 1/30) + (1 - 1/32)) / 2, i.e. half a bin short of 1,
    averaged over the 15- and 16-bin halves;
  * normalisation divides by z = Phi^-1(d), so the ends are exactly -1 and +1;
  * everything is computed in fp64 and rounded once to fp32.

Phi^-1 is the standard library's ``statistics.NormalDist().inv_cdf``.
"""
from statistics import NormalDist

import numpy as np

_ND = NormalDist(0.0, 1.0)


def tail_offset():
    return 0.5 * ((1.0 - 1.0 / (2 * 15)) + (1.0 - 1.0 / (2 * 16)))


def nf4_codebook_f64():
    d = tail_offset()
    z = _ND.inv_cdf(d)
    pos = [_ND.inv_cdf(0.5 + j * (d - 0.5) / 8.0) / z for j in range(1, 9)]
    neg = [-_ND.inv_cdf(0.5 + j * (d - 0.5) / 7.0) / z for j in range(1, 8)]
    values = sorted(neg) + [0.0] + pos
    return np.array(values, dtype=np.float64)


def nf4_codebook():
    """float32[16], ascending; index = the 4-bit code."""
    return nf4_codebook_f64().astype(np.float32)


def nf4_midpoints():
    """Decision boundaries between neighbouring fp32 codewords, exact in fp64."""
    q = nf4_codebook().astype(np.float64)
    return (q[:-1] + q[1:]) / 2.0
