"""INT4 absmax quantization, the baseline of the data-type ablation against NF4.

Pages: "QLoRA 原理精讲", section 2.1 (why not INT4): INT4 maps values onto the
16 integers [-8, 7] with uniform bins, while NF4 gives every bin the same
probability mass under a normal distribution, which the page calls optimal
in the information-theoretic sense for normally distributed weights.
"从LoRA到QLoRA", section 2.1: 8-bit quantization maps a tensor into the integer
range through one quantization constant.

Reading: blocks of 64 and the absmax c1 as for NF4; the 16 levels are
v_i = fl32((i - 8) / 7), i = 0..15 (the integer i - 8 of [-8, 7] over 7, so
that +c1 lands on 7 and -c1 on -7; level -8 is never the nearest); the code
is the level nearest to n = fl32(w / c1), an exact tie going to the lower
code, and an all-zero block gets code 8 (the zero); dequantization is
w' = RNE_bf16(fl32(v[code] * c1)).  Storage is codes + the fp32 absmax
(single quantization), so that the ablation compares data types alone.
"""
import numpy as np

from .bf16 import bf16_bits_to_f32, round_to_bf16_bits
from .quant import BLOCK, block_absmax, pack_codes, unpack_codes

INT4_ZERO_CODE = 8


def int4_levels():
    """float32[16], ascending; index = the 4-bit code."""
    return (np.arange(16, dtype=np.float64) - 8.0) / 7.0


def int4_levels_f32():
    return int4_levels().astype(np.float32)


def int4_midpoints():
    """Decision boundaries between neighbouring fp32 levels, exact in fp64."""
    v = int4_levels_f32().astype(np.float64)
    return (v[:-1] + v[1:]) / 2.0


def int4_encode(w_f32, absmax):
    """code = number of midpoints strictly below n = fl32(w / c1) (ties keep the lower code)."""
    w = np.asarray(w_f32, dtype=np.float32).reshape(-1, BLOCK)
    c1 = np.asarray(absmax, dtype=np.float32).reshape(-1, 1)
    codes = np.full(w.shape, INT4_ZERO_CODE, dtype=np.uint8)
    nz = c1[:, 0] > 0
    if np.any(nz):
        n = w[nz] / c1[nz]                           # fp32 division, correctly rounded
        codes[nz] = np.searchsorted(int4_midpoints(), n.astype(np.float64), side="left").astype(np.uint8)
    return codes.reshape(-1)


def quantize_int4(w_bits):
    """bf16 weight (uint16 bits, numel % 64 == 0) -> (packed codes uint8[numel/2], absmax fp32[numel/64])."""
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16).reshape(-1))
    c1 = block_absmax(w)
    return pack_codes(int4_encode(w, c1)), c1


def dequantize_int4(packed, absmax):
    codes = unpack_codes(packed)
    c1 = np.asarray(absmax, dtype=np.float32).reshape(-1)
    w = int4_levels_f32()[codes].reshape(-1, BLOCK) * c1[:, None]     # fp32 multiply
    return round_to_bf16_bits(w.astype(np.float64)).reshape(-1)


def relative_rms_error(w_bits, wdeq_bits):
    """sqrt(sum (w' - w)^2 / sum w^2) in fp64 (the ablation's figure of merit)."""
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16).reshape(-1)).astype(np.float64)
    d = bf16_bits_to_f32(np.asarray(wdeq_bits, dtype=np.uint16).reshape(-1)).astype(np.float64)
    return float(np.sqrt(np.sum((d - w) ** 2) / np.sum(w * w)))
