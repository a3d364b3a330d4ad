"""bf16 <-> float conversions for the oracle, written from the bf16 format.

bf16 is the compute type of the layer ("从LoRA到QLoRA", section 3; "QLoRA 原理精讲",
section 2.5).  bf16 values are carried as ``uint16`` bit patterns: sign, 8
exponent bits (bias 127, as in IEEE binary32), 7 fraction bits.

``round_to_bf16_bits`` is round-to-nearest, ties to an even significand, applied
ONCE to an exact fp64 value (no intermediate fp32 rounding).
"""
import numpy as np


def bf16_bits_to_f32(u16):
    """Exact widening: the bf16 bits are the top half of the binary32 pattern."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(u16):
    return bf16_bits_to_f32(u16).astype(np.float64)


def round_to_bf16_bits(v):
    """Nearest bf16 to each (finite) value of ``v``; exact ties go to the even significand.

    Written from the format: a normal bf16 has an 8-bit significand, so its
    spacing inside the binade [2^(e-1), 2^e) is 2^(e-8); below the smallest
    normal (2^-126) the spacing is fixed at 2^-133.  ``np.rint`` rounds half to
    even, which is ties-to-even on the integer significand.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("oracle inputs must be finite")
    _, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # 2^-126 = 0.5 * 2^-125 is the smallest normal
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(v / quantum) * quantum      # both steps exact in fp64
    r32 = r.astype(np.float32)              # exact: r has <= 8 significant bits
    if np.any(np.isinf(r32)):
        raise OverflowError("value outside the bf16 range")
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16_bits(x):
    """RNE fp32 -> bf16 (the fp32 value is exact in fp64, so this is one rounding)."""
    return round_to_bf16_bits(np.asarray(x, dtype=np.float32).astype(np.float64))
