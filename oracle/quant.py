"""Blockwise NF4 quantization with double quantization, and its inverse.

Pages: "QLoRA 原理精讲", section 2.1 (the per-block procedure: absmax of the
block, divide to land in [-1, 1], nearest of the 16 codewords, keep codes and
the scale) and section 2.2 with its storage figure (first level: one fp32
constant per 64 weights; second level: those constants quantized to FP8 with
one fp32 super-scale per 256 of them; dequantization runs in reverse order,
super-scale first).  "从LoRA到QLoRA", section 2.3: weights are rescaled by their
absolute maximum into [-1, 1].  The Volcengine article, section 3.2: the block
constants are quantized again to 8 bits in groups of 256.

Readings where the pages are silent:
  * a block is 64 consecutive elements of the row-major flat tensor (numel must
    be a multiple of 64); a group is 256 consecutive blocks; the last group may
    be partial;
  * the NF4 code uses the exact fp32 absmax c1 (exact: the inputs are bf16);
    n = fl32(w / c1); code = number of midpoints strictly below n, so an exact
    tie goes to the lower code; an all-zero block gives code 7 (the zero);
  * two codes per byte, the even element in the high nibble;
  * second level: no centring; s2 = fl32(amax_group / 448) with 448 the largest
    finite E4M3FN value; y = min(fl32(c1 / s2), 448); the FP8 code is the
    E4M3FN value nearest to y, an exact tie going to the lower code; a group
    whose constants are all zero gets s2 = 0 and codes 0;
  * dequantization: c1' = fl32(e4m3(f) * s2), then w' = RNE_bf16(fl32(q[code] * c1')).
"""
import math

import numpy as np

from .bf16 import bf16_bits_to_f32, round_to_bf16_bits
from .codebook import nf4_codebook, nf4_midpoints

BLOCK = 64
GROUP = 256
E4M3_MAX = 448.0
ZERO_CODE = 7


def _check_finite(x):
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle inputs must be finite")


def block_absmax(w_f32):
    """c1 per block of 64 consecutive elements (exact, fp32)."""
    w = np.asarray(w_f32, dtype=np.float32).reshape(-1)
    if w.size % BLOCK:
        raise ValueError("numel must be a multiple of 64")
    _check_finite(w)
    return np.abs(w.reshape(-1, BLOCK)).max(axis=1)


def nf4_encode(w_f32, absmax):
    """4-bit code per element, as in the per-block pseudocode: normalise, nearest codeword.

    code = number of midpoints strictly below n = fl32(w / c1) (``searchsorted``
    with side='left' counts exactly those), so an exact tie keeps the lower code.
    """
    w = np.asarray(w_f32, dtype=np.float32).reshape(-1, BLOCK)
    c1 = np.asarray(absmax, dtype=np.float32).reshape(-1, 1)
    mids = nf4_midpoints()
    codes = np.full(w.shape, ZERO_CODE, dtype=np.uint8)
    step = 1 << 18                                   # blocks per chunk (memory bound only)
    for s in range(0, w.shape[0], step):
        wc, cc = w[s:s + step], c1[s:s + step]
        nz = cc[:, 0] > 0
        if np.any(nz):
            n = wc[nz] / cc[nz]                      # fp32 division, correctly rounded
            codes[s:s + step][nz] = np.searchsorted(mids, n.astype(np.float64), side="left").astype(np.uint8)
    return codes.reshape(-1)


def pack_codes(codes):
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        raise ValueError("need an even number of codes")
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_codes(packed):
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


def e4m3fn_decode(code):
    """Value of an E4M3FN code (sign bit clear): 4 exponent bits (bias 7), 3 fraction bits,
    subnormals when the exponent field is 0; 0x7F is NaN and never produced here."""
    code = int(code)
    if not 0 <= code <= 0x7E:
        raise ValueError("not a finite non-negative E4M3FN code")
    e, f = code >> 3, code & 7
    if e == 0:
        return math.ldexp(f / 8.0, -6)
    return math.ldexp(1.0 + f / 8.0, e - 7)


def e4m3fn_values():
    """fp64 values of codes 0x00..0x7E, ascending with the code."""
    return np.array([e4m3fn_decode(c) for c in range(0x7F)], dtype=np.float64)


def e4m3fn_encode(y):
    """Nearest E4M3FN code to each y in [0, 448]; an exact tie goes to the lower code.

    Differences between an fp32 y and an E4M3 value are exact in fp64, so the
    distance comparison below is exact.  ``argmin`` returns the first (lowest)
    index among equal distances.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64).reshape(-1)
    if np.any(y < 0) or np.any(y > E4M3_MAX):
        raise ValueError("y must lie in [0, 448]")
    vals = e4m3fn_values()
    out = np.empty(y.size, dtype=np.uint8)
    step = 1 << 16
    for s in range(0, y.size, step):
        d = np.abs(y[s:s + step, None] - vals[None, :])
        out[s:s + step] = np.argmin(d, axis=1).astype(np.uint8)
    return out


def double_quantize(c1):
    """Second level: per 256 consecutive constants, fp32 super-scale + FP8 codes."""
    c1 = np.asarray(c1, dtype=np.float32).reshape(-1)
    ngroups = -(-c1.size // GROUP)
    codes = np.zeros(c1.size, dtype=np.uint8)
    supers = np.zeros(ngroups, dtype=np.float32)
    for g in range(ngroups):
        c = c1[g * GROUP:(g + 1) * GROUP]
        amax = c.max()
        if amax == 0:
            continue                                        # s2 = 0, codes 0
        s2 = np.float32(amax) / np.float32(E4M3_MAX)        # fp32 division
        y = np.minimum(c / s2, np.float32(E4M3_MAX))        # fp32 division, clamp
        supers[g] = s2
        codes[g * GROUP:(g + 1) * GROUP] = e4m3fn_encode(y)
    return codes, supers


def double_dequantize_scales(fp8_codes, supers):
    """Reverse order, first step: c1' = fl32(e4m3(f) * s2)."""
    f = np.asarray(fp8_codes, dtype=np.uint8).reshape(-1)
    s2 = np.asarray(supers, dtype=np.float32).reshape(-1)
    vals = e4m3fn_values().astype(np.float32)               # exact in fp32
    g = np.arange(f.size) // GROUP
    return vals[f] * s2[g]                                  # fp32 multiply


def quantize_nf4_dq(w_bits):
    """bf16 weight (uint16 bits, any shape, numel % 64 == 0) ->
    (packed codes uint8[numel/2], FP8 codes uint8[numel/64], super-scales fp32[ceil(numel/16384)])."""
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16).reshape(-1))
    c1 = block_absmax(w)
    codes = nf4_encode(w, c1)
    fp8, supers = double_quantize(c1)
    return pack_codes(codes), fp8, supers


def dequantize_nf4_dq(packed, fp8_codes, supers, numel=None):
    """Storage triple -> bf16 bits (uint16[numel])."""
    codes = unpack_codes(packed)
    if numel is not None and codes.size != numel:
        raise ValueError("numel does not match the packed codes")
    c1p = double_dequantize_scales(fp8_codes, supers)
    if c1p.size * BLOCK != codes.size:
        raise ValueError("one FP8 constant per 64 codes is required")
    q = nf4_codebook()
    w = q[codes].reshape(-1, BLOCK) * c1p[:, None]          # fp32 multiply
    return round_to_bf16_bits(w.astype(np.float64)).reshape(-1)


def dequantize_rows(packed, fp8_codes, supers, N, K, rows):
    """Rows ``rows`` of the dequantized [N, K] weight, as bf16 bits [len(rows), K].

    Same arithmetic as ``dequantize_nf4_dq``, restricted to the blocks of the
    requested rows (blocks never straddle rows since K % 64 == 0)."""
    if K % BLOCK:
        raise ValueError("K must be a multiple of 64")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    bpr = K // BLOCK
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)
    blk = rows[:, None] * bpr + np.arange(bpr)[None, :]             # [R, bpr]
    f = np.asarray(fp8_codes, dtype=np.uint8).reshape(-1)[blk]
    s2 = np.asarray(supers, dtype=np.float32).reshape(-1)[blk // GROUP]
    c1p = e4m3fn_values().astype(np.float32)[f] * s2                # fp32 multiply
    codes = unpack_codes(packed[rows].reshape(-1)).reshape(len(rows), bpr, BLOCK)
    w = nf4_codebook()[codes] * c1p[..., None]
    return round_to_bf16_bits(w.astype(np.float64)).reshape(len(rows), K)


def storage_bytes(numel):
    """Bytes of the storage triple: 4-bit codes + one FP8 code per 64 + one fp32 per 64*256."""
    return numel // 2 + numel // BLOCK + 4 * (-(-numel // (BLOCK * GROUP)))


# ---------------------------------------------------------------- single quantization
#
# The first level alone ("QLoRA 原理精讲", section 2.2, engineering motivation:
# one fp32 scale per 64 weights, 32/64 = 0.5 bits of overhead per weight):
# the same codes as above and the exact fp32 block absmax c1 kept as it is;
# dequantization is w' = RNE_bf16(fl32(q[code] * c1)).

def quantize_nf4_sq(w_bits):
    """bf16 weight (uint16 bits, numel % 64 == 0) -> (packed codes uint8[numel/2], absmax fp32[numel/64])."""
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16).reshape(-1))
    c1 = block_absmax(w)
    return pack_codes(nf4_encode(w, c1)), c1


def dequantize_nf4_sq(packed, absmax):
    """(packed codes, fp32 absmax) -> bf16 bits (uint16[numel])."""
    codes = unpack_codes(packed)
    c1 = np.asarray(absmax, dtype=np.float32).reshape(-1)
    if c1.size * BLOCK != codes.size:
        raise ValueError("one absmax per 64 codes is required")
    w = nf4_codebook()[codes].reshape(-1, BLOCK) * c1[:, None]      # fp32 multiply
    return round_to_bf16_bits(w.astype(np.float64)).reshape(-1)


def dequantize_rows_sq(packed, absmax, N, K, rows):
    """Rows ``rows`` of the dequantized [N, K] weight (single quantization), bf16 bits [len(rows), K]."""
    if K % BLOCK:
        raise ValueError("K must be a multiple of 64")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    bpr = K // BLOCK
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)
    c1 = np.asarray(absmax, dtype=np.float32).reshape(N, bpr)[rows]
    codes = unpack_codes(packed[rows].reshape(-1)).reshape(len(rows), bpr, BLOCK)
    w = nf4_codebook()[codes] * c1[..., None]
    return round_to_bf16_bits(w.astype(np.float64)).reshape(len(rows), K)


def storage_bytes_sq(numel):
    """Bytes of the single-quantization pair: 4-bit codes + one fp32 per 64."""
    return numel // 2 + 4 * (numel // BLOCK)
