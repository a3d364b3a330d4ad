"""The fp16 compute type: the layer's 16-bit tensors in IEEE half precision.

Pages: "QLoRA 原理精讲", section 3, pitfall 4: on GPUs without bfloat16 the
compute dtype is switched to FP16.  Reading: everything the bf16 path rounds
to bf16 is rounded to fp16 instead (nearest, ties to even, with subnormals):
the dequantized weight w' = RNE_fp16(fl32(q[code] * c1')), and Y, dX, dA, dB
and the merged weight from their fp64 values; the weights given to the
quantizer may be fp16 (converted exactly to fp32, then quantized as before).
The storage format does not change.
"""
import numpy as np

from .quant import (BLOCK, block_absmax, double_quantize, double_dequantize_scales, e4m3fn_values, GROUP,
                    nf4_encode, pack_codes, unpack_codes)
from .codebook import nf4_codebook


def f16_bits_to_f64(u16):
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_to_f16_bits(v):
    """Nearest fp16 to each value (ties to even, subnormals, overflow to inf)."""
    with np.errstate(over="ignore"):                 # rounding past 65504 to inf is the definition
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def quantize_nf4_dq_f16(w_bits):
    """fp16 weight bits -> storage triple (the same steps as for bf16 weights)."""
    w = np.asarray(w_bits, dtype=np.uint16).reshape(-1).view(np.float16).astype(np.float32)
    c1 = block_absmax(w)
    codes = nf4_encode(w, c1)
    fp8, supers = double_quantize(c1)
    return pack_codes(codes), fp8, supers


def dequantize_nf4_dq_f16(packed, fp8_codes, supers):
    """Storage triple -> fp16 bits: w' = RNE_fp16(fl32(q[code] * c1'))."""
    codes = unpack_codes(packed)
    c1p = double_dequantize_scales(fp8_codes, supers)
    w = nf4_codebook()[codes].reshape(-1, BLOCK) * c1p[:, None]          # fp32 multiply
    return round_to_f16_bits(w.astype(np.float64)).reshape(-1)


def dequantize_rows_f16(packed, fp8_codes, supers, N, K, rows):
    """Rows ``rows`` of the dequantized [N, K] weight as fp16 bits."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    bpr = K // BLOCK
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)
    blk = rows[:, None] * bpr + np.arange(bpr)[None, :]
    f = np.asarray(fp8_codes, dtype=np.uint8).reshape(-1)[blk]
    s2 = np.asarray(supers, dtype=np.float32).reshape(-1)[blk // GROUP]
    c1p = e4m3fn_values().astype(np.float32)[f] * s2
    codes = unpack_codes(packed[rows].reshape(-1)).reshape(len(rows), bpr, BLOCK)
    w = nf4_codebook()[codes] * c1p[..., None]
    return round_to_f16_bits(w.astype(np.float64)).reshape(len(rows), K)


def linear_fwd_f16(x_bits, wdeq_bits, a_bits, b_bits, scaling):
    """Y = X W'^T + s (X A) B in fp64 from fp16 operands, rounded once to fp16."""
    x, w = f16_bits_to_f64(x_bits), f16_bits_to_f64(wdeq_bits)
    y = x @ w.T
    if a_bits is not None:
        y = y + float(np.float32(scaling)) * ((x @ f16_bits_to_f64(a_bits)) @ f16_bits_to_f64(b_bits))
    return round_to_f16_bits(y)


def linear_fwd_at_f16(x_bits, wdeq_rows_bits, a_bits, b_bits, scaling, t_idx, n_idx):
    """Sampled Y[t_idx[i], n_idx[i]] (``wdeq_rows_bits`` holds rows n_idx of W')."""
    x = f16_bits_to_f64(x_bits)[np.asarray(t_idx)]
    w = f16_bits_to_f64(wdeq_rows_bits)
    y = np.sum(x * w, axis=1)
    if a_bits is not None:
        xa = x @ f16_bits_to_f64(a_bits)
        y = y + float(np.float32(scaling)) * np.sum(xa * f16_bits_to_f64(b_bits)[:, np.asarray(n_idx)].T, axis=1)
    return round_to_f16_bits(y)


def linear_bwd_f16(dy_bits, x_bits, wdeq_bits, a_bits, b_bits, scaling):
    """(dX, dA, dB) as fp16 bits: dX = dY W' + s (dY B^T) A^T, dA = s X^T (dY B^T), dB = s (X A)^T dY."""
    dy, w = f16_bits_to_f64(dy_bits), f16_bits_to_f64(wdeq_bits)
    dx = dy @ w
    if a_bits is None:
        return round_to_f16_bits(dx), None, None
    s = float(np.float32(scaling))
    a, b, x = f16_bits_to_f64(a_bits), f16_bits_to_f64(b_bits), f16_bits_to_f64(x_bits)
    g = dy @ b.T
    dx = dx + s * (g @ a.T)
    return round_to_f16_bits(dx), round_to_f16_bits(s * (x.T @ g)), round_to_f16_bits(s * ((x @ a).T @ dy))


def merge_lora_f16(wdeq_bits, a_bits, b_bits, scaling):
    """W_m = RNE_fp16(W' + s (A B)^T)."""
    w = f16_bits_to_f64(wdeq_bits)
    if a_bits is None:
        return round_to_f16_bits(w)
    return round_to_f16_bits(w + float(np.float32(scaling)) * (f16_bits_to_f64(a_bits) @ f16_bits_to_f64(b_bits)).T)
