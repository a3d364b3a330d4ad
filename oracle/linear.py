"""The QLoRA linear layer: forward, input gradient and LoRA gradients, in fp64.

Pages: the Volcengine article, section 3.4 defines QLoRA for one linear layer
of the quantized base (its equation was lost in extraction); "从LoRA到QLoRA",
section 1.3 and 3.1: the 4-bit base is frozen, dequantized to bf16 for the
forward and backward passes, and gradients flow through it into the LoRA
adapters, whose weights (and only those) get gradients; "QLoRA 原理精讲", section
3 (pitfall 1): the adapters A and B stay in bf16.  The LoRA update of a frozen
W0 is the product of two rank-r matrices (Volcengine article, section 2.1,
formula lost).

Reading of the lost equation (layout: X [T,K], W [N,K], A [K,r], B [r,N]):
    Y  = X W'^T + s (X A) B
    dX = dY W'   + s (dY B^T) A^T
    dA = s X^T (dY B^T)
    dB = s (X A)^T dY
with W' the double-dequantized bf16 weight and s = alpha / r.  Every product
is accumulated exactly enough in fp64 (numpy BLAS) and each output is rounded
once to bf16 (nearest, ties to even).
"""
import numpy as np

from .bf16 import bf16_bits_to_f64, round_to_bf16_bits


def _f64(bits, shape=None):
    a = bf16_bits_to_f64(bits)
    return a.reshape(shape) if shape is not None else a


def linear_fwd_f64(x_bits, wdeq_bits, a_bits, b_bits, scaling):
    """Y = X W'^T + s (X A) B in fp64, unrounded.  ``a_bits is None`` means r = 0 (no LoRA term)."""
    x = _f64(x_bits)
    w = _f64(wdeq_bits)
    y = x @ w.T
    if a_bits is not None:
        a = _f64(a_bits)
        b = _f64(b_bits)
        y = y + float(np.float32(scaling)) * ((x @ a) @ b)
    return y


def linear_fwd(x_bits, wdeq_bits, a_bits, b_bits, scaling):
    """Y as bf16 bits [T, N] (one rounding of the fp64 result)."""
    return round_to_bf16_bits(linear_fwd_f64(x_bits, wdeq_bits, a_bits, b_bits, scaling))


def linear_bwd_f64(dy_bits, x_bits, wdeq_bits, a_bits, b_bits, scaling):
    """(dX, dA, dB) in fp64, unrounded; dA/dB are None without LoRA or without X."""
    dy = _f64(dy_bits)
    w = _f64(wdeq_bits)
    dx = dy @ w
    if a_bits is None:
        return dx, None, None
    s = float(np.float32(scaling))
    a = _f64(a_bits)
    b = _f64(b_bits)
    g = dy @ b.T                     # [T, r]
    dx = dx + s * (g @ a.T)
    da = db = None
    if x_bits is not None:
        x = _f64(x_bits)
        da = s * (x.T @ g)
        db = s * ((x @ a).T @ dy)
    return dx, da, db


def linear_bwd(dy_bits, x_bits, wdeq_bits, a_bits, b_bits, scaling):
    """(dX, dA, dB) as bf16 bits, each rounded once from fp64."""
    dx, da, db = linear_bwd_f64(dy_bits, x_bits, wdeq_bits, a_bits, b_bits, scaling)
    r = lambda v: None if v is None else round_to_bf16_bits(v)
    return r(dx), r(da), r(db)


def lora_grads(x_bits, dy_bits, a_bits, b_bits, scaling):
    """(dA, dB) alone, bf16 bits."""
    x, dy = _f64(x_bits), _f64(dy_bits)
    a, b = _f64(a_bits), _f64(b_bits)
    s = float(np.float32(scaling))
    da = s * (x.T @ (dy @ b.T))
    db = s * ((x @ a).T @ dy)
    return round_to_bf16_bits(da), round_to_bf16_bits(db)


def linear_fwd_at(x_bits, wdeq_rows_bits, a_bits, b_bits, scaling, t_idx, n_idx):
    """Sampled forward outputs Y[t_idx[i], n_idx[i]], computed one by one.

    ``wdeq_rows_bits`` maps each entry of n_idx to its dequantized row of W
    (shape [len(n_idx), K])."""
    x = _f64(x_bits)
    w = _f64(wdeq_rows_bits)
    t_idx = np.asarray(t_idx)
    n_idx = np.asarray(n_idx)
    y = np.einsum("ik,ik->i", x[t_idx], w)
    if a_bits is not None:
        a, b = _f64(a_bits), _f64(b_bits)
        xa = x[t_idx] @ a                                   # [S, r]
        y = y + float(np.float32(scaling)) * np.einsum("ij,ji->i", xa, b[:, n_idx])
    return round_to_bf16_bits(y)


def linear_bwd_dx_at(dy_bits, wdeq_cols_bits, a_bits, b_bits, scaling, t_idx, k_idx):
    """Sampled input gradients dX[t_idx[i], k_idx[i]]; ``wdeq_cols_bits`` is [len(k_idx), N]
    holding column k of W' for each sample."""
    dy = _f64(dy_bits)
    wc = _f64(wdeq_cols_bits)
    t_idx = np.asarray(t_idx)
    k_idx = np.asarray(k_idx)
    v = np.einsum("in,in->i", dy[t_idx], wc)
    if a_bits is not None:
        a, b = _f64(a_bits), _f64(b_bits)
        g = dy[t_idx] @ b.T                                 # [S, r]
        v = v + float(np.float32(scaling)) * np.einsum("ij,ij->i", g, a[k_idx])
    return round_to_bf16_bits(v)
