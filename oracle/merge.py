"""Merging the LoRA adapter into the dequantized base weight, in fp64.

Pages: "QLoRA 原理精讲" (1.2.3), section 2.5 (the LoRA/QLoRA comparison table:
after merging, inference runs at the base model's speed because the adapter
can be merged back into BF16 weights) and section 3, pitfall 3 (the second
deployment path merges the LoRA weights back and works from the merged BF16
weights).

Reading: the adapted layer computes Y = X W'^T + s (X A) B, which equals
X (W' + s (A B)^T)^T, so the merged weight is
    W_m = W' + s (A B)^T          [N, K],  (A B)^T[n][k] = sum_j A[k][j] B[j][n]
with W' the double-dequantized bf16 base weight, s = alpha / r taken in fp32
(as the ABI passes it), the sum formed in fp64 and W_m rounded once to bf16
(nearest, ties to even).  With no adapter (r = 0) W_m is W'.
"""
import numpy as np

from .bf16 import bf16_bits_to_f64, round_to_bf16_bits


def merge_lora_f64(wdeq_bits, a_bits, b_bits, scaling):
    """W' + s (A B)^T in fp64, unrounded; ``wdeq_bits`` [N, K], ``a_bits`` [K, r], ``b_bits`` [r, N]."""
    w = bf16_bits_to_f64(wdeq_bits)
    if a_bits is None:
        return w
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    return w + float(np.float32(scaling)) * (a @ b).T


def merge_lora(wdeq_bits, a_bits, b_bits, scaling):
    """The merged weight as bf16 bits [N, K] (one rounding of the fp64 value)."""
    return round_to_bf16_bits(merge_lora_f64(wdeq_bits, a_bits, b_bits, scaling))


def merge_lora_rows(wdeq_rows_bits, a_bits, b_bits, scaling, n_idx):
    """Rows ``n_idx`` of the merged weight (bf16 bits [len(n_idx), K]); ``wdeq_rows_bits``
    holds the dequantized base rows n_idx, so a large layer can be checked row by row."""
    w = bf16_bits_to_f64(wdeq_rows_bits)
    if a_bits is None:
        return round_to_bf16_bits(w)
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)[:, np.asarray(n_idx)]
    return round_to_bf16_bits(w + float(np.float32(scaling)) * (a @ b).T)
