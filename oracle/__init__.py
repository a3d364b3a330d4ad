"""Plain CPU oracle for the QLoRA frozen-base linear layer (NF4 + double quantization).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check and to time the GPU path.

Every function here is a slow, direct transcription of what the pages define,
in fp64 where the pages leave the precision open.  It shares no code, tables or
helpers with the HIP library; the seeded input generators live in their own
module and carry none of the method's arithmetic.

Sources (titles of the pages, with the part each function follows):
  * "QLoRA 原理精讲" (1.2.3), section 2.1 (NF4, per-block absmax, nearest
    codeword) and section 2.2 with its storage figure (double quantization,
    reverse-order dequantization).
  * "从LoRA到QLoRA：量化技术如何改变预训练模型的微调方式", sections 2.2-2.3 (quantile
    data type normalised to [-1, 1]) and 3.1 (bf16 compute, only LoRA weights
    receive gradients).
  * "QLoRA 原理精讲", section 2.1 (why not INT4: the uniform 16-level baseline
    of the data-type ablation).
  * "QLoRA 原理精讲", section 3 pitfall 4 (the fp16 compute dtype).
  * "QLoRA 原理精讲", section 2.5 and section 3 pitfall 3 (merging the adapter
    back into BF16 weights).
  * The Volcengine article on LoRA / Q-LoRA / PortLLM, sections 3.1, 3.2 and 3.4
    (its formulas were lost in extraction; the readings used are listed in the
    module docstrings).

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``
(closed forms, invariants, brute force, library cross-checks); none is
"parity unpinned".
"""

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits, round_to_bf16_bits, bf16_bits_to_f64
from .codebook import nf4_codebook, nf4_codebook_f64, nf4_midpoints
from .quant import (
    BLOCK, GROUP, E4M3_MAX,
    block_absmax, nf4_encode, pack_codes, unpack_codes,
    e4m3fn_values, e4m3fn_encode, e4m3fn_decode,
    double_quantize, double_dequantize_scales,
    quantize_nf4_dq, dequantize_nf4_dq, dequantize_rows, storage_bytes,
    quantize_nf4_sq, dequantize_nf4_sq, dequantize_rows_sq, storage_bytes_sq,
)
from .linear import (
    linear_fwd, linear_bwd, linear_fwd_f64, linear_bwd_f64, linear_fwd_at, linear_bwd_dx_at,
    lora_grads,
)
from .merge import merge_lora, merge_lora_f64, merge_lora_rows
from .f16 import (
    f16_bits_to_f64, round_to_f16_bits, quantize_nf4_dq_f16, dequantize_nf4_dq_f16, dequantize_rows_f16,
    linear_fwd_f16, linear_fwd_at_f16, linear_bwd_f16, merge_lora_f16,
)
from .int4 import (
    int4_levels, int4_levels_f32, int4_midpoints, int4_encode, quantize_int4, dequantize_int4,
    relative_rms_error,
)

__all__ = [n for n in dir() if not n.startswith("_")]
