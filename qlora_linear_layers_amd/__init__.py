"""MI355X-native QLoRA frozen-base linear layer: NF4 + double quantization,
double dequantization and the fused forward / backward, as hand-written HIP
kernels for gfx950 behind a C ABI (``include/qlora.h``).

The HIP library is loaded on first use by ``qlora_linear_layers_amd.api``; a
missing or unbuilt library raises instead of falling back to anything else.
"""
__version__ = "0.1.0"
