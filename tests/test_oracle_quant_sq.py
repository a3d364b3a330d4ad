"""Pins of the single-quantization oracle (codes + one fp32 absmax per 64
weights, no second level): "QLoRA 原理精讲", section 2.2, the engineering
motivation (first level alone: an fp32 scale per 64 weights, 0.5 bit each)."""
import json
import os

import numpy as np

import oracle
from qlora_linear_layers_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _w(cfg=1, outliers=False, shape=(32, 4096)):
    rng = synth.rng_for(cfg, 0, 0, synth.ROLE_W)
    return synth.outlier_weight_bf16(rng, shape) if outliers else synth.normal_bf16(rng, shape, 0.02)


def test_codes_are_the_first_level_of_double_quantization():
    for outl in (False, True):
        w = _w(outliers=outl)
        p_sq, c1 = oracle.quantize_nf4_sq(w)
        p_dq, _, _ = oracle.quantize_nf4_dq(w)
        assert np.array_equal(p_sq, p_dq)
        assert c1.dtype == np.float32 and c1.size == w.size // 64


def test_exactly_representable_constants_give_the_double_quantized_weight():
    # every block's absmax is 0.4375 = 448 * 2^-10: s2 = 2^-10 and the FP8 code of
    # 448 reproduce c1 exactly, so both formats dequantize to the same bits
    rng = np.random.default_rng(3)
    w = rng.uniform(-0.43, 0.43, (64, 256)).astype(np.float32)
    w[np.arange(64), rng.integers(0, 256, 64)] = 0.4375
    w = w.reshape(-1, 64)
    w[np.arange(w.shape[0]), rng.integers(0, 64, w.shape[0])] = -0.4375
    bits = synth.to_bf16_bits(w.reshape(-1))
    p, c1 = oracle.quantize_nf4_sq(bits)
    assert np.all(c1 == np.float32(0.4375))
    pd, f, s = oracle.quantize_nf4_dq(bits)
    assert np.array_equal(oracle.double_dequantize_scales(f, s), c1)
    assert np.array_equal(oracle.dequantize_nf4_sq(p, c1), oracle.dequantize_nf4_dq(pd, f, s))


def test_error_bound_without_a_scale_term():
    w_bits = _w()
    p, c1 = oracle.quantize_nf4_sq(w_bits)
    wd = oracle.bf16_bits_to_f32(oracle.dequantize_nf4_sq(p, c1)).astype(np.float64)
    w = oracle.bf16_bits_to_f32(w_bits).astype(np.float64).reshape(-1)
    gap = np.diff(oracle.nf4_codebook().astype(np.float64)).max() / 2
    bound = gap * np.repeat(c1.astype(np.float64), 64) + np.abs(wd) * 2.0 ** -8
    assert np.all(np.abs(wd - w) <= bound)
    # the element holding the block maximum comes back to within bf16 rounding
    blk = np.abs(w.reshape(-1, 64))
    idx = blk.argmax(axis=1)
    got = np.abs(wd.reshape(-1, 64)[np.arange(blk.shape[0]), idx])
    assert np.all(np.abs(got - blk.max(axis=1)) <= blk.max(axis=1) * 2.0 ** -8)


def test_roundtrip_idempotent_rows_and_zero_blocks():
    w = _w(outliers=True)
    p, c1 = oracle.quantize_nf4_sq(w)
    wd = oracle.dequantize_nf4_sq(p, c1)
    p2, _ = oracle.quantize_nf4_sq(wd)
    assert np.array_equal(p, p2)
    N, K = w.shape
    rows = [0, 5, 31, 5]
    assert np.array_equal(oracle.dequantize_rows_sq(p, c1, N, K, rows), wd.reshape(N, K)[rows])
    z = np.zeros(128, np.uint16)
    pz, cz = oracle.quantize_nf4_sq(z)
    assert np.all(cz == 0) and np.all(pz == 0x77)
    assert np.array_equal(oracle.dequantize_nf4_sq(pz, cz), z)


def test_storage_matches_the_pages_overhead():
    with open(os.path.join(GOLDEN, "memory_arithmetic.json")) as fh:
        g = {e["id"]: e for e in json.load(fh)["entries"]}
    n = 64 * 1000
    over = 8 * oracle.storage_bytes_sq(n) / n - 4
    assert over == g["fp32_scale_overhead_bits"]["value"]
    P = 70e9
    assert abs(P * over / 8 / 1e9 - g["fp32_scale_overhead_70b_gb"]["value"]) <= g["fp32_scale_overhead_70b_gb"]["tol"]
