"""GPU parity of the INT4 absmax baseline of the data-type ablation ("QLoRA 原理精讲",
section 2.1): bit-exact codes, absmax and dequantized bf16 against the oracle,
including ratios on and next to the INT4 decision midpoints, and the ablation's
error figures computed from the GPU results."""
import numpy as np
import pytest
import torch

import oracle
from qlora_linear_layers_amd import api, synth
from helpers import bits_of, say, to_dev

pytestmark = pytest.mark.gpu


def _check(w_bits, shape, name):
    say(f"[int4] {name} shape={shape}")
    qw = api.int4_quantize(to_dev(w_bits, shape))
    torch.cuda.synchronize()
    rc, ra = oracle.quantize_int4(w_bits)
    c, a = qw.codes.cpu().numpy(), qw.absmax.cpu().numpy()
    assert np.array_equal(c, rc), f"{name}: codes differ at {np.flatnonzero(c != rc)[:8]}"
    assert np.array_equal(a.view(np.uint32), ra.view(np.uint32)), f"{name}: absmax differs"
    wd = bits_of(api.int4_dequantize(qw)).reshape(-1)
    assert np.array_equal(wd, oracle.dequantize_int4(rc, ra)), f"{name}: dequantized values differ"
    return wd


def test_normal_and_outlier_weights():
    w = synth.layer_inputs(1, 0, 0, synth.Linear("w", 4096, 4096), 0, 0)["w"]
    _check(w, (4096, 4096), "4096x4096 N(0,0.02)")
    w = synth.outlier_weight_bf16(synth.rng_for(5, 0, 0, synth.ROLE_W), (1024, 8192))
    _check(w, (1024, 8192), "70B k-shape slice with outliers")


def test_ratios_on_the_midpoints_and_edge_blocks():
    rng = np.random.default_rng(31)
    nb = 640
    x = np.zeros((nb, 64), np.float32)
    for b in range(nb):
        c1 = float(2.0 ** rng.integers(-20, 20)) * 14.0
        k = rng.integers(-14, 15, 64).astype(np.float32)
        x[b] = k * np.float32(c1 / 14.0)                  # ratios k / 14: on INT4 midpoints for odd k
        x[b, rng.integers(0, 64)] = c1 if b % 2 else -c1
        if b % 3 == 0:                                    # neighbours of the midpoints, one bf16 step away
            bits = synth.to_bf16_bits(x[b])
            step = np.where(rng.random(64) < 0.5, 1, -1).astype(np.int32)
            step[(bits & 0x7FFF) == 0] = 0                # zeros stay zero (no step into NaN codes)
            x[b] = oracle.bf16_bits_to_f32((bits.astype(np.int32) + step).astype(np.uint16))
            x[b, 0] = c1
    x[0] = 0.0                                            # all-zero block
    x[1] *= 2.0 ** -110                                   # tiny magnitudes
    _check(synth.to_bf16_bits(x), x.shape, "midpoint ratios")


def test_ablation_errors_from_gpu_results():
    w = synth.normal_bf16(synth.rng_for(1, 0, 0, synth.ROLE_W), (512, 4096), 0.02)
    wi = _check(w, (512, 4096), "ablation normal")
    wn = bits_of(api.nf4_dequantize(api.nf4_quantize(to_dev(w, (512, 4096))))).reshape(-1)
    en, ei = oracle.relative_rms_error(w, wn), oracle.relative_rms_error(w, wi)
    say(f"  relative rms error: NF4 {en:.4f}, INT4 {ei:.4f}")
    rn, ra = oracle.quantize_nf4_sq(w)
    assert en == oracle.relative_rms_error(w, oracle.dequantize_nf4_sq(rn, ra))
    assert en < ei
