"""Pins of the INT4 absmax baseline and of the data-type ablation ("QLoRA 原理精讲",
section 2.1: INT4 bins are uniform over [-8, 7]; NF4 bins carry equal probability
under a normal distribution)."""
import numpy as np

import oracle
from qlora_linear_layers_amd import synth


def test_levels_and_closed_form_code():
    v = oracle.int4_levels()
    assert v[8] == 0 and v[15] == 1 and v[1] == -1 and np.allclose(np.diff(v), 1 / 7)
    rng = np.random.default_rng(1)
    w = synth.to_bf16_bits(rng.standard_normal(64 * 2000).astype(np.float32))
    wf = oracle.bf16_bits_to_f32(w)
    c1 = oracle.block_absmax(wf)
    n = (wf.reshape(-1, 64) / c1[:, None]).astype(np.float32).astype(np.float64).reshape(-1)
    codes = oracle.int4_encode(wf, c1).astype(np.int64)
    # brute force: the nearest fp32 level (distances exact in fp64), first index on ties
    dist = np.abs(n[:, None] - oracle.int4_levels_f32().astype(np.float64)[None, :])
    assert np.array_equal(codes, np.argmin(dist, axis=1))
    # closed form: round half down of 7 n (exact in fp64); it may differ only where
    # fp32 rounding of the levels moves a midpoint across n
    want = np.ceil(7 * n - 0.5).astype(np.int64) + 8
    near = np.abs(7 * n - np.floor(7 * n) - 0.5) < 1e-6
    assert np.all((codes == want) | near) and near.mean() < 1e-2
    assert codes.min() >= 1                          # -8 is never the nearest level


def test_error_bound_zero_blocks_and_mirror():
    rng = np.random.default_rng(2)
    wf = (rng.standard_normal(64 * 500) * 0.02).astype(np.float32)
    wf[:64] = 0
    w = synth.to_bf16_bits(wf)
    p, c1 = oracle.quantize_int4(w)
    codes = oracle.unpack_codes(p)
    assert np.all(codes[:64] == 8)
    wd = oracle.bf16_bits_to_f32(oracle.dequantize_int4(p, c1)).astype(np.float64)
    x = oracle.bf16_bits_to_f32(w).astype(np.float64)
    bound = np.repeat(c1.astype(np.float64), 64) / 14 * (1 + 1e-6) + np.abs(wd) * 2.0 ** -8
    assert np.all(np.abs(wd - x) <= bound)
    # mirrored weights give mirrored codes (16 - code) away from ties
    pm, _ = oracle.quantize_int4(w ^ np.uint16(0x8000))
    cm = oracle.unpack_codes(pm).astype(np.int64)
    nz = codes != 8
    assert np.mean(cm[nz] == 16 - codes[nz].astype(np.int64)) > 0.999


def test_ablation_normal_favours_nf4_uniform_favours_int4():
    """The claim under test, on seeded data: NF4 has the lower error on normal
    weights (with and without outliers); uniform weights reverse it."""
    rng = synth.rng_for(1, 0, 0, synth.ROLE_W)
    cases = {
        "normal": synth.normal_bf16(rng, (64, 4096), 0.02),
        "outliers": synth.outlier_weight_bf16(synth.rng_for(5, 0, 0, synth.ROLE_W), (64, 4096)),
        "uniform": synth.to_bf16_bits(np.random.default_rng(3).uniform(-1, 1, 64 * 4096).astype(np.float32)),
    }
    err = {}
    for name, w in cases.items():
        pn, cn = oracle.quantize_nf4_sq(w)
        pi, ci = oracle.quantize_int4(w)
        err[name] = (oracle.relative_rms_error(w, oracle.dequantize_nf4_sq(pn, cn)),
                     oracle.relative_rms_error(w, oracle.dequantize_int4(pi, ci)))
    assert err["normal"][0] < err["normal"][1]
    assert err["outliers"][0] < err["outliers"][1]
    assert err["uniform"][1] < err["uniform"][0]
