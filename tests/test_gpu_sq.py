"""GPU parity of the single-quantization variant (codes + fp32 block absmax,
"QLoRA 原理精讲" section 2.2, the first level alone) against the oracle:
bit-exact codes, absmax and dequantized bf16; the forward, backward, decode
and merge paths under the tolerances of their double-quantized counterparts."""
import numpy as np
import pytest
import torch

import oracle
from qlora_linear_layers_amd import api, synth
from helpers import assert_gemm_close, bits_of, say, to_dev, to_dev_f32, to_dev_u8
from test_gpu_merge import _assert_merge_close

pytestmark = pytest.mark.gpu


def _check_quant(w_bits, shape, name):
    say(f"[quant sq] {name} shape={shape}")
    qw = api.nf4_quantize(to_dev(w_bits, shape))
    torch.cuda.synchronize()
    rc, ra = oracle.quantize_nf4_sq(w_bits)
    c, a = qw.codes.cpu().numpy(), qw.absmax.cpu().numpy()
    assert np.array_equal(c, rc), f"{name}: packed codes differ at {np.flatnonzero(c != rc)[:8]}"
    assert np.array_equal(a.view(np.uint32), ra.view(np.uint32)), f"{name}: absmax differs"
    wd = bits_of(api.nf4_dequantize(qw)).reshape(-1)
    rd = oracle.dequantize_nf4_sq(rc, ra)
    assert np.array_equal(wd, rd), f"{name}: dequantized bf16 differ at {np.flatnonzero(wd != rd)[:8]}"


def test_quantize_dequantize_bit_exact():
    w = synth.layer_inputs(1, 0, 0, synth.Linear("w", 4096, 4096), 0, 0)["w"]
    _check_quant(w, (4096, 4096), "4096x4096 N(0,0.02)")
    rng = np.random.default_rng(21)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    x[0:3] = 0.0                                          # all-zero blocks
    x[3] *= 1e-38                                         # bf16 subnormals
    x[4] *= 2.0 ** -100                                   # exact-division path
    x[5] *= 1e30
    _check_quant(synth.to_bf16_bits(x), x.shape, "300 blocks, edge magnitudes")
    w = synth.outlier_weight_bf16(synth.rng_for(5, 0, 0, synth.ROLE_W), (1024, 8192))
    _check_quant(w, (1024, 8192), "70B k-shape slice with outliers")


def test_oracle_storage_dequantizes_like_the_oracle():
    """Codes and absmax written by the oracle, dequantized on the GPU."""
    w = synth.layer_inputs(9, 0, 0, synth.Linear("w", 384, 512), 0, 0)["w"]
    rc, ra = oracle.quantize_nf4_sq(w)
    qw = api.NF4WeightSQ(to_dev_u8(rc), to_dev_f32(ra), 384, 512)
    assert np.array_equal(bits_of(api.nf4_dequantize(qw)).reshape(-1), oracle.dequantize_nf4_sq(rc, ra))


def _linear(name, lin, T, r, s, cfg=9, check_bwd=True):
    say(f"[linear sq] {name}: T={T} N={lin.N} K={lin.K} r={r} s={s}")
    d = synth.layer_inputs(cfg, 0, 0, lin, T, r, with_dy=True)
    qw = api.nf4_quantize(to_dev(d["w"], (lin.N, lin.K)))
    rc, ra = oracle.quantize_nf4_sq(d["w"])
    wd = oracle.dequantize_nf4_sq(rc, ra).reshape(lin.N, lin.K)
    x = to_dev(d["x"], (T, lin.K))
    a = to_dev(d["a"], (lin.K, r)) if r else None
    b = to_dev(d["b"], (r, lin.N)) if r else None
    ra_, rb_ = (d["a"], d["b"]) if r else (None, None)
    y = api.qlora_linear_fwd(x, qw, a, b, s)
    torch.cuda.synchronize()
    assert_gemm_close(bits_of(y), oracle.linear_fwd(d["x"], wd, ra_, rb_, s), f"{name} Y")
    if not check_bwd:
        return
    dy = to_dev(d["dy"], (T, lin.N))
    dx, da, db = api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x if r else None, lora_grads=bool(r))
    torch.cuda.synchronize()
    rdx, rda, rdb = oracle.linear_bwd(d["dy"], d["x"], wd, ra_, rb_, s)
    assert_gemm_close(bits_of(dx), rdx, f"{name} dX")
    if r:
        assert_gemm_close(bits_of(da), rda, f"{name} dA")
        assert_gemm_close(bits_of(db), rdb, f"{name} dB")


def test_linear_prefill_shapes():
    _linear("ragged", synth.Linear("t", 448, 320), T=300, r=16, s=1.0)
    _linear("multi-tile", synth.Linear("t", 768, 1024), T=520, r=64, s=0.25)
    _linear("r=0", synth.Linear("t", 512, 256), T=64, r=0, s=0.0)


def test_linear_decode_shapes():
    for T in (1, 5, 16):
        _linear(f"T={T}", synth.Linear("t", 384, 512), T=T, r=16, s=0.5)


def test_one_hot_rows_give_the_dequantized_weight():
    """X = one-hot rows: Y reproduces rows of W' exactly (single-quantization layout)."""
    lin = synth.Linear("t", 320, 256)
    d = synth.layer_inputs(9, 0, 0, lin, 0, 0)
    qw = api.nf4_quantize(to_dev(d["w"], (lin.N, lin.K)))
    wd = bits_of(api.nf4_dequantize(qw))
    x = torch.zeros((lin.K, lin.K), dtype=torch.bfloat16, device="cuda")
    x.fill_diagonal_(1.0)
    assert np.array_equal(bits_of(api.qlora_linear_fwd(x, qw)), wd.T.copy())
    dy = torch.zeros((lin.N, lin.N), dtype=torch.bfloat16, device="cuda")
    dy.fill_diagonal_(1.0)
    dx, _, _ = api.qlora_linear_bwd_input(dy, qw)
    assert np.array_equal(bits_of(dx), wd)


def test_linear_7b_gate_sampled():
    lin = synth.LLAMA7B[4]
    T, r, s = 512, 64, 0.25
    say(f"[linear sq sampled] {lin.name}: T={T} N={lin.N} K={lin.K} r={r}")
    d = synth.layer_inputs(3, 0, 4, lin, T, r, with_dy=True)
    qw = api.nf4_quantize(to_dev(d["w"], (lin.N, lin.K)))
    rc, ra = oracle.quantize_nf4_sq(d["w"])
    x, a, b = to_dev(d["x"], (T, lin.K)), to_dev(d["a"], (lin.K, r)), to_dev(d["b"], (r, lin.N))
    y = bits_of(api.qlora_linear_fwd(x, qw, a, b, s))
    rng = np.random.default_rng(77)
    t, n = rng.integers(0, T, 192), rng.integers(0, lin.N, 192)
    wrows = oracle.dequantize_rows_sq(rc, ra, lin.N, lin.K, n)
    assert_gemm_close(y[t, n], oracle.linear_fwd_at(d["x"], wrows, d["a"], d["b"], s, t, n), "Y samples")


def test_merge():
    lin = synth.Linear("t", 200, 448)
    r, s = 72, 6.0
    d = synth.layer_inputs(9, 0, 0, lin, 0, r)
    qw = api.nf4_quantize(to_dev(d["w"], (lin.N, lin.K)))
    rc, ra = oracle.quantize_nf4_sq(d["w"])
    wd = oracle.dequantize_nf4_sq(rc, ra).reshape(lin.N, lin.K)
    a, b = to_dev(d["a"], (lin.K, r)), to_dev(d["b"], (r, lin.N))
    got = bits_of(api.qlora_merge_lora(qw, a, b, s))
    _assert_merge_close(got, oracle.merge_lora(wd, d["a"], d["b"], s), wd, d["a"], d["b"], s, "merge sq")
    assert np.array_equal(bits_of(api.qlora_merge_lora(qw)), wd)
