"""GPU parity of the LoRA merge W_m = RNE_bf16(W' + s (A B)^T) ("QLoRA 原理精讲",
section 2.5 and section 3 pitfall 3) against the fp64 oracle rounded once.

Tolerance, from the arithmetic: the kernel forms the rank-r sum in fp32 (each
bf16 x bf16 product is exact; r additions) and adds W' with one fused
multiply-add, so before the bf16 rounding it lies within
    e = 2^-24 |W_m| + |s| r 2^-24 sum_j |A[k][j] B[j][n]|
of the exact value.  An element can therefore differ from the oracle only
where the exact value sits within e of a bf16 rounding boundary:
    |gpu - ref| <= ulp_bf16(ref) + 2 e
and at most 1e-3 of the elements may differ at all (a systematic error would
move far more).  Without an adapter (r = 0) or with s = 0 the result is W'
itself, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from qlora_linear_layers_amd import api, synth
from helpers import bits_of, f64_of_bits, say, to_dev

pytestmark = pytest.mark.gpu


def _ulp_bf16(v):
    _, e = np.frexp(np.abs(v))
    return np.where(v == 0, 2.0 ** -133, np.ldexp(1.0, e - 8))


def _assert_merge_close(got, ref, wd, a, b, s, what):
    g, r = f64_of_bits(got), f64_of_bits(ref)
    rank = a.shape[1]
    absab = np.abs(f64_of_bits(a)) @ np.abs(f64_of_bits(b))           # [K, N]
    e = 2.0 ** -24 * np.abs(r) + abs(s) * rank * 2.0 ** -24 * absab.T
    bound = _ulp_bf16(r) + 2 * e
    diff = np.abs(g - r)
    frac = float(np.mean(got != ref))
    worst = float(np.max(diff / bound))
    say(f"  {what}: differing {frac:.2e}, worst diff / bound {worst:.3f}")
    assert worst <= 1.0, what
    assert frac <= 1e-3, what


def _setup(lin, r, cfg=9):
    d = synth.layer_inputs(cfg, 0, 0, lin, 0, r)
    qw = api.nf4_quantize_dq(to_dev(d["w"], (lin.N, lin.K)))
    rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
    return d, qw, (rc, rf, rs)


@pytest.mark.parametrize("N,K,r,s", [(384, 320, 16, 0.5), (104, 512, 72, 48.0), (64, 64, 8, 2.0),
                                     (256, 1024, 256, 0.25), (192, 448, 136, 16.0), (136, 768, 64, -8.0)])
def test_merge_small(N, K, r, s):
    lin = synth.Linear("t", N, K)
    say(f"[merge] N={N} K={K} r={r} s={s}")
    d, qw, (rc, rf, rs) = _setup(lin, r)
    wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(N, K)
    a, b = to_dev(d["a"], (K, r)), to_dev(d["b"], (r, N))
    got = bits_of(api.qlora_merge_lora(qw, a, b, s))
    torch.cuda.synchronize()
    ref = oracle.merge_lora(wd, d["a"], d["b"], s)
    _assert_merge_close(got, ref, wd, d["a"], d["b"], s, f"N={N} K={K} r={r}")


def test_merge_without_adapter_is_the_base_weight():
    lin = synth.Linear("t", 192, 320)
    d, qw, (rc, rf, rs) = _setup(lin, 32)
    wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
    assert np.array_equal(bits_of(api.qlora_merge_lora(qw)), wd)
    a, b = to_dev(d["a"], (lin.K, 32)), to_dev(d["b"], (32, lin.N))
    assert np.array_equal(bits_of(api.qlora_merge_lora(qw, a, b, 0.0)), wd)


def test_merge_is_deterministic():
    lin = synth.Linear("t", 320, 512)
    d, qw, _ = _setup(lin, 64)
    a, b = to_dev(d["a"], (lin.K, 64)), to_dev(d["b"], (64, lin.N))
    first = bits_of(api.qlora_merge_lora(qw, a, b, 3.0))
    assert np.array_equal(bits_of(api.qlora_merge_lora(qw, a, b, 3.0)), first)


def test_merge_7b_q_full():
    lin = synth.LLAMA7B[0]
    say(f"[merge] 7B {lin.name} {lin.N}x{lin.K} r=64 (full)")
    d, qw, (rc, rf, rs) = _setup(lin, 64, cfg=3)
    wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
    a, b = to_dev(d["a"], (lin.K, 64)), to_dev(d["b"], (64, lin.N))
    s = synth.TRAIN_7B["scaling"]
    got = bits_of(api.qlora_merge_lora(qw, a, b, s))
    torch.cuda.synchronize()
    _assert_merge_close(got, oracle.merge_lora(wd, d["a"], d["b"], s), wd, d["a"], d["b"], s, "q 4096x4096")


def test_merge_several_tiles_per_workgroup():
    """N = 8192, K = 2880, r = 64, in full: a workgroup walks three 256-wide k
    tiles of its 64-row block (an odd count, so the pair after the third is
    empty), and the last tile of every row holds only 64 valid k."""
    lin = synth.Linear("t", 8192, 2880)
    say(f"[merge] {lin.N}x{lin.K} r=64 (full, three k tiles per workgroup)")
    d, qw, (rc, rf, rs) = _setup(lin, 64, cfg=5)
    wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
    a, b = to_dev(d["a"], (lin.K, 64)), to_dev(d["b"], (64, lin.N))
    got = bits_of(api.qlora_merge_lora(qw, a, b, 0.75))
    torch.cuda.synchronize()
    _assert_merge_close(got, oracle.merge_lora(wd, d["a"], d["b"], 0.75), wd, d["a"], d["b"], 0.75, "8192x2880")


@pytest.mark.parametrize("idx", [4, 6])
def test_merge_7b_sampled_rows(idx):
    lin = synth.LLAMA7B[idx]
    say(f"[merge] 7B {lin.name} {lin.N}x{lin.K} r=64 (96 rows)")
    d, qw, (rc, rf, rs) = _setup(lin, 64, cfg=3)
    a, b = to_dev(d["a"], (lin.K, 64)), to_dev(d["b"], (64, lin.N))
    s = synth.TRAIN_7B["scaling"]
    got = bits_of(api.qlora_merge_lora(qw, a, b, s))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(idx).choice(lin.N, 96, replace=False))
    wrows = oracle.dequantize_rows(rc, rf, rs, lin.N, lin.K, rows)
    ref = oracle.merge_lora_rows(wrows, d["a"], d["b"], s, rows)
    _assert_merge_close(got[rows], ref, wrows, d["a"], d["b"][:, rows], s, f"{lin.name} rows")
