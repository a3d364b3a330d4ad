"""GPU parity of the fused backward (QLORA_BWD_FUSED_GRADS): the dX kernel also
forms the adapter gradients dA = s X^T (dY B^T) and dB = s (X A)^T dY of its
256-token tile, and one launch adds the tiles.  dX must be the same bits as
the unfused backward (the dX arithmetic is unchanged); dA and dB are checked
against the fp64 oracle rounded once (max relative error <= 1e-2 with the rms
floor, mean absolute error <= 1e-3 rms), since they sum in another order."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from qlora_linear_layers_amd import api, synth
from helpers import assert_gemm_close, bits_of, say, to_dev

pytestmark = pytest.mark.gpu


def _case(lin, T, r, cfg=9):
    d = synth.layer_inputs(cfg, 0, 0, lin, T, r, with_dy=True)
    qw = api.nf4_quantize_dq(to_dev(d["w"], (lin.N, lin.K)))
    rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
    wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
    t = dict(x=to_dev(d["x"], (T, lin.K)), a=to_dev(d["a"], (lin.K, r)), b=to_dev(d["b"], (r, lin.N)),
             dy=to_dev(d["dy"], (T, lin.N)))
    return d, qw, wd, t


# (name, weight [N, K], T, r, s): ragged tiles in every dimension, padded ranks,
# more gradient blocks than waves and fewer, one-tile token groups (T < 1024)
# and two-tile groups with a ragged last group (T = 1100: five tiles), and a
# T <= 96 backward (its forward runs decode windows)
CASES = [
    ("ragged", synth.Linear("t", 448, 320), 300, 16, 1.0),
    ("multi-tile", synth.Linear("t", 768, 1024), 520, 64, 0.25),
    ("rank 136", synth.Linear("t", 448, 320), 300, 136, 0.5),
    ("rank 256 at T = 129", synth.Linear("t", 1088, 576), 129, 256, 0.25),
    ("one k tile", synth.Linear("t", 2112, 256), 260, 64, 0.25),
    ("many k tiles", synth.Linear("t", 192, 2560), 300, 16, 1.0),
    ("five token tiles", synth.Linear("t", 704, 384), 1100, 24, 0.5),
    ("four token tiles, rank 192", synth.Linear("t", 320, 448), 1024, 136, 0.25),
    ("T = 40", synth.Linear("t", 640, 448), 40, 24, 0.5),
]


@pytest.mark.parametrize("name,lin,T,r,s", CASES, ids=[c[0] for c in CASES])
def test_fused_backward_against_oracle(name, lin, T, r, s):
    say(f"[fused bwd] {name}: T={T} N={lin.N} K={lin.K} r={r} s={s}")
    d, qw, wd, t = _case(lin, T, r)
    dx_u, _, _ = api.qlora_linear_bwd_input(t["dy"], qw, t["a"], t["b"], s, x=t["x"], lora_grads=True)
    dx, da, db = api.qlora_linear_bwd_input(t["dy"], qw, t["a"], t["b"], s, x=t["x"], lora_grads=True,
                                            fused_grads=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(dx), bits_of(dx_u)), f"{name}: fused dX differs from the unfused dX"
    rdx, rda, rdb = oracle.linear_bwd(d["dy"], d["x"], wd, d["a"], d["b"], s)
    assert_gemm_close(bits_of(dx), rdx, f"{name} dX")
    assert_gemm_close(bits_of(da), rda, f"{name} dA")
    assert_gemm_close(bits_of(db), rdb, f"{name} dB")


@pytest.mark.parametrize("T", [333, 64])
def test_fused_backward_reusing_the_forward(T):
    """Both flags: s X A from the forward's workspace (T = 333), or recomputed
    because the decode-window forward keeps none (T = 64); the same bits as the
    fused backward that recomputes it, and deterministic over repeated calls."""
    lin = synth.Linear("t", 640, 448)
    r, s = 24, 0.5
    d, qw, wd, t = _case(lin, T, r)
    ref = [bits_of(v) for v in api.qlora_linear_bwd_input(t["dy"], qw, t["a"], t["b"], s, x=t["x"],
                                                            lora_grads=True, fused_grads=True)]
    n = api.qlora_workspace_bytes_bwd(T, lin.K, lin.N, r, api.FUSED_GRADS | api.REUSE_FORWARD)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        api.qlora_linear_fwd(t["x"], qw, t["a"], t["b"], s, workspace=ws)
        got = [bits_of(v) for v in api.qlora_linear_bwd_input(t["dy"], qw, t["a"], t["b"], s, x=t["x"],
                                                                lora_grads=True, workspace=ws, reuse_forward=True,
                                                                fused_grads=True)]
        for what, u, v in zip(("dX", "dA", "dB"), got, ref):
            assert np.array_equal(u, v), what


@pytest.mark.parametrize("which", ["dA", "dB"])
def test_fused_backward_one_gradient(which):
    """Only one of d_lora_a / d_lora_b asked for (through the C ABI): the other
    stays untouched, the one asked for matches the oracle."""
    lin = synth.Linear("t", 704, 576)
    T, r, s = 300, 32, 0.75
    d, qw, wd, t = _case(lin, T, r)
    dx = torch.empty((T, lin.K), dtype=torch.bfloat16, device="cuda")
    da = torch.full((lin.K, r), 7.0, dtype=torch.bfloat16, device="cuda")
    db = torch.full((r, lin.N), 7.0, dtype=torch.bfloat16, device="cuda")
    flags = api.FUSED_GRADS
    ws = torch.empty(api.qlora_workspace_bytes_bwd(T, lin.K, lin.N, r, flags), dtype=torch.uint8, device="cuda")
    p = lambda v: ctypes.c_void_p(v.data_ptr())
    st = api.lib().qlora_linear_bwd_input(
        p(t["dy"]), T, lin.K, lin.N, p(qw.codes), p(qw.absmax_fp8), p(qw.superscale), p(t["a"]), p(t["b"]), r,
        ctypes.c_float(s), p(dx), p(t["x"]), p(da) if which == "dA" else None, p(db) if which == "dB" else None,
        p(ws), ws.numel(), flags, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    rdx, rda, rdb = oracle.linear_bwd(d["dy"], d["x"], wd, d["a"], d["b"], s)
    assert_gemm_close(bits_of(dx), rdx, "dX")
    if which == "dA":
        assert_gemm_close(bits_of(da), rda, "dA")
        assert bool((db == 7.0).all()), "dB was written"
    else:
        assert_gemm_close(bits_of(db), rdb, "dB")
        assert bool((da == 7.0).all()), "dA was written"


def test_fused_backward_7b_q_full():
    """The LLaMA-7B q projection at T = 4096, r = 64, s = 0.25, with the forward's
    s X A reused: dX equal to the unfused backward, every dA and dB element
    against the oracle."""
    lin = synth.LLAMA7B[0]
    T, r, s = 4096, 64, 16.0 / 64
    say(f"[fused bwd] LLaMA-7B q: T={T} N={lin.N} K={lin.K} r={r}")
    d, qw, wd, t = _case(lin, T, r, cfg=3)
    dx_u, _, _ = api.qlora_linear_bwd_input(t["dy"], qw, t["a"], t["b"], s, x=t["x"], lora_grads=True)
    ws = torch.empty(api.qlora_workspace_bytes_bwd(T, lin.K, lin.N, r, api.FUSED_GRADS | api.REUSE_FORWARD),
                     dtype=torch.uint8, device="cuda")
    api.qlora_linear_fwd(t["x"], qw, t["a"], t["b"], s, workspace=ws)
    dx, da, db = api.qlora_linear_bwd_input(t["dy"], qw, t["a"], t["b"], s, x=t["x"], lora_grads=True,
                                            workspace=ws, reuse_forward=True, fused_grads=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(dx), bits_of(dx_u))
    rda, rdb = oracle.lora_grads(d["x"], d["dy"], d["a"], d["b"], s)
    assert_gemm_close(bits_of(da), rda, "dA (full)")
    assert_gemm_close(bits_of(db), rdb, "dB (full)")


def test_fused_backward_fp16_and_single_quantization():
    """The flag on the fp16 compute type and on single-quantized weights: dX
    equal to the unfused call of the same variant, dA and dB against their
    oracles."""
    lin, T, r, s = synth.Linear("t", 448, 320), 300, 16, 1.0
    # fp16
    d = synth.layer_inputs_f16(9, 0, 0, lin, T, r, with_dy=True)
    h = lambda bits, shape: torch.from_numpy(np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
                                             .view(np.int16)).view(torch.float16).reshape(shape).cuda()
    qw = api.nf4_quantize_dq(h(d["w"], (lin.N, lin.K)))
    rc, rf, rs = oracle.quantize_nf4_dq_f16(d["w"])
    wd = oracle.dequantize_nf4_dq_f16(rc, rf, rs).reshape(lin.N, lin.K)
    x, a, b, dy = h(d["x"], (T, lin.K)), h(d["a"], (lin.K, r)), h(d["b"], (r, lin.N)), h(d["dy"], (T, lin.N))
    dx_u, _, _ = api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x, lora_grads=True)
    dx, da, db = api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x, lora_grads=True, fused_grads=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(dx), bits_of(dx_u)), "fp16 dX"
    _, rda, rdb = oracle.linear_bwd_f16(d["dy"], d["x"], wd, d["a"], d["b"], s)
    for what, got, ref in (("fp16 dA", da, rda), ("fp16 dB", db, rdb)):
        g, rr = oracle.f16_bits_to_f64(bits_of(got)).reshape(-1), oracle.f16_bits_to_f64(ref).reshape(-1)
        rms = np.sqrt(np.mean(rr * rr))
        err = np.abs(g - rr)
        assert float(np.max(err / np.maximum(np.abs(rr), rms))) <= 1e-2 and float(np.mean(err) / rms) <= 1e-3, what
    # single quantization
    d = synth.layer_inputs(9, 0, 0, lin, T, r, with_dy=True)
    qw = api.nf4_quantize(to_dev(d["w"], (lin.N, lin.K)))
    rc, ra = oracle.quantize_nf4_sq(d["w"])
    wd = oracle.dequantize_nf4_sq(rc, ra).reshape(lin.N, lin.K)
    x, a, b = to_dev(d["x"], (T, lin.K)), to_dev(d["a"], (lin.K, r)), to_dev(d["b"], (r, lin.N))
    dy = to_dev(d["dy"], (T, lin.N))
    dx_u, _, _ = api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x, lora_grads=True)
    dx, da, db = api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x, lora_grads=True, fused_grads=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(dx), bits_of(dx_u)), "single-quantization dX"
    _, rda, rdb = oracle.linear_bwd(d["dy"], d["x"], wd, d["a"], d["b"], s)
    assert_gemm_close(bits_of(da), rda, "single-quantization dA")
    assert_gemm_close(bits_of(db), rdb, "single-quantization dB")
