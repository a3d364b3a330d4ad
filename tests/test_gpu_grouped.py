"""GPU parity of the grouped decode forward (several independent layers in one
launch pair): each output must be bit-identical to the single-layer call, which
the decode tests pin to the oracle, and a ragged group of mixed shapes is also
checked against the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
from qlora_linear_layers_amd import api, synth
from helpers import assert_gemm_close, bits_of, say, to_dev

pytestmark = pytest.mark.gpu


def _layer(cfg, idx, lin, T, r):
    d = synth.layer_inputs(cfg, 0, idx, lin, T, r)
    qw = api.nf4_quantize_dq(to_dev(d["w"], (lin.N, lin.K)))
    x = to_dev(d["x"], (T, lin.K))
    a = to_dev(d["a"], (lin.K, r)) if r else None
    b = to_dev(d["b"], (r, lin.N)) if r else None
    return d, qw, x, a, b


def _group_vs_single(cfg, lins, T, r, s):
    layers = [_layer(cfg, i, lin, T, r) for i, lin in enumerate(lins)]
    probs = [(x, qw, a, b, s, torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda"))
             for lin, (_, qw, x, a, b) in zip(lins, layers)]
    got = api.qlora_linear_fwd_grouped(probs)
    torch.cuda.synchronize()
    for lin, (_, qw, x, a, b), y in zip(lins, layers, got):
        ref = api.qlora_linear_fwd(x, qw, a, b, s)
        assert np.array_equal(bits_of(y), bits_of(ref)), f"{lin.name} {lin.N}x{lin.K} T={T}: grouped != single"
    return layers, got


@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_7b_layer_set_matches_single_calls(T):
    say(f"[grouped] LLaMA-7B layer set, T={T}, r=64")
    _group_vs_single(2, synth.LLAMA7B, T, 64, 0.25)


def test_dependency_stages():
    """The groups a decode step can launch together: q/k/v, gate/up (and o, down alone)."""
    for stage in ((0, 1, 2), (4, 5), (3,), (6,)):
        say(f"[grouped] stage {[synth.LLAMA7B[i].name for i in stage]} T=8")
        _group_vs_single(2, [synth.LLAMA7B[i] for i in stage], 8, 64, 0.25)


def test_ragged_mixed_shapes_against_oracle():
    """Eight problems (the maximum), N not a multiple of 128 and K not a multiple of
    512 (partial row blocks and k splits), against the oracle and the single calls."""
    lins = [synth.Linear(f"p{i}", n, k) for i, (n, k) in enumerate(
        [(320, 448), (64, 64), (1024, 576), (192, 1088), (448, 320), (128, 2048), (576, 704), (64, 1024)])]
    T, r, s = 5, 24, 0.75
    say(f"[grouped] ragged group of {len(lins)}, T={T}, r={r}")
    layers, got = _group_vs_single(9, lins, T, r, s)
    for lin, (d, _, _, _, _), y in zip(lins, layers, got):
        rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
        wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
        assert_gemm_close(bits_of(y), oracle.linear_fwd(d["x"], wd, d["a"], d["b"], s), f"{lin.name} Y")


def test_no_adapter_group():
    lins = [synth.Linear("a", 512, 256), synth.Linear("b", 256, 768)]
    say("[grouped] r=0 group, T=3")
    layers, got = _group_vs_single(9, lins, 3, 0, 0.0)
    for lin, (d, _, _, _, _), y in zip(lins, layers, got):
        rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
        wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
        assert_gemm_close(bits_of(y), oracle.linear_fwd(d["x"], wd, None, None, 0.0), f"{lin.name} Y")


def test_repeat_calls_are_identical():
    lins = synth.LLAMA7B[:3]
    layers = [_layer(2, i, lin, 4, 64) for i, lin in enumerate(lins)]
    outs = []
    for _ in range(2):
        probs = [(x, qw, a, b, 0.25, torch.empty((4, lin.N), dtype=torch.bfloat16, device="cuda"))
                 for lin, (_, qw, x, a, b) in zip(lins, layers)]
        outs.append([bits_of(y) for y in api.qlora_linear_fwd_grouped(probs)])
    for u, v in zip(*outs):
        assert np.array_equal(u, v)


def _oracle_y(d, lin, s):
    rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
    wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
    return oracle.linear_fwd(d["x"], wd, d["a"], d["b"], s)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8])
def test_valu_product_ragged_against_oracle(T):
    """The decode product as VALU dot products (no matrix-core instruction): the
    ragged group of mixed shapes against the oracle, and against the MFMA form."""
    lins = [synth.Linear(f"p{i}", n, k) for i, (n, k) in enumerate(
        [(320, 448), (64, 64), (1024, 576), (192, 1088), (448, 320), (128, 2048), (576, 704), (64, 1024)])]
    r, s = 24, 0.75
    say(f"[grouped] VALU product, ragged group of {len(lins)}, T={T}, r={r}")
    layers = [_layer(9, i, lin, T, r) for i, lin in enumerate(lins)]
    outs = {}
    for prod in ("valu", "mfma"):
        probs = [(x, qw, a, b, s, torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda"))
                 for lin, (_, qw, x, a, b) in zip(lins, layers)]
        outs[prod] = [bits_of(y) for y in api.qlora_linear_fwd_grouped(probs, product=prod)]
    for lin, (d, _, _, _, _), yv, ym in zip(lins, layers, outs["valu"], outs["mfma"]):
        ref = _oracle_y(d, lin, s)
        assert_gemm_close(yv, ref, f"{lin.name} Y (VALU)")
        assert_gemm_close(ym, ref, f"{lin.name} Y (MFMA)")


def test_valu_product_7b_shapes_full():
    """The VALU product on the LLaMA-7B q, gate and down shapes (one group, r = 64,
    s = 0.25) at T = 1, 4, 8: every output against the oracle; a repeated call
    gives the same bits."""
    lins = [synth.LLAMA7B[i] for i in (0, 4, 6)]
    data = [synth.layer_inputs(2, 0, i, lin, 8, 64) for i, lin in zip((0, 4, 6), lins)]
    qws = [api.nf4_quantize_dq(to_dev(d["w"], (lin.N, lin.K))) for d, lin in zip(data, lins)]
    wds = []
    for d, lin in zip(data, lins):
        rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
        wds.append(oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K))
    ab = [(to_dev(d["a"], (lin.K, 64)), to_dev(d["b"], (64, lin.N))) for d, lin in zip(data, lins)]
    for T in (1, 4, 8):
        say(f"[grouped] VALU product, LLaMA-7B q/gate/down, T={T}, r=64 (full outputs)")
        runs = []
        for _ in range(2):
            probs = [(to_dev(d["x"][:T], (T, lin.K)), qw, a, b, 0.25,
                      torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda"))
                     for d, lin, qw, (a, b) in zip(data, lins, qws, ab)]
            runs.append([bits_of(y) for y in api.qlora_linear_fwd_grouped(probs, product="valu")])
        for u, v in zip(*runs):
            assert np.array_equal(u, v)
        for d, lin, wd, y in zip(data, lins, wds, runs[0]):
            ref = oracle.linear_fwd(d["x"][:T], wd, d["a"], d["b"], 0.25)
            assert_gemm_close(y, ref, f"{lin.name} Y (VALU) T={T}")


def test_valu_product_rejects_more_than_8_tokens():
    lin = synth.Linear("a", 256, 256)
    _, qw, x, a, b = _layer(9, 0, lin, 9, 8)
    with pytest.raises(RuntimeError):
        api.qlora_linear_fwd_grouped([(x, qw, a, b, 1.0, torch.empty((9, 256), dtype=torch.bfloat16,
                                                                      device="cuda"))], product="valu")
