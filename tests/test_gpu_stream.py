"""GPU parity of the 70B-shaped streaming quantization: all 80 layers of
{q 8192x8192, k/v 1024x8192, o 8192x8192, gate/up 28672x8192, down 8192x28672}
with 0.1% Student-t(3) outliers, quantized and dequantized with one layer
resident.  The weights are drawn on the device; the bf16 bytes that the
oracle checks are copied back from there, so both sides see the same input.

Groups of 256 blocks are independent, so the oracle checks two random groups
of every tensor of every layer bit for bit (codes, FP8 codes, super-scale,
dequantized bf16), and the whole k-projection of the first and the last layer.
The packed total of the stack is checked against the storage closed form
(4 + 8/64 + 32/16384 bits per weight)."""
import numpy as np
import pytest
import torch

import oracle
from qlora_linear_layers_amd import synth
from qlora_linear_layers_amd.stream import LayerStream
from helpers import bits_of, say

pytestmark = pytest.mark.gpu


def _check_group(lin, l, g, w, qw, wd):
    e0, e1 = g * 16384, (g + 1) * 16384
    wb = bits_of(w.view(-1)[e0:e1])
    rc, rf, rs = oracle.quantize_nf4_dq(wb)
    where = f"layer {l} {lin.name} group {g}"
    assert np.array_equal(qw.codes[e0 // 2:e1 // 2].cpu().numpy(), rc), f"{where}: codes"
    assert np.array_equal(qw.absmax_fp8[e0 // 64:e1 // 64].cpu().numpy(), rf), f"{where}: FP8 codes"
    assert qw.superscale[g].cpu().numpy().view(np.uint32) == rs[0].view(np.uint32), f"{where}: super-scale"
    assert np.array_equal(bits_of(wd.view(-1)[e0:e1]), oracle.dequantize_nf4_dq(rc, rf, rs)), f"{where}: dequant"


def _check_full(lin, l, w, qw, wd):
    wb = bits_of(w).reshape(-1)
    rc, rf, rs = oracle.quantize_nf4_dq(wb)
    where = f"layer {l} {lin.name} (full)"
    assert np.array_equal(qw.codes.cpu().numpy(), rc), f"{where}: codes"
    assert np.array_equal(qw.absmax_fp8.cpu().numpy(), rf), f"{where}: FP8 codes"
    assert np.array_equal(qw.superscale.cpu().numpy().view(np.uint32), rs.view(np.uint32)), f"{where}: super-scales"
    assert np.array_equal(bits_of(wd).reshape(-1), oracle.dequantize_nf4_dq(rc, rf, rs)), f"{where}: dequant"


def test_stream_70b_all_layers():
    cfg = synth.STREAM_70B
    layers, L = cfg["layers"], cfg["n_layers"]
    rng = np.random.default_rng(15)
    seen = {"outliers": 0}

    def on_layer(l, ws, qws, wds):
        torch.cuda.synchronize()
        if l % 8 == 0 or l == L - 1:
            say(f"[stream 70B] layer {l}")
        for ti, (lin, w, qw, wd) in enumerate(zip(layers, ws, qws, wds)):
            if ti == 1 and l in (0, L - 1):
                _check_full(lin, l, w, qw, wd)
            ngroups = qw.superscale.numel()
            for g in rng.choice(ngroups, size=2, replace=False):
                _check_group(lin, l, int(g), w, qw, wd)
        # the outlier recipe is live: N(0, 0.02) alone never reaches 0.2 (10 sigma) in 855M draws
        seen["outliers"] += int(max(float(w.abs().max()) for w in ws) > 0.2)

    res = LayerStream([(lin.N, lin.K) for lin in layers]).run(
        lambda l: synth.device_layer_weights(cfg["config"], l, layers, outliers=True), L, on_layer, timed=False)
    params = L * sum(lin.N * lin.K for lin in layers)
    assert params == 68_451_041_280
    closed = L * sum(oracle.storage_bytes(lin.N * lin.K) for lin in layers)
    assert res["packed_bytes"] == closed == 35_311_779_840
    assert 8 * res["packed_bytes"] == params * (4 * 16384 + 8 * 256 + 32) // 16384
    assert seen["outliers"] == L
