"""The no-allocation forward (qlora_linear_fwd_noalloc, for callers that cannot
allocate device memory) against qlora_linear_fwd: the same kernels, so the
outputs must be identical bit for bit wherever qlora_linear_fwd's workspace fits
the static scratch.  Where its split-k partials would not, the no-allocation
call splits the reduction over fewer workgroups, and the two outputs, each
rounded once from an fp32 sum in another order, are held to the GEMM tolerance
(max relative error <= 1e-2 with the rms floor, mean absolute error <= 1e-3
rms).  Two calls in a row on each path, the second smaller than the first (the
shared static scratch keeps the first call's contents), over the decode,
16-token-window and MFMA-tile routes (split-k and not)."""
import numpy as np
import pytest
import torch

from qlora_linear_layers_amd import api, synth
from helpers import assert_gemm_close, bits_of, say, to_dev

pytestmark = pytest.mark.gpu


def _case(lin, T, r, s, seed):
    d = synth.layer_inputs(9, seed, 0, lin, T, r)
    qw = api.nf4_quantize_dq(to_dev(d["w"], (lin.N, lin.K)))
    x = to_dev(d["x"], (T, lin.K))
    a = to_dev(d["a"], (lin.K, r)) if r else None
    b = to_dev(d["b"], (r, lin.N)) if r else None
    return qw, x, a, b


@pytest.mark.parametrize("first,second", [
    ((synth.Linear("t", 4096, 4096), 8, 64), (synth.Linear("t", 1024, 2048), 3, 16)),       # decode
    ((synth.Linear("t", 2048, 1024), 90, 64), (synth.Linear("t", 512, 768), 40, 24)),       # windows
    ((synth.Linear("t", 1024, 2048), 700, 64), (synth.Linear("t", 640, 448), 333, 0)),      # split-k MFMA tiles
    ((synth.Linear("t", 2048, 1024), 520, 136), (synth.Linear("t", 384, 256), 5, 8)),       # across routes
    ((synth.Linear("t", 4096, 4096), 4096, 16), (synth.Linear("t", 512, 256), 200, 16)),    # one round of tiles
    ((synth.Linear("t", 4096, 4096), 512, 16), (synth.Linear("t", 1024, 2048), 700, 64)),   # fewer splits, then all
])
def test_noalloc_matches_workspace_forward(first, second):
    for i, (lin, T, r) in enumerate((first, second)):
        # bit-equal unless qlora_linear_fwd's own workspace exceeds the scratch
        exact = api.qlora_workspace_bytes(T, lin.K, lin.N, r) <= api.lib().qlora_noalloc_scratch_bytes()
        say(f"[noalloc] call {i}: N={lin.N} K={lin.K} T={T} r={r} exact={exact}")
        qw, x, a, b = _case(lin, T, r, 0.5, i)
        ref = bits_of(api.qlora_linear_fwd(x, qw, a, b, 0.5))
        y = torch.full((T, lin.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = bits_of(api.qlora_linear_fwd_noalloc(x, qw, a, b, 0.5, out=y))
        torch.cuda.synchronize()
        if exact:
            assert np.array_equal(got, ref), (i, lin, T, r)
        else:
            assert_gemm_close(got, ref, f"call {i} against qlora_linear_fwd")


def test_noalloc_rejects_oversized_without_touching_outputs():
    lin = synth.Linear("t", 11008, 4096)
    qw, x, a, b = _case(lin, 96, 64, 0.25, 0)           # 16-token windows of 11008 rows: 34 MB of partials
    y = torch.zeros((96, lin.N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.QLoraError) as e:
        api.qlora_linear_fwd_noalloc(x, qw, a, b, 0.25, out=y)
    assert e.value.status == 5                           # QLORA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not torch.any(y != 0)
