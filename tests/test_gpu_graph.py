"""HIP graph capture of the layer's entry points.  Each case records its calls
once into a torch.cuda.CUDAGraph (workspaces and outputs made beforehand, so
nothing allocates while capturing; the library issues no memset nodes), then
replays the graph several times with eager work between the replays (new
input values copied in, outputs overwritten, device synchronizations) and
checks every replay against the eager calls on the same inputs, bit for bit:
the kernels are the same, so the graph must reproduce them exactly."""
import numpy as np
import pytest
import torch

from qlora_linear_layers_amd import api, synth
from helpers import bits_of, say

pytestmark = pytest.mark.gpu


def _weights(lin, r, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    qw = api.nf4_quantize_dq(torch.randn((lin.N, lin.K), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16))
    a = torch.randn((lin.K, r), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16)
    b = torch.randn((r, lin.N), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16)
    return qw, a, b


def _capture(fn):
    """Warm up on a side stream, then record fn into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, inputs, outputs, eager, reps=3):
    """Replay `g` reps times, each time with fresh input values copied into the
    captured input tensors and the outputs overwritten first; compare with the
    eager calls on the same values."""
    for rep in range(reps):
        gen = torch.Generator(device="cuda").manual_seed(1000 + rep)
        for t in inputs:
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits_of(t).copy() for t in outputs]
        ref = eager()
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(got, ref)):
            assert np.array_equal(u, bits_of(v)), f"replay {rep}, output {i}"


def test_graph_decode_step_of_the_7b_layer_set():
    """The seven LLaMA-7B linears at T = 4, r = 64, in one grouped decode
    launch pair."""
    T, r, s = 4, 64, 0.25
    say(f"[graph] 7B decode step, T={T}")
    ws_ = [_weights(lin, r, i) for i, lin in enumerate(synth.LLAMA7B)]
    xs = [torch.empty((T, lin.K), dtype=torch.bfloat16, device="cuda") for lin in synth.LLAMA7B]
    ys = [torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda") for lin in synth.LLAMA7B]
    for x in xs:
        x.normal_()
    probs = [(x, qw, a, b, s, y) for x, (qw, a, b), y in zip(xs, ws_, ys)]
    arr_ws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    g = _capture(lambda: api.qlora_linear_fwd_grouped(probs, workspace=arr_ws))

    def eager():
        outs = [torch.empty_like(y) for y in ys]
        api.qlora_linear_fwd_grouped([(x, qw, a, b, s, o) for x, (qw, a, b), o in zip(xs, ws_, outs)])
        return outs
    _replays(g, xs, ys, eager)


def test_graph_split_k_training_step():
    """The LLaMA-7B q projection at T = 512 (split-k forward and dX): forward,
    then dX, dA and dB with the forward's s X A reused, in one graph."""
    lin, T, r, s = synth.LLAMA7B[0], 512, 64, 0.25
    say(f"[graph] split-k training step, T={T} N={lin.N} K={lin.K}")
    qw, a, b = _weights(lin, r, 7)
    x = torch.randn((T, lin.K), device="cuda").to(torch.bfloat16)
    dy = torch.randn((T, lin.N), device="cuda").to(torch.bfloat16)
    ws = torch.empty(api.qlora_workspace_bytes_bwd(T, lin.K, lin.N, r, api.REUSE_FORWARD), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, lin.K), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((lin.K, r), dtype=torch.bfloat16, device="cuda")
    db = torch.empty((r, lin.N), dtype=torch.bfloat16, device="cuda")

    def step():
        api.qlora_linear_fwd(x, qw, a, b, s, workspace=ws, out=y)
        api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x, lora_grads=True, workspace=ws, dx=dx, d_lora_a=da,
                                   d_lora_b=db, reuse_forward=True)
    g = _capture(step)

    def eager():
        y2 = api.qlora_linear_fwd(x, qw, a, b, s)
        return [y2, *api.qlora_linear_bwd_input(dy, qw, a, b, s, x=x, lora_grads=True)]
    _replays(g, [x, dy], [y, dx, da, db], eager)


def test_graph_no_allocation_forward():
    """qlora_linear_fwd_noalloc (static scratch, no workspace argument) at the
    decode size and at a split-k size, captured together."""
    s = 0.5
    cases = [(synth.Linear("t", 4096, 4096), 8, 16), (synth.Linear("t", 2048, 1024), 520, 64)]
    say("[graph] no-allocation forward")
    tensors = []
    for i, (lin, T, r) in enumerate(cases):
        qw, a, b = _weights(lin, r, 20 + i)
        x = torch.empty((T, lin.K), dtype=torch.bfloat16, device="cuda").normal_()
        y = torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda")
        tensors.append((x, qw, a, b, y))

    def fwd():
        for x, qw, a, b, y in tensors:
            api.qlora_linear_fwd_noalloc(x, qw, a, b, s, out=y)
    g = _capture(fwd)

    def eager():
        return [api.qlora_linear_fwd(x, qw, a, b, s) for x, qw, a, b, _ in tensors]
    _replays(g, [t[0] for t in tensors], [t[4] for t in tensors], eager)
