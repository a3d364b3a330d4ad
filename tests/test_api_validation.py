"""Host-side argument checks of the Python binding: every tensor's shape is
checked against (T, K, N, r) and the storage sizes before anything reaches the
C ABI (which trusts the sizes it is given).  CPU tensors suffice: the shape
checks come first, then the device checks."""
import pytest
import torch

from qlora_linear_layers_amd import api

N, K, T, R = 192, 128, 5, 8


def _qw(n=N, k=K, short=None):
    num = n * k
    sizes = {"codes": num // 2, "absmax_fp8": num // 64, "superscale": -(-num // 16384)}
    if short:
        sizes[short] -= 1
    return api.NF4Weight(torch.zeros(sizes["codes"], dtype=torch.uint8),
                         torch.zeros(sizes["absmax_fp8"], dtype=torch.uint8),
                         torch.zeros(sizes["superscale"], dtype=torch.float32), n, k)


def _t(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_forward_shapes_checked():
    qw = _qw()
    _raises(lambda: api.qlora_linear_fwd(_t(T, K + 64), qw), "x has shape")
    _raises(lambda: api.qlora_linear_fwd(_t(T, K, 1), qw), "x must be 2-D")
    _raises(lambda: api.qlora_linear_fwd(_t(T, K), qw, _t(K, R), _t(R + 8, N)), "lora_b has shape")
    _raises(lambda: api.qlora_linear_fwd(_t(T, K), qw, _t(K + 64, R), _t(R, N)), "lora_a has shape")
    _raises(lambda: api.qlora_linear_fwd(_t(T, K), qw, _t(K, R), None), "together")
    _raises(lambda: api.qlora_linear_fwd(_t(T, K), qw, out=_t(T, N + 64)), "out has shape")
    # correct shapes on the CPU get past the shape checks and stop at the device check
    _raises(lambda: api.qlora_linear_fwd(_t(T, K), qw, _t(K, R), _t(R, N)), "GPU tensor")


def test_backward_shapes_checked():
    qw = _qw()
    a, b = _t(K, R), _t(R, N)
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N + 64), qw), "dy has shape")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, a, b, x=_t(T + 1, K), lora_grads=True), "x has shape")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, dx=_t(T, K + 64)), "dx has shape")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, a, b, x=_t(T, K), lora_grads=True,
                                               d_lora_a=_t(K, R + 8)), "d_lora_a has shape")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, a, b, x=_t(T, K), lora_grads=True,
                                               d_lora_b=_t(R, N - 64)), "d_lora_b has shape")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, a, b, lora_grads=True), "needs x")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, lora_grads=True, x=_t(T, K)), "needs the adapters")
    _raises(lambda: api.qlora_linear_bwd_input(_t(T, N), qw, a, b, x=_t(T, K), lora_grads=True), "GPU tensor")


def test_storage_sizes_checked():
    for short, name in (("codes", "codes"), ("absmax_fp8", "absmax_fp8"), ("superscale", "superscale")):
        if short == "superscale" and -(-N * K // 16384) == 1:
            qw = _qw(n=N * 64, short=short)        # a size with more than one super-scale
            x = _t(T, K)
        else:
            qw, x = _qw(short=short), _t(T, K)
        _raises(lambda: api.qlora_linear_fwd(x, qw), f"{name} has shape")
        _raises(lambda: api.nf4_dequantize_dq(qw), f"{name} has shape")
        _raises(lambda: api.qlora_merge_lora(qw), f"{name} has shape")
    sq = api.NF4WeightSQ(torch.zeros(N * K // 2, dtype=torch.uint8), torch.zeros(N * K // 64 - 1), N, K)
    _raises(lambda: api.nf4_dequantize(sq), "absmax has shape")


def test_merge_and_dequantize_outputs_checked():
    qw = _qw()
    _raises(lambda: api.qlora_merge_lora(qw, out=_t(K, N)), "out has shape")
    _raises(lambda: api.qlora_merge_lora(qw, _t(K, R), _t(R, N + 8)), "lora_b has shape")
    _raises(lambda: api.nf4_dequantize_dq(qw, out=_t(N, K - 64)), "elements")
    _raises(lambda: api.nf4_quantize_dq_into(_t(N + 1, K), qw), "elements")


def test_grouped_problems_checked():
    qw = _qw()
    good = (_t(T, K), qw, _t(K, R), _t(R, N), 0.5, _t(T, N))
    _raises(lambda: api.qlora_linear_fwd_grouped([good, (_t(T, K), qw, _t(K, R), _t(R, N), 0.5, _t(T, N + 64))]),
            "do not match")
    _raises(lambda: api.qlora_linear_fwd_grouped([good, (_t(T, K), qw, _t(K, R), _t(R + 8, N), 0.5, _t(T, N))]),
            "lora_b has shape")
    _raises(lambda: api.qlora_linear_fwd_grouped([good, (_t(T, K), qw, _t(K, 2 * R), _t(2 * R, N), 0.5,
                                                         _t(T, N))]), "same rank")
    _raises(lambda: api.nf4_quantize_dq_grouped([_t(N, K)], [_qw(short="codes")]), "codes has shape")
