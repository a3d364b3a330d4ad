"""Shared helpers for the tests: bf16 bit arrays <-> torch tensors, tolerance check."""
import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits, shape=None):
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    if shape is not None:
        t = t.reshape(shape)
    return t.cuda()


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def to_dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bits_of(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of_bits(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_errors(got_bits, ref_bits):
    """(max relative error with the rms floor, MAE / rms) of bf16 outputs against the bf16-rounded oracle."""
    g = f64_of_bits(got_bits).reshape(-1)
    r = f64_of_bits(ref_bits).reshape(-1)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    if rms == 0:
        return float(np.max(np.abs(g - r), initial=0.0)), 0.0
    err = np.abs(g - r)
    return float(np.max(err / np.maximum(np.abs(r), rms))), float(np.mean(err) / rms)


MAX_REL = 1e-2
MAE_REL = 1e-3


def assert_gemm_close(got_bits, ref_bits, what):
    mx, mae = gemm_errors(got_bits, ref_bits)
    say(f"  {what}: max_rel={mx:.3e} mae/rms={mae:.3e}")
    assert mx <= MAX_REL and mae <= MAE_REL, f"{what}: max_rel {mx:.3e}, mae/rms {mae:.3e}"
