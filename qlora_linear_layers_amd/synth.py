"""Seeded synthetic inputs for the QLoRA linear layer, shared by the tests, the
benchmark and the CPU baseline.

This module only draws random numbers and names workload shapes: it holds none
of the quantization or GEMM arithmetic.  Every tensor is drawn in fp32 from its
own stream ``PCG64(SeedSequence([config, layer, tensor, role]))`` and rounded
once to bf16 (by torch's CPU conversion); bf16 tensors are returned as uint16
bit patterns so that the GPU path and the oracle consume the same bytes.

Distributions: weights W ~ N(0, 0.02) (standard deviation), activations X and
upstream gradients dY ~ N(0, 1), LoRA factors A and B ~ N(0, 0.01).  The 70B
streaming workload also replaces 0.1% of the weights (mask u < 0.001 from the
same stream) with 0.1 * Student-t(3).
"""
from dataclasses import dataclass

import numpy as np
import torch

ROLE_W, ROLE_X, ROLE_A, ROLE_B, ROLE_DY = 0, 1, 2, 3, 4


def rng_for(config, layer, tensor, role):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, layer, tensor, role])))


def to_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(f32):
    """fp32 draws -> IEEE half bits (nearest even), for the fp16 compute-type workloads."""
    return np.asarray(f32, dtype=np.float32).astype(np.float16).view(np.uint16)


def layer_inputs_f16(config, layer_idx, lin_idx, lin, T, r, with_dy=False):
    """layer_inputs with every tensor drawn the same way and rounded to fp16 instead of bf16."""
    g = lambda role: rng_for(config, layer_idx, lin_idx, role)
    out = dict(w=to_f16_bits(g(ROLE_W).standard_normal((lin.N, lin.K), dtype=np.float32) * np.float32(0.02)))
    if T:
        out["x"] = to_f16_bits(g(ROLE_X).standard_normal((T, lin.K), dtype=np.float32))
    if r:
        out["a"] = to_f16_bits(g(ROLE_A).standard_normal((lin.K, r), dtype=np.float32) * np.float32(0.01))
        out["b"] = to_f16_bits(g(ROLE_B).standard_normal((r, lin.N), dtype=np.float32) * np.float32(0.01))
    if with_dy:
        out["dy"] = to_f16_bits(g(ROLE_DY).standard_normal((T, lin.N), dtype=np.float32))
    return out


def normal_bf16(rng, shape, std):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def outlier_weight_bf16(rng, shape, std=0.02, frac=0.001, scale=0.1):
    w = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    u = rng.random(shape, dtype=np.float32)
    t = rng.standard_t(3, size=shape).astype(np.float32) * np.float32(scale)
    w = np.where(u < frac, t, w)
    return to_bf16_bits(w)


@dataclass(frozen=True)
class Linear:
    name: str
    N: int          # output features (rows of W)
    K: int          # input features


LLAMA7B = (Linear("q", 4096, 4096), Linear("k", 4096, 4096), Linear("v", 4096, 4096),
           Linear("o", 4096, 4096), Linear("gate", 11008, 4096), Linear("up", 11008, 4096),
           Linear("down", 4096, 11008))
LLAMA65B = (Linear("q", 8192, 8192), Linear("k", 8192, 8192), Linear("v", 8192, 8192),
            Linear("o", 8192, 8192), Linear("gate", 22016, 8192), Linear("up", 22016, 8192),
            Linear("down", 8192, 22016))
LLAMA70B = (Linear("q", 8192, 8192), Linear("k", 1024, 8192), Linear("v", 1024, 8192),
            Linear("o", 8192, 8192), Linear("gate", 28672, 8192), Linear("up", 28672, 8192),
            Linear("down", 8192, 28672))

# Workload table: (config id, description, layer set, tokens, rank, scaling)
SINGLE_LAYER = dict(config=1, layers=(Linear("w", 4096, 4096),), T=16, r=16, scaling=1.0)
DECODE_7B = dict(config=2, layers=LLAMA7B, T=(1, 4, 8), r=64, scaling=16.0 / 64)
TRAIN_7B = dict(config=3, layers=LLAMA7B, T=4096, r=64, scaling=16.0 / 64)
LAYER_65B = dict(config=4, layers=LLAMA65B, T=2048, r=64, scaling=16.0 / 64)
STREAM_70B = dict(config=5, layers=LLAMA70B, n_layers=80)


def layer_inputs(config, layer_idx, lin_idx, lin, T, r, with_dy=False, outliers=False):
    """Seeded bf16 inputs (uint16 bits) of one linear: W [N,K], X [T,K], A [K,r], B [r,N], dY [T,N]."""
    g = lambda role: rng_for(config, layer_idx, lin_idx, role)
    if outliers:
        w = outlier_weight_bf16(g(ROLE_W), (lin.N, lin.K))
    else:
        w = normal_bf16(g(ROLE_W), (lin.N, lin.K), 0.02)
    out = dict(w=w)
    if T:
        out["x"] = normal_bf16(g(ROLE_X), (T, lin.K), 1.0)
    if r:
        out["a"] = normal_bf16(g(ROLE_A), (lin.K, r), 0.01)
        out["b"] = normal_bf16(g(ROLE_B), (r, lin.N), 0.01)
    if with_dy:
        out["dy"] = normal_bf16(g(ROLE_DY), (T, lin.N), 1.0)
    return out


# ----------------------------------------------------------------- on-device draws
#
# The 65B- and 70B-shaped workloads are too large to draw with numpy on the host
# in reasonable time (68.5 G values for the 70B stack).  These draw the same
# distributions with torch's seeded device generator instead; the seed of each
# tensor still comes from SeedSequence([config, layer, tensor, role]).  Tests
# that check such tensors against the oracle copy the drawn bf16 bytes back to
# the host, so both sides still consume the same bytes.

def device_generator(config, layer, tensor, role, device="cuda"):
    seed = int(np.random.SeedSequence([config, layer, tensor, role]).generate_state(1, np.uint64)[0]) >> 1
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_normal_bf16(g, shape, std, device="cuda"):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.mul_(std).to(torch.bfloat16)


def device_outlier_weight_bf16(g, shape, std=0.02, frac=0.001, scale=0.1, device="cuda"):
    """N(0, std) with a fraction `frac` of the entries (mask u < frac) replaced by
    scale * t3, where t3 = z / sqrt(chi2_3 / 3) is drawn from its definition
    (z and the three normals of chi2_3 independent standard normals)."""
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    idx = torch.nonzero(u.view(-1) < frac).view(-1)
    del u
    z = torch.randn(idx.numel(), generator=g, device=device, dtype=torch.float32)
    chi2 = torch.randn((idx.numel(), 3), generator=g, device=device, dtype=torch.float32).square_().sum(1)
    w.view(-1)[idx] = z / torch.sqrt(chi2 / 3.0) * scale
    return w.to(torch.bfloat16)


def device_layer_weights(config, layer, layers, outliers=False, device="cuda"):
    """bf16 weights [N, K] of every linear of one layer, drawn on the device."""
    out = []
    for ti, lin in enumerate(layers):
        g = device_generator(config, layer, ti, ROLE_W, device)
        if outliers:
            out.append(device_outlier_weight_bf16(g, (lin.N, lin.K), device=device))
        else:
            out.append(device_normal_bf16(g, (lin.N, lin.K), 0.02, device=device))
    return out


def device_layer_inputs(config, layer, ti, lin, T, r, with_dy=False, device="cuda"):
    """X [T,K], A [K,r], B [r,N] and optionally dY [T,N] of one linear, drawn on the device."""
    g = lambda role: device_generator(config, layer, ti, role, device)
    out = dict(x=device_normal_bf16(g(ROLE_X), (T, lin.K), 1.0, device),
               a=device_normal_bf16(g(ROLE_A), (lin.K, r), 0.01, device),
               b=device_normal_bf16(g(ROLE_B), (r, lin.N), 0.01, device))
    if with_dy:
        out["dy"] = device_normal_bf16(g(ROLE_DY), (T, lin.N), 1.0, device)
    return out
