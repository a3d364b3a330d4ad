"""Pins of the fp16 compute-type oracle ("QLoRA 原理精讲", section 3 pitfall 4)."""
import struct

import numpy as np

import oracle
from qlora_linear_layers_amd import synth


def _struct_f16(v):
    """CPython's own correctly rounded double -> half conversion (an independent routine)."""
    try:
        return struct.unpack("<H", struct.pack("<e", v))[0]
    except OverflowError:
        return 0x7C00 if v > 0 else 0xFC00


def test_rounding_matches_an_independent_implementation():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        # exact ties between neighbouring halves, subnormal ties, the overflow edge
                        (np.arange(1, 2048) + 0.5) * 2.0 ** -10, (np.arange(1, 64) + 0.5) * 2.0 ** -24,
                        [65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0]])
    got = oracle.round_to_f16_bits(v)
    want = np.array([_struct_f16(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.f16_bits_to_f64(got[:20000]), got[:20000].view(np.float16).astype(np.float64))


def test_dequantize_is_the_bf16_product_rounded_to_fp16():
    w = synth.normal_bf16(synth.rng_for(1, 0, 0, synth.ROLE_W), (16, 4096), 0.02)
    p, f, s = oracle.quantize_nf4_dq(w)
    wd16 = oracle.f16_bits_to_f64(oracle.dequantize_nf4_dq_f16(p, f, s))
    wd = oracle.bf16_bits_to_f64(oracle.dequantize_nf4_dq(p, f, s))
    # both round the same fp32 product: they agree to the coarser (bf16) rounding
    assert np.all(np.abs(wd16 - wd) <= np.abs(wd16) * 2.0 ** -8 + 2.0 ** -24)
    assert np.mean(wd16 != wd) > 0.5                    # and fp16 keeps bits that bf16 drops
    rows = [0, 7, 15]
    assert np.array_equal(oracle.dequantize_rows_f16(p, f, s, 16, 4096, rows),
                          oracle.dequantize_nf4_dq_f16(p, f, s).reshape(16, 4096)[rows])


def test_quantize_from_fp16_equals_quantize_of_the_same_values():
    # fp16 weights that are also exact bf16 values quantize exactly like their bf16 bits
    rng = np.random.default_rng(2)
    x = synth.to_bf16_bits(rng.standard_normal(64 * 300).astype(np.float32) * 0.02)
    xf = oracle.bf16_bits_to_f32(x)
    h = xf.astype(np.float16)
    same = h.astype(np.float32) == xf
    x16 = np.where(same, h.view(np.uint16), np.uint16(0))
    xb = np.where(same, x, np.uint16(0))
    a, b = oracle.quantize_nf4_dq_f16(x16), oracle.quantize_nf4_dq(xb)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_layer_and_merge_closed_forms():
    rng = np.random.default_rng(3)
    T, K, N, r = 3, 64, 5, 2
    f = lambda *sh: rng.standard_normal(sh).astype(np.float16).view(np.uint16)
    x, w, a, b = f(T, K), f(N, K), f(K, r), f(r, N)
    X, W, A, B = (oracle.f16_bits_to_f64(v) for v in (x, w, a, b))
    s = 0.5
    # brute-force loops against the matrix forms
    y = np.array([[sum(X[t, k] * W[n, k] for k in range(K)) + s * sum(sum(X[t, k] * A[k, j] for k in range(K)) * B[j, n]
                                                                     for j in range(r)) for n in range(N)] for t in range(T)])
    assert np.array_equal(oracle.linear_fwd_f16(x, w, a, b, s), oracle.round_to_f16_bits(y))
    assert np.array_equal(oracle.linear_fwd_at_f16(x, w[[1, 4]], a, b, s, [0, 2], [1, 4]),
                          oracle.round_to_f16_bits(y[[0, 2], [1, 4]]))
    # the backward is pinned below (exact rational sums, adjoint identity, directional derivatives)
    wm = oracle.merge_lora_f16(w, a, b, s)
    assert np.array_equal(wm, oracle.round_to_f16_bits(W + s * np.multiply.outer(B[0], A[:, 0])
                                                       + s * np.multiply.outer(B[1], A[:, 1])))


def _small_f16(T, K, N, r, seed, lora_std=0.01):
    rng = np.random.default_rng(seed)
    f = lambda sh, std: synth.to_f16_bits(rng.standard_normal(sh).astype(np.float32) * np.float32(std))
    x, w, a, b, dy = f((T, K), 1.0), f((N, K), 0.02), f((K, r), lora_std), f((r, N), lora_std), f((T, N), 1.0)
    p, fq, sq = oracle.quantize_nf4_dq_f16(w)
    wd = oracle.dequantize_nf4_dq_f16(p, fq, sq).reshape(N, K)
    return x, wd, a, b, dy


def test_backward_brute_force_exact_sums():
    """dX, dA, dB of the fp16 oracle against exact rational sums over the loop
    definitions, each rounded once to fp16 (an independent computation: no BLAS,
    no fp64 accumulation)."""
    from fractions import Fraction
    x, wd, a, b, dy = _small_f16(T=4, K=64, N=3, r=3, seed=11)
    s = 0.25
    F = lambda bits: [[Fraction(float(v)) for v in row] for row in oracle.f16_bits_to_f64(bits)]
    X, W, A, B, D = F(x), F(wd), F(a), F(b), F(dy)
    T, K, N, r = len(X), len(X[0]), len(W), len(B)
    S = Fraction(s)
    G = [[sum(D[t][n] * B[j][n] for n in range(N)) for j in range(r)] for t in range(T)]
    XA = [[sum(X[t][k] * A[k][j] for k in range(K)) for j in range(r)] for t in range(T)]
    dx = [[float(sum(D[t][n] * W[n][k] for n in range(N)) + S * sum(G[t][j] * A[k][j] for j in range(r)))
           for k in range(K)] for t in range(T)]
    da = [[float(S * sum(X[t][k] * G[t][j] for t in range(T))) for j in range(r)] for k in range(K)]
    db = [[float(S * sum(XA[t][j] * D[t][n] for t in range(T))) for n in range(N)] for j in range(r)]
    gdx, gda, gdb = oracle.linear_bwd_f16(dy, x, wd, a, b, s)
    # Fraction -> float is correctly rounded, and the fp16 rounding of a double that
    # is itself the nearest double to the exact value is the nearest fp16 unless the
    # exact value sits within 2^-53 relative of an fp16 midpoint (none does here)
    assert np.array_equal(gdx, oracle.round_to_f16_bits(np.array(dx)))
    assert np.array_equal(gda, oracle.round_to_f16_bits(np.array(da)))
    assert np.array_equal(gdb, oracle.round_to_f16_bits(np.array(db)))


def _fwd_f64_f16(x, wd, a, b, s):
    """The forward in fp64 from fp16 operands, by explicit loops over numpy rows
    (the matrix algebra of the oracle's backward is what this pins)."""
    X, W, A, B = (oracle.f16_bits_to_f64(v) for v in (x, wd, a, b))
    T, N = X.shape[0], W.shape[0]
    y = np.empty((T, N))
    for t in range(T):
        xa = np.array([np.dot(X[t], A[:, j]) for j in range(A.shape[1])])
        for n in range(N):
            y[t, n] = np.dot(X[t], W[n]) + float(np.float32(s)) * np.dot(xa, B[:, n])
    return y


def test_backward_adjoint_identity():
    """The forward is linear in X, so its input gradient is the adjoint map:
    <Y(X), dY> = <X, dX(dY)>.  Y is the fp64 loop forward; dX is the fp16
    oracle's, so the identity holds up to one fp16 rounding per element.  The
    adapters are scaled up so that the LoRA term of dX is far above that."""
    x, wd, a, b, dy = _small_f16(T=6, K=192, N=9, r=4, seed=12, lora_std=0.25)
    s = 2.0
    y = _fwd_f64_f16(x, wd, a, b, s)
    # the oracle rounds dX to fp16; compare against the rounded adjoint, and check
    # the rounded value brackets the exact inner product within fp16 resolution
    dx16 = oracle.f16_bits_to_f64(oracle.linear_bwd_f16(dy, x, wd, a, b, s)[0])
    DY, X = oracle.f16_bits_to_f64(dy), oracle.f16_bits_to_f64(x)
    lhs = float(np.sum(y * DY))
    rhs = float(np.sum(X * dx16))
    # |rhs - <X, dX_exact>| <= sum |X| |dX| 2^-11 (one fp16 rounding per element)
    bound = float(np.sum(np.abs(X) * np.abs(dx16))) * 2.0 ** -11 + 1e-12
    assert abs(lhs - rhs) <= bound


def test_lora_grads_directional_derivative():
    """L(A, B) = <Y, dY> is linear in A for fixed B (and in B for fixed A), so
    L(A + U) - L(A) = <dA, U> exactly; dA, dB of the fp16 oracle must agree with
    these directional derivatives to their fp16 rounding."""
    x, wd, a, b, dy = _small_f16(T=5, K=128, N=6, r=3, seed=13)
    s = 0.25
    _, da16, db16 = oracle.linear_bwd_f16(dy, x, wd, a, b, s)
    rng = np.random.default_rng(14)
    DY = oracle.f16_bits_to_f64(dy)
    l0 = np.sum(_fwd_f64_f16(x, wd, a, b, s) * DY)
    for which, g16 in (("a", da16), ("b", db16)):
        base = a if which == "a" else b
        u = synth.to_f16_bits(rng.standard_normal(base.shape).astype(np.float32))
        pert = oracle.round_to_f16_bits(oracle.f16_bits_to_f64(base) + oracle.f16_bits_to_f64(u))
        delta = oracle.f16_bits_to_f64(pert) - oracle.f16_bits_to_f64(base)
        args = (x, wd, pert, b, s) if which == "a" else (x, wd, a, pert, s)
        l1 = np.sum(_fwd_f64_f16(*args) * DY)
        g = oracle.f16_bits_to_f64(g16)
        bound = float(np.sum(np.abs(g) * np.abs(delta))) * 2.0 ** -11 + 1e-9 * max(1.0, abs(l1))
        assert abs((l1 - l0) - np.sum(g * delta)) <= bound, which
