"""The C ABI library on the host: it loads, exports every symbol the header
declares, its own codebook (an independent inverse-normal) equals the
oracle's bit for bit, and argument validation rejects bad calls before any
launch (these calls never reach the GPU)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from qlora_linear_layers_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, NULL, SHAPE, ALIGN, VALUE, WORKSPACE = 0, 1, 2, 3, 4, 5
FAKE = 1 << 20           # a 16-byte aligned non-NULL address; never dereferenced on these paths
MIS = FAKE + 8           # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        pytest.skip("library not built")
    return api.lib()


def _declared():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_exports_match_header(L):
    from qlora_linear_layers_amd import calib
    names = _declared()
    assert set(names) == set(api.EXPORTS) | set(calib.EXPORTS), names
    for n in names:
        assert hasattr(L, n)


def test_calibration_validation(L):
    from qlora_linear_layers_amd import calib
    c = calib._lib()
    assert c.qlora_calib_copy(None, FAKE, 16, None) == 1
    assert c.qlora_calib_copy(FAKE, FAKE, 24, None) == 1
    assert c.qlora_calib_copy(MIS, FAKE, 16, None) == 1
    assert c.qlora_calib_mfma(FAKE, FAKE, 0, 10, None) == 1
    assert c.qlora_calib_mfma_flops(256, 10) == 256 * 4 * 10 * 16 * 32 * 32 * 16 * 2


def test_codebook_bit_exact(L):
    got = api.nf4_build_codebook().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.nf4_codebook().view(np.uint32))
    assert L.nf4_build_codebook(None) == NULL


def test_workspace_upto_covers_every_token_count(L):
    """qlora_workspace_bytes is not monotone in T (16 < T <= 96 keeps one set of
    split partials per 16-token window); the _upto size is the maximum over T."""
    for K, N, r in ((4096, 11008, 64), (11008, 4096, 64), (448, 320, 24), (256, 256, 0)):
        sizes = [L.qlora_workspace_bytes(T, K, N, r) for T in range(1, 301)]
        for T_max in (1, 16, 17, 100, 128, 129, 300):
            assert L.qlora_workspace_bytes_upto(T_max, K, N, r) == max(sizes[:T_max])
    assert L.qlora_workspace_bytes(96, 4096, 11008, 64) > L.qlora_workspace_bytes(4096, 4096, 11008, 64)
    assert L.qlora_workspace_bytes_upto(0, 4096, 4096, 64) == 0


def test_noalloc_forward_validation(L):
    """The no-allocation forward checks its arguments like qlora_linear_fwd and
    rejects sizes whose workspace exceeds its static scratch, before anything
    touches a device.  Accepted sizes then need the device (this machine has
    none: QLORA_ERR_DEVICE), which separates accepted from rejected sizes here."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("accepted sizes would launch kernels on these fake pointers")
    DEVICE = 6
    f = L.qlora_linear_fwd_noalloc
    assert L.qlora_noalloc_scratch_bytes() == 32 << 20

    def call(T, K, N, r, **kw):
        a = dict(x=FAKE, codes=FAKE, f8=FAKE, sup=FAKE, la=FAKE if r else None, lb=FAKE if r else None, s=0.25,
                 y=FAKE)
        a.update(kw)
        return f(a["x"], T, K, N, a["codes"], a["f8"], a["sup"], a["la"], a["lb"], r, a["s"], a["y"], None)

    assert call(16, 256, 256, 16, x=None) == NULL
    assert call(16, 256, 256, 16, y=MIS) == ALIGN
    assert call(16, 250, 256, 16) == SHAPE
    assert call(16, 256, 256, 16, s=math.inf) == VALUE
    # T <= 16 decode of every 7B and 65B linear with r = 64 fits; so does T = 4096 on the 7B shapes
    for K, N in ((4096, 4096), (4096, 11008), (11008, 4096), (8192, 8192), (8192, 22016), (22016, 8192)):
        for T in (1, 8, 16):
            assert call(T, K, N, 64) == DEVICE, (T, K, N)
    for K, N in ((4096, 4096), (4096, 11008), (11008, 4096)):
        assert call(4096, K, N, 64) == DEVICE
        # mid-size T on the 7B shapes: the split-k partials are held to the scratch
        for T in (256, 512, 1024, 2048):
            assert L.qlora_workspace_bytes(T, K, N, 64) > 0
            assert call(T, K, N, 64) == DEVICE, (T, K, N)
            assert call(T, K, N, 0) == DEVICE, (T, K, N)
    # windows of the 7B gate at T = 96 (one decode workspace per 16-token window) do not
    assert call(96, 4096, 11008, 64) == WORKSPACE
    assert call(1 << 20, 1024, 1024, 64) == WORKSPACE


def test_status_strings(L):
    for s in range(7):
        assert L.qlora_status_string(s)
    assert L.qlora_status_string(99) == b"unknown status"


def test_quantize_validation(L):
    q = L.nf4_quantize_dq
    assert q(None, 64, FAKE, FAKE, FAKE, None) == NULL
    assert q(FAKE, 63, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 0, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, -64, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(MIS, 64, FAKE, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 64, FAKE, MIS, FAKE, None) == ALIGN
    d = L.nf4_dequantize_dq
    assert d(FAKE, FAKE, None, 64, FAKE, None) == NULL
    assert d(FAKE, FAKE, FAKE, 100, FAKE, None) == SHAPE
    assert d(FAKE, FAKE, FAKE, 64, MIS, None) == ALIGN


def _fwd(L, **kw):
    a = dict(x=FAKE, T=16, K=256, N=256, codes=FAKE, f8=FAKE, sup=FAKE, la=FAKE, lb=FAKE, r=16, s=1.0,
             y=FAKE, ws=FAKE, wsb=1 << 40, st=None)
    a.update(kw)
    return L.qlora_linear_fwd(a["x"], a["T"], a["K"], a["N"], a["codes"], a["f8"], a["sup"], a["la"], a["lb"],
                              a["r"], a["s"], a["y"], a["ws"], a["wsb"], a["st"])


def test_fwd_validation(L):
    assert _fwd(L, x=None) == NULL
    assert _fwd(L, la=None) == NULL
    assert _fwd(L, T=0) == SHAPE
    assert _fwd(L, K=100) == SHAPE
    assert _fwd(L, N=32) == SHAPE
    assert _fwd(L, r=12) == SHAPE
    assert _fwd(L, r=264) == SHAPE
    assert _fwd(L, T=1 << 20, K=2048) == SHAPE      # T*K above 2^30
    assert _fwd(L, r=0) == SHAPE            # adapters given with r = 0
    assert _fwd(L, y=MIS) == ALIGN
    assert _fwd(L, s=math.inf) == VALUE
    assert _fwd(L, s=math.nan) == VALUE
    assert _fwd(L, ws=None) == WORKSPACE
    assert _fwd(L, wsb=16) == WORKSPACE


def _bwd(L, **kw):
    a = dict(dy=FAKE, T=16, K=256, N=256, codes=FAKE, f8=FAKE, sup=FAKE, la=FAKE, lb=FAKE, r=16, s=1.0,
             dx=FAKE, x=FAKE, da=FAKE, db=FAKE, ws=FAKE, wsb=1 << 40, flags=0, st=None)
    a.update(kw)
    return L.qlora_linear_bwd_input(a["dy"], a["T"], a["K"], a["N"], a["codes"], a["f8"], a["sup"], a["la"],
                                    a["lb"], a["r"], a["s"], a["dx"], a["x"], a["da"], a["db"], a["ws"], a["wsb"],
                                    a["flags"], a["st"])


def test_bwd_validation(L):
    assert _bwd(L, dy=None) == NULL
    assert _bwd(L, x=None) == NULL            # grads requested without X
    assert _bwd(L, lb=None) == NULL
    assert _bwd(L, T=-1) == SHAPE
    assert _bwd(L, r=0, la=None, lb=None) == SHAPE   # grads requested with r = 0
    assert _bwd(L, da=MIS) == ALIGN
    assert _bwd(L, s=math.inf) == VALUE
    assert _bwd(L, flags=4) == VALUE          # unknown flag bit
    assert _bwd(L, flags=1 << 31) == VALUE
    assert _bwd(L, wsb=0) == WORKSPACE
    # the fused gradients need their own, larger workspace (one fp32 partial per 256-token tile)
    T, K, N, r = 300, 256, 320, 16
    plain = L.qlora_workspace_bytes_bwd(T, K, N, r, 0)
    fused = L.qlora_workspace_bytes_bwd(T, K, N, r, api.FUSED_GRADS)
    assert fused > 0 and plain > 0
    assert _bwd(L, T=T, K=K, N=N, r=r, wsb=fused - 1, flags=api.FUSED_GRADS) == WORKSPACE
    assert _bwd(L, T=T, K=K, N=N, r=r, wsb=fused - 1, flags=api.FUSED_GRADS | api.REUSE_FORWARD) == WORKSPACE
    assert _bwd(L, T=T, K=K, N=N, r=r, wsb=fused - 1, flags=api.FUSED_GRADS | 4) == VALUE


def test_workspace_bytes_bwd(L):
    f = L.qlora_workspace_bytes_bwd
    for T, K, N, r in ((300, 256, 320, 16), (4096, 4096, 11008, 64), (2048, 22016, 8192, 64), (17, 64, 64, 256)):
        plain, fused = f(T, K, N, r, 0), f(T, K, N, r, api.FUSED_GRADS)
        assert f(T, K, N, r, api.REUSE_FORWARD) == plain
        assert f(T, K, N, r, api.REUSE_FORWARD | api.FUSED_GRADS) == fused
        # the two layouts share everything up to the gradient partials: plain holds the k_grad
        # partials, fused one [K + N][r_pad] fp32 block per group of 256-token tiles instead
        # (two tiles per group from four tiles on)
        r_pad = -(-r // 64) * 64
        tiles = -(-T // 256)
        tiles = -(-tiles // 2) if tiles >= 4 else tiles
        ceil256 = lambda v: -(-v // 256) * 256
        assert fused - ceil256(tiles * K * r_pad * 4) - ceil256(tiles * N * r_pad * 4) < plain
        assert fused >= ceil256(tiles * K * r_pad * 4) + ceil256(tiles * N * r_pad * 4)
        assert plain >= L.qlora_workspace_bytes(T, K, N, r) or T <= 96
    assert f(16, 100, 64, 16, 0) == 0                      # rejected sizes
    assert f(300, 256, 320, 16, 4) == 0                    # unknown flag
    # without an adapter there are no gradients: the scale table alone
    assert f(300, 256, 320, 0, api.FUSED_GRADS) == f(300, 256, 320, 0, 0) == (256 // 64) * 320 * 4


def test_workspace_bytes(L):
    # no adapter: the larger of the forward's and the backward's needs.  The
    # forward at T <= 16 keeps the decode path's split partials [K/512][T][N]
    # fp32, at 16 < T <= 96 one such set per 16-token window; the backward
    # keeps the dX kernel's block scales [K/64][N] fp32 and, while dX has too
    # few 256 x 256 tiles for the chip, S (2..16) fp32 partial tiles [S][K][T
    # rounded up to 4]
    scl = (4096 // 64) * 4096 * 4

    def dx_splits(T, n):
        ldp = -(-T // 4) * 4
        S, rest = divmod(n - scl, 4096 * ldp * 4)
        return S if rest == 0 else -1

    for T, fwd in ((16, (4096 // 512) * 16 * 4096 * 4), (1, (4096 // 512) * 1 * 4096 * 4),
                   (64, 4 * (4096 // 512) * 16 * 4096 * 4), (40, 3 * (4096 // 512) * 16 * 4096 * 4)):
        n = L.qlora_workspace_bytes(T, 4096, 4096, 0)
        assert n >= fwd and n >= scl
        assert n == fwd or 2 <= dx_splits(T, n) <= 16, (T, n)
    # T > 96 runs 256 x 256 MFMA tiles: with 256 or more tiles only the scale table ...
    assert L.qlora_workspace_bytes(4096, 4096, 4096, 0) == scl
    # ... with fewer, the forward and dX split their reductions and keep S fp32
    # partial tiles [S][N or K][T rounded up to 4] (2 <= S <= 16, at most
    # 64 MiB, at least 4 k tiles per split); on a square weight both take the
    # same S, so the backward's scale table plus its partials is the larger
    for T in (129, 300, 333, 700, 2048):
        n = L.qlora_workspace_bytes(T, 4096, 4096, 0)
        assert n % 256 == 0 and 2 <= dx_splits(T, n) <= 16 and n <= scl + (64 << 20), (T, n)
    assert L.qlora_workspace_bytes(1 << 23, 4096, 4096, 16) == 0                     # T too large
    assert L.qlora_workspace_bytes(16, 100, 4096, 16) == 0
    a = L.qlora_workspace_bytes(4096, 4096, 11008, 64)
    b = L.qlora_workspace_bytes(4096, 4096, 11008, 16)
    assert a > 0 and b > 0 and a % 256 == 0


def _merge(L, codes=FAKE, f=FAKE, s2=FAKE, K=128, N=64, la=FAKE, lb=FAKE, r=16, s=0.5, w=FAKE):
    return L.qlora_merge_lora(codes, f, s2, K, N, la, lb, r, s, w, None)


def test_merge_validation(L):
    assert _merge(L, codes=None) == NULL
    assert _merge(L, w=None) == NULL
    assert _merge(L, la=None) == NULL              # adapter half missing with r > 0
    assert _merge(L, K=100) == SHAPE               # K not a multiple of 64
    assert _merge(L, N=0) == SHAPE
    assert _merge(L, N=100) == SHAPE             # N not a multiple of 8
    assert _merge(L, r=12) == SHAPE                # r not a multiple of 8
    assert _merge(L, r=264) == SHAPE               # above the rank limit
    assert _merge(L, r=0) == SHAPE                 # adapter pointers given with r = 0
    assert _merge(L, K=1 << 21) == SHAPE
    assert _merge(L, K=1 << 20, N=1 << 12) == SHAPE   # N*K = 2^32
    assert _merge(L, w=MIS) == ALIGN
    assert _merge(L, lb=MIS) == ALIGN
    assert _merge(L, s=math.nan) == VALUE


def test_single_quantization_validation(L):
    assert L.nf4_quantize(None, 64, FAKE, FAKE, None) == NULL
    assert L.nf4_quantize(FAKE, 64, FAKE, None, None) == NULL
    assert L.nf4_quantize(FAKE, 96, FAKE, FAKE, None) == SHAPE
    assert L.nf4_quantize(FAKE, 64, FAKE, MIS, None) == ALIGN
    assert L.nf4_dequantize(FAKE, None, 64, FAKE, None) == NULL
    assert L.nf4_dequantize(FAKE, FAKE, 0, FAKE, None) == SHAPE
    assert L.nf4_dequantize(FAKE, MIS, 64, FAKE, None) == ALIGN
    f = L.qlora_linear_fwd_sq
    assert f(FAKE, 16, 128, 128, FAKE, None, None, None, 0, 1.0, FAKE, FAKE, 1 << 30, None) == NULL
    assert f(FAKE, 16, 100, 128, FAKE, FAKE, None, None, 0, 1.0, FAKE, FAKE, 1 << 30, None) == SHAPE
    assert f(FAKE, 16, 128, 128, FAKE, MIS, None, None, 0, 1.0, FAKE, FAKE, 1 << 30, None) == ALIGN
    assert f(FAKE, 16, 128, 128, FAKE, FAKE, None, None, 0, math.inf, FAKE, FAKE, 1 << 30, None) == VALUE
    assert f(FAKE, 16, 128, 128, FAKE, FAKE, None, None, 0, 1.0, FAKE, None, 0, None) == WORKSPACE
    b = L.qlora_linear_bwd_input_sq
    assert b(FAKE, 64, 128, 128, FAKE, None, FAKE, FAKE, 16, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0,
             None) == NULL
    assert b(FAKE, 64, 128, 128, FAKE, FAKE, FAKE, FAKE, 16, 1.0, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, 0,
             None) == NULL                                # grads without X
    assert b(FAKE, 64, 128, 128, FAKE, FAKE, FAKE, FAKE, 16, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 4,
             None) == VALUE
    m = L.qlora_merge_lora_sq
    assert m(FAKE, None, 128, 64, FAKE, FAKE, 16, 0.5, FAKE, None) == NULL
    assert m(FAKE, FAKE, 128, 60, FAKE, FAKE, 16, 0.5, FAKE, None) == SHAPE
    assert m(FAKE, MIS, 128, 64, FAKE, FAKE, 16, 0.5, FAKE, None) == ALIGN


def test_int4_validation(L):
    assert L.int4_quantize(None, 64, FAKE, FAKE, None) == NULL
    assert L.int4_quantize(FAKE, 65, FAKE, FAKE, None) == SHAPE
    assert L.int4_quantize(FAKE, 64, MIS, FAKE, None) == ALIGN
    assert L.int4_dequantize(FAKE, None, 64, FAKE, None) == NULL
    assert L.int4_dequantize(FAKE, FAKE, -64, FAKE, None) == SHAPE
    assert L.int4_dequantize(FAKE, FAKE, 64, MIS, None) == ALIGN


def test_f16_validation(L):
    assert L.nf4_quantize_dq_f16(None, 64, FAKE, FAKE, FAKE, None) == NULL
    assert L.nf4_quantize_dq_f16(FAKE, 63, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.nf4_dequantize_dq_f16(FAKE, FAKE, FAKE, 64, MIS, None) == ALIGN
    f = L.qlora_linear_fwd_f16
    assert f(FAKE, 16, 128, 128, FAKE, FAKE, None, None, None, 0, 1.0, FAKE, FAKE, 1 << 30, None) == NULL
    assert f(FAKE, 16, 128, 100, FAKE, FAKE, FAKE, None, None, 0, 1.0, FAKE, FAKE, 1 << 30, None) == SHAPE
    assert f(FAKE, 16, 128, 128, FAKE, FAKE, FAKE, None, None, 0, math.nan, FAKE, FAKE, 1 << 30, None) == VALUE
    b = L.qlora_linear_bwd_input_f16
    assert b(FAKE, 64, 128, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 1.0, FAKE, FAKE, FAKE, FAKE, None, 0, 0,
             None) == WORKSPACE
    m = L.qlora_merge_lora_f16
    assert m(FAKE, FAKE, FAKE, 128, 64, FAKE, None, 16, 0.5, FAKE, None) == NULL
    assert m(FAKE, FAKE, FAKE, 96, 64, FAKE, FAKE, 16, 0.5, FAKE, None) == SHAPE


def _problems(n, over=None):
    arr = (api.LinearProblem * n)()
    for i in range(n):
        d = dict(x=FAKE, codes=FAKE, absmax_fp8=FAKE, superscale=FAKE, lora_a=FAKE, lora_b=FAKE, y=FAKE,
                 K=256, N=512, scaling=0.25)
        d.update((over or {}).get(i, {}))
        arr[i] = api.LinearProblem(**d)
    return arr


def test_grouped_validation(L):
    f, wb = L.qlora_linear_fwd_grouped, L.qlora_grouped_workspace_bytes
    big = 1 << 40
    assert f(3, None, 8, 16, FAKE, big, None) == NULL
    assert f(0, _problems(1), 8, 16, FAKE, big, None) == SHAPE
    assert f(9, _problems(9), 8, 16, FAKE, big, None) == SHAPE            # above QLORA_MAX_GROUP
    assert f(2, _problems(2), 17, 16, FAKE, big, None) == SHAPE           # above QLORA_GROUPED_MAX_T
    assert f(2, _problems(2), 0, 16, FAKE, big, None) == SHAPE
    assert f(2, _problems(2), 8, 12, FAKE, big, None) == SHAPE            # rank not a multiple of 8
    assert f(2, _problems(2, {1: dict(K=100)}), 8, 16, FAKE, big, None) == SHAPE
    assert f(2, _problems(2, {1: dict(y=None)}), 8, 16, FAKE, big, None) == NULL
    assert f(2, _problems(2, {1: dict(lora_b=None)}), 8, 16, FAKE, big, None) == NULL
    assert f(2, _problems(2), 8, 0, FAKE, big, None) == SHAPE             # adapters given with r = 0
    assert f(2, _problems(2, {0: dict(codes=MIS)}), 8, 16, FAKE, big, None) == ALIGN
    assert f(2, _problems(2, {1: dict(scaling=math.nan)}), 8, 16, FAKE, big, None) == VALUE
    assert f(2, _problems(2), 8, 16, MIS, big, None) == ALIGN
    assert f(2, _problems(2), 8, 16, None, big, None) == WORKSPACE
    assert f(2, _problems(2), 8, 16, FAKE, 16, None) == WORKSPACE
    # workspace: each problem's split partials [K/512][T][N] and adapter partials [K/256][T][r_pad], 256-aligned
    one = (256 // 512 + 1) * 8 * 512 * 4 + (256 // 256) * 8 * 64 * 4
    assert wb(3, _problems(3), 8, 16) == 3 * one
    assert wb(9, _problems(9), 8, 16) == 0
    assert wb(2, _problems(2, {1: dict(N=100)}), 8, 16) == 0


def test_grouped_product_validation(L):
    f = L.qlora_linear_fwd_grouped_ex
    big = 1 << 40
    assert f(2, _problems(2), 8, 16, 3, FAKE, big, None) == VALUE          # unknown decode product
    assert f(2, _problems(2), 8, 16, 1 << 31, FAKE, big, None) == VALUE
    assert f(2, _problems(2), 9, 16, api.QLORA_DECODE_VALU, FAKE, big, None) == VALUE   # VALU product: T <= 8
    assert f(2, _problems(2), 17, 16, api.QLORA_DECODE_MFMA, FAKE, big, None) == SHAPE
    assert f(2, _problems(2, {1: dict(K=100)}), 8, 16, api.QLORA_DECODE_VALU, FAKE, big, None) == SHAPE
    assert f(2, _problems(2), 8, 16, api.QLORA_DECODE_VALU, FAKE, 16, None) == WORKSPACE
    assert f(2, _problems(2), 8, 16, api.QLORA_DECODE_MFMA, None, big, None) == WORKSPACE


def _tensors(n, over=None):
    arr = (api.NF4Tensor * n)()
    for i in range(n):
        d = dict(w=FAKE, numel=64 * 300, codes=FAKE, absmax_fp8=FAKE, superscale=FAKE)
        d.update((over or {}).get(i, {}))
        arr[i] = api.NF4Tensor(**d)
    return arr


def test_grouped_quantize_validation(L):
    for f in (L.nf4_quantize_dq_grouped, L.nf4_dequantize_dq_grouped):
        assert f(2, None, None) == NULL
        assert f(0, _tensors(1), None) == SHAPE
        assert f(17, _tensors(17), None) == SHAPE                          # above QLORA_MAX_TENSORS
        assert f(2, _tensors(2, {1: dict(numel=100)}), None) == SHAPE
        assert f(2, _tensors(2, {1: dict(numel=0)}), None) == SHAPE
        assert f(2, _tensors(2, {0: dict(numel=(1 << 43) + 64)}), None) == SHAPE
        assert f(2, _tensors(2, {1: dict(codes=None)}), None) == NULL
        assert f(2, _tensors(2, {0: dict(w=MIS)}), None) == ALIGN
        assert f(2, _tensors(2, {1: dict(superscale=MIS)}), None) == ALIGN
    # single-tensor calls share the element limit
    assert L.nf4_quantize_dq(FAKE, (1 << 43) + 64, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.nf4_dequantize_dq(FAKE, FAKE, FAKE, (1 << 43) + 64, FAKE, None) == SHAPE
