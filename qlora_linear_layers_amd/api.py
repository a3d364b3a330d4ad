"""Thin Python binding over the C ABI of ``libqlora_mi355x.so`` (``include/qlora.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  torch provides device memory (tensors) and the current stream.  The
names match the C entry points.  A missing library raises ``RuntimeError``;
there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_mi355x.so")

_c_p = ctypes.c_void_p
_c_i64 = ctypes.c_int64
_SIGS = {
    "nf4_build_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
    "nf4_quantize_dq": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "nf4_dequantize_dq": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_p, _c_p]),
    "qlora_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "qlora_workspace_bytes_upto": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "qlora_workspace_bytes_bwd": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_uint]),
    "qlora_linear_fwd": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                        ctypes.c_float, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "qlora_linear_bwd_input": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                              ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t,
                                              ctypes.c_uint, _c_p]),
    "qlora_merge_lora": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, ctypes.c_float, _c_p,
                                        _c_p]),
    "nf4_quantize": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_p, _c_p]),
    "nf4_dequantize": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_p, _c_p]),
    "int4_quantize": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_p, _c_p]),
    "int4_dequantize": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_p, _c_p]),
    "qlora_linear_fwd_sq": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                           ctypes.c_float, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "qlora_linear_bwd_input_sq": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                                 ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t,
                                                 ctypes.c_uint, _c_p]),
    "qlora_merge_lora_sq": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, ctypes.c_float, _c_p,
                                           _c_p]),
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                                ctypes.c_float, _c_p, _c_p]),
    "qlora_noalloc_scratch_bytes": (ctypes.c_size_t, []),
}


class LinearProblem(ctypes.Structure):
    """qlora_linear_problem: one layer of a grouped decode forward."""
    _fields_ = [("x", _c_p), ("codes", _c_p), ("absmax_fp8", _c_p), ("superscale", _c_p), ("lora_a", _c_p),
                ("lora_b", _c_p), ("y", _c_p), ("K", _c_i64), ("N", _c_i64), ("scaling", ctypes.c_float)]


_SIGS["qlora_grouped_workspace_bytes"] = (ctypes.c_size_t, [ctypes.c_int, ctypes.POINTER(LinearProblem), _c_i64,
                                                            _c_i64])
_SIGS["qlora_linear_fwd_grouped"] = (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(LinearProblem), _c_i64, _c_i64,
                                                    _c_p, ctypes.c_size_t, _c_p])
_SIGS["qlora_linear_fwd_grouped_ex"] = (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(LinearProblem), _c_i64, _c_i64,
                                                       ctypes.c_uint, _c_p, ctypes.c_size_t, _c_p])
QLORA_DECODE_MFMA = 1
QLORA_DECODE_VALU = 2


class NF4Tensor(ctypes.Structure):
    """nf4_tensor: one tensor of a grouped quantize / dequantize."""
    _fields_ = [("w", _c_p), ("numel", _c_i64), ("codes", _c_p), ("absmax_fp8", _c_p), ("superscale", _c_p)]


_SIGS["nf4_quantize_dq_grouped"] = (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(NF4Tensor), _c_p])
_SIGS["nf4_dequantize_dq_grouped"] = (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(NF4Tensor), _c_p])
# fp16 compute type: the same arguments as the bf16 entry point of the same stem
for _n in ("nf4_quantize_dq", "nf4_dequantize_dq", "qlora_linear_fwd", "qlora_linear_bwd_input", "qlora_merge_lora"):
    _SIGS[_n + "_f16"] = _SIGS[_n]
EXPORTS = tuple(_SIGS)

REUSE_FORWARD = 1   # QLORA_BWD_REUSE_FORWARD
FUSED_GRADS = 2     # QLORA_BWD_FUSED_GRADS

_lib = None


class QLoraError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} ({lib().qlora_status_string(status).decode()})")
        self.status = status


def lib():
    """Load the in-tree HIP library (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise QLoraError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_HALF = (torch.bfloat16, torch.float16)


def _ct(t, name):
    """Compute type of a 16-bit tensor: '' for bf16, '_f16' for fp16."""
    if t.dtype not in _HALF:
        raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    return "_f16" if t.dtype == torch.float16 else ""


def _entry(stem, ct, qw):
    """C entry point for a compute type and a storage format."""
    if isinstance(qw, NF4WeightSQ):
        if ct:
            raise ValueError("single quantization has no fp16 entry points")
        return stem + "_sq"
    return stem + ct


def _shape(t, shape, name):
    """Raise ValueError unless tensor `t` (if given) has exactly `shape`."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_storage(qw):
    """The storage tensors of a quantized weight must hold exactly what its (N, K) needs:
    the C ABI trusts the sizes, so a mismatch would read past an allocation."""
    n = qw.N * qw.K
    if qw.N < 1 or qw.K < 1 or n % 64:
        raise ValueError(f"quantized weight [{qw.N}, {qw.K}]: N*K must be a positive multiple of 64")
    _shape(qw.codes.reshape(-1), (n // 2,), "codes")
    if isinstance(qw, NF4WeightSQ):
        _shape(qw.absmax.reshape(-1), (n // 64,), "absmax")
    else:
        _shape(qw.absmax_fp8.reshape(-1), (n // 64,), "absmax_fp8")
        _shape(qw.superscale.reshape(-1), (-(-n // 16384),), "superscale")


def _check_adapters(lora_a, lora_b, K, N):
    """Rank of the adapter pair A [K, r], B [r, N] (0 without an adapter)."""
    if (lora_a is None) != (lora_b is None):
        raise ValueError("lora_a and lora_b are given together or not at all")
    if lora_a is None:
        return 0
    if lora_a.dim() != 2:
        raise ValueError(f"lora_a must be 2-D [K, r], got shape {tuple(lora_a.shape)}")
    r = lora_a.shape[1]
    _shape(lora_a, (K, r), "lora_a")
    _shape(lora_b, (r, N), "lora_b")
    return r


@dataclass
class NF4Weight:
    """Storage triple of a quantized [N, K] weight (device tensors)."""
    codes: torch.Tensor       # uint8 [N*K/2]
    absmax_fp8: torch.Tensor  # uint8 [N*K/64]
    superscale: torch.Tensor  # float32 [ceil(N*K/16384)]
    N: int
    K: int

    @property
    def numel(self):
        return self.N * self.K

    def nbytes(self):
        return self.codes.numel() + self.absmax_fp8.numel() + 4 * self.superscale.numel()


@dataclass
class NF4WeightSQ:
    """Single-quantization pair of an [N, K] weight (device tensors): no second level."""
    codes: torch.Tensor       # uint8 [N*K/2]
    absmax: torch.Tensor      # float32 [N*K/64]
    N: int
    K: int

    @property
    def numel(self):
        return self.N * self.K

    def nbytes(self):
        return self.codes.numel() + 4 * self.absmax.numel()


def nf4_build_codebook():
    out = (ctypes.c_float * 16)()
    _check("nf4_build_codebook", lib().nf4_build_codebook(out))
    return torch.tensor(list(out), dtype=torch.float32)


def nf4_quantize_dq(w):
    """bf16 (or fp16) weight [N, K] (or flat) on the GPU -> NF4Weight."""
    ct = _ct(w, "w")
    _dev(w, w.dtype, "w")
    numel = w.numel()
    N, K = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, numel)
    codes = torch.empty(numel // 2, dtype=torch.uint8, device=w.device)
    fp8 = torch.empty(max(numel // 64, 1), dtype=torch.uint8, device=w.device)
    sup = torch.empty(max(-(-numel // 16384), 1), dtype=torch.float32, device=w.device)
    fn = "nf4_quantize_dq" + ct
    _check(fn, getattr(lib(), fn)(_ptr(w), numel, _ptr(codes), _ptr(fp8), _ptr(sup), _stream()))
    return NF4Weight(codes, fp8, sup, N, K)


def nf4_quantize_dq_into(w, qw):
    """Quantize into an existing NF4Weight (no allocation)."""
    fn = "nf4_quantize_dq" + _ct(w, "w")
    _check_storage(qw)
    if w.numel() != qw.numel:
        raise ValueError(f"w has {w.numel()} elements, the storage holds {qw.numel}")
    _dev(w, w.dtype, "w")
    _check(fn, getattr(lib(), fn)(_ptr(w), w.numel(), _ptr(qw.codes), _ptr(qw.absmax_fp8), _ptr(qw.superscale),
                                  _stream()))


def nf4_dequantize_dq(qw, out=None, dtype=torch.bfloat16):
    """NF4Weight -> [N, K] on the GPU, bf16 or (dtype / out fp16) fp16."""
    _check_storage(qw)
    if out is not None and out.numel() != qw.numel:
        raise ValueError(f"out has {out.numel()} elements, the weight has {qw.numel}")
    if out is None:
        out = torch.empty((qw.N, qw.K), dtype=dtype, device=qw.codes.device)
    fn = "nf4_dequantize_dq" + _ct(out, "out")
    _dev(out, out.dtype, "out")
    _check(fn, getattr(lib(), fn)(_ptr(qw.codes), _ptr(qw.absmax_fp8), _ptr(qw.superscale), qw.numel, _ptr(out),
                                  _stream()))
    return out


MAX_TENSORS = 16         # QLORA_MAX_TENSORS


def _tensor_array(ws, qws):
    if len(ws) != len(qws):
        raise ValueError("one storage triple per weight")
    arr = (NF4Tensor * len(ws))()
    for i, (w, qw) in enumerate(zip(ws, qws)):   # every size first, then the device checks
        _check_storage(qw)
        if w.numel() != qw.numel:
            raise ValueError(f"tensor {i}: {w.numel()} elements, storage for {qw.numel}")
    for i, (w, qw) in enumerate(zip(ws, qws)):
        _dev(w, torch.bfloat16, "w")
        arr[i] = NF4Tensor(w.data_ptr(), w.numel(), qw.codes.data_ptr(), qw.absmax_fp8.data_ptr(),
                           qw.superscale.data_ptr())
    return arr


def nf4_quantize_dq_grouped(ws, qws=None):
    """Quantize up to 16 bf16 weights in one launch; returns (or fills) one NF4Weight per weight."""
    if qws is None:
        qws = []
        for w in ws:
            numel = w.numel()
            N, K = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, numel)
            qws.append(NF4Weight(torch.empty(numel // 2, dtype=torch.uint8, device=w.device),
                                 torch.empty(max(numel // 64, 1), dtype=torch.uint8, device=w.device),
                                 torch.empty(max(-(-numel // 16384), 1), dtype=torch.float32, device=w.device), N, K))
    _check("nf4_quantize_dq_grouped", lib().nf4_quantize_dq_grouped(len(ws), _tensor_array(ws, qws), _stream()))
    return qws


def nf4_dequantize_dq_grouped(qws, outs=None):
    """Dequantize up to 16 NF4Weights to bf16 in one launch; returns (or fills) the [N, K] outputs."""
    if outs is None:
        outs = [torch.empty((q.N, q.K), dtype=torch.bfloat16, device=q.codes.device) for q in qws]
    _check("nf4_dequantize_dq_grouped", lib().nf4_dequantize_dq_grouped(len(qws), _tensor_array(outs, qws),
                                                                           _stream()))
    return outs


def nf4_quantize(w):
    """bf16 weight [N, K] (or flat) on the GPU -> NF4WeightSQ (single quantization)."""
    _dev(w, torch.bfloat16, "w")
    numel = w.numel()
    N, K = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, numel)
    codes = torch.empty(numel // 2, dtype=torch.uint8, device=w.device)
    absmax = torch.empty(max(numel // 64, 1), dtype=torch.float32, device=w.device)
    _check("nf4_quantize", lib().nf4_quantize(_ptr(w), numel, _ptr(codes), _ptr(absmax), _stream()))
    return NF4WeightSQ(codes, absmax, N, K)


def nf4_dequantize(qw, out=None):
    """NF4WeightSQ -> bf16 [N, K] on the GPU."""
    _check_storage(qw)
    if out is not None and out.numel() != qw.numel:
        raise ValueError(f"out has {out.numel()} elements, the weight has {qw.numel}")
    if out is None:
        out = torch.empty((qw.N, qw.K), dtype=torch.bfloat16, device=qw.codes.device)
    _dev(out, torch.bfloat16, "out")
    _check("nf4_dequantize", lib().nf4_dequantize(_ptr(qw.codes), _ptr(qw.absmax), qw.numel, _ptr(out), _stream()))
    return out


def int4_quantize(w):
    """bf16 weight on the GPU -> NF4WeightSQ-shaped pair holding INT4 absmax codes (ablation baseline)."""
    _dev(w, torch.bfloat16, "w")
    numel = w.numel()
    N, K = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, numel)
    codes = torch.empty(numel // 2, dtype=torch.uint8, device=w.device)
    absmax = torch.empty(max(numel // 64, 1), dtype=torch.float32, device=w.device)
    _check("int4_quantize", lib().int4_quantize(_ptr(w), numel, _ptr(codes), _ptr(absmax), _stream()))
    return NF4WeightSQ(codes, absmax, N, K)


def int4_dequantize(qw, out=None):
    _check_storage(qw)
    if out is not None and out.numel() != qw.numel:
        raise ValueError(f"out has {out.numel()} elements, the weight has {qw.numel}")
    if out is None:
        out = torch.empty((qw.N, qw.K), dtype=torch.bfloat16, device=qw.codes.device)
    _dev(out, torch.bfloat16, "out")
    _check("int4_dequantize", lib().int4_dequantize(_ptr(qw.codes), _ptr(qw.absmax), qw.numel, _ptr(out),
                                                     _stream()))
    return out


def _scale_args(qw):
    """(entry-point suffix, block-constant pointers) of either storage format."""
    if isinstance(qw, NF4WeightSQ):
        return "_sq", (_ptr(qw.absmax),)
    return "", (_ptr(qw.absmax_fp8), _ptr(qw.superscale))


def qlora_workspace_bytes(T, K, N, r):
    return int(lib().qlora_workspace_bytes(T, K, N, r))


def qlora_workspace_bytes_upto(T_max, K, N, r):
    """Workspace bytes that serve every call with 1 <= T <= T_max tokens."""
    return int(lib().qlora_workspace_bytes_upto(T_max, K, N, r))


def qlora_workspace_bytes_bwd(T, K, N, r, flags):
    return int(lib().qlora_workspace_bytes_bwd(T, K, N, r, flags))


def workspace_for(T, K, N, r, device):
    n = qlora_workspace_bytes(T, K, N, r)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def qlora_linear_fwd(x, qw, lora_a=None, lora_b=None, scaling=1.0, workspace=None, out=None):
    """Y = X W'^T + scaling (X A) B; x [T, K] -> y [T, N], bf16 or fp16 (the _f16 entry point).
    `qw` is an NF4Weight (double quantization) or an NF4WeightSQ (single quantization, _sq)."""
    ct = _ct(x, "x")
    _check_storage(qw)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [T, K], got shape {tuple(x.shape)}")
    T, K = x.shape
    _shape(x, (T, qw.K), "x")
    r = _check_adapters(lora_a, lora_b, qw.K, qw.N)
    _shape(out, (T, qw.N), "out")
    _dev(x, x.dtype, "x")
    _dev(lora_a, x.dtype, "lora_a")
    _dev(lora_b, x.dtype, "lora_b")
    if out is None:
        out = torch.empty((T, qw.N), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = workspace_for(T, K, qw.N, r, x.device)
    _dev(out, x.dtype, "out")
    sc = _scale_args(qw)[1]
    fn = _entry("qlora_linear_fwd", ct, qw)
    _check(fn, getattr(lib(), fn)(
        _ptr(x), T, K, qw.N, _ptr(qw.codes), *sc, _ptr(lora_a), _ptr(lora_b),
        r, float(scaling), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def qlora_linear_fwd_noalloc(x, qw, lora_a=None, lora_b=None, scaling=1.0, out=None):
    """qlora_linear_fwd with the library's static scratch instead of a workspace
    (for callers that cannot allocate; `out` must then be given).  bf16 and
    double quantization only."""
    if x.dtype != torch.bfloat16 or isinstance(qw, NF4WeightSQ):
        raise TypeError("the no-allocation forward takes bf16 tensors and double-quantized weights")
    _check_storage(qw)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [T, K], got shape {tuple(x.shape)}")
    T = x.shape[0]
    _shape(x, (T, qw.K), "x")
    r = _check_adapters(lora_a, lora_b, qw.K, qw.N)
    _shape(out, (T, qw.N), "out")
    for t, name in ((x, "x"), (lora_a, "lora_a"), (lora_b, "lora_b"), (out, "out")):
        _dev(t, torch.bfloat16, name)
    if out is None:
        out = torch.empty((T, qw.N), dtype=torch.bfloat16, device=x.device)
    _check("qlora_linear_fwd_noalloc", lib().qlora_linear_fwd_noalloc(
        _ptr(x), T, qw.K, qw.N, _ptr(qw.codes), _ptr(qw.absmax_fp8), _ptr(qw.superscale), _ptr(lora_a),
        _ptr(lora_b), r, float(scaling), _ptr(out), _stream()))
    return out


MAX_GROUP = 8            # QLORA_MAX_GROUP
GROUPED_MAX_T = 16       # QLORA_GROUPED_MAX_T


def _grouped_array(problems, T, r):
    arr = (LinearProblem * len(problems))()
    for i, pr in enumerate(problems):          # every shape first, then the device checks
        x, qw, a, b, scaling, y = pr
        if isinstance(qw, NF4WeightSQ):
            raise TypeError("the grouped forward takes double-quantized weights (NF4Weight)")
        _check_storage(qw)
        if tuple(x.shape) != (T, qw.K) or tuple(y.shape) != (T, qw.N):
            raise ValueError(f"problem {i}: x {tuple(x.shape)} / out {tuple(y.shape)} do not match T={T}, "
                             f"K={qw.K}, N={qw.N}")
        if _check_adapters(a, b, qw.K, qw.N) != r:
            raise ValueError(f"problem {i}: every problem of a group has the same rank")
    for i, pr in enumerate(problems):
        x, qw, a, b, scaling, y = pr
        for t, name in ((x, "x"), (a, "lora_a"), (b, "lora_b"), (y, "out")):
            _dev(t, torch.bfloat16, name)
        arr[i] = LinearProblem(x.data_ptr(), qw.codes.data_ptr(), qw.absmax_fp8.data_ptr(), qw.superscale.data_ptr(),
                               None if a is None else a.data_ptr(), None if b is None else b.data_ptr(),
                               y.data_ptr(), qw.K, qw.N, float(scaling))
    return arr


def qlora_grouped_workspace_bytes(problems):
    """Workspace bytes of qlora_linear_fwd_grouped for a list of
    (x, qw, lora_a, lora_b, scaling, out) problems."""
    T = problems[0][0].shape[0]
    r = 0 if problems[0][2] is None else problems[0][2].shape[1]
    arr = _grouped_array(problems, T, r)
    return int(lib().qlora_grouped_workspace_bytes(len(problems), arr, T, r))


def qlora_linear_fwd_grouped(problems, workspace=None, product=None):
    """Decode forward of up to 8 independent layers in one launch pair.  Each
    problem is (x [T, K] bf16, NF4Weight, lora_a or None, lora_b or None,
    scaling, out [T, N] bf16); every problem has the same T (<= 16) and rank.
    Writes each out exactly as qlora_linear_fwd would.  `product` None keeps
    the library's choice; "mfma" or "valu" (T <= 8) picks the decode product
    (qlora_linear_fwd_grouped_ex)."""
    flags = {None: 0, "mfma": QLORA_DECODE_MFMA, "valu": QLORA_DECODE_VALU}.get(product)
    if flags is None:
        raise ValueError(f"product must be None, 'mfma' or 'valu', not {product!r}")
    T = problems[0][0].shape[0]
    r = 0 if problems[0][2] is None else problems[0][2].shape[1]
    arr = _grouped_array(problems, T, r)
    if workspace is None:
        n = int(lib().qlora_grouped_workspace_bytes(len(problems), arr, T, r))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=problems[0][0].device)
    if flags:
        _check("qlora_linear_fwd_grouped_ex", lib().qlora_linear_fwd_grouped_ex(
            len(problems), arr, T, r, flags, _ptr(workspace), workspace.numel(), _stream()))
    else:
        _check("qlora_linear_fwd_grouped", lib().qlora_linear_fwd_grouped(
            len(problems), arr, T, r, _ptr(workspace), workspace.numel(), _stream()))
    return [pr[5] for pr in problems]


def qlora_linear_bwd_input(dy, qw, lora_a=None, lora_b=None, scaling=1.0, x=None, lora_grads=False,
                           workspace=None, dx=None, d_lora_a=None, d_lora_b=None, reuse_forward=False,
                           fused_grads=False):
    """dX (and dA, dB when lora_grads) for upstream gradient dy [T, N] bf16.  With
    reuse_forward, `workspace` must be the one the forward of the same x, A, scaling
    just used (s X A is taken from it).  With fused_grads the dX kernel also forms
    dA and dB (QLORA_BWD_FUSED_GRADS); the workspace must then hold
    qlora_workspace_bytes_bwd(T, K, N, r, flags) bytes."""
    if reuse_forward and workspace is None:
        raise ValueError("reuse_forward needs the forward's workspace")
    ct = _ct(dy, "dy")
    _check_storage(qw)
    if dy.dim() != 2:
        raise ValueError(f"dy must be 2-D [T, N], got shape {tuple(dy.shape)}")
    T, N, K = dy.shape[0], qw.N, qw.K
    _shape(dy, (T, N), "dy")
    r = _check_adapters(lora_a, lora_b, K, N)
    if lora_grads and r == 0:
        raise ValueError("lora_grads needs the adapters")
    if lora_grads and x is None:
        raise ValueError("lora_grads needs x")
    _shape(x, (T, K), "x")
    _shape(dx, (T, K), "dx")
    if lora_grads:
        _shape(d_lora_a, (K, r), "d_lora_a")
        _shape(d_lora_b, (r, N), "d_lora_b")
    _dev(dy, dy.dtype, "dy")
    _dev(x, dy.dtype, "x")
    _dev(lora_a, dy.dtype, "lora_a")
    _dev(lora_b, dy.dtype, "lora_b")
    if dx is None:
        dx = torch.empty((T, K), dtype=dy.dtype, device=dy.device)
    if lora_grads:
        if d_lora_a is None:
            d_lora_a = torch.empty((K, r), dtype=dy.dtype, device=dy.device)
        if d_lora_b is None:
            d_lora_b = torch.empty((r, N), dtype=dy.dtype, device=dy.device)
    _dev(dx, dy.dtype, "dx")
    if lora_grads:
        _dev(d_lora_a, dy.dtype, "d_lora_a")
        _dev(d_lora_b, dy.dtype, "d_lora_b")
    flags = (REUSE_FORWARD if reuse_forward else 0) | (FUSED_GRADS if fused_grads else 0)
    if workspace is None:
        n = qlora_workspace_bytes_bwd(T, K, N, r, flags) if fused_grads else qlora_workspace_bytes(T, K, N, r)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dy.device)
    sc = _scale_args(qw)[1]
    fn = _entry("qlora_linear_bwd_input", ct, qw)
    _check(fn, getattr(lib(), fn)(
        _ptr(dy), T, K, N, _ptr(qw.codes), *sc, _ptr(lora_a), _ptr(lora_b),
        r, float(scaling), _ptr(dx), _ptr(x), _ptr(d_lora_a) if lora_grads else None,
        _ptr(d_lora_b) if lora_grads else None, _ptr(workspace), workspace.numel(), flags, _stream()))
    return (dx, d_lora_a, d_lora_b) if lora_grads else (dx, None, None)


def qlora_merge_lora(qw, lora_a=None, lora_b=None, scaling=1.0, out=None, dtype=None):
    """W_m = RNE_16(W' + scaling (A B)^T) -> [N, K] (W' itself without an adapter), in the
    dtype of the adapters (else of `out`, else `dtype`, else bf16)."""
    dt = lora_a.dtype if lora_a is not None else (out.dtype if out is not None else (dtype or torch.bfloat16))
    _check_storage(qw)
    r = _check_adapters(lora_a, lora_b, qw.K, qw.N)
    _shape(out, (qw.N, qw.K), "out")
    _dev(lora_a, dt, "lora_a")
    _dev(lora_b, dt, "lora_b")
    if out is None:
        out = torch.empty((qw.N, qw.K), dtype=dt, device=qw.codes.device)
    _dev(out, dt, "out")
    sc = _scale_args(qw)[1]
    fn = _entry("qlora_merge_lora", _ct(out, "out"), qw)
    _check(fn, getattr(lib(), fn)(
        _ptr(qw.codes), *sc, qw.K, qw.N, _ptr(lora_a), _ptr(lora_b), r, float(scaling), _ptr(out), _stream()))
    return out


# The _sq entry points under their C names (the wrappers above pick them for an NF4WeightSQ).
def qlora_linear_fwd_sq(x, qw, lora_a=None, lora_b=None, scaling=1.0, workspace=None, out=None):
    assert isinstance(qw, NF4WeightSQ)
    return qlora_linear_fwd(x, qw, lora_a, lora_b, scaling, workspace, out)


def qlora_linear_bwd_input_sq(dy, qw, lora_a=None, lora_b=None, scaling=1.0, x=None, lora_grads=False,
                              workspace=None, dx=None, d_lora_a=None, d_lora_b=None, reuse_forward=False,
                              fused_grads=False):
    assert isinstance(qw, NF4WeightSQ)
    return qlora_linear_bwd_input(dy, qw, lora_a, lora_b, scaling, x, lora_grads, workspace, dx, d_lora_a, d_lora_b,
                                  reuse_forward, fused_grads)


def qlora_merge_lora_sq(qw, lora_a=None, lora_b=None, scaling=1.0, out=None):
    assert isinstance(qw, NF4WeightSQ)
    return qlora_merge_lora(qw, lora_a, lora_b, scaling, out)
