"""Binding of the calibration kernels (``include/qlora_calib.h``): the device's
achievable streaming bandwidth and bf16 MFMA rate, measured beside the layer's
kernels.  Argument marshalling only; they are not part of the QLoRA path."""
import ctypes

import torch

from . import api

_SIGS = {
    "qlora_calib_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "qlora_calib_mfma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]),
    "qlora_calib_mfma_flops": (ctypes.c_double, [ctypes.c_int, ctypes.c_int]),
}
EXPORTS = tuple(_SIGS)
_bound = False


def _lib():
    global _bound
    L = api.lib()
    if not _bound:
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _bound = True
    return L


def stream_copy(src, dst):
    """dst <- src (contiguous GPU tensors of the same byte size, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    if _lib().qlora_calib_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                               api._stream()) != 0:
        raise RuntimeError("qlora_calib_copy failed")


def mfma_loop(seed, out, workgroups, iters):
    """Run the MFMA-only loop; returns the flops it performs.  seed: >= 128 int32
    words on the GPU; out: >= workgroups * 256 float32 on the GPU."""
    if seed.numel() < 128 or seed.element_size() != 4 or out.numel() < workgroups * 256 or out.dtype != torch.float32:
        raise ValueError("seed needs 128 32-bit words, out workgroups * 256 floats")
    L = _lib()
    if L.qlora_calib_mfma(ctypes.c_void_p(seed.data_ptr()), ctypes.c_void_p(out.data_ptr()), workgroups, iters,
                          api._stream()) != 0:
        raise RuntimeError("qlora_calib_mfma failed")
    return L.qlora_calib_mfma_flops(workgroups, iters)
