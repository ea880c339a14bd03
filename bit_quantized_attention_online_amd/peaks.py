"""Binding of libqk4v8_peaks.so (include/qk4v8_peaks.h): argument marshalling
only.  Each call enqueues one microbenchmark launch on the current stream and
returns the work it executes; the caller times it with events."""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqk4v8_peaks.so")
_lib = None

EXPORTED = ["qk4v8_peak_hbm_read", "qk4v8_peak_mfma", "qk4v8_peak_exp2"]
FMT_FP8, FMT_FP4, FMT_BF16 = 0, 4, 16


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_attention_online_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.qk4v8_peak_hbm_read.restype = ctypes.c_int
        L.qk4v8_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.qk4v8_peak_mfma.restype = ctypes.c_int
        L.qk4v8_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.c_void_p]
        L.qk4v8_peak_exp2.restype = ctypes.c_int
        L.qk4v8_peak_exp2.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.c_void_p]
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def hbm_read(buf, sink):
    """Stream-read every byte of the device tensor ``buf`` once; returns bytes."""
    n = buf.numel() * buf.element_size()
    _check(lib().qk4v8_peak_hbm_read(buf.data_ptr(), n, sink.data_ptr(), _stream()), "qk4v8_peak_hbm_read")
    return n


def mfma(fmt, iters, sink):
    """MFMA loop (FMT_FP4 / FMT_FP8: scaled 32x32x64, FMT_BF16: 32x32x16); returns flops."""
    f = ctypes.c_double(0)
    _check(lib().qk4v8_peak_mfma(fmt, iters, sink.data_ptr(), ctypes.byref(f), _stream()), "qk4v8_peak_mfma")
    return f.value


def exp2(iters, sink):
    """v_exp_f32 loop; returns the lane-exponentials executed."""
    f = ctypes.c_double(0)
    _check(lib().qk4v8_peak_exp2(iters, sink.data_ptr(), ctypes.byref(f), _stream()), "qk4v8_peak_exp2")
    return f.value
