"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Holds none of the optimizer's arithmetic: only the counter-based generator
(synth_core.h) and the workload recipes (workloads.py).  Host arrays are
filled by libsynth.so, device buffers by libsynth_dev.so; both give the same
fp32 values for the same (seed, stream, index).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_host = None
_dev = None

# array ids used in the stream number
X, M, V, G, LAYER_SCALE, SEL = 1, 2, 3, 4, 5, 6


def stream_id(array, step=0, worker=0):
    return (array << 40) | (step << 20) | worker


def host_lib():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        _host = ctypes.CDLL(path)
        u64, i64, i32, d, P = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                               ctypes.c_void_p)
        _host.synth_fill_normal.argtypes = [u64, u64, i64, i64, d, d, P]
        _host.synth_fill_uniform.argtypes = [u64, u64, i64, i64, d, d, P]
        _host.synth_normal_f64.argtypes = [u64, u64, i64, i64, P]
        _host.synth_layer_log_scales.argtypes = [u64, u64, i32, d, d, P]
        _host.synth_fill_index.argtypes = [u64, u64, i64, i64, i32, P]
        _host.synth_ln_unit_host.argtypes = [u64]
        _host.synth_ln_unit_host.restype = d
        _host.synth_sqrt_host.argtypes = [d]
        _host.synth_sqrt_host.restype = d
        _host.synth_cos2pi_host.argtypes = [u64]
        _host.synth_cos2pi_host.restype = d
        _host.synth_mix64_host.argtypes = [u64]
        _host.synth_mix64_host.restype = u64
        _host.synth_num_threads.restype = ctypes.c_int
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libsynth_dev.so is not built (run __graft_entry__.build())")
        _dev = ctypes.CDLL(path)
        u64, i64, d, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        _dev.synth_dev_fill_normal.argtypes = [u64, u64, i64, i64, d, d, P, P]
        _dev.synth_dev_fill_uniform.argtypes = [u64, u64, i64, i64, d, d, P, P]
        _dev.synth_dev_fill_normal.restype = ctypes.c_int
        _dev.synth_dev_fill_uniform.restype = ctypes.c_int
    return _dev


def normal_host(out, seed, stream, offset, mean, std):
    assert out.dtype == np.float32 and out.flags.c_contiguous
    host_lib().synth_fill_normal(seed, stream, offset, out.size, mean, std, out.ctypes.data)
    return out


def uniform_host(out, seed, stream, offset, lo, hi):
    assert out.dtype == np.float32 and out.flags.c_contiguous
    host_lib().synth_fill_uniform(seed, stream, offset, out.size, lo, hi, out.ctypes.data)
    return out


def _torch_stream(stream):
    import torch
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def normal_dev(t, seed, stream, offset, mean, std, cuda_stream=None):
    """Fill a contiguous float32 CUDA tensor (or a window of one) on device."""
    assert t.is_cuda and t.is_contiguous()
    rc = dev_lib().synth_dev_fill_normal(seed, stream, offset, t.numel(), mean, std, t.data_ptr(),
                                         _torch_stream(cuda_stream))
    if rc:
        raise RuntimeError(f"synth_dev_fill_normal failed ({rc})")
    return t


def uniform_dev(t, seed, stream, offset, lo, hi, cuda_stream=None):
    assert t.is_cuda and t.is_contiguous()
    rc = dev_lib().synth_dev_fill_uniform(seed, stream, offset, t.numel(), lo, hi, t.data_ptr(),
                                          _torch_stream(cuda_stream))
    if rc:
        raise RuntimeError(f"synth_dev_fill_uniform failed ({rc})")
    return t


def layer_log_scales(seed, L, lo_exp10, hi_exp10):
    out = np.empty(L, np.float64)
    host_lib().synth_layer_log_scales(seed, stream_id(LAYER_SCALE), L, lo_exp10, hi_exp10,
                                      out.ctypes.data)
    return out


def index_host(out, seed, stream, offset, nb):
    """Fill the int32 array `out` with uniform integers in [0, nb)."""
    assert out.dtype == np.int32 and out.flags.c_contiguous
    host_lib().synth_fill_index(seed, stream, offset, out.size, nb, out.ctypes.data)
    return out
