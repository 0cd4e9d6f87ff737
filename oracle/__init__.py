"""ctypes binding of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the optimizer library.  Arrays are
numpy arrays on the host; every call runs the plain single-threaded C code.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ONEBIT_ORACLE_LIB lets the mutation test load a deliberately broken build.
_LIB_PATH = os.environ.get("ONEBIT_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

ONEBIT = 0
IDENTITY = 1


class HParams(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in
                ("beta1", "beta2", "eta", "lr", "weight_decay", "c_min", "c_max", "f_min", "f_max",
                 "kappa")] + [("rho_mode", ctypes.c_int32), ("c_avg_decay", ctypes.c_float),
                              ("bias_step", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        _lib.oracle_chunk_scale.argtypes = [P, i64, i32, P]
        _lib.oracle_chunk_scale.restype = ctypes.c_float
        _lib.oracle_compress_ef.argtypes = [i64, i32, P, P, P, P]
        _lib.oracle_decompress.argtypes = [i64, i32, P, P, P]
        _lib.oracle_average.argtypes = [i64, i32, i32, P, P, P]
        _lib.oracle_average_packed.argtypes = [i64, i32, i32, P, P, P, P, P]
        _lib.oracle_warmup_step.argtypes = [i32, P, i32, P, P, P, P, P, P, ctypes.POINTER(HParams)]
        _lib.oracle_freeze.argtypes = [i32, i64, i32, P, P, P, P, P, i32, P, P,
                                       ctypes.POINTER(HParams)]
        _lib.oracle_compressed_step.argtypes = [i32, P, i32, i32, P, P, P, P, P, P, P, P, P, P, P,
                                                P, P, P, ctypes.POINTER(HParams), i32]
        _lib.oracle_adam_warmup_step.argtypes = [i64, i32, P, P, P, P, ctypes.POINTER(HParams)]
        _lib.oracle_adam_compressed_step.argtypes = [i64, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                                     ctypes.POINTER(HParams), i32]
        _lib.oracle_sparse_step.argtypes = [i32, P, i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                            ctypes.POINTER(HParams)]
        for f in ("oracle_compress_ef", "oracle_decompress", "oracle_average",
                  "oracle_average_packed", "oracle_warmup_step", "oracle_freeze",
                  "oracle_compressed_step", "oracle_adam_warmup_step",
                  "oracle_adam_compressed_step", "oracle_sparse_step"):
            getattr(_lib, f).restype = None
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    assert isinstance(a, np.ndarray) and a.dtype == np.float32 and a.flags.c_contiguous
    return a


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[_ptr(a) for a in arrays])
    return arr


def _words_out(n):
    """An output array of sign words, all ones until the oracle writes it
    (so a word it failed to write shows)."""
    return np.full(n, 0xFFFFFFFF, np.uint32)


def _f32_out(n):
    """An fp32 output array, NaN until the oracle writes it."""
    return np.full(n, np.nan, np.float32)


def num_chunks(n, C):
    return (n + C - 1) // C


def hparams(**kw):
    return HParams(**kw)


def chunk_scale(z, C):
    z = _f32(np.ascontiguousarray(z, dtype=np.float32))
    scratch = np.empty(C, np.float32)
    return float(lib().oracle_chunk_scale(_ptr(z), z.size, C, _ptr(scratch)))


def compress_ef(inp, err, C):
    """err is updated in place; returns (bits uint32[K*C/32], scales f32[K])."""
    n = inp.size
    K = num_chunks(n, C)
    bits = _words_out(K * C // 32)
    scales = _f32_out(K)
    lib().oracle_compress_ef(n, C, _ptr(_f32(inp)), _ptr(_f32(err)), _ptr(bits), _ptr(scales))
    return bits, scales


def decompress(bits, scales, n, C):
    out = np.empty(n, np.float32)
    lib().oracle_decompress(n, C, _ptr(bits), _ptr(scales), _ptr(out))
    return out


def average(bits_w, scales_w, n, C):
    W = len(bits_w)
    a = np.empty(n, np.float32)
    lib().oracle_average(n, C, W, _ptr_array(bits_w), _ptr_array(scales_w), _ptr(a))
    return a


def average_packed(bits_w, scales_w, err_s, C):
    n = err_s.size
    K = num_chunks(n, C)
    W = len(bits_w)
    bits = _words_out(K * C // 32)
    scales = _f32_out(K)
    lib().oracle_average_packed(n, C, W, _ptr_array(bits_w), _ptr_array(scales_w),
                                _ptr(_f32(err_s)), _ptr(bits), _ptr(scales))
    return bits, scales


def warmup_step(numels, grads, x, m, v, c_sum, hp):
    """x, m, v, c_sum updated in place; returns c (per tensor)."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    L = numels.size
    c_out = np.empty(L, np.float32)
    lib().oracle_warmup_step(L, _ptr(numels), len(grads), _ptr_array([_f32(g) for g in grads]),
                             _ptr(_f32(x)), _ptr(_f32(m)), _ptr(_f32(v)), _ptr(_f32(c_sum)),
                             _ptr(c_out), ctypes.byref(hp))
    return c_out


def freeze(numels, v, v_fresh, err_w, err_s, c_sum, T_w, c_avg, f_prev, hp=None):
    numels = np.asarray(numels, dtype=np.int64)
    lib().oracle_freeze(numels.size, int(numels.sum()), len(err_w), _ptr(_f32(v)),
                        _ptr(_f32(v_fresh)), _ptr_array([_f32(e) for e in err_w]),
                        _ptr(_f32(err_s)), _ptr(_f32(c_sum)), T_w, _ptr(_f32(c_avg)),
                        _ptr(_f32(f_prev)), None if hp is None else ctypes.byref(hp))


def compressed_step(numels, C, grads, err_w, err_s, x, m, v_frozen, v_fresh, c_avg, f_prev, hp,
                    compressor=ONEBIT):
    """State arrays updated in place.  Returns a dict with the per-tensor c,
    the workers' and the server's packed signs and scales."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    L = numels.size
    N = int(numels.sum())
    W = len(grads)
    K = num_chunks(N, C)
    c_out = np.empty(L, np.float32)
    bits_w = [_words_out(K * C // 32) for _ in range(W)]
    scales_w = [_f32_out(K) for _ in range(W)]
    bits_s = _words_out(K * C // 32)
    scales_s = _f32_out(K)
    lib().oracle_compressed_step(
        L, _ptr(numels), C, W, _ptr_array([_f32(g) for g in grads]),
        _ptr_array([_f32(e) for e in err_w]), _ptr(_f32(err_s)), _ptr(_f32(x)), _ptr(_f32(m)),
        _ptr(_f32(v_frozen)), _ptr(_f32(v_fresh)), _ptr(_f32(c_avg)), _ptr(_f32(f_prev)),
        _ptr(c_out), _ptr_array(bits_w), _ptr_array(scales_w), _ptr(bits_s), _ptr(scales_s),
        ctypes.byref(hp), compressor)
    return {"c": c_out, "bits_w": bits_w, "scales_w": scales_w, "bits_s": bits_s,
            "scales_s": scales_s}


def adam_warmup_step(grads, x, m, v, hp):
    """1-bit Adam's warmup: one Adam step; x, m, v updated in place."""
    lib().oracle_adam_warmup_step(x.size, len(grads), _ptr_array([_f32(g) for g in grads]),
                                  _ptr(_f32(x)), _ptr(_f32(m)), _ptr(_f32(v)), ctypes.byref(hp))


def adam_compressed_step(C, grads, err_w, err_s, x, m, v_frozen, hp, compressor=ONEBIT):
    """1-bit Adam's compression-stage step; state updated in place.  Returns
    the workers' and the server's packed signs and scales."""
    n = x.size
    W = len(grads)
    K = num_chunks(n, C)
    bits_w = [_words_out(K * C // 32) for _ in range(W)]
    scales_w = [_f32_out(K) for _ in range(W)]
    bits_s = _words_out(K * C // 32)
    scales_s = _f32_out(K)
    lib().oracle_adam_compressed_step(
        n, C, W, _ptr_array([_f32(g) for g in grads]), _ptr_array([_f32(e) for e in err_w]),
        _ptr(_f32(err_s)), _ptr(_f32(x)), _ptr(_f32(m)), _ptr(_f32(v_frozen)),
        _ptr_array(bits_w), _ptr_array(scales_w), _ptr(bits_s), _ptr(scales_s), ctypes.byref(hp),
        compressor)
    return {"bits_w": bits_w, "scales_w": scales_w, "bits_s": bits_s, "scales_s": scales_s}


def sparse_step(numels, C, nsel, sel, grads, err_w, x, m, v_frozen, v_fresh, c_avg, hp):
    """SLAMB-style sparse compression step; state updated in place.  Returns
    the workers' transmitted values and the server's averages (nsel*64 per
    chunk)."""
    numels = np.asarray(numels, dtype=np.int64)
    N = int(numels.sum())
    K = num_chunks(N, C)
    W = len(grads)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    assert sel.size == K
    vals_w = [_f32_out(K * nsel * 64) for _ in range(W)]
    vals_s = _f32_out(K * nsel * 64)
    lib().oracle_sparse_step(
        numels.size, numels.ctypes.data, C, W, nsel, sel.ctypes.data,
        _ptr_array([_f32(g) for g in grads]), _ptr_array([_f32(e) for e in err_w]), _ptr(_f32(x)),
        _ptr(_f32(m)), _ptr(_f32(v_frozen)), _ptr(_f32(v_fresh)), _ptr(_f32(c_avg)),
        _ptr_array(vals_w), _ptr(vals_s), ctypes.byref(hp))
    return {"vals_w": vals_w, "vals_s": vals_s}
