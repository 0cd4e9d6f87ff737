"""Python binding of libonebit.so: the 1-bit LAMB per-step optimizer and
compression pass on one MI355X GPU.

Argument marshalling only.  Every function has the name and the argument
order of its C counterpart in include/onebit.h; array arguments are CUDA
(HIP) tensors of the documented dtype (or raw device addresses as ints),
lists stand for the host arrays of worker pointers, `stream` defaults to
torch's current stream.  Every step of the path runs in the library's HIP
kernels; if the library is not built, importing this package raises.
"""
import ctypes
import os

__all__ = [
    "ONEBIT_OK", "ONEBIT_EINVAL", "ONEBIT_EALIGN", "ONEBIT_EUNSUPPORTED", "ONEBIT_EHIP",
    "ONEBIT_ENOMEM", "OnebitError", "onebit_hparams", "LayerTable", "onebit_layer_table_create",
    "onebit_layer_table_destroy", "onebit_layer_table_info", "onebit_workspace_size",
    "onebit_lamb_warmup_step", "onebit_lamb_freeze", "onebit_compress_ef", "onebit_average_packed",
    "onebit_lamb_compressed_step", "onebit_lamb_compress_average", "onebit_lamb_rescale_update",
    "onebit_decompress", "onebit_last_error", "onebit_version", "onebit_adam_warmup_step",
    "onebit_adam_compressed_step", "onebit_sparse_compressed_step", "ONEBIT_RHO_MAX",
    "ONEBIT_RHO_NORM_RATIO",
    "LIB_PATH",
]

ONEBIT_OK, ONEBIT_EINVAL, ONEBIT_EALIGN, ONEBIT_EUNSUPPORTED, ONEBIT_EHIP, ONEBIT_ENOMEM = range(6)
ONEBIT_STATUS_NONFINITE_WORKER = 1
ONEBIT_STATUS_NONFINITE_SERVER = 2
ONEBIT_STATUS_NONFINITE_TRUST = 4
ONEBIT_STATUS_NONFINITE_RHO = 8
ONEBIT_MAX_WORKERS = 16

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libonebit.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class onebit_hparams(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in
                ("beta1", "beta2", "eta", "lr", "weight_decay", "c_min", "c_max", "f_min", "f_max",
                 "kappa")] + [("rho_mode", ctypes.c_int32), ("c_avg_decay", ctypes.c_float),
                              ("bias_step", ctypes.c_int32)]


ONEBIT_RHO_MAX = 0
ONEBIT_RHO_NORM_RATIO = 1


_lib.onebit_layer_table_create.argtypes = [_P, _i32, _i32, ctypes.POINTER(_P)]
_lib.onebit_layer_table_destroy.argtypes = [_P]
_lib.onebit_layer_table_info.argtypes = [_P, _P, _P, _P]
_lib.onebit_workspace_size.argtypes = [_P, _i32, ctypes.POINTER(ctypes.c_size_t)]
_lib.onebit_lamb_warmup_step.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P,
                                         ctypes.POINTER(onebit_hparams), _P, _P, _P]
_lib.onebit_lamb_freeze.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _i32, _P, _P,
                                    ctypes.POINTER(onebit_hparams), _P]
_lib.onebit_compress_ef.argtypes = [_i64, _i32, _P, _P, _P, _P, _P, _P]
_lib.onebit_average_packed.argtypes = [_i64, _i32, _i32, _P, _P, _P, _P, _P, _P, _P]
_lib.onebit_lamb_compressed_step.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, ctypes.POINTER(onebit_hparams), _P,
                                             _P, _P]
_lib.onebit_lamb_compress_average.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.POINTER(onebit_hparams), _P, _P, _P]
_lib.onebit_lamb_rescale_update.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            ctypes.POINTER(onebit_hparams), _P, _P, _P]
_lib.onebit_decompress.argtypes = [_i64, _i32, _P, _P, _P, _P]
_lib.onebit_adam_warmup_step.argtypes = [_i64, _i32, _P, _P, _P, _P, ctypes.POINTER(onebit_hparams),
                                         _P]
_lib.onebit_adam_compressed_step.argtypes = [_i64, _i32, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, ctypes.POINTER(onebit_hparams), _P, _P]
_lib.onebit_sparse_compressed_step.argtypes = [_P, _i32, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               _P, ctypes.POINTER(onebit_hparams), _P, _P]
_lib.onebit_last_error.restype = ctypes.c_char_p
_lib.onebit_version.restype = ctypes.c_char_p
for _f in ("onebit_layer_table_create", "onebit_layer_table_destroy", "onebit_layer_table_info",
           "onebit_workspace_size", "onebit_lamb_warmup_step", "onebit_lamb_freeze",
           "onebit_compress_ef", "onebit_average_packed", "onebit_lamb_compressed_step",
           "onebit_lamb_compress_average", "onebit_lamb_rescale_update", "onebit_decompress"):
    getattr(_lib, _f).restype = ctypes.c_int


class OnebitError(RuntimeError):
    def __init__(self, code, fn, msg):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


def _check(rc, fn):
    if rc != ONEBIT_OK:
        raise OnebitError(rc, fn, onebit_last_error())


def _ptr(a):
    """Device address of a tensor, an int address, or None (NULL)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _ptr_list(items):
    if items is None:
        return None
    return (ctypes.c_void_p * len(items))(*[_ptr(a) for a in items])


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def onebit_last_error():
    return _lib.onebit_last_error().decode()


def onebit_version():
    return _lib.onebit_version().decode()


def onebit_layer_table_create(numels, chunk):
    """Returns the raw descriptor handle (int); see LayerTable for RAII."""
    arr = (ctypes.c_int64 * len(numels))(*[int(n) for n in numels])
    out = ctypes.c_void_p()
    _check(_lib.onebit_layer_table_create(arr, len(numels), chunk, ctypes.byref(out)),
           "onebit_layer_table_create")
    return out.value


def onebit_layer_table_destroy(handle):
    _check(_lib.onebit_layer_table_destroy(handle), "onebit_layer_table_destroy")


def onebit_layer_table_info(handle):
    N, K, S = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.onebit_layer_table_info(handle, ctypes.byref(N), ctypes.byref(K), ctypes.byref(S)),
           "onebit_layer_table_info")
    return N.value, K.value, S.value


def onebit_workspace_size(handle, W):
    b = ctypes.c_size_t()
    _check(_lib.onebit_workspace_size(handle, W, ctypes.byref(b)), "onebit_workspace_size")
    return b.value


class LayerTable:
    """Owns an onebit_layer_table handle."""

    def __init__(self, numels, chunk=4096):
        self.numels = [int(n) for n in numels]
        self.chunk = chunk
        self.handle = onebit_layer_table_create(self.numels, chunk)
        self.N, self.K, self.n_segments = onebit_layer_table_info(self.handle)
        self.L = len(self.numels)

    def workspace_size(self, W):
        return onebit_workspace_size(self.handle, W)

    def close(self):
        if self.handle:
            onebit_layer_table_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def _as_parameter_(self):
        return ctypes.c_void_p(self.handle)


def _h(table):
    return table.handle if isinstance(table, LayerTable) else table


def onebit_lamb_warmup_step(table, W, grads, x, m, v, c_sum, c_out, hp, ws, status=None,
                            stream=None):
    _check(_lib.onebit_lamb_warmup_step(_h(table), W, _ptr_list(grads), _ptr(x), _ptr(m), _ptr(v),
                                        _ptr(c_sum), _ptr(c_out), ctypes.byref(hp), _ptr(ws),
                                        _ptr(status), _stream(stream)),
           "onebit_lamb_warmup_step")


def onebit_lamb_freeze(table, W, v, v_fresh, err_w, err_s, c_sum, T_w, c_avg, f_prev, hp=None,
                       stream=None):
    _check(_lib.onebit_lamb_freeze(_h(table), W, _ptr(v), _ptr(v_fresh), _ptr_list(err_w),
                                   _ptr(err_s), _ptr(c_sum), T_w, _ptr(c_avg), _ptr(f_prev),
                                   None if hp is None else ctypes.byref(hp), _stream(stream)),
           "onebit_lamb_freeze")


def onebit_compress_ef(n, chunk, inp, err, bits, scales, status=None, stream=None):
    _check(_lib.onebit_compress_ef(n, chunk, _ptr(inp), _ptr(err), _ptr(bits), _ptr(scales),
                                   _ptr(status), _stream(stream)),
           "onebit_compress_ef")


def onebit_average_packed(n, chunk, W, bits_w, scales_w, err_s, bits_out, scales_out, status=None,
                          stream=None):
    _check(_lib.onebit_average_packed(n, chunk, W, _ptr_list(bits_w), _ptr_list(scales_w),
                                      _ptr(err_s), _ptr(bits_out), _ptr(scales_out), _ptr(status),
                                      _stream(stream)),
           "onebit_average_packed")


def onebit_lamb_compressed_step(table, W, grads, err_w, err_s, x, m, v_frozen, v_fresh, c_avg,
                                f_prev, c_out, bits_w, scales_w, bits_s, scales_s, hp, ws,
                                status=None, stream=None):
    _check(_lib.onebit_lamb_compressed_step(
        _h(table), W, _ptr_list(grads), _ptr_list(err_w), _ptr(err_s), _ptr(x), _ptr(m),
        _ptr(v_frozen), _ptr(v_fresh), _ptr(c_avg), _ptr(f_prev), _ptr(c_out), _ptr_list(bits_w),
        _ptr_list(scales_w), _ptr(bits_s), _ptr(scales_s), ctypes.byref(hp), _ptr(ws),
        _ptr(status), _stream(stream)),
        "onebit_lamb_compressed_step")


def onebit_lamb_compress_average(table, W, grads, err_w, err_s, m, v_frozen, v_fresh, bits_w,
                                 scales_w, bits_s, scales_s, hp, ws, status=None, stream=None):
    _check(_lib.onebit_lamb_compress_average(
        _h(table), W, _ptr_list(grads), _ptr_list(err_w), _ptr(err_s), _ptr(m), _ptr(v_frozen),
        _ptr(v_fresh), _ptr_list(bits_w), _ptr_list(scales_w), _ptr(bits_s), _ptr(scales_s),
        ctypes.byref(hp), _ptr(ws), _ptr(status), _stream(stream)),
        "onebit_lamb_compress_average")


def onebit_lamb_rescale_update(table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev, c_out, hp,
                               ws, status=None, stream=None):
    _check(_lib.onebit_lamb_rescale_update(
        _h(table), _ptr(bits_s), _ptr(scales_s), _ptr(x), _ptr(m), _ptr(v_frozen), _ptr(c_avg),
        _ptr(f_prev), _ptr(c_out), ctypes.byref(hp), _ptr(ws), _ptr(status), _stream(stream)),
        "onebit_lamb_rescale_update")


def onebit_decompress(n, chunk, bits, scales, out, stream=None):
    _check(_lib.onebit_decompress(n, chunk, _ptr(bits), _ptr(scales), _ptr(out), _stream(stream)),
           "onebit_decompress")


def onebit_adam_warmup_step(n, W, grads, x, m, v, hp, stream=None):
    _check(_lib.onebit_adam_warmup_step(n, W, _ptr_list(grads), _ptr(x), _ptr(m), _ptr(v),
                                        ctypes.byref(hp), _stream(stream)),
           "onebit_adam_warmup_step")


def onebit_adam_compressed_step(n, chunk, W, grads, err_w, err_s, x, m, v_frozen, bits_w,
                                scales_w, bits_s, scales_s, hp, status=None, stream=None):
    _check(_lib.onebit_adam_compressed_step(
        n, chunk, W, _ptr_list(grads), _ptr_list(err_w), _ptr(err_s), _ptr(x), _ptr(m),
        _ptr(v_frozen), _ptr_list(bits_w), _ptr_list(scales_w), _ptr(bits_s), _ptr(scales_s),
        ctypes.byref(hp), _ptr(status), _stream(stream)),
        "onebit_adam_compressed_step")


def onebit_sparse_compressed_step(table, W, nsel, sel, grads, err_w, x, m, v_frozen, v_fresh,
                                  c_avg, vals_w, vals_s, hp, status=None, stream=None):
    _check(_lib.onebit_sparse_compressed_step(
        _h(table), W, nsel, _ptr(sel), _ptr_list(grads), _ptr_list(err_w), _ptr(x), _ptr(m),
        _ptr(v_frozen), _ptr(v_fresh), _ptr(c_avg), _ptr_list(vals_w), _ptr(vals_s),
        ctypes.byref(hp), _ptr(status), _stream(stream)),
        "onebit_sparse_compressed_step")
