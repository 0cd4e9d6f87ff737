"""Python binding of libonebit.so: the 1-bit LAMB per-step optimizer and
compression pass on one MI355X GPU.

Argument marshalling only.  Every function has the name and the argument
order of its C counterpart in include/onebit.h; array arguments are CUDA
(HIP) tensors of the documented dtype (or raw device addresses as ints),
lists stand for the host arrays of worker pointers, `stream` defaults to
torch's current stream.  Every step of the path runs in the library's HIP
kernels; if the library is not built, importing this package raises.

Before a call reaches the library, tensors are checked for what the C side
cannot see: that they live on the current GPU, are contiguous, have the documented
dtype and hold at least the bytes the call touches, and that a list holds
at least W worker entries (OnebitError with ONEBIT_EINVAL otherwise).  When
a scalar argument (n, chunk, W, nsel) is itself invalid, the sizes are not
checked and the library reports the error.  Raw integer addresses are
passed through unchecked.
"""
import ctypes
import os

__all__ = [
    "ONEBIT_OK", "ONEBIT_EINVAL", "ONEBIT_EALIGN", "ONEBIT_EUNSUPPORTED", "ONEBIT_EHIP",
    "ONEBIT_ENOMEM", "OnebitError", "onebit_hparams", "LayerTable", "onebit_layer_table_create",
    "onebit_layer_table_destroy", "onebit_layer_table_info", "onebit_workspace_size",
    "onebit_lamb_warmup_step", "onebit_lamb_warmup_step_carry", "onebit_lamb_freeze",
    "onebit_compress_ef", "onebit_average_packed",
    "onebit_lamb_compressed_step", "onebit_lamb_compressed_step_noalloc",
    "onebit_lamb_compress_average", "onebit_lamb_rescale_update",
    "onebit_decompress", "onebit_last_error", "onebit_version", "onebit_adam_warmup_step",
    "onebit_adam_compressed_step", "onebit_sparse_compressed_step", "onebit_worker_compress",
    "onebit_lamb_rescale_stats", "onebit_adam_update", "onebit_sparse_worker",
    "onebit_sparse_average", "onebit_sparse_update", "ONEBIT_RHO_MAX",
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

# The arrays come from torch, so the library must share torch's HIP runtime:
# torch is imported first, and libonebit.so's HIP calls then bind to the
# runtime it loaded.  Loaded the other way round, the process can end up with
# two runtimes, and the library's sees no device.
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - the binding's host checks need no GPU
    pass

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
_lib.onebit_lamb_warmup_step_carry.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P, _P, _i32,
                                               ctypes.POINTER(onebit_hparams), _P, _P, _P]
_lib.onebit_lamb_freeze.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _i32, _P, _P,
                                    ctypes.POINTER(onebit_hparams), _P]
_lib.onebit_compress_ef.argtypes = [_i64, _i32, _P, _P, _P, _P, _P, _P]
_lib.onebit_average_packed.argtypes = [_i64, _i32, _i32, _P, _P, _P, _P, _P, _P, _P]
_lib.onebit_lamb_compressed_step.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, ctypes.POINTER(onebit_hparams), _P,
                                             _P, _P]
_lib.onebit_lamb_compressed_step_noalloc.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                     _P, _P, _P, _P, _P,
                                                     ctypes.POINTER(onebit_hparams), _P, _P]
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
_lib.onebit_worker_compress.argtypes = [_i64, _i32, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.POINTER(onebit_hparams), _P, _P]
_lib.onebit_lamb_rescale_stats.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.POINTER(onebit_hparams), _P, _P]
_lib.onebit_adam_update.argtypes = [_i64, _i32, _P, _P, _P, _P, _P, ctypes.POINTER(onebit_hparams),
                                    _P]
_lib.onebit_sparse_worker.argtypes = [_i64, _i32, _i32, _P, _P, _P, _P, _P,
                                      ctypes.POINTER(onebit_hparams), _P]
_lib.onebit_sparse_average.argtypes = [_i64, _i32, _P, _P, _P]
_lib.onebit_sparse_update.argtypes = [_P, _i32, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.POINTER(onebit_hparams), _P, _P]
_lib.onebit_last_error.restype = ctypes.c_char_p
_lib.onebit_version.restype = ctypes.c_char_p
for _f in ("onebit_layer_table_create", "onebit_layer_table_destroy", "onebit_layer_table_info",
           "onebit_workspace_size", "onebit_lamb_warmup_step", "onebit_lamb_warmup_step_carry",
           "onebit_lamb_freeze",
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


_F32, _WORDS, _ANY = "f32", "words", "any"


def _chunk_ok(chunk):
    return isinstance(chunk, int) and 64 <= chunk <= (1 << 24) and chunk & (chunk - 1) == 0


def _W_ok(W):
    return isinstance(W, int) and 1 <= W <= ONEBIT_MAX_WORKERS


def _bad(fn, msg):
    return OnebitError(ONEBIT_EINVAL, fn, "binding: " + msg)


def _ptr(a, fn="", name="", nbytes=None, kind=_ANY):
    """Device address of a tensor, an int address, or None (NULL).  A
    tensor must be on the GPU, contiguous, of the kind's dtype, and hold at
    least nbytes (when given)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    import torch
    if not a.is_cuda:
        raise _bad(fn, f"{name} is not a GPU tensor")
    if a.device.index != torch.cuda.current_device():
        raise _bad(fn, f"{name} is on {a.device}, the current device is "
                       f"cuda:{torch.cuda.current_device()}")
    if not a.is_contiguous():
        raise _bad(fn, f"{name} is not contiguous")
    if kind == _F32 and a.dtype != torch.float32:
        raise _bad(fn, f"{name} has dtype {a.dtype}, float32 expected")
    if kind == _WORDS and a.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise _bad(fn, f"{name} has dtype {a.dtype}, 32-bit words expected")
    if nbytes is not None and a.numel() * a.element_size() < nbytes:
        raise _bad(fn, f"{name} holds {a.numel() * a.element_size()} bytes, the call touches "
                       f"{nbytes}")
    return a.data_ptr()


def _ptr_list(items, fn="", name="", W=None, nbytes=None, kind=_ANY):
    """Host array of the entries' device addresses; at least W entries."""
    if items is None:
        return None
    if W is not None and _W_ok(W) and len(items) < W:
        raise _bad(fn, f"{name} has {len(items)} entries, W = {W}")
    return (ctypes.c_void_p * len(items))(
        *[_ptr(a, fn, f"{name}[{i}]", nbytes, kind) for i, a in enumerate(items)])


class _Sizes:
    """Bytes an entry point touches per kind of array, or None where the
    scalar arguments are invalid (the library then reports the error)."""

    def __init__(self, n=None, chunk=None, L=None, ws=None):
        ok = n is not None and n >= 0 and _chunk_ok(chunk)
        K = -(-n // chunk) if ok else None
        self.elems = 4 * n if ok else None             # one fp32 per element
        self.words = 4 * (K * chunk // 32) if ok else None
        self.scales = 4 * K if ok else None
        self.tensors = 4 * L if L is not None else None
        self.ws = ws
        self.K = K


def _table_sizes(table, W=None):
    if isinstance(table, LayerTable):
        ws = table.workspace_size(W) if W is not None and _W_ok(W) else None
        return _Sizes(table.N, table.chunk, table.L, ws)
    return _Sizes()                                     # raw handle: sizes unknown here


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
    fn, z = "onebit_lamb_warmup_step", _table_sizes(table, W)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    t = lambda a, nm: _ptr(a, fn, nm, z.tensors, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_warmup_step(_h(table), W, _ptr_list(grads, fn, "grads", W, z.elems, _F32),
                                        e(x, "x"), e(m, "m"), e(v, "v"), t(c_sum, "c_sum"),
                                        t(c_out, "c_out"), ctypes.byref(hp),
                                        _ptr(ws, fn, "ws", z.ws), _ptr(status, fn, "status", 4),
                                        _stream(stream)), fn)


def onebit_lamb_warmup_step_carry(table, W, grads, x, m, v, c_sum, c_out, x_sq, x_sq_valid, hp,
                                  ws, status=None, stream=None):
    fn, z = "onebit_lamb_warmup_step_carry", _table_sizes(table, W)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    t = lambda a, nm: _ptr(a, fn, nm, z.tensors, _F32)  # noqa: E731
    segs = 8 * table.n_segments if isinstance(table, LayerTable) else None
    if x_sq is not None and not isinstance(x_sq, int):
        import torch
        if x_sq.dtype != torch.float64:
            raise _bad(fn, f"x_sq has dtype {x_sq.dtype}, float64 expected")
    _check(_lib.onebit_lamb_warmup_step_carry(
        _h(table), W, _ptr_list(grads, fn, "grads", W, z.elems, _F32), e(x, "x"), e(m, "m"),
        e(v, "v"), t(c_sum, "c_sum"), t(c_out, "c_out"), _ptr(x_sq, fn, "x_sq", segs), x_sq_valid,
        ctypes.byref(hp), _ptr(ws, fn, "ws", z.ws), _ptr(status, fn, "status", 4),
        _stream(stream)), fn)


def onebit_lamb_freeze(table, W, v, v_fresh, err_w, err_s, c_sum, T_w, c_avg, f_prev, hp=None,
                       stream=None):
    fn, z = "onebit_lamb_freeze", _table_sizes(table)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    t = lambda a, nm: _ptr(a, fn, nm, z.tensors, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_freeze(_h(table), W, e(v, "v"), e(v_fresh, "v_fresh"),
                                   _ptr_list(err_w, fn, "err_w", W, z.elems, _F32),
                                   e(err_s, "err_s"), t(c_sum, "c_sum"), T_w, t(c_avg, "c_avg"),
                                   t(f_prev, "f_prev"), None if hp is None else ctypes.byref(hp),
                                   _stream(stream)), fn)


def onebit_compress_ef(n, chunk, inp, err, bits, scales, status=None, stream=None):
    fn, z = "onebit_compress_ef", _Sizes(n, chunk)
    _check(_lib.onebit_compress_ef(n, chunk, _ptr(inp, fn, "in", z.elems, _F32),
                                   _ptr(err, fn, "err", z.elems, _F32),
                                   _ptr(bits, fn, "bits", z.words, _WORDS),
                                   _ptr(scales, fn, "scales", z.scales, _F32),
                                   _ptr(status, fn, "status", 4), _stream(stream)), fn)


def onebit_average_packed(n, chunk, W, bits_w, scales_w, err_s, bits_out, scales_out, status=None,
                          stream=None):
    fn, z = "onebit_average_packed", _Sizes(n, chunk)
    _check(_lib.onebit_average_packed(n, chunk, W, _ptr_list(bits_w, fn, "bits_w", W, z.words, _WORDS),
                                      _ptr_list(scales_w, fn, "scales_w", W, z.scales, _F32),
                                      _ptr(err_s, fn, "err_s", z.elems, _F32),
                                      _ptr(bits_out, fn, "bits_out", z.words, _WORDS),
                                      _ptr(scales_out, fn, "scales_out", z.scales, _F32),
                                      _ptr(status, fn, "status", 4), _stream(stream)), fn)


def onebit_lamb_compressed_step(table, W, grads, err_w, err_s, x, m, v_frozen, v_fresh, c_avg,
                                f_prev, c_out, bits_w, scales_w, bits_s, scales_s, hp, ws,
                                status=None, stream=None):
    fn, z = "onebit_lamb_compressed_step", _table_sizes(table, W)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    t = lambda a, nm: _ptr(a, fn, nm, z.tensors, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_compressed_step(
        _h(table), W, _ptr_list(grads, fn, "grads", W, z.elems, _F32),
        _ptr_list(err_w, fn, "err_w", W, z.elems, _F32), e(err_s, "err_s"), e(x, "x"), e(m, "m"),
        e(v_frozen, "v_frozen"), e(v_fresh, "v_fresh"), t(c_avg, "c_avg"), t(f_prev, "f_prev"),
        t(c_out, "c_out"), _ptr_list(bits_w, fn, "bits_w", W, z.words, _WORDS),
        _ptr_list(scales_w, fn, "scales_w", W, z.scales, _F32),
        _ptr(bits_s, fn, "bits_s", z.words, _WORDS), _ptr(scales_s, fn, "scales_s", z.scales, _F32),
        ctypes.byref(hp), _ptr(ws, fn, "ws", z.ws), _ptr(status, fn, "status", 4),
        _stream(stream)), fn)


def onebit_lamb_compressed_step_noalloc(table, W, grads, err_w, err_s, x, m, v_frozen, v_fresh,
                                        c_avg, f_prev, c_out, bits_w, scales_w, bits_s, scales_s,
                                        hp, status=None, stream=None):
    """onebit_lamb_compressed_step with the library's static scratch in place
    of a workspace: the call allocates nothing (see include/onebit.h)."""
    fn, z = "onebit_lamb_compressed_step_noalloc", _table_sizes(table, W)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    t = lambda a, nm: _ptr(a, fn, nm, z.tensors, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_compressed_step_noalloc(
        _h(table), W, _ptr_list(grads, fn, "grads", W, z.elems, _F32),
        _ptr_list(err_w, fn, "err_w", W, z.elems, _F32), e(err_s, "err_s"), e(x, "x"), e(m, "m"),
        e(v_frozen, "v_frozen"), e(v_fresh, "v_fresh"), t(c_avg, "c_avg"), t(f_prev, "f_prev"),
        t(c_out, "c_out"), _ptr_list(bits_w, fn, "bits_w", W, z.words, _WORDS),
        _ptr_list(scales_w, fn, "scales_w", W, z.scales, _F32),
        _ptr(bits_s, fn, "bits_s", z.words, _WORDS), _ptr(scales_s, fn, "scales_s", z.scales, _F32),
        ctypes.byref(hp), _ptr(status, fn, "status", 4), _stream(stream)), fn)


def onebit_lamb_compress_average(table, W, grads, err_w, err_s, m, v_frozen, v_fresh, bits_w,
                                 scales_w, bits_s, scales_s, hp, ws, status=None, stream=None):
    fn, z = "onebit_lamb_compress_average", _table_sizes(table, W)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_compress_average(
        _h(table), W, _ptr_list(grads, fn, "grads", W, z.elems, _F32),
        _ptr_list(err_w, fn, "err_w", W, z.elems, _F32), e(err_s, "err_s"), e(m, "m"),
        e(v_frozen, "v_frozen"), e(v_fresh, "v_fresh"),
        _ptr_list(bits_w, fn, "bits_w", W, z.words, _WORDS),
        _ptr_list(scales_w, fn, "scales_w", W, z.scales, _F32),
        _ptr(bits_s, fn, "bits_s", z.words, _WORDS), _ptr(scales_s, fn, "scales_s", z.scales, _F32),
        ctypes.byref(hp), _ptr(ws, fn, "ws", z.ws), _ptr(status, fn, "status", 4),
        _stream(stream)), fn)


def onebit_lamb_rescale_update(table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev, c_out, hp,
                               ws, status=None, stream=None):
    fn, z = "onebit_lamb_rescale_update", _table_sizes(table, 1)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    t = lambda a, nm: _ptr(a, fn, nm, z.tensors, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_rescale_update(
        _h(table), _ptr(bits_s, fn, "bits_s", z.words, _WORDS),
        _ptr(scales_s, fn, "scales_s", z.scales, _F32), e(x, "x"), e(m, "m"),
        e(v_frozen, "v_frozen"), t(c_avg, "c_avg"), t(f_prev, "f_prev"), t(c_out, "c_out"),
        ctypes.byref(hp), _ptr(ws, fn, "ws", z.ws), _ptr(status, fn, "status", 4),
        _stream(stream)), fn)


def onebit_decompress(n, chunk, bits, scales, out, stream=None):
    fn, z = "onebit_decompress", _Sizes(n, chunk)
    _check(_lib.onebit_decompress(n, chunk, _ptr(bits, fn, "bits", z.words, _WORDS),
                                  _ptr(scales, fn, "scales", z.scales, _F32),
                                  _ptr(out, fn, "out", z.elems, _F32), _stream(stream)), fn)


def onebit_adam_warmup_step(n, W, grads, x, m, v, hp, stream=None):
    fn = "onebit_adam_warmup_step"
    nb = 4 * n if isinstance(n, int) and n >= 0 else None
    e = lambda a, nm: _ptr(a, fn, nm, nb, _F32)  # noqa: E731
    _check(_lib.onebit_adam_warmup_step(n, W, _ptr_list(grads, fn, "grads", W, nb, _F32),
                                        e(x, "x"), e(m, "m"), e(v, "v"), ctypes.byref(hp),
                                        _stream(stream)), fn)


def onebit_adam_compressed_step(n, chunk, W, grads, err_w, err_s, x, m, v_frozen, bits_w,
                                scales_w, bits_s, scales_s, hp, status=None, stream=None):
    fn, z = "onebit_adam_compressed_step", _Sizes(n, chunk)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    _check(_lib.onebit_adam_compressed_step(
        n, chunk, W, _ptr_list(grads, fn, "grads", W, z.elems, _F32),
        _ptr_list(err_w, fn, "err_w", W, z.elems, _F32), e(err_s, "err_s"), e(x, "x"), e(m, "m"),
        e(v_frozen, "v_frozen"), _ptr_list(bits_w, fn, "bits_w", W, z.words, _WORDS),
        _ptr_list(scales_w, fn, "scales_w", W, z.scales, _F32),
        _ptr(bits_s, fn, "bits_s", z.words, _WORDS), _ptr(scales_s, fn, "scales_s", z.scales, _F32),
        ctypes.byref(hp), _ptr(status, fn, "status", 4), _stream(stream)), fn)


def onebit_sparse_compressed_step(table, W, nsel, sel, grads, err_w, x, m, v_frozen, v_fresh,
                                  c_avg, vals_w, vals_s, hp, status=None, stream=None):
    fn, z = "onebit_sparse_compressed_step", _table_sizes(table)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    nsel_ok = z.K is not None and isinstance(nsel, int) and 1 <= nsel <= table.chunk // 64
    per = 4 * z.K * nsel * 64 if nsel_ok else None
    _check(_lib.onebit_sparse_compressed_step(
        _h(table), W, nsel, _ptr(sel, fn, "sel", z.scales, _WORDS),
        _ptr_list(grads, fn, "grads", W, z.elems, _F32),
        _ptr_list(err_w, fn, "err_w", W, z.elems, _F32), e(x, "x"), e(m, "m"),
        e(v_frozen, "v_frozen"), e(v_fresh, "v_fresh"), _ptr(c_avg, fn, "c_avg", z.tensors, _F32),
        _ptr_list(vals_w, fn, "vals_w", W, per, _F32), _ptr(vals_s, fn, "vals_s", per, _F32),
        ctypes.byref(hp), _ptr(status, fn, "status", 4), _stream(stream)), fn)


def onebit_worker_compress(n, chunk, grad, err_w, m, bits_m, scales_m, bits_w, scales_w, hp,
                           status=None, stream=None):
    fn, z = "onebit_worker_compress", _Sizes(n, chunk)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    _check(_lib.onebit_worker_compress(
        n, chunk, e(grad, "grad"), e(err_w, "err_w"), e(m, "m"),
        _ptr(bits_m, fn, "bits_m", z.words, _WORDS), _ptr(scales_m, fn, "scales_m", z.scales, _F32),
        _ptr(bits_w, fn, "bits_w", z.words, _WORDS), _ptr(scales_w, fn, "scales_w", z.scales, _F32),
        ctypes.byref(hp), _ptr(status, fn, "status", 4), _stream(stream)), fn)


def onebit_lamb_rescale_stats(table, bits_s, scales_s, m, bits_m, scales_m, v_frozen, v_fresh, hp,
                              ws, stream=None):
    fn, z = "onebit_lamb_rescale_stats", _table_sizes(table, 1)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    _check(_lib.onebit_lamb_rescale_stats(
        _h(table), _ptr(bits_s, fn, "bits_s", z.words, _WORDS),
        _ptr(scales_s, fn, "scales_s", z.scales, _F32), e(m, "m"),
        _ptr(bits_m, fn, "bits_m", z.words, _WORDS), _ptr(scales_m, fn, "scales_m", z.scales, _F32),
        e(v_frozen, "v_frozen"), e(v_fresh, "v_fresh"), ctypes.byref(hp), _ptr(ws, fn, "ws", z.ws),
        _stream(stream)), fn)


def onebit_adam_update(n, chunk, bits_s, scales_s, x, m, v_frozen, hp, stream=None):
    fn, z = "onebit_adam_update", _Sizes(n, chunk)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    _check(_lib.onebit_adam_update(
        n, chunk, _ptr(bits_s, fn, "bits_s", z.words, _WORDS),
        _ptr(scales_s, fn, "scales_s", z.scales, _F32), e(x, "x"), e(m, "m"), e(v_frozen, "v_frozen"),
        ctypes.byref(hp), _stream(stream)), fn)


def onebit_sparse_worker(n, chunk, nsel, sel, grad, err_w, m, vals_w, hp, stream=None):
    fn, z = "onebit_sparse_worker", _Sizes(n, chunk)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    ok = z.K is not None and isinstance(nsel, int) and 1 <= nsel <= chunk // 64
    per = 4 * z.K * nsel * 64 if ok else None
    _check(_lib.onebit_sparse_worker(
        n, chunk, nsel, _ptr(sel, fn, "sel", z.scales, _WORDS), e(grad, "grad"), e(err_w, "err_w"),
        e(m, "m"), _ptr(vals_w, fn, "vals_w", per, _F32), ctypes.byref(hp), _stream(stream)), fn)


def onebit_sparse_average(count, W, vals_w, vals_s, stream=None):
    fn = "onebit_sparse_average"
    nb = 4 * count if isinstance(count, int) and count >= 0 else None
    _check(_lib.onebit_sparse_average(count, W, _ptr_list(vals_w, fn, "vals_w", W, nb, _F32),
                                      _ptr(vals_s, fn, "vals_s", nb, _F32), _stream(stream)), fn)


def onebit_sparse_update(table, nsel, sel, vals_s, x, m, v_frozen, v_fresh, c_avg, hp, status=None,
                         stream=None):
    fn, z = "onebit_sparse_update", _table_sizes(table)
    e = lambda a, nm: _ptr(a, fn, nm, z.elems, _F32)  # noqa: E731
    ok = z.K is not None and isinstance(nsel, int) and 1 <= nsel <= table.chunk // 64
    per = 4 * z.K * nsel * 64 if ok else None
    _check(_lib.onebit_sparse_update(
        _h(table), nsel, _ptr(sel, fn, "sel", z.scales, _WORDS), _ptr(vals_s, fn, "vals_s", per, _F32),
        e(x, "x"), e(m, "m"), e(v_frozen, "v_frozen"), e(v_fresh, "v_fresh"),
        _ptr(c_avg, fn, "c_avg", z.tensors, _F32), ctypes.byref(hp), _ptr(status, fn, "status", 4),
        _stream(stream)), fn)
