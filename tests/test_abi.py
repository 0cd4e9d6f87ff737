"""The C ABI without a GPU: the library loads, exports every entry point
that include/onebit.h declares, and rejects bad arguments with the
documented codes before it touches the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "onebit.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(onebit_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def ob():
    import communication_compressed_optimizer_amd as ob
    return ob


def test_header_lists_the_entry_points():
    names = declared_functions()
    for fn in ("onebit_layer_table_create", "onebit_layer_table_destroy", "onebit_lamb_warmup_step",
               "onebit_lamb_freeze", "onebit_compress_ef", "onebit_average_packed",
               "onebit_lamb_compressed_step", "onebit_decompress", "onebit_workspace_size",
               "onebit_adam_warmup_step", "onebit_adam_compressed_step"):
        assert fn in names


def test_library_exports_every_declared_symbol(ob):
    lib = ctypes.CDLL(ob.LIB_PATH)
    missing = [fn for fn in declared_functions() if not hasattr(lib, fn)]
    assert not missing
    # and the Python binding carries the same names
    assert all(hasattr(ob, fn) for fn in declared_functions())


def test_version_and_empty_error(ob):
    assert "gfx950" in ob.onebit_version()


def test_argument_checks(ob):
    lib = ob._lib
    P = ctypes.c_void_p
    # n < 0, bad chunk, NULL, misaligned: all rejected before any launch
    assert lib.onebit_compress_ef(-1, 4096, None, None, None, None, None, None) == ob.ONEBIT_EINVAL
    assert lib.onebit_compress_ef(10, 1000, None, None, None, None, None, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_compress_ef(10, 32, None, None, None, None, None, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_compress_ef(10, 4096, None, P(4096), P(4096), P(4096), None, None) == \
        ob.ONEBIT_EINVAL
    assert "in is NULL" in ob.onebit_last_error()
    assert lib.onebit_compress_ef(10, 4096, P(4100), P(4096), P(4096), P(4096), None, None) == \
        ob.ONEBIT_EALIGN
    assert lib.onebit_compress_ef(0, 4096, None, None, None, None, None, None) == ob.ONEBIT_OK
    # the status word takes 32-bit atomics
    assert lib.onebit_compress_ef(10, 4096, P(4096), P(4096), P(4096), P(4096), P(4098), None) == \
        ob.ONEBIT_EALIGN
    assert "status is not 4-byte aligned" in ob.onebit_last_error()
    arr2 = (P * 2)(4096, 4096)
    assert lib.onebit_average_packed(10, 4096, 0, arr2, arr2, P(4096), P(4096), P(4096), None,
                                     None) == ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_average_packed(10, 4096, 17, arr2, arr2, P(4096), P(4096), P(4096), None,
                                     None) == ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_decompress(5, 4096, P(4096), P(4096), P(4098), None) == ob.ONEBIT_EALIGN
    # at most 2^30 - 1 chunks per buffer, and fewer than 2^32 work-items in
    # the launch (below 1024 elements a chunk takes one 64-wide wave, so at
    # chunk 64 fewer than 2^32 elements), refused before any pointer is read
    big = (1 << 30) * 1024
    assert lib.onebit_compress_ef(big, 1024, *[P(4096)] * 4, None, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert "n too large" in ob.onebit_last_error()
    assert lib.onebit_compress_ef(1 << 32, 64, *[P(4096)] * 4, None, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert "at most 67108863 chunks of 64" in ob.onebit_last_error()
    assert lib.onebit_decompress((1 << 32) - 63, 64, P(4096), P(4096), P(4096), None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_average_packed(big, 1024, 2, arr2, arr2, P(4096), P(4096), P(4096), None,
                                     None) == ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_decompress(big, 1024, P(4096), P(4096), P(4096), None) == \
        ob.ONEBIT_EUNSUPPORTED


def test_table_checks(ob):
    lib = ob._lib
    out = ctypes.c_void_p()
    numels = (ctypes.c_int64 * 3)(10, 0, 5)
    assert lib.onebit_layer_table_create(numels, 3, 4096, ctypes.byref(out)) == ob.ONEBIT_EINVAL
    assert lib.onebit_layer_table_create(numels, 0, 4096, ctypes.byref(out)) == ob.ONEBIT_EINVAL
    numels = (ctypes.c_int64 * 1)(10)
    assert lib.onebit_layer_table_create(numels, 1, 3000, ctypes.byref(out)) == \
        ob.ONEBIT_EUNSUPPORTED
    for chunk in (1 << 25, 3 << 15, (1 << 24) + 64, 32):
        assert lib.onebit_layer_table_create(numels, 1, chunk, ctypes.byref(out)) == \
            ob.ONEBIT_EUNSUPPORTED
        assert "[64, 2^24]" in ob.onebit_last_error()
    assert lib.onebit_layer_table_destroy(None) == ob.ONEBIT_OK
    # sizes whose sum would overflow int64, or that exceed 2^30 - 1 chunks,
    # are refused before anything is allocated
    numels = (ctypes.c_int64 * 3)(1 << 62, 1 << 62, 1 << 62)
    assert lib.onebit_layer_table_create(numels, 3, 4096, ctypes.byref(out)) == \
        ob.ONEBIT_EUNSUPPORTED
    assert "too many chunks" in ob.onebit_last_error()
    numels = (ctypes.c_int64 * 1)(1 << 32)
    assert lib.onebit_layer_table_create(numels, 1, 64, ctypes.byref(out)) == \
        ob.ONEBIT_EUNSUPPORTED
    assert "too many chunks" in ob.onebit_last_error()
    numels = (ctypes.c_int64 * 2)((1 << 29) * 4096, (1 << 29) * 4096)
    assert lib.onebit_layer_table_create(numels, 2, 4096, ctypes.byref(out)) == \
        ob.ONEBIT_EUNSUPPORTED
    assert not out.value
    hp = ob.onebit_hparams(weight_decay=0.01)
    assert lib.onebit_lamb_warmup_step(None, 1, None, None, None, None, None, None,
                                       ctypes.byref(hp), None, None, None) == ob.ONEBIT_EINVAL


def test_adam_argument_checks(ob):
    lib = ob._lib
    P = ctypes.c_void_p
    hp = ob.onebit_hparams(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3)
    bad_wd = ob.onebit_hparams(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3, weight_decay=0.01)
    g = (P * 2)(4096, 4096)
    hpr = ctypes.byref(hp)
    assert lib.onebit_adam_warmup_step(-1, 2, g, P(4096), P(4096), P(4096), hpr, None) == \
        ob.ONEBIT_EINVAL
    assert lib.onebit_adam_warmup_step(10, 0, g, P(4096), P(4096), P(4096), hpr, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_adam_warmup_step(10, 2, g, P(4096), P(4096), P(4096), ctypes.byref(bad_wd),
                                       None) == ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_adam_warmup_step(10, 2, g, P(4100), P(4096), P(4096), hpr, None) == \
        ob.ONEBIT_EALIGN
    assert lib.onebit_adam_warmup_step(10, 2, None, P(4096), P(4096), P(4096), hpr, None) == \
        ob.ONEBIT_EINVAL
    assert lib.onebit_adam_warmup_step(0, 2, None, None, None, None, hpr, None) == ob.ONEBIT_OK
    args = [g, g, P(4096), P(4096), P(4096), P(4096), None, None, P(4096), P(4096)]
    assert lib.onebit_adam_compressed_step(10, 3000, 2, *args, hpr, None, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_adam_compressed_step(10, 4096, 17, *args, hpr, None, None) == \
        ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_adam_compressed_step(-5, 4096, 2, *args, hpr, None, None) == \
        ob.ONEBIT_EINVAL
    bad = list(args)
    bad[3] = None                     # x (m may be NULL: packed momentum)
    assert lib.onebit_adam_compressed_step(10, 4096, 2, *bad, hpr, None, None) == ob.ONEBIT_EINVAL
    assert "x is NULL" in ob.onebit_last_error()
    bad = list(args)
    bad[4] = P(4100)                  # m misaligned
    assert lib.onebit_adam_compressed_step(10, 4096, 2, *bad, hpr, None, None) == ob.ONEBIT_EALIGN
    bad = list(args)
    bad[5] = P(4104)                  # v_frozen misaligned
    assert lib.onebit_adam_compressed_step(10, 4096, 2, *bad, hpr, None, None) == ob.ONEBIT_EALIGN
    bad = list(args)
    bad[1] = (P * 2)(4096, 0)         # err_w[1] NULL
    assert lib.onebit_adam_compressed_step(10, 4096, 2, *bad, hpr, None, None) == ob.ONEBIT_EINVAL
    assert lib.onebit_adam_compressed_step(0, 4096, 2, *[None] * 10, hpr, None, None) == \
        ob.ONEBIT_OK


def test_package_refuses_to_load_without_library(tmp_path):
    """No fallback: without libonebit.so the package import fails loudly."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "communication_compressed_optimizer_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "communication_compressed_optimizer_amd", "__init__.py"), pkg)
    res = subprocess.run([sys.executable, "-c", "import communication_compressed_optimizer_amd"],
                         cwd=tmp_path, capture_output=True, text=True)
    assert res.returncode != 0 and "is not built" in res.stderr


def test_torch_is_loaded_before_the_library():
    """The binding imports torch before it loads libonebit.so, so that the
    library's HIP calls bind to the runtime torch's tensors live in (loaded
    the other way round a process can hold two runtimes)."""
    import subprocess
    import sys
    code = ("import sys; import communication_compressed_optimizer_amd as ob; "
            "assert 'torch' in sys.modules, 'torch not loaded'; print('ok')")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0 and "ok" in res.stdout, res.stderr[-2000:]


def test_binding_checks_tensors_before_the_library(ob):
    """Host tensors and short worker lists are rejected by the binding
    itself (a host address or a missing worker pointer would reach the
    GPU otherwise)."""
    import torch
    host = torch.zeros(4096, dtype=torch.float32)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress_ef(4096, 4096, host, host, None, None)
    assert ei.value.code == ob.ONEBIT_EINVAL and "not a GPU tensor" in str(ei.value)
    hp = ob.onebit_hparams(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_adam_warmup_step(4096, 4, [None] * 3, None, None, None, hp)
    assert ei.value.code == ob.ONEBIT_EINVAL and "3 entries, W = 4" in str(ei.value)
    # invalid scalars are left to the library, which names them
    assert ob._Sizes(10, 3000).elems is None and ob._Sizes(-1, 4096).elems is None
    z = ob._Sizes(4097, 4096)
    assert (z.K, z.elems, z.words, z.scales) == (2, 4 * 4097, 4 * 2 * 128, 8)
    # chunks are powers of two from 64 to 2^24
    z = ob._Sizes(5, 1 << 24)
    assert (z.K, z.elems, z.words, z.scales) == (1, 20, 4 * (1 << 19), 4)
    assert ob._Sizes(5, 1 << 25).elems is None and ob._Sizes(5, 32).elems is None
    assert ob._Sizes(5, 3 << 15).elems is None


def test_share_entry_point_checks(ob):
    """One GPU's share: argument errors come back as codes without a GPU."""
    lib = ob._lib
    P = ctypes.c_void_p
    hp = ob.onebit_hparams(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3)
    hpr = ctypes.byref(hp)
    args = [P(4096), P(4096), P(4096), None, None, P(4096), P(4096)]
    assert lib.onebit_worker_compress(10, 3000, *args, hpr, None, None) == ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_worker_compress(-1, 4096, *args, hpr, None, None) == ob.ONEBIT_EINVAL
    assert lib.onebit_worker_compress(0, 4096, *[None] * 7, hpr, None, None) == ob.ONEBIT_OK
    bad = list(args)
    bad[2] = None                     # no fp32 momentum and no packed one
    assert lib.onebit_worker_compress(10, 4096, *bad, hpr, None, None) == ob.ONEBIT_EINVAL
    assert "m is NULL" in ob.onebit_last_error()
    bad = list(args)
    bad[0] = P(4100)                  # grad misaligned
    assert lib.onebit_worker_compress(10, 4096, *bad, hpr, None, None) == ob.ONEBIT_EALIGN
    bad = list(args)
    bad[5] = P(4100)                  # sign words may start at any 4-byte boundary
    bad[6] = P(4098)                  # but not at 2 bytes
    assert lib.onebit_worker_compress(10, 4096, *bad, hpr, None, None) == ob.ONEBIT_EALIGN
    assert "scales_w is not 4-byte aligned" in ob.onebit_last_error()
    assert lib.onebit_lamb_rescale_stats(None, P(4096), P(4096), P(4096), None, None, P(4096),
                                         P(4096), hpr, P(4096), None) == ob.ONEBIT_EINVAL
    # sparse stage
    assert lib.onebit_sparse_worker(10, 4096, 0, P(4096), P(4096), P(4096), P(4096), P(4096), hpr,
                                    None) == ob.ONEBIT_EINVAL                  # nsel = 0
    assert lib.onebit_sparse_worker(10, 4096, 65, P(4096), P(4096), P(4096), P(4096), P(4096), hpr,
                                    None) == ob.ONEBIT_EINVAL                  # nsel > chunk/64
    assert lib.onebit_sparse_worker(10, 4096, 1, P(4096), P(4096), P(4096), None, P(4096), hpr,
                                    None) == ob.ONEBIT_EINVAL                  # m NULL
    assert lib.onebit_sparse_average(6, 2, None, P(4096), None) == ob.ONEBIT_EINVAL   # 6 % 4
    assert lib.onebit_sparse_average(8, 17, None, P(4096), None) == ob.ONEBIT_EUNSUPPORTED
    assert lib.onebit_sparse_average(0, 2, None, None, None) == ob.ONEBIT_OK
    assert lib.onebit_sparse_update(None, 1, P(4096), P(4096), P(4096), P(4096), P(4096), P(4096),
                                    P(4096), hpr, None, None) == ob.ONEBIT_EINVAL



def test_written_arrays_may_not_overlap(ob):
    """A written array that overlaps another argument of the call is refused
    before any launch; read-only arrays may overlap each other."""
    lib = ob._lib
    P = ctypes.c_void_p
    n, C = 8192, 4096                       # 32 KiB of fp32, 2 chunks: 1 KiB of words, 8 B of scales
    base = 1 << 20
    inp, err, bits, scales = base, base + 32768, base + 65536, base + 65536 + 1024
    assert lib.onebit_compress_ef(n, C, P(inp), P(inp + 16384), P(bits), P(scales), None,
                                  None) == ob.ONEBIT_EINVAL
    assert "err overlaps in" in ob.onebit_last_error()
    assert lib.onebit_compress_ef(n, C, P(inp), P(err), P(err + 1020), P(scales), None,
                                  None) == ob.ONEBIT_EINVAL      # bits starts inside err
    assert lib.onebit_compress_ef(n, C, P(inp), P(err), P(bits), P(bits + 1020), None,
                                  None) == ob.ONEBIT_EINVAL      # scales inside bits
    assert lib.onebit_compress_ef(n, C, P(inp), P(err), P(bits), P(scales), P(scales + 4),
                                  None) == ob.ONEBIT_EINVAL      # status inside scales
    assert "status overlaps scales" in ob.onebit_last_error()
    hp = ob.onebit_hparams(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3)
    hpr = ctypes.byref(hp)
    # two workers reading one gradient buffer is allowed; writing one error
    # buffer from both is not
    g = (P * 2)(inp, inp)
    e = (P * 2)(err, err)
    x, m, v = base + 4 * 32768, base + 5 * 32768, base + 6 * 32768
    assert lib.onebit_adam_warmup_step(n, 2, g, P(x), P(inp), P(v), hpr, None) == \
        ob.ONEBIT_EINVAL                                          # m is a gradient buffer
    assert "overlaps grads[0]" in ob.onebit_last_error()
    args = [g, e, P(base + 7 * 32768), P(x), P(m), P(v), None, None, P(bits), P(scales)]
    assert lib.onebit_adam_compressed_step(n, C, 2, *args, hpr, None, None) == ob.ONEBIT_EINVAL
    assert "err_w[1] overlaps err_w[0]" in ob.onebit_last_error()
    arr = (P * 2)(bits, bits)
    sc = (P * 2)(scales, scales)
    assert lib.onebit_average_packed(n, C, 2, arr, sc, P(err), P(bits), P(base + 3 * 32768),
                                     None, None) == ob.ONEBIT_EINVAL   # output over an input
    assert "bits_out overlaps bits_w[0]" in ob.onebit_last_error()
    assert lib.onebit_decompress(n, C, P(bits), P(scales), P(bits - 16), None) == \
        ob.ONEBIT_EINVAL
    assert lib.onebit_sparse_average(64, 2, (P * 2)(inp, inp), P(inp + 128), None) == \
        ob.ONEBIT_EINVAL


HP_BASE = dict(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3, c_min=0.01, c_max=10.0, f_min=0.5,
               f_max=4.0, kappa=0.1)
INF, NAN = float("inf"), float("nan")
# Outside the domains the method gives them ("1-bit LAMB", Background on LAMB:
# beta1, beta2 decay factors; eta keeps the denominator away from 0;
# clip(x, a, b) = min{max{x, a}, b} needs a <= b): every one is EINVAL.
HP_BAD = [("beta1", 1.0), ("beta1", -0.1), ("beta1", NAN), ("beta2", 1.0), ("beta2", 1.5),
          ("beta2", NAN), ("eta", -1e-8), ("eta", INF), ("eta", NAN), ("lr", INF), ("lr", -INF),
          ("lr", NAN), ("weight_decay", -0.1), ("c_min", 20.0), ("c_min", -1.0), ("c_min", NAN),
          ("c_max", NAN), ("c_max", 0.001), ("f_min", 5.0), ("f_min", -0.5), ("f_max", NAN),
          ("f_max", 0.1), ("kappa", -0.1), ("kappa", INF), ("kappa", NAN), ("c_avg_decay", 1.0)]
# Edges inside the domains.
HP_GOOD = [("beta1", 0.0), ("beta2", 0.0), ("eta", 0.0), ("lr", -1e-3), ("c_max", INF),
           ("f_max", INF), ("kappa", 0.0), ("c_min", 10.0), ("f_min", 4.0), ("kappa", 5.0)]


def _hp(ob, **kw):
    return ob.onebit_hparams(**dict(HP_BASE, **kw))


@pytest.mark.parametrize("field,value", HP_BAD)
def test_hparam_outside_domain_is_refused(ob, field, value):
    """Every entry point that takes hp refuses a field outside its domain with
    EINVAL before it enqueues anything.  The calls pass n = 0 (or NULL
    tables), so nothing could be launched even if the check let them
    through."""
    lib = ob._lib
    P = ctypes.c_void_p
    hpr = ctypes.byref(_hp(ob, **{field: value}))
    name = field.split("_")[0]
    calls = [
        lambda: lib.onebit_worker_compress(0, 4096, *[None] * 7, hpr, None, None),
        lambda: lib.onebit_adam_warmup_step(0, 2, None, None, None, None, hpr, None),
        lambda: lib.onebit_adam_compressed_step(0, 4096, 2, *[None] * 10, hpr, None, None),
        lambda: lib.onebit_adam_update(0, 4096, None, None, None, None, None, hpr, None),
        lambda: lib.onebit_sparse_worker(0, 4096, 1, *[None] * 5, hpr, None),
    ]
    for call in calls:
        assert call() == ob.ONEBIT_EINVAL, field
        assert name in ob.onebit_last_error() or "clip bounds" in ob.onebit_last_error() or \
            "soft thresholds" in ob.onebit_last_error(), ob.onebit_last_error()
    # and through the binding (argument marshalling only: the library refuses)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_worker_compress(0, 4096, None, None, None, None, None, None, None,
                                  _hp(ob, **{field: value}), None, 0)
    assert ei.value.code == ob.ONEBIT_EINVAL


@pytest.mark.parametrize("field,value", HP_GOOD)
def test_hparam_domain_edges_are_accepted(ob, field, value):
    lib = ob._lib
    hpr = ctypes.byref(_hp(ob, **{field: value}))
    assert lib.onebit_worker_compress(0, 4096, *[None] * 7, hpr, None, None) == ob.ONEBIT_OK
    assert lib.onebit_adam_warmup_step(0, 2, None, None, None, None, hpr, None) == ob.ONEBIT_OK


def test_invalid_struct_reported_before_the_adam_mode_refusal(ob):
    """A struct that is invalid and also asks for weight decay in the 1-bit
    Adam mode is reported as invalid (EINVAL), not as unsupported."""
    lib = ob._lib
    hp = _hp(ob, beta1=1.0, weight_decay=0.01)
    assert lib.onebit_adam_warmup_step(0, 2, None, None, None, None, ctypes.byref(hp), None) == \
        ob.ONEBIT_EINVAL
    hp = _hp(ob, weight_decay=0.01)
    assert lib.onebit_adam_warmup_step(0, 2, None, None, None, None, ctypes.byref(hp), None) == \
        ob.ONEBIT_EUNSUPPORTED


def test_ceiling_library_loads_without_a_gpu():
    """The pure-traffic ceiling kernels bench.py times beside the step: the
    library loads, exports its three entry points and refuses bad arguments
    before any launch (n = 0 launches nothing)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "communication_compressed_optimizer_amd",
                                   "libonebit_ceiling.so"))
    P = ctypes.c_void_p
    for fn in ("onebit_ceiling_read", "onebit_ceiling_copy", "onebit_ceiling_phase1"):
        assert hasattr(lib, fn)
    lib.onebit_ceiling_read.argtypes = [ctypes.c_int64, P, P, P]
    lib.onebit_ceiling_copy.argtypes = [ctypes.c_int64, P, P, P]
    lib.onebit_ceiling_phase1.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P, P, P, P, P,
                                          ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32, P]
    assert lib.onebit_ceiling_read(-1, P(16), P(16), None) == 1
    assert lib.onebit_ceiling_read(4095, P(16), P(16), None) == 0       # no whole chunk
    assert lib.onebit_ceiling_copy(100, None, P(16), None) == 1
    arr = (P * 2)(16, 16)
    assert lib.onebit_ceiling_phase1(4096, 17, P(16), arr, arr, None, P(16), P(16), P(16), P(16),
                                     0, 0, 0, None) == 1                   # W > 16
    assert lib.onebit_ceiling_phase1(4096, 2, P(16), arr, arr, None, P(16), P(16), P(16), P(16),
                                     0, 3, 0, None) == 1                   # mode 3
    assert lib.onebit_ceiling_phase1(4096, 2, P(16), arr, arr, None, P(16), P(16), P(16), P(16),
                                     0, 0, 200000, None) == 1              # more LDS than a CU has
    assert lib.onebit_ceiling_phase1(4095, 2, P(16), arr, arr, None, P(16), P(16), P(16), P(16),
                                     0, 0, 0, None) == 0


def test_warmup_carry_argument_checks(ob):
    """The carried warmup needs its x_sq array: NULL is refused before the
    table is looked at (no GPU needed)."""
    lib = ob._lib
    P = ctypes.c_void_p
    hp = _hp(ob)
    assert lib.onebit_lamb_warmup_step_carry(P(16), 2, None, None, None, None, None, None, None, 0,
                                             ctypes.byref(hp), None, None, None) == ob.ONEBIT_EINVAL
    assert "x_sq is NULL" in ob.onebit_last_error()
