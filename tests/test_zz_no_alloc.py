"""onebit_lamb_compressed_step_noalloc, the compression step that allocates
nothing (its workspace is the library's static per-device scratch), against
onebit_lamb_compressed_step with a caller's workspace, through the C ABI.

Two calls in a row on the scratch, the second on a smaller table than the
first, every output bit for bit (the step's own arithmetic is shared, so the
bar is exact); then the norm-ratio reading (which uses another region of the
scratch) and packed momentum; and a table whose workspace would exceed the
scratch is refused before anything is launched."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import communication_compressed_optimizer_amd as ob  # noqa: E402
from synth.workloads import Workload  # noqa: E402

from tests.harness import DevRun  # noqa: E402

LARGE = [30522 * 16, 1, 4095, 4097, 100, 8192, 17, 1024 * 1024, 3] * 3     # 4.6 M elements
SMALL = [5, 7, 11, 13] * 40 + [2048 * 3 + 1]


def _noalloc_step(r, step, packed=False):
    r.x_sq_valid = 0
    r.fill_grads(step)
    ob.onebit_lamb_compressed_step_noalloc(r.table, r.wl.W, r.g, r.e, r.err_s, r.x,
                                           None if packed else r.m, r.v, r.vf, r.c_avg, r.f_prev,
                                           r.c_out, r.bits_w, r.scales_w, r.bits_s, r.scales_s,
                                           r.hp, r.status)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _same(a, b, packed=False):
    names = ["x", "vf", "err_s", "f_prev", "c_out", "bits_s", "scales_s"] + \
        ([] if packed else ["m"])
    for k in names:
        assert torch.equal(_bits(getattr(a, k)), _bits(getattr(b, k))), k
    for w in range(a.wl.W):
        assert torch.equal(_bits(a.e[w]), _bits(b.e[w])), ("e", w)
        assert torch.equal(a.bits_w[w], b.bits_w[w]), ("bits_w", w)
        assert torch.equal(_bits(a.scales_w[w]), _bits(b.scales_w[w])), ("scales_w", w)


@pytest.mark.parametrize("rho_mode", [ob.ONEBIT_RHO_MAX, ob.ONEBIT_RHO_NORM_RATIO])
def test_noalloc_equals_workspace_step(rho_mode):
    # the first call at W = 8 (the persistent pass A), the second on a smaller
    # table at W = 2 (one workgroup per chunk)
    for numels, W in ((LARGE, 8), (SMALL, 2)):
        wl = Workload("noalloc", numels, W=W, init="frozen")
        a, b = DevRun(wl), DevRun(wl)
        for r in (a, b):
            r.hp.rho_mode = rho_mode
        a.compressed_step(0)
        _noalloc_step(b, 0)
        torch.cuda.synchronize()
        _same(a, b)
        assert int(b.status.item()) == 0


def test_noalloc_packed_momentum():
    wl = Workload("noalloc", SMALL, W=3, init="frozen")
    a, b = DevRun(wl), DevRun(wl)
    a.compressed_step(0)
    _noalloc_step(b, 0)
    for step in (1, 2):
        a.compressed_step(step, packed=True)
        _noalloc_step(b, step, packed=True)
    torch.cuda.synchronize()
    _same(a, b, packed=True)


def test_noalloc_refuses_a_table_beyond_its_scratch():
    """About 1.1 M segments need more than the 16 MiB scratch: refused with
    EUNSUPPORTED before any array is looked at (NULL arrays here)."""
    table = ob.LayerTable([1024 * 1_100_000], 1024)
    ws = table.workspace_size(2)
    assert ws > 16 << 20
    hp = ob.onebit_hparams(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3)
    rc = ob._lib.onebit_lamb_compressed_step_noalloc(
        ctypes.c_void_p(table.handle), 2, *[None] * 14, ctypes.byref(hp), None, None)
    assert rc == ob.ONEBIT_EUNSUPPORTED
    assert "scratch" in ob.onebit_last_error()


def test_noalloc_step_replays_from_a_graph():
    """The callers it is for: captured once in a HIP graph (the scratch
    address was looked up when the table was made, so the capture holds
    kernel launches only) and replayed three times, with eager work and
    synchronizations between the replays; every replay equals an eager
    workspace step bit for bit."""
    wl = Workload("noalloc", SMALL, W=3, init="frozen")
    a, b = DevRun(wl), DevRun(wl)
    for r in (a, b):
        r.fill_grads(0)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ob.onebit_lamb_compressed_step_noalloc(b.table, 3, b.g, b.e, b.err_s, b.x, b.m, b.v,
                                               b.vf, b.c_avg, b.f_prev, b.c_out, b.bits_w,
                                               b.scales_w, b.bits_s, b.scales_s, b.hp, b.status)
    torch.cuda.synchronize()
    for _ in range(3):
        a.compressed_step(0, fill=False)
        g.replay()
        torch.cuda.synchronize()
        _same(a, b)
        a.x.add_(0.0)                       # eager work between the replays
