"""The entry points under HIP graph capture: every call only enqueues kernels
on the given stream (no allocation, no memset, no host synchronization), so
a captured step replays as the eager step.  Each replay is checked against
an eager run of the same step, with eager work and synchronizations between
the replays."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from synth.workloads import Workload  # noqa: E402

from tests.harness import DevRun  # noqa: E402
from tests.test_gpu_sharded import Sharded  # noqa: E402

TABLE = [4096 * 3 + 100, 1, 777, 2 * 4096, 5000, 3]
STATE = ("x", "m", "v", "vf", "err_s", "bits_s", "scales_s", "c_sum", "c_avg", "f_prev", "c_out")


def _same(a, b, extra=()):
    torch.cuda.synchronize()
    for k in STATE + tuple(extra):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    for w in range(a.wl.W):
        assert torch.equal(a.e[w], b.e[w]), f"e{w}"
        if a.bits_w is not None:
            assert torch.equal(a.bits_w[w], b.bits_w[w]), f"bits_w{w}"


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("W", [4, 8])
def test_lamb_steps_replay_as_eager(W):
    wl = Workload("graph", TABLE, W=W, init="fresh", grad_std=0.02)
    a, b = DevRun(wl), DevRun(wl)
    for r in (a, b):
        r.fill_grads(0)
    gw = _capture(lambda: b.warmup_step(0, fill=False))
    for _ in range(3):
        a.warmup_step(0, fill=False)
        gw.replay()
        _same(a, b)
        a.x.add_(0.0)                       # eager work between the replays
    for r in (a, b):
        r.freeze(3)
    gc = _capture(lambda: b.compressed_step(0, fill=False))
    gp = _capture(lambda: b.compressed_step(0, fill=False, packed=True))
    a.compressed_step(0, fill=False)
    gc.replay()
    _same(a, b)
    for _ in range(3):
        a.compressed_step(0, fill=False, packed=True)
        gp.replay()
        _same(a, b)
        torch.cuda.synchronize()


def test_carried_warmup_replays_as_eager():
    """The warmup step with the parameters' squared norm carried: after one
    eager step has written x_sq, the carried step is captured and replayed
    three times against the eager carried step."""
    wl = Workload("graph", TABLE, W=3, init="fresh", grad_std=0.02)
    a, b = DevRun(wl, carry_norm=True), DevRun(wl, carry_norm=True)
    for r in (a, b):
        r.fill_grads(0)
        r.warmup_step(0, fill=False)        # x_sq written; later steps skip reading x
    g = _capture(lambda: b.warmup_step(1, fill=False))
    for _ in range(3):
        a.warmup_step(1, fill=False)
        g.replay()
        _same(a, b, extra=("x_sq",))
        a.x.add_(0.0)


def test_adam_and_sparse_steps_replay_as_eager():
    wl = Workload("graph", [5 * 4096 + 17], W=3, init="frozen")
    a, b = DevRun(wl), DevRun(wl)
    for r in (a, b):
        r.fill_grads(0)
    ga = _capture(lambda: b.adam_compressed_step(0, fill=False))
    for _ in range(3):
        a.adam_compressed_step(0, fill=False)
        ga.replay()
        _same(a, b)
    wl2 = Workload("graph", TABLE, W=3, init="frozen")
    c, d = DevRun(wl2), DevRun(wl2)
    for r in (c, d):
        r.fill_grads(0)
        r.sparse_step(0, 2, fill=False)     # allocates the value buffers and selection
    gs = _capture(lambda: d.ob.onebit_sparse_compressed_step(
        d.table, 3, 2, d.sel, d.g, d.e, d.x, d.m, d.v, d.vf, d.c_avg, d.vals_w, d.vals_s, d.hp,
        d.status))
    for _ in range(3):
        c.ob.onebit_sparse_compressed_step(c.table, 3, 2, c.sel, c.g, c.e, c.x, c.m, c.v, c.vf,
                                           c.c_avg, c.vals_w, c.vals_s, c.hp, c.status)
        gs.replay()
        _same(c, d, extra=("vals_s",))


def test_share_steps_replay_as_eager():
    """One GPU's share (worker compressions, the served chunk ranges, the
    replicas' statistics and updates) captured once and replayed."""
    wl = Workload("graph", TABLE, W=3, init="frozen")
    a, b = DevRun(wl), DevRun(wl)
    for r in (a, b):
        r.fill_grads(0)
    sa, sb = Sharded(a), Sharded(b)
    g = _capture(lambda: sb.step())
    for _ in range(3):
        sa.step()
        g.replay()
        torch.cuda.synchronize()
        for p in sa.replicas:
            for k in ("x", "m", "vf", "f_prev", "c_out"):
                assert torch.equal(getattr(sa, k)[p], getattr(sb, k)[p]), (p, k)
        for k in ("err_s", "bits_s", "scales_s"):
            assert torch.equal(getattr(sa, k), getattr(sb, k)), k
        for w in range(wl.W):
            assert torch.equal(sa.e[w], sb.e[w]) and torch.equal(sa.bits_w[w], sb.bits_w[w])
        a.x.add_(0.0)                       # eager work between the replays

