"""GPU parity of the SLAMB-style sparse compression stage: the HIP library,
called through its C ABI, against the CPU oracle on the same seeded inputs
and the same seeded block selection.  Every output is element-wise, so
every array must match bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import communication_compressed_optimizer_amd as ob  # noqa: E402
from synth.workloads import Workload, WORKLOADS  # noqa: E402

from tests.harness import (DevRun, HostRun, assert_parity, compare_sparse,  # noqa: E402
                           compare_state)
from tests.test_gpu_workloads import block_windows  # noqa: E402

RAGGED = [4096 * 3 + 100, 1, 777, 2 * 4096, 5000, 3]


@pytest.mark.parametrize("nsel", [1, 5, 64])
@pytest.mark.parametrize("W", [1, 3, 8])
def test_sparse_step_parity(nsel, W):
    wl = Workload("sparse", RAGGED, W=W, init="frozen")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        d.sparse_step(step, nsel)
        h.sparse_step(step, nsel)
        assert_parity(compare_sparse(d, h), f"step {step}")
    assert int(d.status.item()) == 0


@pytest.mark.parametrize("chunk", [1024, 16384])
def test_sparse_other_chunks(chunk):
    wl = Workload("sparse", RAGGED + [3 * chunk + 9], W=4, chunk=chunk, init="frozen")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.sparse_step(step, 2)
        h.sparse_step(step, 2)
        assert_parity(compare_sparse(d, h), f"step {step}")


def test_sparse_after_lamb_warmup():
    """LAMB warmup, freeze, then the sparse stage: GPU and oracle each on
    their own state (the warmup part to its tolerance, the rest exact)."""
    wl = Workload("sparse", RAGGED, W=4, init="fresh", grad_std=0.02)
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        d.warmup_step(step)
        h.warmup_step(step)
    d.freeze(3)
    h.freeze(3)
    assert_parity(compare_state(d, h, stage="warmup"), "freeze")
    # adopt the GPU's warmup result (x and c_avg carry the warmup's
    # order-dependent norms) so that the sparse stage is compared exactly
    h.load_from(d.window(0, wl.N))
    for step in range(3, 8):
        d.sparse_step(step, 4)
        h.sparse_step(step, 4)
        assert_parity(compare_sparse(d, h), f"sparse {step}")


def test_sparse_worker_values_optional():
    wl = Workload("sparse", RAGGED, W=3, init="frozen")
    a, b = DevRun(wl), DevRun(wl, store_worker_bits=False)
    a.sparse_step(0, 3)
    b.sparse_step(0, 3)
    for k in ("x", "m", "vf", "vals_s"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k


def test_sparse_argument_checks():
    wl = Workload("sparse", [4096], W=2, init="frozen")
    d = DevRun(wl)
    d.sparse_step(0, 1)
    sel = d.sel
    for nsel in (0, 65):
        with pytest.raises(ob.OnebitError) as ei:
            ob.onebit_sparse_compressed_step(d.table, 2, nsel, sel, d.g, d.e, d.x, d.m, d.v, d.vf,
                                             d.c_avg, None, d.vals_s, d.hp)
        assert ei.value.code == ob.ONEBIT_EINVAL
    hp = ob.onebit_hparams(**{f: getattr(d.hp, f) for f, _ in ob.onebit_hparams._fields_})
    hp.weight_decay = 0.01
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_sparse_compressed_step(d.table, 2, 1, sel, d.g, d.e, d.x, d.m, d.v, d.vf,
                                         d.c_avg, None, d.vals_s, hp)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED


def test_sparse_bert_large_windows():
    """The BERT-Large table, W = 8, 1/64 of the blocks per step: two steps at
    full size, windows checked against the oracle."""
    base = WORKLOADS["bert_large"]
    wl = Workload("sparse_bert_large", base.numels, W=8, init="frozen")
    d = DevRun(wl)
    hosts = [HostRun(wl, lo, hi) for lo, hi in block_windows(wl, chunks=48)]
    for step in range(2):
        d.sparse_step(step, 1)
        for h in hosts:
            h.sparse_step(step, 1)
            assert_parity(compare_sparse(d, h), f"step {step} window [{h.lo}, {h.hi})")
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nsel", [1, 7])
def test_sparse_update_reads_momentum_on_the_selection_only(nsel):
    """onebit_sparse_update needs the previous momentum only where a block
    was transmitted: with m set to NaN everywhere else, every output is the
    same bit for bit (m ends 0 there either way)."""
    wl = Workload("sparse", RAGGED, W=2, init="frozen")
    C, K, N = wl.chunk, wl.K, wl.N
    d = DevRun(wl)
    sel_h = wl.selection(0)
    sel = torch.from_numpy(sel_h).cuda()
    vals = torch.randn(K * nsel * 64, device="cuda") * 1e-3
    on = np.zeros(K * C, bool)                       # the selection, chunk by chunk
    for k in range(K):
        b0 = int(sel_h[k]) % (C // 64)
        for j in range(nsel):
            b = (b0 + j) % (C // 64)
            on[k * C + b * 64:k * C + (b + 1) * 64] = True
    on = torch.from_numpy(on[:N]).cuda()
    outs = []
    for poison in (False, True):
        x, m, vf = d.x.clone(), d.m.clone(), d.vf.clone()
        if poison:
            m[~on] = float("nan")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ob.onebit_sparse_update(d.table, nsel, sel, vals, x, m, d.v, vf, d.c_avg, d.hp, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        outs.append((x, m, vf))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert not torch.any(outs[1][1][~on])                 # m is 0 off the selection
