"""GPU parity of the 1-bit Adam mode: the HIP library, called through its C
ABI, against the CPU oracle on the same seeded inputs.

1-bit Adam has no per-tensor quantity, so every output -- parameters,
moments, errors, packed signs and scales -- must match bit for bit.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import communication_compressed_optimizer_amd as ob  # noqa: E402
from synth.workloads import Workload, WORKLOADS  # noqa: E402

from tests.harness import DevRun, HostRun, assert_parity, compare_adam  # noqa: E402
from tests.test_gpu_workloads import block_windows  # noqa: E402

# flat sizes: several full chunks plus a ragged tail, an exact multiple of
# the chunk, a single partial chunk, a single element
SIZES = [3 * 4096 + 777, 5 * 4096, 1000, 1]


def _flat(n, W, chunk=4096, init="fresh"):
    return Workload("adam", [n], W=W, chunk=chunk, init=init,
                    grad_std=0.02 if init == "fresh" else 1e-3)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("W", [1, 3, 8, 16])
def test_adam_warmup_parity(n, W):
    wl = _flat(n, W)
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        d.adam_warmup_step(step)
        h.adam_warmup_step(step)
        assert_parity(compare_adam(d, h), f"warmup step {step}")


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("W", [1, 3, 8, 16])
def test_adam_compressed_parity(n, W):
    """From a frozen state: two compression steps."""
    wl = _flat(n, W, init="frozen")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.adam_compressed_step(step)
        h.adam_compressed_step(step)
        assert_parity(compare_adam(d, h), f"step {step}")
    assert int(d.status.item()) == 0


@pytest.mark.parametrize("chunk", [1024, 2048, 8192, 16384])
def test_adam_compressed_other_chunks(chunk):
    wl = _flat(3 * chunk + 9, 4, chunk=chunk, init="frozen")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.adam_compressed_step(step)
        h.adam_compressed_step(step)
        assert_parity(compare_adam(d, h), f"step {step}")


def test_adam_trajectory():
    """Fresh state: 4 Adam warmup steps, then (errors zero, v frozen) 6
    compression steps, GPU and oracle each on their own state."""
    wl = _flat(7 * 4096 + 1234, 4)
    d, h = DevRun(wl), HostRun(wl)
    step = 0
    for _ in range(4):
        d.adam_warmup_step(step)
        h.adam_warmup_step(step)
        step += 1
    assert_parity(compare_adam(d, h), "after warmup")
    for _ in range(6):
        d.adam_compressed_step(step)
        h.adam_compressed_step(step)
        assert_parity(compare_adam(d, h), f"compression {step}")
        step += 1
    assert int(d.status.item()) == 0


def test_adam_worker_outputs_optional():
    """Without worker sign/scale arrays the step computes the same state."""
    wl = _flat(3 * 4096 + 5, 3, init="frozen")
    a, b = DevRun(wl), DevRun(wl, store_worker_bits=False)
    a.adam_compressed_step(0)
    b.adam_compressed_step(0)
    for k in ("x", "m", "err_s", "bits_s", "scales_s"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    for w in range(3):
        assert torch.equal(a.e[w], b.e[w])


def test_adam_empty_is_a_no_op():
    wl = _flat(4096, 2, init="frozen")
    d = DevRun(wl)
    x0 = d.x.clone()
    ob.onebit_adam_warmup_step(0, 2, d.g, d.x, d.m, d.v, d.hp)
    ob.onebit_adam_compressed_step(0, 4096, 2, d.g, d.e, d.err_s, d.x, d.m, d.v, d.bits_w,
                                   d.scales_w, d.bits_s, d.scales_s, d.hp, d.status)
    torch.cuda.synchronize()
    assert torch.equal(d.x, x0)


def test_adam_status_flags():
    wl = _flat(2 * 4096 + 17, 2, init="frozen")
    d = DevRun(wl)
    d.fill_grads(0)
    d.g[1][4096 + 3] = float("inf")
    d.adam_compressed_step(0, fill=False)
    torch.cuda.synchronize()
    st = int(d.status.item())
    assert st & ob.ONEBIT_STATUS_NONFINITE_WORKER and st & ob.ONEBIT_STATUS_NONFINITE_SERVER


def test_adam_binding_rejects_bad_arguments():
    wl = _flat(4096, 2, init="frozen")
    d = DevRun(wl)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_adam_compressed_step(4096, 3000, 2, d.g, d.e, d.err_s, d.x, d.m, d.v, None,
                                       None, d.bits_s, d.scales_s, d.hp)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_adam_warmup_step(4095, 2, d.g, d.x[1:], d.m, d.v, d.hp)
    assert ei.value.code == ob.ONEBIT_EALIGN


def test_adam_bert_large_windows():
    """BERT-Large's 333,563,904 parameters as one flat buffer, W = 8: one
    Adam warmup step and two compression steps at full size, windows
    checked against the oracle."""
    base = WORKLOADS["bert_large"]
    wl = Workload("adam_bert_large", base.numels, W=8, init="fresh", grad_std=1e-3)
    d = DevRun(wl)
    hosts = [HostRun(wl, lo, hi) for lo, hi in block_windows(wl, chunks=48)]
    d.adam_warmup_step(0)
    for h in hosts:
        h.adam_warmup_step(0)
    for step in (1, 2):
        d.adam_compressed_step(step)
        for h in hosts:
            h.adam_compressed_step(step)
            assert_parity(compare_adam(d, h), f"step {step} window [{h.lo}, {h.hi})")
    assert int(d.status.item()) == 0
    del d
    torch.cuda.empty_cache()
