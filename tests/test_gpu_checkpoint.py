"""Checkpoint and resume inside the compression stage.

The error buffers are state: error compensation feeds each step's
compression error into the next step ("1-bit LAMB" page, Related work), and
the rescale carries f_prev and the fresh variance from step to step (Section
4 summary).  After the warmup, the freeze and two compression steps every
one of them has moved away from its initial value.  The whole state is then
written to disk with torch.save, loaded with torch.load(weights_only=True)
into freshly allocated, NaN-poisoned buffers, and stepped on: the resumed run
must equal the uninterrupted one bit for bit, and the oracle (run from the
start on its own state) to the parity bar.  With packed momentum the
momentum is the server's packed output (bits_s, scales_s), which the
checkpoint then carries instead of m.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from synth.workloads import Workload  # noqa: E402

from tests.harness import DevRun, HostRun, assert_parity, compare_state  # noqa: E402

TABLE = [1, 3, 4095, 4097, 100, 8192, 17, 256 * 256, 1000 * 64]

# the compression stage's state; with packed momentum bits_s/scales_s are
# the momentum and m is not part of it
STATE = ("x", "m", "v", "vf", "err_s", "c_sum", "c_avg", "f_prev", "bits_s", "scales_s")


def _state(run, packed):
    d = {k: getattr(run, k) for k in STATE if not (packed and k == "m")}
    d["e"] = list(run.e)
    return d


def _save(run, path, packed, step):
    blob = {k: (v.cpu() if not isinstance(v, list) else [t.cpu() for t in v])
            for k, v in _state(run, packed).items()}
    blob["step"] = step
    torch.save(blob, path)


def _load(run, path, packed):
    blob = torch.load(path, weights_only=True)
    for k, v in _state(run, packed).items():
        if isinstance(v, list):
            for dst, src in zip(v, blob[k]):
                dst.copy_(src)
        else:
            v.copy_(blob[k])
    return blob["step"]


def _poison(run):
    """Every array of a fresh run set to NaN (or all-ones words), so that a
    value the checkpoint failed to restore cannot pass for a right one."""
    for k in ("x", "m", "v", "vf", "err_s", "c_sum", "c_avg", "f_prev", "c_out", "scales_s"):
        getattr(run, k).fill_(float("nan"))
    run.bits_s.fill_(-1)
    for t in run.e:
        t.fill_(float("nan"))
    for t in run.bits_w:
        t.fill_(-1)
    for t in run.scales_w:
        t.fill_(float("nan"))


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("W", [1, 3, 8])
def test_resume_inside_compression_stage(tmp_path, packed, W):
    wl = Workload("checkpoint", TABLE, W=W, init="fresh", grad_std=0.02)
    a, h = DevRun(wl), HostRun(wl)
    step = 0
    for _ in range(3):
        a.warmup_step(step)
        h.warmup_step(step)
        step += 1
    a.freeze(3)
    h.freeze(3)
    for _ in range(2):
        # the first compression step needs the warmup's fp32 m; with packed
        # momentum every later one reads bits_s/scales_s instead
        a.compressed_step(step, packed=packed and step > 3)
        h.compressed_step(step)
        step += 1
    torch.cuda.synchronize()
    # the carried state has moved away from its starting values (with one
    # worker the server recompresses a constant-magnitude chunk, exactly, so
    # its error stays 0)
    assert all(float(t.abs().max()) > 0 for t in a.e)
    assert (float(a.err_s.abs().max()) > 0) == (W > 1)
    assert float((a.f_prev - 1).abs().max()) > 0
    path = tmp_path / "state.pt"
    _save(a, path, packed, step)

    b = DevRun(wl)
    _poison(b)
    assert _load(b, path, packed) == step
    for _ in range(3):
        for r in (a, b):
            r.compressed_step(step, packed=packed)
        h.compressed_step(step)
        step += 1
        torch.cuda.synchronize()
        names = ["x", "vf", "err_s", "f_prev", "c_out", "bits_s", "scales_s"] + \
            ([] if packed else ["m"])
        for k in names:
            assert torch.equal(_bits(getattr(a, k)), _bits(getattr(b, k))), (k, step)
        for w in range(W):
            assert torch.equal(_bits(a.e[w]), _bits(b.e[w])), ("e", w, step)
            assert torch.equal(a.bits_w[w], b.bits_w[w]) and \
                torch.equal(_bits(a.scales_w[w]), _bits(b.scales_w[w])), ("worker", w, step)
        # and the resumed run against the oracle, which never stopped
        if packed:
            b.m.copy_(b.momentum_from_packed())
        assert_parity(compare_state(b, h), f"resumed, step {step}")
    assert int(b.status.item()) == 0


def test_resume_from_raw_files(tmp_path):
    """The same checkpoint written as raw little-endian arrays (numpy .npy,
    no pickling) and read back: the state is nothing but its arrays."""
    wl = Workload("checkpoint", TABLE, W=2, init="frozen")
    a = DevRun(wl)
    for step in range(2):
        a.compressed_step(step)
    torch.cuda.synchronize()
    arrays = {k: v for k, v in _state(a, False).items() if k != "e"}
    for k, v in arrays.items():
        np.save(tmp_path / f"{k}.npy", v.cpu().numpy())
    for w, t in enumerate(a.e):
        np.save(tmp_path / f"e{w}.npy", t.cpu().numpy())
    b = DevRun(wl)
    _poison(b)
    for k in arrays:
        getattr(b, k).copy_(torch.from_numpy(np.load(tmp_path / f"{k}.npy", allow_pickle=False)))
    for w in range(wl.W):
        b.e[w].copy_(torch.from_numpy(np.load(tmp_path / f"e{w}.npy", allow_pickle=False)))
    for step in range(2, 4):
        for r in (a, b):
            r.compressed_step(step)
    torch.cuda.synchronize()
    for k in ("x", "m", "vf", "err_s", "f_prev", "bits_s", "scales_s"):
        assert torch.equal(_bits(getattr(a, k)), _bits(getattr(b, k))), k
