"""Seeded random tables against the oracle: tensor counts, sizes (including
ones that end exactly on a chunk boundary), chunk sizes, worker counts,
modes (1-bit LAMB, 1-bit Adam, the sparse stage, and one GPU's share of a
W-GPU LAMB step) and variant readings drawn from a fixed seed, a short
trajectory each.  The bar is the one of the other parity tests."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import communication_compressed_optimizer_amd as ob  # noqa: E402
from synth.workloads import Workload  # noqa: E402

from tests.harness import (DevRun, HostRun, assert_parity, compare_adam,  # noqa: E402
                           compare_sparse, compare_state)
from tests.test_gpu_sharded import Sharded  # noqa: E402


def _table(r, chunk):
    L = int(r.integers(1, 24))
    sizes = []
    for _ in range(L):
        kind = r.random()
        if kind < 0.15:
            sizes.append(int(chunk * r.integers(1, 4)))                 # whole chunks
        elif kind < 0.3:
            sizes.append(int(r.integers(1, 8)))                         # tiny
        else:
            sizes.append(int(np.exp(r.uniform(0, np.log(3 * chunk)))) + 1)
    return sizes


@pytest.mark.parametrize("seed", range(60))
def test_random_table(seed):
    r = np.random.default_rng(1000 + seed)
    chunk = int(r.choice([64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]))
    W = int(r.integers(1, 17))
    numels = _table(r, chunk)
    mode = ["lamb", "lamb", "adam", "sparse", "share"][seed % 5]
    wl = Workload("random", numels, W=W, chunk=chunk, init="fresh", grad_std=0.02,
                  layer_scaled=bool(r.random() < 0.5), seed=seed)
    d, h = DevRun(wl, carry_norm=seed % 3 == 0), HostRun(wl)
    if mode == "lamb":
        variant = dict(rho_mode=int(r.integers(0, 2)),
                       c_avg_decay=float(r.choice([0.0, 0.8])),
                       weight_decay=float(r.choice([0.0, 0.01])))
        for run in (d, h):
            for k, v in variant.items():
                setattr(run.hp, k, v)
        bias = bool(r.random() < 0.5)
        for step in range(2):
            for run in (d, h):
                run.hp.bias_step = step + 1 if bias else 0
                run.warmup_step(step)
            assert_parity(compare_state(d, h, stage="warmup"), f"seed {seed} warmup {step}")
        for run in (d, h):
            run.hp.bias_step = 0
            run.freeze(2)
        for step in range(2, 5):
            d.compressed_step(step, packed=step > 2 and seed % 2 == 1)
            if step > 2 and seed % 2 == 1:
                d.m.copy_(d.momentum_from_packed())
            h.compressed_step(step)
            assert_parity(compare_state(d, h), f"seed {seed} compression {step}")
    elif mode == "adam":
        n = wl.N
        for step in range(2):
            d.adam_warmup_step(step)
            h.adam_warmup_step(step)
        for step in range(2, 5):
            d.adam_compressed_step(step)
            h.adam_compressed_step(step)
            assert_parity(compare_adam(d, h), f"seed {seed} adam {step} (n={n})")
    elif mode == "share":
        # one GPU's share on W simulated GPUs against the oracle, from a frozen state
        wlf = Workload("random", numels, W=W, chunk=chunk, init="frozen", grad_std=1e-3,
                       layer_scaled=bool(r.random() < 0.5), seed=seed)
        d, h = DevRun(wlf), HostRun(wlf)
        d.hp.rho_mode = h.hp.rho_mode = int(r.integers(0, 2))
        sh = Sharded(d, replicas=sorted({0, W - 1}))
        for step in range(3):
            d.fill_grads(step)
            sh.step()
            h.compressed_step(step)
            for p in sh.replicas:
                assert_parity(compare_state(None, h, d=sh.window(p)), f"seed {seed} share {step}")
    else:
        nsel = int(r.integers(1, chunk // 64 + 1))
        for step in range(2):
            d.warmup_step(step)
            h.warmup_step(step)
        d.freeze(2)
        h.freeze(2)
        h.load_from(d.window(0, wl.N))
        for step in range(2, 5):
            d.sparse_step(step, nsel)
            h.sparse_step(step, nsel)
            assert_parity(compare_sparse(d, h), f"seed {seed} sparse {step} (nsel={nsel})")
    assert int(d.status.item()) == 0, f"seed {seed}: status {int(d.status.item())}"
    assert ob.onebit_last_error() == ""
