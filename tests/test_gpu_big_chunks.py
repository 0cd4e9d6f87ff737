"""Chunks longer than 16384 elements (2^15 up to 2^24) on the GPU, against
the oracle.

Such a chunk is one workgroup of 256 threads over its 4096-element blocks,
held in registers at 2^15 and 2^16 and walked twice beyond.  Its scale is the canonical stride-halving tree over the whole
chunk, formed as a pairwise tree over the blocks in bit-reversed order and
then the tree of one block, so signs, scales and errors must equal the
oracle's bit for bit, as for the shorter chunks; a block past the end of
the last chunk adds exact zeros.  The compression steps run as their per-GPU
parts in order (every worker's compression, the server's average, the
statistics, the update), which needs the workers' sign words and scales and,
for 1-bit LAMB, the fp32 momentum; the sparse stage keeps chunks of at most
16384.  Covered: the codec (up to a chunk of 2^24), the LAMB warmup (plain
and with the norm carried), the freeze, the compression step under both rho
rules, the 1-bit Adam mode with fp32 and packed momentum, one GPU's share
equal to the fused step (packed momentum included), the allocation-free
step, and the refusals.
Tables are ragged: tensors shorter than a block, tensors straddling blocks
and chunks, a last chunk that ends inside a block with whole blocks past it.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import communication_compressed_optimizer_amd as ob  # noqa: E402
import oracle  # noqa: E402
from synth.workloads import Workload  # noqa: E402

from tests.harness import (DevRun, HostRun, assert_parity, compare_adam,  # noqa: E402
                           compare_state)
from tests.test_gpu_sharded import Sharded, _assert_equals_fused  # noqa: E402

BIG = [1 << 15, 1 << 16]


def _normals(n, seed, std=1.0):
    return (np.random.default_rng(seed).standard_normal(n) * std).astype(np.float32)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def _table(C):
    """Tensors shorter than a block, equal to and longer than a chunk,
    straddling blocks and chunks, ending half way into the last chunk."""
    return [1, 3, C - 1, C + 1, 100, 2 * C, 17, 4096 + 5, 5 * C + C // 2 + 9]


def _codec(n, C, seed=11):
    K = oracle.num_chunks(n, C)
    inp, err = _normals(n, seed, 1e-3), _normals(n, seed + 1, 1e-4)
    inp[::97] = 0.0
    d_in, d_err = _dev(inp), _dev(err)
    d_bits = torch.full((K * C // 32,), -1, dtype=torch.int32, device="cuda")
    d_sc = torch.full((K,), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ob.onebit_compress_ef(n, C, d_in, d_err, d_bits, d_sc, status)
    bits, scales = oracle.compress_ef(inp, err, C)
    assert np.array_equal(_bits(d_bits), bits)
    assert np.array_equal(_bits(d_sc), scales.view(np.uint32))
    assert np.array_equal(_bits(d_err), err.view(np.uint32))
    # the server's average of W = 3 packed workers, recompressed with its error
    W = 3
    bits_w, scales_w = [], []
    for w in range(W):
        b, s = oracle.compress_ef(_normals(n, seed + 100 + w, 1e-3), np.zeros(n, np.float32), C)
        bits_w.append(b)
        scales_w.append(s)
    err_s = _normals(n, seed + 200, 1e-4)
    d_err_s = _dev(err_s)
    ob.onebit_average_packed(n, C, W, [_dev(b.view(np.int32)) for b in bits_w],
                             [_dev(s) for s in scales_w], d_err_s, d_bits, d_sc, status)
    b, s = oracle.average_packed(bits_w, scales_w, err_s, C)
    assert np.array_equal(_bits(d_bits), b)
    assert np.array_equal(_bits(d_sc), s.view(np.uint32))
    assert np.array_equal(_bits(d_err_s), err_s.view(np.uint32))
    out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ob.onebit_decompress(n, C, d_bits, d_sc, out)
    assert np.array_equal(out.cpu().numpy(), oracle.decompress(b, s, n, C))
    assert int(status.item()) == 0


@pytest.mark.parametrize("C", BIG + [1 << 20])
@pytest.mark.parametrize("n_of", [lambda C: 1, lambda C: C - 1, lambda C: C,
                                  lambda C: 2 * C + 3 * 4096 + 5, lambda C: 3 * C + C // 2],
                         ids=["1", "C-1", "C", "2C+3blk+5", "3.5C"])
def test_codec_big_chunks(C, n_of):
    _codec(n_of(C), C)


def test_codec_chunk_2_24():
    """The longest chunk: one whole chunk of 2^24 and a second that ends one
    element into its second block."""
    _codec((1 << 24) + 4097, 1 << 24, seed=21)


@pytest.mark.parametrize("C,W", [(1 << 15, 1), (1 << 15, 4), (1 << 16, 4), (1 << 20, 2)])
def test_lamb_trajectory_big_chunks(C, W):
    """Three warmup steps (the norm carried for W > 1), the freeze, then
    compression steps under both rho rules, GPU and oracle each on their own
    state."""
    wl = Workload("big", _table(C), W=W, chunk=C, init="fresh", grad_std=0.02)
    d, h = DevRun(wl, carry_norm=W > 1), HostRun(wl)
    step = 0
    for _ in range(3):
        d.warmup_step(step)
        h.warmup_step(step)
        step += 1
    assert_parity(compare_state(d, h, stage="warmup"), "after warmup")
    d.freeze(3)
    h.freeze(3)
    for rho in (ob.ONEBIT_RHO_MAX, ob.ONEBIT_RHO_MAX, ob.ONEBIT_RHO_NORM_RATIO):
        d.hp.rho_mode = h.hp.rho_mode = rho
        d.compressed_step(step)
        h.compressed_step(step)
        step += 1
        assert_parity(compare_state(d, h), f"step {step - 1}, rho mode {rho}")
    assert int(d.status.item()) == 0


def test_many_tensors_in_one_block():
    """Hundreds of tiny tensors inside the first block of a chunk of 2^15,
    then tensors over block and chunk boundaries: the per-block segment
    statistics loop over many tensors."""
    C = 1 << 15
    numels = [1 + (i * 7) % 13 for i in range(400)] + [C + 3, 4096 * 3 + 1, 2 * C + 77]
    wl = Workload("big_tiny", numels, W=3, chunk=C, init="fresh", grad_std=0.02)
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.warmup_step(step)
        h.warmup_step(step)
    assert_parity(compare_state(d, h, stage="warmup"), "after warmup")
    d.freeze(2)
    h.freeze(2)
    for step, rho in ((2, ob.ONEBIT_RHO_MAX), (3, ob.ONEBIT_RHO_NORM_RATIO)):
        d.hp.rho_mode = h.hp.rho_mode = rho
        d.compressed_step(step)
        h.compressed_step(step)
        assert_parity(compare_state(d, h), f"rho mode {rho}")


@pytest.mark.parametrize("C", BIG)
def test_compressed_step_exact_big_chunks(C):
    """From a frozen state the compression step has no order-dependent sum:
    two steps, W = 8, every array exact."""
    wl = Workload("big", _table(C), W=8, chunk=C, init="frozen", grad_std=1e-3)
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.compressed_step(step)
        h.compressed_step(step)
        rep = compare_state(d, h)
        assert_parity(rep, f"step {step}")
        assert rep["x"]["max_abs"] == 0.0


@pytest.mark.parametrize("C", BIG + [1 << 20])
def test_adam_big_chunks(C):
    wl = Workload("big", [3 * C + 4096 + 7], W=4, chunk=C, init="fresh", grad_std=0.02)
    d, h = DevRun(wl), HostRun(wl)
    step = 0
    for _ in range(2):
        d.adam_warmup_step(step)
        h.adam_warmup_step(step)
        step += 1
    for packed in (False, True, True):
        d.adam_compressed_step(step, packed=packed)
        h.adam_compressed_step(step)
        step += 1
        if packed:
            d.m.copy_(d.momentum_from_packed())
        assert_parity(compare_adam(d, h), f"step {step - 1}, packed={packed}")
    assert int(d.status.item()) == 0


@pytest.mark.parametrize("C", BIG)
def test_share_big_chunks(C):
    """One GPU's share entry points equal the fused step bit for bit: fp32
    momentum, then the packed momentum against the fused step's fp32 one
    (the momentum is the server's output either way)."""
    wl = Workload("big", _table(C), W=3, chunk=C, init="frozen")
    f, s = DevRun(wl), DevRun(wl)
    sh = Sharded(s)
    for step in range(3):
        packed = step > 0
        f.fill_grads(step)
        s.fill_grads(step)
        f.compressed_step(step, fill=False)
        sh.step(packed=packed)
        torch.cuda.synchronize()
        _assert_equals_fused(sh, f, packed)


def test_big_chunk_refusals():
    """What chunks over 16384 do not take: the fused LAMB step without the
    workers' sign words or with packed momentum, the sparse stage, and
    chunks past 2^24 or not a power of two."""
    C = 1 << 15
    wl = Workload("big", _table(C), W=2, chunk=C, init="frozen")
    d = DevRun(wl)
    x0 = d.x.clone()
    with pytest.raises(ob.OnebitError) as ei:
        d.compressed_step(0, packed=True)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED
    d2 = DevRun(wl, store_worker_bits=False)
    with pytest.raises(ob.OnebitError) as ei:
        d2.compressed_step(0)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED
    with pytest.raises(ob.OnebitError) as ei:
        d2.adam_compressed_step(0)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED
    with pytest.raises(ob.OnebitError) as ei:
        d.sparse_step(0, 1)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(d.x, x0) and torch.equal(d2.x, x0)     # nothing ran
    for bad in (1 << 25, 3 << 15, (1 << 24) + 64):
        with pytest.raises(ob.OnebitError):
            ob.LayerTable([100], bad)


def test_noalloc_big_chunks():
    """The allocation-free step at chunks of 2^15 and 2^20 equals the step
    with a caller's workspace bit for bit, the second call on a smaller
    table; packed momentum is refused there as in the fused step."""
    from tests.test_zz_no_alloc import _noalloc_step, _same
    for C, numels, W in ((1 << 15, _table(1 << 15), 4), (1 << 20, [5, 3 << 20, 7], 2)):
        wl = Workload("big_noalloc", numels, W=W, chunk=C, init="frozen")
        a, b = DevRun(wl), DevRun(wl)
        for step in range(2):
            a.compressed_step(step)
            _noalloc_step(b, step)
        torch.cuda.synchronize()
        _same(a, b)
        assert int(b.status.item()) == 0
        with pytest.raises(ob.OnebitError) as ei:
            _noalloc_step(b, 2, packed=True)
        assert ei.value.code == ob.ONEBIT_EUNSUPPORTED


@pytest.mark.parametrize("seed", range(12))
def test_random_table_big_chunks(seed):
    """Seeded random tables at chunks of 2^15 to 2^18 (held in registers,
    then walked twice at lr = 5 and 6), random W and variant readings: two
    warmup steps and three compression steps of 1-bit LAMB, or 1-bit Adam
    with packed momentum, against the oracle."""
    r = np.random.default_rng(5000 + seed)
    chunk = int(r.choice([1 << 15, 1 << 16, 1 << 17, 1 << 18]))
    W = int(r.integers(1, 9))
    L = int(r.integers(1, 12))
    numels = []
    for _ in range(L):
        kind = r.random()
        if kind < 0.15:
            numels.append(int(chunk * r.integers(1, 3)))
        elif kind < 0.3:
            numels.append(int(r.integers(1, 8)))
        else:
            numels.append(int(np.exp(r.uniform(0, np.log(2 * chunk)))) + 1)
    wl = Workload("random_big", numels, W=W, chunk=chunk, init="fresh", grad_std=0.02,
                  layer_scaled=bool(r.random() < 0.5), seed=seed)
    d, h = DevRun(wl, carry_norm=seed % 3 == 0), HostRun(wl)
    if seed % 4 != 3:
        variant = dict(rho_mode=int(r.integers(0, 2)), c_avg_decay=float(r.choice([0.0, 0.8])),
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
            d.compressed_step(step)
            h.compressed_step(step)
            assert_parity(compare_state(d, h), f"seed {seed} compression {step}")
    else:
        for step in range(2):
            d.adam_warmup_step(step)
            h.adam_warmup_step(step)
        for step in range(2, 5):
            d.adam_compressed_step(step, packed=step > 2)
            h.adam_compressed_step(step)
            if step > 2:
                d.m.copy_(d.momentum_from_packed())
            assert_parity(compare_adam(d, h), f"seed {seed} adam {step}")
    assert int(d.status.item()) == 0
