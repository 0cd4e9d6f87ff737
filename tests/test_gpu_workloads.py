"""GPU parity on the full-size workloads.

The GPU runs the whole table; the oracle runs windows of it that start on a
chunk boundary (chunk-local state is exact there; per-tensor values are
compared for the tensors wholly inside a window).  Inputs of both sides come
from the same seeded generator (device fill on the GPU, host fill for the
oracle, bit-identical by construction and by test_synth_device_matches_host).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from synth.workloads import WORKLOADS  # noqa: E402

from tests.harness import DevRun, HostRun, assert_parity, compare_state  # noqa: E402


def block_windows(wl, chunks=120):
    """Windows of `chunks` chunks around the small tensors (bias, LayerNorm)
    of the first and of the last encoder block (the latter reaching the
    ragged last chunk), plus the first chunks."""
    C, K = wl.chunk, wl.K
    off = wl.offsets
    first_block = 1 if wl.L % 16 == 1 else 0   # an embedding precedes the blocks
    i_bo = first_block + 7          # Wo bias of the first block
    i_b2 = wl.L - 3                 # b2 of the last block
    wins = [(0, min(K, 64))]
    for i in (i_bo, i_b2):
        k = int(off[i]) // C
        lo = max(0, k - chunks // 2)
        wins.append((lo, min(K, lo + chunks)))
    return [(lo * C, min(wl.N, hi * C)) for lo, hi in sorted(set(wins))]


def test_bert_large_step():
    """BERT-Large table, W = 8: the configuration's 10 compression steps, GPU
    and oracle each on their own state, windows checked after every step."""
    wl = WORKLOADS["bert_large"]
    d = DevRun(wl)
    hosts = [HostRun(wl, lo, hi) for lo, hi in block_windows(wl)]
    for step in range(wl.compression_steps):
        d.compressed_step(step)
        torch.cuda.synchronize()
        for h in hosts:
            h.compressed_step(step)
            assert_parity(compare_state(d, h), f"step {step} window [{h.lo}, {h.hi})")
    assert int(d.status.item()) == 0


def covering_windows(wl, chunks=16384):
    """Chunk-aligned windows of at most `chunks` chunks that together cover
    every chunk, each starting at the first chunk of the first tensor the
    previous window does not hold whole, so that every tensor lies wholly
    inside some window (tensors are shorter than a window)."""
    C, K, N = wl.chunk, wl.K, wl.N
    off = wl.offsets
    wins, lo = [], 0
    while True:
        hi = min(K, lo + chunks)
        wins.append((lo, hi))
        if hi == K:
            break
        l = int(np.searchsorted(off, hi * C, side="right")) - 1   # tensor holding element hi*C
        lo = int(off[l]) // C
    return [(lo * C, min(N, hi * C)) for lo, hi in wins]


def whole_buffer_parity(d, wl, run_host, stage="compression", chunks=8192, threads=4):
    """Compare the GPU state d with the oracle over the WHOLE buffer.  The
    oracle runs covering_windows(wl, chunks), each window on its own state
    (run_host(h) steps it), on a few threads: the oracle and the input
    generator are C calls that release the interpreter lock, and a few
    windows at a time keep host memory bounded.  Every chunk-local array is
    compared element by element, and the per-tensor values on every tensor
    (each lies wholly inside some window)."""
    C, off = wl.chunk, wl.offsets
    wins = covering_windows(wl, chunks)
    covered = np.zeros(wl.K, bool)
    whole = np.zeros(wl.L, bool)
    for lo, hi in wins:
        covered[lo // C:-(-hi // C)] = True
        whole |= (off[:-1] >= lo) & (off[1:] <= hi)
    assert covered.all() and whole.all()
    torch.cuda.synchronize()

    def one(win):
        lo, hi = win
        h = HostRun(wl, lo, hi)
        run_host(h)
        rep = compare_state(d, h, stage=stage)
        return lo, hi, rep, -(-hi // C) - lo // C, h.full.size

    n_chunks = n_tensors = 0
    with ThreadPoolExecutor(max(1, min(threads, os.cpu_count() or 1))) as ex:
        for lo, hi, rep, nc, nt in ex.map(one, wins):
            assert_parity(rep, f"window [{lo}, {hi})")
            last = f"bits_w{wl.W - 1}"
            if last in rep:                         # every worker sign word of the window
                assert rep[last]["n"] == nc * C // 32
            n_chunks += nc
            n_tensors += nt
    assert n_chunks >= wl.K and n_tensors >= wl.L
    return wins


@pytest.mark.timeout(900)
def test_bert_large_whole_buffer():
    """BERT-Large table, W = 8, two compression steps (the second one
    compensating the first one's errors), compared against the oracle over
    the WHOLE buffer: every chunk's signs, scales and errors of all eight
    workers and of the server, m, v_fresh, and the parameters and per-tensor
    coefficients of every tensor.  Under error feedback a wrong sign anywhere
    is carried into every later step ("1-bit LAMB" page, Related work), so
    no chunk is left to sampling."""
    wl = WORKLOADS["bert_large"]
    d = DevRun(wl)
    for step in range(2):
        d.compressed_step(step)
    torch.cuda.synchronize()
    assert int(d.status.item()) == 0

    def run_host(h):
        for step in range(2):
            h.compressed_step(step)

    whole_buffer_parity(d, wl, run_host, threads=8)


@pytest.mark.timeout(900)
def test_mixed_warmup_whole_buffer():
    """BERT-Large table with per-tensor gradient scales, W = 8: two LAMB
    warmup steps, the second with the parameters' squared norm carried over
    from the first, compared against the oracle over the whole buffer: m and
    v of every element bit for bit, and the parameters, trust ratios and
    their running sums of every tensor within the bar (the segment sums of
    the carried norm are indexed deep into the table here)."""
    wl = WORKLOADS["mixed"]
    d = DevRun(wl, carry_norm=True)
    for step in range(2):
        d.warmup_step(step)
    torch.cuda.synchronize()
    assert int(d.status.item()) == 0

    def run_host(h):
        for step in range(2):
            h.warmup_step(step)

    whole_buffer_parity(d, wl, run_host, stage="warmup")


@pytest.mark.timeout(900)
def test_mixed_switch_whole_buffer():
    """The Mixed configuration through the switch, over the WHOLE buffer: its
    20 LAMB warmup steps (the parameters' squared norm carried from step to
    step on the GPU), the freeze, then two compression steps with the
    adaptive layerwise rescale, against the oracle on tensor-aligned windows
    covering the buffer: every chunk's signs, scales and errors of the eight
    workers and of the server, m and v_fresh bit for bit, and the
    parameters, the warmup coefficients' averages, f_prev and c of every
    tensor within the bar ("1-bit LAMB" page, Section 4 summary: the
    warmup stage preconditions the compression stage)."""
    wl = WORKLOADS["mixed"]
    n_comp = 2
    d = DevRun(wl, carry_norm=True)
    step = 0
    for _ in range(wl.warmup_steps):
        d.warmup_step(step)
        step += 1
    d.freeze(wl.warmup_steps)
    for _ in range(n_comp):
        d.compressed_step(step)
        step += 1
    torch.cuda.synchronize()
    assert int(d.status.item()) == 0

    def run_host(h):
        s = 0
        for _ in range(wl.warmup_steps):
            h.warmup_step(s)
            s += 1
        h.freeze(wl.warmup_steps)
        for _ in range(n_comp):
            h.compressed_step(s)
            s += 1

    # 22 steps of eight workers' gradients per window: the host's input
    # generation dominates, so eight windows at a time (about 27 GB)
    whole_buffer_parity(d, wl, run_host, threads=8)


def test_mixed_warmup_to_compression():
    """BERT-Large table with per-tensor gradient scales: 20 LAMB warmup steps
    (the parameters' squared norm carried from step to step), freeze, 20
    compression steps, GPU and oracle each on their own state."""
    wl = WORKLOADS["mixed"]
    d = DevRun(wl, carry_norm=True)         # every warmup step after the first skips reading x
    hosts = [HostRun(wl, lo, hi) for lo, hi in block_windows(wl, chunks=64)]
    step = 0
    for _ in range(wl.warmup_steps):
        d.warmup_step(step)
        for h in hosts:
            h.warmup_step(step)
        step += 1
    torch.cuda.synchronize()
    for h in hosts:
        assert_parity(compare_state(d, h, stage="warmup"), f"after warmup, window [{h.lo}, {h.hi})")
    d.freeze(wl.warmup_steps)
    for h in hosts:
        h.freeze(wl.warmup_steps)
    for _ in range(wl.compression_steps):
        d.compressed_step(step)
        for h in hosts:
            h.compressed_step(step)
        step += 1
    torch.cuda.synchronize()
    for h in hosts:
        assert_parity(compare_state(d, h), f"after compression, window [{h.lo}, {h.hi})")
    assert int(d.status.item()) == 0


@pytest.mark.timeout(1200)
def test_bert_xl_step():
    """BERT-XL table (2.83e9 parameters, W = 4, about 150 GB of state): one
    compression step compared against the oracle over the whole buffer
    (691,493 chunks, element indices up to 2.83e9)."""
    torch.cuda.empty_cache()
    wl = WORKLOADS["bert_xl"]
    free, _ = torch.cuda.mem_get_info()
    need = wl.N * 4 * (5 + 2 * wl.W) * 1.02
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} free")
    d = DevRun(wl, store_worker_bits=False)
    d.compressed_step(0)
    torch.cuda.synchronize()
    assert int(d.status.item()) == 0
    wins = whole_buffer_parity(d, wl, lambda h: h.compressed_step(0))
    assert wins[-1][1] == wl.N > 2**31
    del d
    torch.cuda.empty_cache()


def test_bert_xl_share_step():
    """BERT-XL table (2.83e9 parameters, W = 4): one compression step through
    one GPU's share entry points instead of the fused step -- each worker's
    compression, the W chunk ranges as server, then one replica's statistics
    and update, in place on one state -- windows checked against the oracle
    like the fused step (the windows around the last block lie past element
    2^31)."""
    import communication_compressed_optimizer_amd as ob
    torch.cuda.empty_cache()
    wl = WORKLOADS["bert_xl"]
    C, N, K, W = wl.chunk, wl.N, wl.K, wl.W
    words = K * C // 32
    free, _ = torch.cuda.mem_get_info()
    need = wl.N * 4 * (5 + 2 * wl.W) * 1.02 + W * 4 * (words + K)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} free")
    d = DevRun(wl, store_worker_bits=False)
    bits_w = [torch.empty(words, dtype=torch.int32, device="cuda") for _ in range(W)]
    scales_w = [torch.empty(K, dtype=torch.float32, device="cuda") for _ in range(W)]
    d.fill_grads(0)
    for p in range(W):
        ob.onebit_worker_compress(N, C, d.g[p], d.e[p], d.m, None, None, bits_w[p], scales_w[p],
                                  d.hp, d.status)
    for p in range(W):
        k0, k1 = K * p // W, K * (p + 1) // W
        lo, hi, w0, w1 = k0 * C, min(k1 * C, N), k0 * C // 32, k1 * C // 32
        ob.onebit_average_packed(hi - lo, C, W, [b[w0:w1] for b in bits_w],
                                 [s[k0:k1] for s in scales_w], d.err_s[lo:hi], d.bits_s[w0:w1],
                                 d.scales_s[k0:k1], d.status)
    ob.onebit_lamb_rescale_stats(d.table, d.bits_s, d.scales_s, d.m, None, None, d.v, d.vf, d.hp,
                                 d.ws)
    ob.onebit_lamb_rescale_update(d.table, d.bits_s, d.scales_s, d.x, d.m, d.v, d.c_avg, d.f_prev,
                                  d.c_out, d.hp, d.ws, d.status)
    torch.cuda.synchronize()
    wins = block_windows(wl, chunks=64)
    assert wins[-1][1] > 2**31
    for lo, hi in wins:
        h = HostRun(wl, lo, hi)
        h.compressed_step(0)
        assert_parity(compare_state(d, h), f"window [{lo}, {hi})")
    assert int(d.status.item()) == 0
    del d, bits_w, scales_w
    torch.cuda.empty_cache()
