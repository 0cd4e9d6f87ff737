"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs.

Signs, scales, errors, moments and the fresh variance must match bit for
bit; parameters and per-tensor coefficients within rel 1e-5 / abs 1e-7
(they are bit-exact in the compression stage too, where no order-dependent
sum is involved, and that is reported).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import communication_compressed_optimizer_amd as ob  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from synth.workloads import HPARAMS, Workload, WORKLOADS  # noqa: E402

from tests.harness import DevRun, HostRun, assert_parity, compare_state  # noqa: E402


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def normals(n, stream, std=1.0, seed=0, offset=0):
    out = np.empty(n, np.float32)
    return synth.normal_host(out, seed, stream, offset, 0.0, std)


# ---------------------------------------------------------------------------
# the generator itself: device fill == host fill, bit for bit
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,offset", [(1, 0), (1000, 7), (3_000_001, 123_456_789_012)])
def test_synth_device_matches_host(n, offset):
    t = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.normal_dev(t, 5, synth.stream_id(synth.G, 3, 2), offset, 0.25, 1e-3)
    h = np.empty(n, np.float32)
    synth.normal_host(h, 5, synth.stream_id(synth.G, 3, 2), offset, 0.25, 1e-3)
    assert np.array_equal(host(t).view(np.uint32), h.view(np.uint32))
    synth.uniform_dev(t, 5, 77, offset, 1e-8, 1e-4)
    synth.uniform_host(h, 5, 77, offset, 1e-8, 1e-4)
    assert np.array_equal(host(t).view(np.uint32), h.view(np.uint32))


# ---------------------------------------------------------------------------
# codec entry points
# ---------------------------------------------------------------------------
CODEC_CASES = [(1, 4096), (4095, 4096), (4097, 4096), (129_792, 4096), (3 * 4096 + 2816, 4096),
               (1_000_003, 1024), (70_001, 2048), (50_000, 8192), (100_001, 16384),
               (16 * 1024 * 1024, 4096)]


@pytest.mark.parametrize("n,C", CODEC_CASES)
def test_compress_ef_parity(n, C):
    K = oracle.num_chunks(n, C)
    inp = normals(n, 11, 1e-3)
    err = normals(n, 12, 1e-4)
    inp[::97] = 0.0
    inp[5::101] = -0.0
    d_in, d_err = dev(inp), dev(err)
    d_bits = torch.full((K * C // 32,), -1, dtype=torch.int32, device="cuda")
    d_sc = torch.full((K,), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ob.onebit_compress_ef(n, C, d_in, d_err, d_bits, d_sc, status)
    bits, scales = oracle.compress_ef(inp, err, C)
    assert np.array_equal(u32(d_bits), bits)
    assert np.array_equal(host(d_sc).view(np.uint32), scales.view(np.uint32))
    assert np.array_equal(host(d_err).view(np.uint32), err.view(np.uint32))
    assert int(status.item()) == 0


def test_compress_ef_zero_chunk_and_empty():
    C = 4096
    n = 2 * C
    inp = np.zeros(n, np.float32)
    inp[C:] = 1.0
    err = np.zeros(n, np.float32)
    d_in, d_err = dev(inp), dev(err)
    d_bits = torch.zeros(n // 32, dtype=torch.int32, device="cuda")
    d_sc = torch.zeros(2, dtype=torch.float32, device="cuda")
    ob.onebit_compress_ef(n, C, d_in, d_err, d_bits, d_sc)
    assert np.all(u32(d_bits) == 0xFFFFFFFF) and host(d_sc).tolist() == [0.0, 1.0]
    assert np.all(host(d_err) == 0)
    ob.onebit_compress_ef(0, C, None, None, None, None)  # n = 0 does nothing


def test_compress_ef_subnormal_values():
    """fp32 subnormals are kept on both sides (no flush to zero): chunks of
    subnormal inputs, of values whose squares underflow, of huge values whose
    squares overflow the sum, and normal chunks, bit for bit."""
    C = 4096
    n = 5 * C + 123
    r = np.random.default_rng(7)
    inp = f32(r.standard_normal(n))
    inp[:C] *= np.float32(1e-39)                 # subnormal inputs
    inp[C:2 * C] *= np.float32(1e-25)            # squares underflow to subnormal or zero
    inp[2 * C:3 * C] *= np.float32(3e18)         # squares near the top of the range
    inp[3 * C:3 * C + 7] = np.float32(1.4e-45)   # the smallest subnormal
    err = f32(r.standard_normal(n) * 1e-41)
    K = oracle.num_chunks(n, C)
    d_in, d_err = dev(inp), dev(err)
    d_bits = torch.zeros(K * C // 32, dtype=torch.int32, device="cuda")
    d_sc = torch.zeros(K, dtype=torch.float32, device="cuda")
    ob.onebit_compress_ef(n, C, d_in, d_err, d_bits, d_sc)
    bits, scales = oracle.compress_ef(inp, err, C)
    assert np.array_equal(u32(d_bits), bits)
    assert np.array_equal(host(d_sc).view(np.uint32), scales.view(np.uint32))
    assert np.array_equal(host(d_err).view(np.uint32), err.view(np.uint32))
    # squares of subnormals underflow to 0, so that chunk's scale is 0 and its
    # errors carry the subnormal sums in + err, kept (not flushed) on both sides
    assert scales[0] == 0.0 and np.count_nonzero(err[:C]) > C // 2


def test_compressed_step_tiny_state():
    """A compression step whose momentum, gradients and variances are tiny
    (subnormal products along the way), bit for bit against the oracle."""
    numels = [4096 * 2 + 5, 777]
    wl = Workload("tiny_state", numels, W=3, init="frozen")
    d, h = DevRun(wl), HostRun(wl)
    for t_d, a_h, sc in ((d.m, h.m, 1e-36), (d.v, h.v, 1e-30), (d.vf, h.vf, 1e-30)):
        a_h *= np.float32(sc)
        t_d.copy_(dev(a_h))
    for step in range(2):
        h.fill_grads(step)
        for w in range(wl.W):
            h.g[w] *= np.float32(1e-35)
            d.g[w].copy_(dev(h.g[w]))
        d.compressed_step(step, fill=False)
        h.compressed_step(step, fill=False)
        assert_parity(compare_state(d, h), f"step {step}")


def f32(a):
    return np.asarray(a, dtype=np.float32)


def test_status_flags_nonfinite():
    C, n = 4096, 4096 * 2
    inp = np.ones(n, np.float32)
    inp[5000] = np.inf
    d_in, d_err = dev(inp), dev(np.zeros(n, np.float32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ob.onebit_compress_ef(n, C, d_in, d_err, torch.zeros(n // 32, dtype=torch.int32, device="cuda"),
                          torch.zeros(2, dtype=torch.float32, device="cuda"), status)
    assert int(status.item()) == ob.ONEBIT_STATUS_NONFINITE_WORKER


@pytest.mark.parametrize("W", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n,C", [(129_792, 4096), (3 * 4096 + 5, 4096), (20_000, 1024)])
def test_average_packed_parity(W, n, C):
    K = oracle.num_chunks(n, C)
    bits_w, scales_w = [], []
    for w in range(W):
        b, s = oracle.compress_ef(normals(n, 100 + w, 1e-3), np.zeros(n, np.float32), C)
        bits_w.append(b)
        scales_w.append(s)
    err_s = normals(n, 200, 1e-4)
    d_err = dev(err_s)
    d_bits = torch.full((K * C // 32,), -1, dtype=torch.int32, device="cuda")
    d_sc = torch.zeros(K, dtype=torch.float32, device="cuda")
    ob.onebit_average_packed(n, C, W, [dev(b.view(np.int32)) for b in bits_w],
                             [dev(s) for s in scales_w], d_err, d_bits, d_sc)
    b, s = oracle.average_packed(bits_w, scales_w, err_s, C)
    assert np.array_equal(u32(d_bits), b)
    assert np.array_equal(host(d_sc).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(host(d_err).view(np.uint32), err_s.view(np.uint32))


@pytest.mark.parametrize("n,C", [(129_792, 4096), (4097, 4096), (5000, 1024)])
def test_decompress_parity(n, C):
    bits, scales = oracle.compress_ef(normals(n, 300), np.zeros(n, np.float32), C)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    ob.onebit_decompress(n, C, dev(bits.view(np.int32)), dev(scales), out)
    assert np.array_equal(host(out), oracle.decompress(bits, scales, n, C))


# ---------------------------------------------------------------------------
# optimizer steps on ragged tables
# ---------------------------------------------------------------------------
RAGGED = [
    [1, 3, 4095, 4097, 100, 8192, 17],       # chunks straddle up to 4 tensors
    [4096 * 3],                               # chunk-aligned single tensor
    [5, 7, 11, 13] * 300 + [2048 * 3 + 1],   # many tiny tensors per chunk
    [256 * 256, 256, 1000 * 64],              # the three-tensor table
    [10, 20, 30],                             # the whole table inside one partial chunk
    [1],                                      # a single element
]


def _ragged_workload(numels, W, chunk=4096, init="frozen"):
    return Workload("ragged", numels, W=W, chunk=chunk, init=init,
                    grad_std=0.02 if init == "fresh" else 1e-3)


@pytest.mark.parametrize("numels", RAGGED)
@pytest.mark.parametrize("W", [1, 3, 8, 16])
def test_compressed_step_parity(numels, W):
    wl = _ragged_workload(numels, W)
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.compressed_step(step)
        h.compressed_step(step)
        rep = compare_state(d, h)
        assert_parity(rep, f"step {step}")
        assert rep["x"]["max_abs"] == 0.0          # no order-dependent sum in this stage
    assert int(d.status.item()) == 0


@pytest.mark.parametrize("chunk", [1024, 2048, 8192, 16384])
def test_compressed_step_other_chunks(chunk):
    wl = _ragged_workload(RAGGED[0] + [3 * chunk + 9], 4, chunk=chunk)
    d, h = DevRun(wl), HostRun(wl)
    d.compressed_step(0)
    h.compressed_step(0)
    assert_parity(compare_state(d, h))


@pytest.mark.parametrize("numels", RAGGED)
@pytest.mark.parametrize("W", [1, 2, 8])
def test_warmup_step_parity(numels, W):
    wl = _ragged_workload(numels, W, init="fresh")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        d.warmup_step(step)
        h.warmup_step(step)
        assert_parity(compare_state(d, h, stage="warmup"), f"warmup step {step}")


def _segment_sums_host(wl, x):
    """Per-(chunk, tensor) sums of x^2 in float64, segments numbered chunk by
    chunk and within a chunk tensor by tensor (an independent enumeration)."""
    C, N = wl.chunk, wl.N
    off = wl.offsets
    x = x.astype(np.float64)
    out = []
    for k in range(wl.K):
        lo, hi = k * C, min((k + 1) * C, N)
        for l in range(len(off) - 1):
            a, b = max(lo, int(off[l])), min(hi, int(off[l + 1]))
            if a < b:
                out.append(float(np.sum(x[a:b] * x[a:b])))
    return np.array(out)


@pytest.mark.parametrize("numels", RAGGED)
@pytest.mark.parametrize("variant", ["plain", "bias", "weight_decay"])
def test_warmup_norm_carry_is_bit_identical(numels, variant):
    """onebit_lamb_warmup_step_carry (x's squared norm carried from one step's
    update pass to the next step) against onebit_lamb_warmup_step (x read in
    every step): four steps, then an outside change to x announced with
    x_sq_valid = 0, then two more steps.  Every output is equal bit for bit,
    and after each carried step x_sq holds the per-segment sums of the
    updated x^2 (float64 sums on the host, to the rounding of the order)."""
    wl = _ragged_workload(numels, 3, init="fresh")
    a, b = DevRun(wl), DevRun(wl, carry_norm=True)
    assert b.x_sq.numel() == b.table.n_segments
    if variant == "weight_decay":
        a.hp.weight_decay = b.hp.weight_decay = 0.01
    for step in range(7):
        if step == 4:                         # x changed outside the warmup
            for r in (a, b):
                r.x.mul_(-0.5)
            b.x_sq_valid = 0
        for r in (a, b):
            if variant == "bias":
                r.hp.bias_step = step + 1
            r.warmup_step(step)
        torch.cuda.synchronize()
        for name in ("x", "m", "v", "c_sum", "c_out"):
            assert torch.equal(getattr(a, name).view(torch.int32), getattr(b, name).view(torch.int32)), \
                (name, step)
        want = _segment_sums_host(wl, host(b.x))
        got = host(b.x_sq)
        assert np.allclose(got, want, rtol=1e-11, atol=0), step


def test_freeze_parity():
    wl = _ragged_workload(RAGGED[0], 3, init="fresh")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        d.warmup_step(step)
        h.warmup_step(step)
    d.freeze(3)
    h.freeze(3)
    assert_parity(compare_state(d, h, stage="warmup"))
    for w in range(3):
        assert torch.count_nonzero(d.e[w]).item() == 0
    assert torch.equal(d.vf, d.v)


# ---------------------------------------------------------------------------
# whole workloads
# ---------------------------------------------------------------------------
def test_tiny_trajectory():
    """The three-tensor workload end to end: 5 warmup steps, freeze, 5
    compression steps, GPU and oracle each on their own state."""
    wl = WORKLOADS["tiny"]
    d, h = DevRun(wl), HostRun(wl)
    step = 0
    for _ in range(wl.warmup_steps):
        d.warmup_step(step)
        h.warmup_step(step)
        assert_parity(compare_state(d, h, stage="warmup"), f"warmup {step}")
        step += 1
    d.freeze(wl.warmup_steps)
    h.freeze(wl.warmup_steps)
    for _ in range(wl.compression_steps):
        d.compressed_step(step)
        h.compressed_step(step)
        assert_parity(compare_state(d, h), f"compression {step}")
        step += 1
    assert int(d.status.item()) == 0


def test_tiny_strict_per_step():
    """Each step from an identical state: the oracle adopts the GPU state
    before every step."""
    wl = WORKLOADS["tiny"]
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        h.load_from(d.window(0, wl.N))
        d.warmup_step(step)
        h.warmup_step(step)
        assert_parity(compare_state(d, h, stage="warmup"))
    d.freeze(3)
    h.freeze(3)
    for step in range(3, 6):
        h.load_from(d.window(0, wl.N))
        d.compressed_step(step)
        h.compressed_step(step)
        assert_parity(compare_state(d, h))


def test_single_layer_16m():
    """One 16M-element tensor, W = 4, one compression step, whole buffer."""
    wl = WORKLOADS["single"]
    d, h = DevRun(wl), HostRun(wl)
    d.compressed_step(0)
    h.compressed_step(0)
    assert_parity(compare_state(d, h))


def test_degenerate_tensors():
    """The method's special cases through 2 LAMB warmup steps, the freeze
    and 3 compression steps, GPU against oracle: a tensor of zero
    parameters (||x|| = 0, so the trust ratio is 1), a tensor whose
    gradients and moments are all zero (||u|| = 0, ratio 1; then whole
    chunks of zeros: scale 0, every sign bit set, errors 0, q = 1), a
    one-element tensor, a one-chunk tensor whose gradients are all
    positive, and gradients of -0.0."""
    C = 4096
    numels = [C, 2 * C, 1, C, 2 * C + 11]
    wl = Workload("degenerate", numels, W=3, chunk=C, init="fresh", grad_std=0.02)
    d, h = DevRun(wl), HostRun(wl)
    off = wl.offsets
    t = [slice(int(off[i]), int(off[i + 1])) for i in range(len(numels))]
    h.x[t[0]] = 0.0
    for a in (h.m, h.v):
        a[t[1]] = 0.0
    for name in ("x", "m", "v"):
        getattr(d, name).copy_(dev(getattr(h, name)))
    d.vf.copy_(d.v)
    h.vf[:] = h.v

    def grads(step):
        h.fill_grads(step)
        for w in range(wl.W):
            g = h.g[w]
            g[t[1]] = 0.0
            g[t[3]] = np.abs(g[t[3]])
            g[t[4]][::7] = -0.0
            d.g[w].copy_(dev(g))

    for step in range(2):
        grads(step)
        d.warmup_step(step, fill=False)
        h.warmup_step(step, fill=False)
        assert_parity(compare_state(d, h, stage="warmup"), f"warmup {step}")
        if step == 0:
            c = host(d.c_out)
            assert c[0] == 1.0 and c[1] == 1.0, c     # ||x|| = 0 and ||u|| = 0
    d.freeze(2)
    h.freeze(2)
    for step in range(2, 5):
        grads(step)
        d.compressed_step(step, fill=False)
        h.compressed_step(step, fill=False)
        assert_parity(compare_state(d, h), f"compression {step}")
        # chunks 1 and 2 hold tensor 1 alone: all zeros
        assert np.all(host(d.scales_s)[1:3] == 0.0)
        assert np.all(u32(d.bits_s)[C // 32:3 * C // 32] == 0xFFFFFFFF)
        assert not torch.any(d.err_s[t[1]] != 0)
    assert int(d.status.item()) == 0


def test_independent_calls_on_two_streams():
    """Two tables, each with its own state and workspace, stepped on two
    streams at once (LAMB compression steps on one, 1-bit Adam steps on the
    other) give bit for bit what each gives alone: the library keeps no
    state between calls beyond the caller's arrays."""
    wa = Workload("streams_a", [4096 * 5 + 3, 100, 4096], W=3, init="frozen")
    wb = Workload("streams_b", [7, 4096 * 2, 999], W=5, init="frozen", seed=1)
    keys = ("x", "m", "v", "vf", "err_s", "bits_s", "scales_s", "c")

    def run(d, wl, step):
        if wl is wa:
            d.compressed_step(step)
        else:
            d.adam_compressed_step(step)

    ref = {}
    for wl in (wa, wb):
        d = DevRun(wl)
        for step in range(3):
            run(d, wl, step)
        torch.cuda.synchronize()
        ref[wl.name] = d.window(0, wl.N)
    da, db = DevRun(wa), DevRun(wb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for step in range(3):
        with torch.cuda.stream(sa):
            run(da, wa, step)
        with torch.cuda.stream(sb):
            run(db, wb, step)
    torch.cuda.synchronize()
    for d, wl in ((da, wa), (db, wb)):
        got = d.window(0, wl.N)
        for k in keys:
            assert np.array_equal(np.asarray(got[k]).view(np.uint32),
                                  np.asarray(ref[wl.name][k]).view(np.uint32)), (wl.name, k)
        for w in range(wl.W):
            assert np.array_equal(got["e"][w].view(np.uint32), ref[wl.name]["e"][w].view(np.uint32))


def test_determinism_and_resume():
    """Two runs are bitwise identical, and a run resumed from a saved state
    equals the uninterrupted one (across the warmup -> compression switch)."""
    wl = _ragged_workload(RAGGED[0], 4, init="fresh")
    a = DevRun(wl)
    for s in range(3):
        a.warmup_step(s)
    saved = {k: getattr(a, k).clone() for k in ("x", "m", "v", "vf", "c_sum")}
    a.freeze(3)
    for s in range(3, 6):
        a.compressed_step(s)
    b = DevRun(wl)
    for k, t in saved.items():
        getattr(b, k).copy_(t)
    b.freeze(3)
    for s in range(3, 6):
        b.compressed_step(s)
    for k in ("x", "m", "v", "vf", "err_s", "bits_s", "scales_s", "f_prev", "c_out"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    for w in range(4):
        assert torch.equal(a.e[w], b.e[w])


def test_two_phase_equals_fused():
    """onebit_lamb_compress_average + onebit_lamb_rescale_update is
    onebit_lamb_compressed_step."""
    wl = _ragged_workload(RAGGED[0], 4)
    a, b = DevRun(wl), DevRun(wl)
    for step in range(2):
        a.compressed_step(step)
        b.fill_grads(step)
        ob.onebit_lamb_compress_average(b.table, 4, b.g, b.e, b.err_s, b.m, b.v, b.vf, b.bits_w,
                                        b.scales_w, b.bits_s, b.scales_s, b.hp, b.ws, b.status)
        ob.onebit_lamb_rescale_update(b.table, b.bits_s, b.scales_s, b.x, b.m, b.v, b.c_avg,
                                      b.f_prev, b.c_out, b.hp, b.ws, b.status)
    for k in ("x", "m", "vf", "err_s", "bits_s", "scales_s", "f_prev", "c_out"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k


def test_worker_packed_outputs_optional():
    """NULL worker sign/scale arrays skip those stores and change nothing else."""
    wl = _ragged_workload(RAGGED[3], 2)
    a, b = DevRun(wl), DevRun(wl, store_worker_bits=False)
    a.compressed_step(0)
    b.compressed_step(0)
    for k in ("x", "m", "vf", "err_s", "bits_s", "scales_s"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k


# ---------------------------------------------------------------------------
# failure handling and elastic membership (forced from the host)
# ---------------------------------------------------------------------------
def test_worker_drop_and_rejoin():
    """A worker leaves for two steps (the step runs with W-1 workers) and
    rejoins with its error buffer reset; GPU and oracle agree throughout."""
    numels = RAGGED[0]
    wl4 = _ragged_workload(numels, 4)
    d, h = DevRun(wl4), HostRun(wl4)
    N = wl4.N
    hp = d.hp
    for step in range(5):
        active = [0, 1, 2] if step in (1, 2) else [0, 1, 2, 3]
        if step == 3:                           # rejoin: its stale error is dropped
            d.e[3].zero_()
            h.e[3][:] = 0
        d.fill_grads(step)
        h.fill_grads(step)
        W = len(active)
        ob.onebit_lamb_compressed_step(
            d.table, W, [d.g[w] for w in active], [d.e[w] for w in active], d.err_s, d.x, d.m, d.v,
            d.vf, d.c_avg, d.f_prev, d.c_out, [d.bits_w[w] for w in active],
            [d.scales_w[w] for w in active], d.bits_s, d.scales_s, hp, d.ws, d.status)
        out = oracle.compressed_step(h.numels, wl4.chunk, [h.g[w] for w in active],
                                     [h.e[w] for w in active], h.err_s, h.x, h.m, h.v, h.vf,
                                     h.c_avg, h.f_prev, h.hp)
        torch.cuda.synchronize()
        for name, a, b in (("x", d.x, h.x), ("m", d.m, h.m), ("vf", d.vf, h.vf),
                           ("err_s", d.err_s, h.err_s)):
            assert np.array_equal(host(a).view(np.uint32), b.view(np.uint32)), (step, name)
        for w in range(4):
            assert np.array_equal(host(d.e[w]).view(np.uint32), h.e[w].view(np.uint32)), (step, w)
        assert np.array_equal(u32(d.bits_s), out["bits_s"])
    assert N > 0 and int(d.status.item()) == 0


def test_status_flags_from_steps():
    """Non-finite gradients set the documented status bits in the warmup and
    in the compression step; the calls still complete."""
    wl = _ragged_workload(RAGGED[0], 2, init="fresh")
    d = DevRun(wl)
    d.fill_grads(0)
    d.g[1][5] = float("nan")
    ob.onebit_lamb_warmup_step(d.table, 2, d.g, d.x, d.m, d.v, d.c_sum, d.c_out, d.hp, d.ws,
                               d.status)
    torch.cuda.synchronize()
    assert int(d.status.item()) & ob.ONEBIT_STATUS_NONFINITE_TRUST
    wl2 = _ragged_workload(RAGGED[0], 2)
    d2 = DevRun(wl2)
    d2.fill_grads(0)
    d2.g[0][100] = float("inf")
    ob.onebit_lamb_compressed_step(d2.table, 2, d2.g, d2.e, d2.err_s, d2.x, d2.m, d2.v, d2.vf,
                                   d2.c_avg, d2.f_prev, d2.c_out, d2.bits_w, d2.scales_w,
                                   d2.bits_s, d2.scales_s, d2.hp, d2.ws, d2.status)
    torch.cuda.synchronize()
    st = int(d2.status.item())
    assert st & ob.ONEBIT_STATUS_NONFINITE_WORKER and st & ob.ONEBIT_STATUS_NONFINITE_SERVER


def test_nan_ratio_rule_matches_oracle():
    """A NaN rescale ratio (here a NaN frozen variance) at a tensor's first
    element, in the middle of another and at the last element of a third.
    Both sides make those tensors' rho NaN (one NaN anywhere, reading R13),
    so their f is clamped from f_prev alone (kp); the other tensors keep
    f = rho = their maximum ratio, below kp here because v_frozen = v_fresh
    = 1 puts every ratio near 1/sqrt(beta2).  The status bit is set, x is
    NaN at exactly those elements, and every other value meets the bar."""
    numels = RAGGED[0]
    wl = _ragged_workload(numels, 3)
    d, h = DevRun(wl), HostRun(wl)
    for run in (d, h):
        run.v[:] = 1.0
        run.vf[:] = 1.0
    off = wl.offsets
    idx = [int(off[2]), int(off[3]) + numels[3] // 2, int(off[6]) - 1]
    for i in idx:
        d.v[i] = float("nan")
        h.v[i] = np.nan
    d.compressed_step(0)
    h.compressed_step(0)
    torch.cuda.synchronize()
    dd = d.window(0, wl.N)
    nan_d, nan_h = np.isnan(dd["x"]), np.isnan(h.x)
    assert np.array_equal(nan_d, nan_h) and sorted(np.flatnonzero(nan_h)) == idx
    dd["x"] = np.where(nan_d, np.float32(0), dd["x"]).astype(np.float32)
    h.x[nan_h] = 0.0
    assert_parity(compare_state(d, h, dd), "NaN ratios")
    kp = np.float32(1) + np.float32(HPARAMS["kappa"])
    for l in range(len(numels)):
        if l in (2, 3, 5):
            assert dd["f_prev"][l] == kp and h.f_prev[l] == kp, l
        else:
            assert 1.0 < dd["f_prev"][l] < kp, (l, dd["f_prev"][l])
    assert int(d.status.item()) & ob.ONEBIT_STATUS_NONFINITE_RHO


def test_binding_rejects_bad_arguments():
    n, C = 4096, 4096
    a = torch.zeros(n + 4, dtype=torch.float32, device="cuda")
    bits = torch.zeros(n // 32, dtype=torch.int32, device="cuda")
    sc = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress_ef(n, C, a[1:], a[:n], bits, sc)      # 4-byte offset
    assert ei.value.code == ob.ONEBIT_EALIGN
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress_ef(n, 3000, a, a, bits, sc)
    assert ei.value.code == ob.ONEBIT_EUNSUPPORTED
    with pytest.raises(ob.OnebitError):
        ob.LayerTable([10, 0, 5])
    ob.onebit_average_packed(0, C, 2, [bits, bits], [sc, sc], a, bits, sc)   # n = 0: nothing
    ob.onebit_decompress(0, C, bits, sc, a)
    assert torch.count_nonzero(a).item() == 0
    # the binding's own checks, before the library: dtype, layout, size, worker count
    strided = torch.zeros(2 * n, dtype=torch.float32, device="cuda")[::2]
    for call in (lambda: ob.onebit_compress_ef(n, C, a.double()[:n], a[:n], bits, sc),
                 lambda: ob.onebit_compress_ef(n, C, strided, a[:n], bits, sc),
                 lambda: ob.onebit_compress_ef(n, C, a[:n - 1], a[:n], bits, sc),
                 lambda: ob.onebit_compress_ef(n, C, a[:n], a[:n], bits.float(), sc),
                 lambda: ob.onebit_compress_ef(n, C, a[:n], a[:n], bits[:-1], sc),
                 lambda: ob.onebit_average_packed(n, C, 2, [bits], [sc, sc], a, bits, sc)):
        with pytest.raises(ob.OnebitError) as ei:
            call()
        assert ei.value.code == ob.ONEBIT_EINVAL and "binding:" in str(ei.value)
    assert torch.count_nonzero(a).item() == 0 and torch.count_nonzero(bits).item() == 0


def test_many_workers_trajectory():
    """W = 16 workers through warmup, freeze and compression on a ragged table."""
    wl = _ragged_workload(RAGGED[0], 16, init="fresh")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(3):
        d.warmup_step(step)
        h.warmup_step(step)
    d.freeze(3)
    h.freeze(3)
    for step in range(3, 6):
        d.compressed_step(step)
        h.compressed_step(step)
        assert_parity(compare_state(d, h), f"step {step}")


@pytest.mark.parametrize("chunk", [1024, 16384])
def test_warmup_other_chunks(chunk):
    wl = _ragged_workload(RAGGED[0] + [2 * chunk + 3], 3, chunk=chunk, init="fresh")
    d, h = DevRun(wl), HostRun(wl)
    for step in range(2):
        d.warmup_step(step)
        h.warmup_step(step)
    assert_parity(compare_state(d, h, stage="warmup"))
