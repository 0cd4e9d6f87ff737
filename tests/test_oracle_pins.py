"""Pins of the CPU oracle against what the method and the mathematics fix.

Nothing here retypes the oracle's formulas: each test checks a property
that holds for the method as described on the 1-bit LAMB page (arXiv
2104.06069) -- a norm identity, an error-feedback identity, a reduction to a
textbook optimizer, a closed form, an invariance, or a brute force on tiny
inputs -- chosen so that a dropped term, a wrong sign or a transposed
operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle

U = 2.0 ** -24
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def hp(**kw):
    base = dict(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3, weight_decay=0.0, c_min=0.01,
                c_max=10.0, f_min=0.5, f_max=4.0, kappa=0.1)
    base.update(kw)
    return oracle.hparams(**base)


def chunk_lengths(n, C):
    return [min(C, n - k * C) for k in range(oracle.num_chunks(n, C))]


# ---------------------------------------------------------------------------
# P1  norm preservation of the 1-bit operator (scale = ||z|| / sqrt(n))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,C", [(4096, 4096), (3 * 4096 + 2816, 4096), (1, 4096), (33, 1024),
                                 (5000, 1024), (4095, 2048)])
def test_p1_norm_preserved(n, C):
    z = f32(rng(1).standard_normal(n) * 0.37)
    err = np.zeros(n, np.float32)
    bits, scales = oracle.compress_ef(z, err, C)
    for k, nk in enumerate(chunk_lengths(n, C)):
        zk = z[k * C:k * C + nk].astype(np.float64)
        norm_z = math.sqrt(math.fsum(zk * zk))
        norm_cz = math.sqrt(nk * float(scales[k]) ** 2)  # ||C[z]|| = s * sqrt(n_k)
        assert abs(norm_cz - norm_z) <= (math.log2(C) + 3) * U * norm_z


def test_p1_zero_padding_not_counted():
    # The partial last chunk is normalised by its valid length only.
    C = 4096
    z = f32(np.full(100, 3.0))
    _, scales = oracle.compress_ef(z, np.zeros(100, np.float32), C)
    assert scales[0] == np.float32(3.0)


# ---------------------------------------------------------------------------
# P2  error feedback: z = C[z] + e, and the error is carried forward
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,C", [(4096 * 2 + 77, 4096), (3000, 1024)])
def test_p2_ef_identity_one_step(n, C):
    z = f32(rng(2).standard_normal(n))
    err = np.zeros(n, np.float32)          # z = in + 0 exactly
    bits, scales = oracle.compress_ef(z, err, C)
    cz = oracle.decompress(bits, scales, n, C).astype(np.float64)
    e = err.astype(np.float64)
    resid = np.abs((cz + e) - z.astype(np.float64))
    half_ulp = np.spacing(np.abs(err)).astype(np.float64) / 2
    assert np.all(resid <= half_ulp)
    # Sterbenz range: z - s is exact, so the identity holds exactly
    s_elem = np.repeat(scales.astype(np.float64), C)[:n]
    exact = (np.abs(z) >= s_elem / 2) & (np.abs(z) <= 2 * s_elem)
    assert exact.sum() > n // 4
    assert np.all(resid[exact] == 0.0)


def test_p2_error_carried_forward():
    # Sum_t C[z_t] + e_T = Sum_t in_t: what is sent tracks what was fed in.
    n, C, T = 4096 + 1000, 4096, 20
    err = np.zeros(n, np.float32)
    sent = np.zeros(n, np.float64)
    fed = np.zeros(n, np.float64)
    r = rng(3)
    for _ in range(T):
        x = f32(r.standard_normal(n) * r.uniform(0.1, 10))
        fed += x
        bits, scales = oracle.compress_ef(x, err, C)
        sent += oracle.decompress(bits, scales, n, C)
    gap = np.abs(sent + err - fed)
    assert np.max(gap) <= 64 * T * U * np.max(np.abs(fed) + np.abs(sent))
    # and the error stays bounded by the scale (it does not accumulate)
    assert np.max(np.abs(err)) < 50 * np.max(np.abs(fed)) / math.sqrt(T)


# ---------------------------------------------------------------------------
# P3  identity compressor => textbook momentum SGD
# ---------------------------------------------------------------------------
def test_p3_identity_compressor_is_momentum_sgd():
    numels = [5000, 300]
    N, W, T = sum(numels), 3, 5
    h = hp(eta=1.0, lr=1.0, kappa=0.0)
    r = rng(4)
    x = np.zeros(N, np.float32)
    m = f32(r.standard_normal(N) * 1e-2)
    v0 = np.zeros(N, np.float32)
    vf = np.zeros(N, np.float32)
    err_w = [np.zeros(N, np.float32) for _ in range(W)]
    err_s = np.zeros(N, np.float32)
    c_avg = np.ones(2, np.float32)
    f_prev = np.ones(2, np.float32)
    xd, md = x.astype(np.float64), m.astype(np.float64)
    for _ in range(T):
        g = [f32(r.standard_normal(N) * 1e-2) for _ in range(W)]
        out = oracle.compressed_step(numels, 4096, g, err_w, err_s, x, m, v0, vf, c_avg, f_prev, h,
                                     compressor=oracle.IDENTITY)
        gbar = np.mean([gi.astype(np.float64) for gi in g], axis=0)
        md = 0.9 * md + 0.1 * gbar
        xd = xd - md
        assert np.all(out["c"] == 1.0)
    assert np.max(np.abs(m - md)) <= 1e-5 * np.max(np.abs(md))
    assert np.max(np.abs(x - xd)) <= 1e-5 * np.max(np.abs(xd))
    assert all(np.all(e == 0) for e in err_w) and np.all(err_s == 0)


# ---------------------------------------------------------------------------
# P4  the average step is the arithmetic mean
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 16])
def test_p4_average_is_mean(W):
    n, C = 4096 + 123, 4096
    K = oracle.num_chunks(n, C)
    r = rng(5 + W)
    bits_w = [r.integers(0, 2 ** 32, size=K * C // 32, dtype=np.uint64).astype(np.uint32)
              for _ in range(W)]
    scales_w = [f32(r.uniform(0.5, 2.0, size=K)) for _ in range(W)]
    a = oracle.average(bits_w, scales_w, n, C).astype(np.float64)
    vals = []
    for b, s in zip(bits_w, scales_w):
        sign = np.unpackbits(b.view(np.uint8), bitorder="little").reshape(K, C)
        vals.append(np.where(sign, 1.0, -1.0) * s.astype(np.float64)[:, None])
    mean = (np.sum(vals, axis=0) / W).reshape(-1)[:n]
    bound = W * U * np.max(np.abs(np.array(vals))) + np.spacing(np.abs(a).astype(np.float32))
    assert np.all(np.abs(a - mean) <= bound)


@pytest.mark.parametrize("W", [2, 4, 8, 16])
def test_p4_identical_workers_exact(W):
    n, C = 2 * 4096, 4096
    z = f32(rng(6).standard_normal(n))
    bits, scales = oracle.compress_ef(z, np.zeros(n, np.float32), C)
    err_s = np.zeros(n, np.float32)
    a = oracle.average([bits] * W, [scales] * W, n, C)
    assert np.array_equal(a, oracle.decompress(bits, scales, n, C))
    b2, s2 = oracle.average_packed([bits] * W, [scales] * W, err_s, C)
    assert np.array_equal(b2, bits) and np.array_equal(s2, scales) and np.all(err_s == 0)


# ---------------------------------------------------------------------------
# P5  trust ratio: the per-tensor step length is gamma * ||x_{t-1}||
# ---------------------------------------------------------------------------
def test_p5_trust_ratio_step_length_tiny_tensors():
    numels = [1, 2, 3, 5, 8, 7]
    N = sum(numels)
    r = rng(7)
    h = hp(lr=0.25, c_min=0.0, c_max=1e30)
    x0 = f32(r.standard_normal(N))
    x, m, v = x0.copy(), f32(r.standard_normal(N) * 0.1), f32(r.uniform(0.01, 1, N))
    c_sum = np.zeros(len(numels), np.float32)
    g = [f32(r.standard_normal(N)) for _ in range(3)]
    c = oracle.warmup_step(numels, g, x, m, v, c_sum, h)
    off = 0
    for l, nl in enumerate(numels):
        sl = slice(off, off + nl)
        xo = x0[sl].astype(np.float64)
        dx = xo - x[sl].astype(np.float64)
        assert abs(np.linalg.norm(dx) / np.linalg.norm(xo) - 0.25) <= 4e-7
        # direction: Adam's m / (sqrt(v) + eta), from the returned moments
        u = m[sl].astype(np.float64) / (np.sqrt(v[sl].astype(np.float64)) + 1e-8)
        cos = dx @ u / (np.linalg.norm(dx) * np.linalg.norm(u))
        assert cos >= 1 - 1e-9
        # and c is ||x|| / ||u||
        assert abs(c[l] - np.linalg.norm(xo) / np.linalg.norm(u)) <= 8 * U * c[l]
        off += nl
    assert np.array_equal(c_sum, c)


def test_p5_clip_applies_to_whole_ratio():
    numels = [64, 64]
    N = 128
    r = rng(8)
    h = hp(lr=0.5, c_min=0.0, c_max=1e-3)
    x0 = f32(r.standard_normal(N))
    x, m, v = x0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
    g = [f32(r.standard_normal(N))]
    c = oracle.warmup_step(numels, g, x, m, v, np.zeros(2, np.float32), h)
    assert np.all(c == np.float32(1e-3))
    u = m.astype(np.float64) / (np.sqrt(v.astype(np.float64)) + 1e-8)
    for l in range(2):
        sl = slice(64 * l, 64 * l + 64)
        dx = np.linalg.norm(x0[sl].astype(np.float64) - x[sl])
        assert abs(dx / (0.5 * 1e-3 * np.linalg.norm(u[sl])) - 1) < 1e-4


def test_p5_zero_norms_give_ratio_one():
    numels = [16, 16]
    h = hp(c_min=0.0, c_max=100.0)
    x = np.concatenate([np.zeros(16), np.ones(16)]).astype(np.float32)
    g = [np.concatenate([np.ones(16), np.zeros(16)]).astype(np.float32)]
    m, v = np.zeros(32, np.float32), np.zeros(32, np.float32)
    c = oracle.warmup_step(numels, g, x, m, v, np.zeros(2, np.float32), h)
    assert np.all(c == 1.0)           # x = 0 in tensor 0, update = 0 in tensor 1
    assert np.all(x[16:] == 1.0)      # no gradient, no move


# ---------------------------------------------------------------------------
# P6  warmup step 1 from m = v = 0: closed form
# ---------------------------------------------------------------------------
def test_p6_first_warmup_step_closed_form():
    numels = [4096, 1000]
    N, W = sum(numels), 4
    r = rng(9)
    h = hp(eta=0.0, c_min=0.0, c_max=1e30)
    x0 = f32(r.standard_normal(N) * 0.02)
    x, m, v = x0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
    g = [f32(r.standard_normal(N) * 1e-3) for _ in range(W)]
    c = oracle.warmup_step(numels, g, x, m, v, np.zeros(2, np.float32), h)
    # the hyper-parameters are the fp32 values of 0.9 and 0.999
    a1 = 1 - float(np.float32(0.9))
    a2 = 1 - float(np.float32(0.999))
    G = np.array([gi.astype(np.float64) for gi in g])
    gbar = G.mean(axis=0)
    gabs = np.abs(G).mean(axis=0)
    assert np.all(np.abs(m - a1 * gbar) <= a1 * 4 * U * gabs + 3 * U * np.abs(a1 * gbar))
    assert np.all(np.abs(v - a2 * gbar ** 2) <= a2 * 10 * U * gabs ** 2 + 4 * U * a2 * gbar ** 2)
    off = 0
    for l, nl in enumerate(numels):
        xn = np.linalg.norm(x0[off:off + nl].astype(np.float64))
        expect = xn * math.sqrt(a2) / (a1 * math.sqrt(nl))
        assert abs(c[l] / expect - 1) <= 1e-5
        off += nl


# ---------------------------------------------------------------------------
# P7  idempotence C[C[z]] = C[z] with zero error, full chunks of 4^k
# ---------------------------------------------------------------------------
def test_p7_sqrt_of_rounded_square_is_identity():
    r = rng(10)
    n = 10_000_000
    t = np.empty(n, np.float32)
    for _ in range(10):                                   # 10^8 floats in 10 slices
        # random 23-bit mantissas with exponents 2^-60 .. 2^59
        bits = (r.integers(67, 187, n, dtype=np.uint32) << 23) | r.integers(0, 1 << 23, n, dtype=np.uint32)
        s = bits.view(np.float32)
        np.multiply(s, s, out=t)
        np.sqrt(t, out=t)
        assert np.array_equal(t, s)


@pytest.mark.parametrize("C", [1024, 4096, 16384])
def test_p7_idempotent(C):
    n = 3 * C
    z = f32(rng(11).standard_normal(n))
    bits, scales = oracle.compress_ef(z, np.zeros(n, np.float32), C)
    cz = oracle.decompress(bits, scales, n, C)
    err2 = np.zeros(n, np.float32)
    bits2, scales2 = oracle.compress_ef(cz, err2, C)
    assert np.array_equal(bits2, bits) and np.array_equal(scales2, scales)
    assert np.all(err2 == 0)


# ---------------------------------------------------------------------------
# P8  sign packing: brute force on tiny vectors
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,C", [(1, 64), (31, 64), (64, 64), (100, 64), (130, 128), (4097, 4096)])
def test_p8_packing(n, C):
    r = rng(12 + n)
    z = f32(r.standard_normal(n))
    z[::7] = 0.0
    z[3::11] = -0.0
    bits, _ = oracle.compress_ef(z, np.zeros(n, np.float32), C)
    K = oracle.num_chunks(n, C)
    want = np.zeros(K * C, np.uint8)
    want[:n] = ~np.signbit(z) | (z == 0)              # z >= 0, with -0 counted as >= 0
    packed = np.packbits(want, bitorder="little").view(np.uint32)
    assert np.array_equal(bits, packed)
    assert int(np.unpackbits(bits.view(np.uint8)).sum()) == int(np.sum(z >= 0))
    # every sign word is written in full: what the output held before does not leak
    dirty = np.full(K * C // 32, 0xFFFFFFFF, np.uint32)
    err0, sc = np.zeros(n, np.float32), np.zeros(K, np.float32)      # kept alive across the call
    oracle.lib().oracle_compress_ef(n, C, oracle._ptr(z), oracle._ptr(err0), oracle._ptr(dirty),
                                    oracle._ptr(sc))
    assert np.array_equal(dirty, packed)


def test_p8_tree_order_against_independent_pairwise():
    # The chunk sum of squares uses the stride-halving tree t[j] += t[j+h],
    # h = C/2 .. 1; an independent vectorised evaluation of the same tree.
    r = rng(13)
    for C in (64, 1024, 4096):
        for n in (C, C - 1, C // 2 + 3, 1):
            z = f32(r.standard_normal(n) * np.exp(r.uniform(-20, 20, n)))
            t = np.zeros(C, np.float32)
            t[:n] = z * z
            while t.size > 1:
                h = t.size // 2
                t = t[:h] + t[h:]
            expect = np.float32(np.sqrt(t[0])) / np.float32(np.sqrt(np.float32(n)))
            assert oracle.chunk_scale(z, C) == expect


# ---------------------------------------------------------------------------
# P9  identity compressor => reconstructed gradient equals the mean gradient
# ---------------------------------------------------------------------------
def test_p9_reconstructed_gradient_identity():
    numels = [3000]
    N, W = 3000, 4
    r = rng(14)
    x = f32(r.standard_normal(N))
    m = f32(r.standard_normal(N) * 1e-3)
    m0 = m.copy()
    vfz = f32(r.uniform(1e-8, 1e-4, N))
    vf = vfz.copy()
    g = [f32(r.standard_normal(N) * 1e-3) for _ in range(W)]
    oracle.compressed_step(numels, 4096, g, [np.zeros(N, np.float32) for _ in range(W)],
                           np.zeros(N, np.float32), x, m, vfz, vf, np.ones(1, np.float32),
                           np.ones(1, np.float32), hp(), compressor=oracle.IDENTITY)
    gbar = np.mean([gi.astype(np.float64) for gi in g], axis=0)
    want = 0.999 * vfz.astype(np.float64) + 0.001 * gbar * gbar
    assert np.max(np.abs(vf - want) / want) < 2e-5
    assert np.allclose(m, 0.9 * m0.astype(np.float64) + 0.1 * gbar, rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# P10 layerwise rescale: closed form with a zero reconstructed gradient, and
#     the soft-threshold truth table
# ---------------------------------------------------------------------------
def _constant_magnitude_state(numels, mus, r):
    N = sum(numels)
    sign = np.where(r.random(N) < 0.5, -1.0, 1.0)
    m = f32(sign * np.repeat(mus, numels))
    return m


def _run_zero_ghat(numels, vfz, vf, f_prev, c_avg, W=4):
    N = sum(numels)
    r = rng(15)
    m = _constant_magnitude_state(numels, r.uniform(1e-4, 1e-2, len(numels)), r)
    beta1 = np.float32(0.9)
    mhat_want = beta1 * m
    x = f32(r.standard_normal(N) * 0.02)
    g = [np.zeros(N, np.float32)] * W
    err_w = [np.zeros(N, np.float32) for _ in range(W)]
    err_s = np.zeros(N, np.float32)
    out = oracle.compressed_step(numels, 4096, g, err_w, err_s, x, m, vfz, vf, c_avg, f_prev, hp())
    assert np.array_equal(m, mhat_want)               # mhat = fl(beta1 m) exactly
    assert all(np.all(e == 0) for e in err_w) and np.all(err_s == 0)
    return out


def test_p10_zero_ghat_closed_form():
    numels = [4096 * 2, 4096]
    N = sum(numels)
    r = rng(16)
    vfz = f32(r.uniform(1e-8, 1e-4, N))
    vf = vfz.copy()
    c_avg = np.array([2.0, 0.5], np.float32)
    out = _run_zero_ghat(numels, vfz, vf, np.ones(2, np.float32), c_avg)
    assert np.array_equal(vf, np.float32(0.999) * vfz)  # ghat = 0: only the decay
    off = 0
    for l, nl in enumerate(numels):
        sl = slice(off, off + nl)
        q = (np.sqrt(vfz[sl].astype(np.float64)) + 1e-8) / (np.sqrt(vf[sl].astype(np.float64)) + 1e-8)
        rho = q.max()
        assert abs(rho - 1 / math.sqrt(0.999)) < 1e-6
        assert abs(out["c"][l] / c_avg[l] - rho) <= 6 * U * rho
        off += nl


def test_p10_soft_threshold_truth_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "soft_threshold_cases.txt"))
            if ln.strip() and not ln.startswith("#")]
    L = len(rows)
    numels = [4096] * L
    N = sum(numels)
    r = rng(17)
    vfz = f32(r.uniform(1e-6, 1e-5, N))
    vf = np.empty(N, np.float32)
    f_prev = np.empty(L, np.float32)
    for l, (_, fp, rho_t, _, _) in enumerate(rows):
        sl = slice(4096 * l, 4096 * l + 4096)
        # rho = max sqrt(vfz / (beta2 vf)) -> choose vf so that the max is near rho_t
        vf[sl] = f32(vfz[sl].astype(np.float64) / (0.999 * float(rho_t) ** 2))
        f_prev[l] = np.float32(float(fp))
    vfz_c, vf_c = vfz.copy(), vf.copy()
    out = _run_zero_ghat(numels, vfz, vf, f_prev, np.ones(L, np.float32))
    for l, (name, _, _, expect, _) in enumerate(rows):
        if expect == "rho":
            sl = slice(4096 * l, 4096 * l + 4096)
            vf_new = np.float32(0.999) * vf_c[sl]
            rho = np.max((np.sqrt(vfz_c[sl].astype(np.float64)) + 1e-8) /
                         (np.sqrt(vf_new.astype(np.float64)) + 1e-8))
            assert abs(out["c"][l] - rho) <= 6 * U * rho, name
        else:
            assert out["c"][l] == np.float32(float.fromhex(expect)), name
    assert np.array_equal(f_prev, out["c"])          # f_prev tracks the new factor (c_avg = 1)


# ---------------------------------------------------------------------------
# P11 power-of-two homogeneity and antisymmetry of the 1-bit operator
# ---------------------------------------------------------------------------
def test_p11_homogeneity_and_antisymmetry():
    n, C = 4096 * 2 + 500, 4096
    z = f32(rng(18).standard_normal(n))
    z[z == 0] = 1.0
    e1 = np.zeros(n, np.float32)
    b1, s1 = oracle.compress_ef(z, e1, C)
    e4 = np.zeros(n, np.float32)
    b4, s4 = oracle.compress_ef(f32(z * 4), e4, C)
    assert np.array_equal(b4, b1) and np.array_equal(s4, s1 * 4) and np.array_equal(e4, e1 * 4)
    en = np.zeros(n, np.float32)
    bn, sn = oracle.compress_ef(f32(-z), en, C)
    valid = np.zeros(oracle.num_chunks(n, C) * C, bool)
    valid[:n] = True
    ub1 = np.unpackbits(b1.view(np.uint8), bitorder="little").astype(bool)
    ubn = np.unpackbits(bn.view(np.uint8), bitorder="little").astype(bool)
    assert np.array_equal(ubn[valid], ~ub1[valid]) and not ubn[~valid].any()
    assert np.array_equal(sn, s1) and np.array_equal(en, -e1)


# ---------------------------------------------------------------------------
# P12 LAMB scale invariance: with eta = 0, g -> 2^k g leaves the update alone
# ---------------------------------------------------------------------------
def test_p12_scale_invariance():
    numels = [2000, 96]
    N = sum(numels)
    r = rng(19)
    h = hp(eta=0.0)
    x0 = f32(r.standard_normal(N) * 0.02)
    gs = [[f32(r.standard_normal(N) * 1e-3) for _ in range(2)] for _ in range(3)]
    res = []
    for scale in (1.0, 4.0, 0.125):
        x, m, v = x0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
        cs = np.zeros(2, np.float32)
        for g in gs:
            oracle.warmup_step(numels, [f32(gi * scale) for gi in g], x, m, v, cs, h)
        res.append((x, cs))
    for x, cs in res[1:]:
        assert np.array_equal(x, res[0][0]) and np.array_equal(cs, res[0][1])


# ---------------------------------------------------------------------------
# P13 determinism and freeze bookkeeping
# ---------------------------------------------------------------------------
def test_p13_determinism_and_freeze():
    numels = [4096, 777]
    N, W = sum(numels), 2
    r = rng(20)
    v = f32(r.uniform(1e-8, 1e-4, N))
    outs = []
    for _ in range(2):
        vf = np.empty(N, np.float32)
        err_w = [f32(r.standard_normal(N)) for _ in range(W)]
        err_s = f32(r.standard_normal(N))
        c_avg = np.empty(2, np.float32)
        f_prev = np.zeros(2, np.float32)
        oracle.freeze(numels, v, vf, err_w, err_s, np.array([3.0, 1.5], np.float32), 3, c_avg, f_prev)
        assert np.array_equal(vf, v) and all(np.all(e == 0) for e in err_w) and np.all(err_s == 0)
        assert np.array_equal(c_avg, [1.0, 0.5]) and np.array_equal(f_prev, [1.0, 1.0])
        rr = rng(21)
        x, m = f32(rr.standard_normal(N)), f32(rr.standard_normal(N) * 1e-3)
        g = [f32(rr.standard_normal(N) * 1e-3) for _ in range(W)]
        out = oracle.compressed_step(numels, 4096, g, err_w, err_s, x, m, v, vf, c_avg, f_prev, hp())
        outs.append((x, m, vf, err_s, out["bits_s"], out["scales_s"], out["c"]))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_p4_server_error_feedback():
    # The server's packed output plus its new error equals the average plus
    # its previous error (the server compensates its own compression error).
    n, C, W = 4096 * 2 + 300, 4096, 3
    r = rng(22)
    bits_w, scales_w = [], []
    for _ in range(W):
        b, s = oracle.compress_ef(f32(r.standard_normal(n)), np.zeros(n, np.float32), C)
        bits_w.append(b)
        scales_w.append(s)
    e_in = f32(r.standard_normal(n) * 0.1)
    e_out = e_in.copy()
    b2, s2 = oracle.average_packed(bits_w, scales_w, e_out, C)
    a = oracle.average(bits_w, scales_w, n, C).astype(np.float64)
    lhs = oracle.decompress(b2, s2, n, C).astype(np.float64) + e_out
    rhs = a + e_in
    # rounding of y = a + e_in to fp32, and of the new error
    bound = np.spacing(np.abs(rhs).astype(np.float32)) + np.spacing(np.abs(e_out))
    assert np.all(np.abs(lhs - rhs) <= bound)
    assert np.max(np.abs(e_out)) > 0


# ---------------------------------------------------------------------------
# P14 1-bit Adam warmup = textbook Adam (torch.optim.Adam, fp64) with its
#     bias correction folded into a per-step learning rate and epsilon
# ---------------------------------------------------------------------------
def _torch_adam_steps(x0, grads_per_step, b1, b2, lr, eta):
    import torch
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eta, foreach=False)
    for t, g in enumerate(grads_per_step, start=1):
        bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
        # torch divides by bc1 and sqrt(bc2); undo both so the step is
        # lr * m / (sqrt(v) + eta) with the raw moments
        opt.param_groups[0]["lr"] = lr * bc1 / math.sqrt(bc2)
        opt.param_groups[0]["eps"] = eta / math.sqrt(bc2)
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("eta", [1e-8, 1e-5])
def test_p14_adam_warmup_is_textbook_adam(eta):
    n, W, T = 6000, 3, 5
    r = rng(30)
    h = hp(eta=eta, lr=1e-3)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    x0 = f32(r.standard_normal(n) * 0.02)
    x, m, v = x0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    gbars = []
    for _ in range(T):
        g = [f32(r.standard_normal(n) * 1e-3) for _ in range(W)]
        oracle.adam_warmup_step(g, x, m, v, h)
        gbars.append(np.mean([gi.astype(np.float64) for gi in g], axis=0))
    xd, md, vd = _torch_adam_steps(x0.astype(np.float64), gbars, b1, b2, 1e-3, float(np.float32(eta)))
    assert np.max(np.abs(m - md)) <= 1e-5 * np.max(np.abs(md))
    assert np.max(np.abs(v - vd)) <= 1e-5 * np.max(np.abs(vd))
    # parameters: T roundings of x plus a small relative error on each step
    assert np.all(np.abs(x - xd) <= T * (U * np.abs(xd) + 1e-5 * 1e-3 * 4))
    assert np.max(np.abs(x - x0)) > 1e-4          # it moved


# ---------------------------------------------------------------------------
# P15 1-bit Adam compression stage with the identity compressor = momentum
#     SGD under the fixed preconditioner diag(1 / (sqrt(v_frozen) + eta))
#     (torch.optim.SGD, fp64, in the coordinates m / d, g / d)
# ---------------------------------------------------------------------------
def test_p15_adam_identity_compressor_is_preconditioned_momentum_sgd():
    import torch
    n, W, T = 5000, 3, 5
    r = rng(31)
    h = hp(eta=1e-4, lr=1e-2)
    b1 = float(np.float32(0.9))
    a1 = float(np.float32(1) - np.float32(0.9))
    x = f32(r.standard_normal(n) * 0.02)
    x0 = x.astype(np.float64)
    m = f32(r.standard_normal(n) * 1e-3)
    vfz = f32(r.uniform(1e-8, 1e-5, n))
    d = np.sqrt(vfz.astype(np.float64)) + float(np.float32(1e-4))
    err_w = [np.zeros(n, np.float32) for _ in range(W)]
    err_s = np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.tensor(x, dtype=torch.float64))
    opt = torch.optim.SGD([p], lr=float(np.float32(1e-2)), momentum=b1, dampening=1 - a1,
                          foreach=False)
    opt.state[p]["momentum_buffer"] = torch.tensor(m.astype(np.float64) / d)
    for _ in range(T):
        g = [f32(r.standard_normal(n) * 1e-3) for _ in range(W)]
        oracle.adam_compressed_step(4096, g, err_w, err_s, x, m, vfz, h, compressor=oracle.IDENTITY)
        gbar = np.mean([gi.astype(np.float64) for gi in g], axis=0)
        p.grad = torch.tensor(gbar / d)
        opt.step()
    xd = p.detach().numpy()
    md = opt.state[p]["momentum_buffer"].numpy() * d
    assert np.max(np.abs(m - md)) <= 1e-5 * np.max(np.abs(md))
    # T roundings of x plus a small relative error on the distance moved
    assert np.all(np.abs(x - xd) <= T * U * np.abs(xd) + 1e-5 * np.max(np.abs(xd - x0)))
    assert np.max(np.abs(xd - x0)) > 1e-3          # it moved
    assert all(np.all(e == 0) for e in err_w) and np.all(err_s == 0)


# ---------------------------------------------------------------------------
# P16 1-bit Adam with chunks of constant magnitude (4^k valid elements): the
#     1-bit operator is exact there (sqrt of a rounded square is the value;
#     power-of-two sums of equal terms are exact), so the 1-bit step equals
#     the identity-compressor step bit for bit, with zero errors
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W", [1, 2])
@pytest.mark.parametrize("carrier", ["momentum", "gradient"])
def test_p16_adam_exact_compression_matches_identity(W, carrier):
    C = 4096
    n = 2 * C + 1024
    r = rng(32 + W)
    mags = f32(np.exp(r.uniform(-8, -3, 3)))
    signs = np.where(r.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    pattern = f32(signs * np.repeat(mags, [C, C, 1024]))
    h = hp(eta=1e-6, lr=1e-2)
    vfz = f32(r.uniform(1e-8, 1e-5, n))
    x0 = f32(r.standard_normal(n) * 0.02)
    if carrier == "momentum":
        m0, g = pattern, [np.zeros(n, np.float32) for _ in range(W)]
    else:
        m0, g = np.zeros(n, np.float32), [pattern.copy() for _ in range(W)]
    res = []
    for comp in (oracle.ONEBIT, oracle.IDENTITY):
        x, m = x0.copy(), m0.copy()
        err_w = [np.zeros(n, np.float32) for _ in range(W)]
        err_s = np.zeros(n, np.float32)
        oracle.adam_compressed_step(C, g, err_w, err_s, x, m, vfz, h, compressor=comp)
        res.append((x, m, err_w, err_s))
    (x1, m1, ew1, es1), (x2, m2, _, _) = res
    assert np.array_equal(x1, x2) and np.array_equal(m1, m2)
    assert all(np.all(e == 0) for e in ew1) and np.all(es1 == 0)
    assert np.max(np.abs(x1 - x0)) > 0


# ---------------------------------------------------------------------------
# Variant readings (all off by default)
# ---------------------------------------------------------------------------
# P17 bias correction: the 1-bit Adam warmup with bias_step = t is exactly
#     textbook Adam (torch.optim.Adam, fp64, its own bias correction)
def test_p17_bias_corrected_adam_warmup_is_torch_adam():
    import torch
    n, W, T = 5000, 2, 6
    r = rng(40)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    eta = 1e-6
    x0 = f32(r.standard_normal(n) * 0.02)
    x, m, v = x0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.Adam([p], lr=float(np.float32(1e-3)), betas=(b1, b2),
                           eps=float(np.float32(eta)), foreach=False)
    for t in range(1, T + 1):
        g = [f32(r.standard_normal(n) * 1e-3) for _ in range(W)]
        oracle.adam_warmup_step(g, x, m, v, hp(eta=eta, bias_step=t))
        p.grad = torch.tensor(np.mean([gi.astype(np.float64) for gi in g], axis=0))
        opt.step()
    xd = p.detach().numpy()
    assert np.all(np.abs(x - xd) <= T * (U * np.abs(xd) + 1e-5 * 1e-3 * 4))
    assert np.max(np.abs(x - x0)) > 5e-3       # bias-corrected steps are ~lr each


# P18 bias correction in the LAMB warmup: step 1 from m = v = 0 has
#     mhat = gbar and vhat = gbar^2, so u = sign(gbar) (eta = 0) and the trust
#     ratio is ||x|| / sqrt(n_l) exactly
def test_p18_bias_corrected_lamb_first_step():
    numels = [4096, 1000, 7]
    N, W = sum(numels), 3
    r = rng(41)
    h = hp(eta=0.0, c_min=0.0, c_max=1e30, bias_step=1)
    x0 = f32(r.standard_normal(N) * 0.02)
    x, m, v = x0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32)
    g = [f32(r.standard_normal(N) * 1e-3) for _ in range(W)]
    c = oracle.warmup_step(numels, g, x, m, v, np.zeros(3, np.float32), h)
    off = 0
    for l, nl in enumerate(numels):
        xn = np.linalg.norm(x0[off:off + nl].astype(np.float64))
        assert abs(c[l] / (xn / math.sqrt(nl)) - 1) <= 1e-6
        # the step moves every parameter of the tensor by about lr * c
        dx = np.abs(x0[off:off + nl].astype(np.float64) - x[off:off + nl])
        assert np.all(np.abs(dx / (1e-3 * float(c[l])) - 1) <= 1e-3)
        off += nl


# P19 weight decay (LAMB): with zero gradient and momentum the update
#     direction is lambda*x, so the trust ratio is 1/lambda and the step
#     scales x by (1 - lr*c*lambda); the same in the compression stage
@pytest.mark.parametrize("lam,c_expect", [(0.5, 2.0), (0.01, 10.0)])
def test_p19_weight_decay_closed_form(lam, c_expect):
    numels = [4096, 333]
    N = sum(numels)
    r = rng(42)
    x0 = f32(r.standard_normal(N) * 0.02)
    x, m = x0.copy(), np.zeros(N, np.float32)
    v = f32(r.uniform(1e-8, 1e-4, N))
    g = [np.zeros(N, np.float32)] * 2
    h = hp(weight_decay=lam)
    c = oracle.warmup_step(numels, g, x, m, v, np.zeros(2, np.float32), h)
    assert np.allclose(c, c_expect, rtol=4 * U, atol=0)      # clipped at c_max = 10 for 0.01
    want = x0.astype(np.float64) * (1 - 1e-3 * c_expect * lam)
    assert np.all(np.abs(x - want) <= 4 * U * np.abs(want))
    # compression stage: m = g = 0 -> mhat = 0, update lr*c*lambda*x
    x1 = x.copy()
    vf = v.copy()
    err_w = [np.zeros(N, np.float32) for _ in range(2)]
    out = oracle.compressed_step(numels, 4096, g, err_w, np.zeros(N, np.float32), x, m, v, vf,
                                 np.ones(2, np.float32), np.ones(2, np.float32), h)
    assert np.all(m == 0)
    off = 0
    for l, nl in enumerate(numels):
        want = x1[off:off + nl].astype(np.float64) * (1 - 1e-3 * float(out["c"][l]) * lam)
        assert np.all(np.abs(x[off:off + nl] - want) <= 4 * U * np.abs(want))
        off += nl


# P20 EMA of the warmup coefficient: after T warmup steps the frozen c_avg is
#     the bias-corrected exponential average of the per-step coefficients
@pytest.mark.parametrize("d", [0.5, 0.9])
def test_p20_ema_c_avg(d):
    numels = [4096, 500, 3]
    N, W, T = sum(numels), 2, 7
    r = rng(43)
    h = hp(c_avg_decay=d)
    x = f32(r.standard_normal(N) * 0.02)
    m, v = np.zeros(N, np.float32), np.zeros(N, np.float32)
    c_sum = np.zeros(3, np.float32)
    cs = []
    for _ in range(T):
        g = [f32(r.standard_normal(N) * 10 ** r.uniform(-4, -2)) for _ in range(W)]
        cs.append(oracle.warmup_step(numels, g, x, m, v, c_sum, h).astype(np.float64))
    c_avg = np.zeros(3, np.float32)
    oracle.freeze(numels, v, v.copy(), [np.zeros(N, np.float32)] * W, np.zeros(N, np.float32),
                  c_sum, T, c_avg, np.zeros(3, np.float32), h)
    wts = np.array([(1 - d) * d ** (T - 1 - t) for t in range(T)])
    want = (wts[:, None] * np.array(cs)).sum(axis=0) / wts.sum()
    assert np.all(np.abs(c_avg - want) <= 4 * T * U * want)
    # and the mean (default) is the plain average
    c_avg2 = np.zeros(3, np.float32)
    oracle.freeze(numels, v, v.copy(), [np.zeros(N, np.float32)] * W, np.zeros(N, np.float32),
                  f32(np.sum(cs, axis=0)), T, c_avg2, np.zeros(3, np.float32))
    assert np.all(np.abs(c_avg2 - np.mean(cs, axis=0)) <= 2 * U * np.mean(cs, axis=0))


# P21 norm-ratio factor: rho = ||sqrt(v_frozen)+eta|| / ||sqrt(v_fresh)+eta||
#     is a weighted mean of the element ratios q, so it equals the common q
#     when they agree, lies between min q and max q, and for two equal halves
#     with equal denominators is the root mean square of the two ratios
def _run_zero_ghat_hp(numels, vfz, vf, h):
    N = sum(numels)
    r = rng(44)
    m = _constant_magnitude_state(numels, r.uniform(1e-4, 1e-2, len(numels)), r)
    x = f32(r.standard_normal(N) * 0.02)
    g = [np.zeros(N, np.float32)] * 2
    err_w = [np.zeros(N, np.float32) for _ in range(2)]
    L = len(numels)
    return oracle.compressed_step(numels, 4096, g, err_w, np.zeros(N, np.float32), x, m, vfz, vf,
                                  np.ones(L, np.float32), np.ones(L, np.float32), h)


def test_p21_norm_ratio_factor():
    numels = [4096, 4096, 4096]
    N = sum(numels)
    r = rng(45)
    h = hp(rho_mode=1, eta=0.0, kappa=1000.0, f_min=0.0, f_max=1e30)
    vfz = np.empty(N, np.float32)
    vf = np.empty(N, np.float32)
    vfz[:4096] = 4e-6                             # tensor 0: every q equal
    vf[:4096] = 1e-6
    vfz[4096:8192] = f32(r.uniform(1e-8, 1e-4, 4096))   # tensor 1: random
    vf[4096:8192] = f32(r.uniform(1e-8, 1e-4, 4096))
    vfz[8192:8192 + 2048] = 9e-6                  # tensor 2: two halves, one denominator
    vfz[8192 + 2048:] = 1e-6
    vf[8192:] = 4e-6
    vfz0, vf0 = vfz.copy(), vf.copy()
    out = _run_zero_ghat_hp(numels, vfz, vf, h)
    vf_new = (np.float32(0.999) * vf0).astype(np.float64)
    q = np.sqrt(vfz0.astype(np.float64)) / np.sqrt(vf_new)
    c = out["c"].astype(np.float64)
    assert abs(c[0] / q[0] - 1) <= 8 * U
    assert q[4096:8192].min() * (1 - 4 * U) <= c[1] <= q[4096:8192].max() * (1 + 4 * U)
    assert abs(c[1] / q[4096:8192].max() - 1) > 1e-3        # not the max reading
    rms = math.sqrt((q[8192] ** 2 + q[-1] ** 2) / 2)
    assert abs(c[2] / rms - 1) <= 8 * U
    # the default reading on the same state is the max
    out2 = _run_zero_ghat_hp(numels, vfz0.copy(), vf0.copy(), hp(eta=0.0, kappa=1000.0, f_min=0.0,
                                                                   f_max=1e30))
    assert abs(out2["c"][1] / q[4096:8192].max() - 1) <= 8 * U


# P27 a NaN rescale ratio anywhere in a tensor makes rho_l NaN (reading R13:
#     one sign bit cannot encode an undefined value, so the tensor has no
#     defined factor).  C10's fminf then drops it, so f is the clamp of
#     f_prev alone: max(min(f_max, kp*f_prev), f_min, km*f_prev) = kp here.
#     A tensor without NaN keeps f = rho = its exact maximum ratio.
@pytest.mark.parametrize("where", [0, 1, 1234, 4094, 4095])
def test_p27_nan_ratio_makes_rho_nan(where):
    numels = [4096, 4096]
    N = sum(numels)
    vfz = np.full(N, 1e-6, np.float32)
    vf = np.full(N, 1e-6, np.float32)
    vfz[where] = np.nan                            # q is NaN at one element of tensor 0
    out = _run_zero_ghat_hp(numels, vfz, vf, hp(eta=0.0))
    kp = np.float32(1.0) + np.float32(0.1)
    assert out["c"][0] == kp                       # c_avg = f_prev = 1
    # tensor 1: every q = sqrt(1e-6) / sqrt(0.999 * 1e-6) in fp32, inside the thresholds
    q = np.sqrt(np.float32(1e-6)) / np.sqrt(np.float32(0.999) * np.float32(1e-6))
    assert 1.0 < q < kp and out["c"][1] == q


# ---------------------------------------------------------------------------
# SLAMB-style sparse compression stage
# ---------------------------------------------------------------------------
def _selected_mask(N, C, nsel, sel):
    """Independent enumeration of the transmitted positions: blocks
    sel[k], sel[k]+1, ... (nsel of them, modulo C/64) of every chunk."""
    mask = np.zeros(N, bool)
    nb = C // 64
    for k, b0 in enumerate(sel):
        for j in range(nsel):
            b = (b0 + j) % nb
            lo = k * C + b * 64
            mask[lo:min(lo + 64, N)] = True
    return mask


def _sparse_state(numels, W, seed, m_std=1e-3):
    N = sum(numels)
    r = rng(seed)
    return dict(x=f32(r.standard_normal(N) * 0.02), m=f32(r.standard_normal(N) * m_std),
                vfz=f32(r.uniform(1e-8, 1e-4, N)), vf=f32(r.uniform(1e-8, 1e-4, N)),
                e=[f32(r.standard_normal(N) * 1e-4) for _ in range(W)],
                g=[f32(r.standard_normal(N) * 1e-3) for _ in range(W)], r=r)


# P22 selection, masking and local error compensation: exactly the chosen
#     blocks are transmitted (in cyclic block order), the momentum is zero
#     elsewhere, nothing outside moves, and transmitted + kept = accumulated
@pytest.mark.parametrize("nsel", [1, 3])
def test_p22_sparse_selection_masking_and_ef(nsel):
    numels = [4096 * 2 + 1000, 700]
    N, C, W = sum(numels), 4096, 3
    st = _sparse_state(numels, W, 50)
    K = oracle.num_chunks(N, C)
    sel = st["r"].integers(0, C // 64, K).astype(np.int32)
    sel[-1] = 27 - (nsel - 1)            # the partial chunk's blocks straddle its end
    mask = _selected_mask(N, C, nsel, sel)
    x0, m0, vf0 = st["x"].copy(), st["m"].copy(), st["vf"].copy()
    e0 = [e.copy() for e in st["e"]]
    out = oracle.sparse_step(numels, C, nsel, sel, st["g"], st["e"], st["x"], st["m"], st["vfz"],
                             st["vf"], np.ones(2, np.float32), hp())
    assert np.all(st["m"][~mask] == 0) and np.all(st["x"][~mask] == x0[~mask])
    assert np.all(st["vf"][~mask] == vf0[~mask])
    assert np.all(st["m"][mask] != 0) and np.all(st["x"][mask] != x0[mask])
    for w in range(W):
        assert np.all(st["e"][w][mask] == 0)
        # transmitted value + kept error = the worker's accumulated momentum
        sent = np.zeros(N, np.float64)
        pos = np.flatnonzero(mask)
        sent[pos] = _gather(out["vals_w"][w], pos, C, nsel, sel)
        b1 = float(np.float32(0.9))
        a1 = float(np.float32(1) - np.float32(0.9))
        t1, t2 = b1 * m0.astype(np.float64), a1 * st["g"][w].astype(np.float64)
        acc = t1 + t2 + e0[w]
        bound = 4 * U * (np.abs(t1) + np.abs(t2) + np.abs(e0[w]))
        assert np.all(np.abs(sent + st["e"][w] - acc) <= bound)
    # the server's values are the workers' mean, in the same order
    vw = np.array([v.astype(np.float64) for v in out["vals_w"]])
    mean = vw.mean(axis=0)
    bound = W * U * np.abs(vw).mean(axis=0) + U * np.abs(mean)
    assert np.all(np.abs(out["vals_s"] - mean) <= bound)
    # per full chunk exactly nsel*64 values; past the buffer's end zeros
    per = nsel * 64
    assert np.count_nonzero(out["vals_s"][:per * (K - 1)]) == per * (K - 1)
    assert np.count_nonzero(out["vals_s"][per * (K - 1):]) == int(mask[(K - 1) * C:].sum())


def _gather(vals, pos, C, nsel, sel):
    """Values at flat positions `pos` from a transmitted array laid out as
    nsel*64 per chunk, blocks in cyclic order from sel[k]."""
    nb = C // 64
    k = pos // C
    j = pos - k * C
    rel = ((j // 64) - sel[k]) % nb
    return vals[k * nsel * 64 + rel * 64 + j % 64].astype(np.float64)


# P23 every block selected and the rescale pinned to 1: the sparse stage is
#     the 1-bit LAMB stage with the identity compressor (and f = 1), which
#     P3 pins to textbook momentum SGD
def test_p23_sparse_dense_limit_is_identity_compressor():
    numels = [4096 + 300, 4096]
    N, C, W = sum(numels), 4096, 2
    h = hp(f_min=1.0, f_max=1.0, kappa=1e6)
    a = _sparse_state(numels, W, 51)
    b = {k: ([e.copy() for e in v] if isinstance(v, list) else v.copy()) for k, v in a.items()
         if k != "r"}
    for e in a["e"] + b["e"]:
        e[:] = 0
    K = oracle.num_chunks(N, C)
    c_avg = np.array([1.5, 0.75], np.float32)
    for step in range(3):
        sel = a["r"].integers(0, C // 64, K).astype(np.int32)
        oracle.sparse_step(numels, C, C // 64, sel, a["g"], a["e"], a["x"], a["m"], a["vfz"],
                           a["vf"], c_avg, h)
        oracle.compressed_step(numels, C, b["g"], b["e"], np.zeros(N, np.float32), b["x"], b["m"],
                               b["vfz"], b["vf"], c_avg, np.ones(2, np.float32), h,
                               compressor=oracle.IDENTITY)
        for k in ("x", "m", "vf"):
            assert np.array_equal(a[k], b[k]), (step, k)
        assert all(np.all(e == 0) for e in a["e"])


# P24 element-wise rescale in closed form: with zero gradients, zero errors
#     and identical workers the average is beta1*m exactly, the reconstructed
#     gradient is 0, v_fresh decays by beta2, and each selected element moves
#     by lr*c*clamp(q)*mhat/(sqrt(v_frozen)+eta) with q from the decayed v_fresh
def test_p24_sparse_elementwise_rescale_closed_form():
    numels = [4096 * 2]
    N, C, W = sum(numels), 4096, 2
    r = rng(52)
    m = f32(np.where(r.random(N) < 0.5, -1.0, 1.0) * 3e-3)
    vfz = f32(r.uniform(1e-6, 1e-5, N))
    vf = f32(vfz.astype(np.float64) * r.uniform(0.01, 100.0, N))   # q from 0.1 to 10
    x = f32(r.standard_normal(N) * 0.02)
    x0, vf0, m0 = x.copy(), vf.copy(), m.copy()
    g = [np.zeros(N, np.float32)] * W
    e = [np.zeros(N, np.float32) for _ in range(W)]
    sel = np.array([5, 60], np.int32)
    nsel = 16
    mask = _selected_mask(N, C, nsel, sel)
    h = hp(eta=0.0)
    oracle.sparse_step(numels, C, nsel, sel, g, e, x, m, vfz, vf, np.array([2.0], np.float32), h)
    mhat = (np.float32(0.9) * m0).astype(np.float64)
    assert np.array_equal(m[mask], mhat[mask].astype(np.float32))
    vf_new = (np.float32(0.999) * vf0)
    assert np.array_equal(vf[mask], vf_new[mask])
    q = np.sqrt(vfz.astype(np.float64)) / np.sqrt(vf_new.astype(np.float64))
    rr = np.clip(q, 0.5, 4.0)
    assert np.any(q[mask] < 0.5) and np.any(q[mask] > 4.0)      # both clamps bind
    want = x0.astype(np.float64) - 1e-3 * 2.0 * rr * mhat / np.sqrt(vfz.astype(np.float64))
    assert np.all(np.abs(x[mask] - want[mask]) <= 2 * U * np.abs(want[mask]) + 8 * U * 1e-3 * 2.0 *
                  np.abs(rr * mhat / np.sqrt(vfz.astype(np.float64)))[mask])


# P25 the warmup coefficients accumulate: after T warmup steps (default
#     reading) c_sum is the sum of the T per-step coefficients the steps
#     returned, and the freeze makes c_avg their mean
def test_p25_warmup_coefficients_accumulate():
    numels = [4096, 500, 3]
    N, W, T = sum(numels), 2, 6
    r = rng(53)
    h = hp(c_min=1e-4)                                        # no coefficient at a clip bound
    x = f32(r.standard_normal(N) * 0.1)
    m, v = np.zeros(N, np.float32), np.zeros(N, np.float32)
    c_sum = np.zeros(3, np.float32)
    cs = []
    for _ in range(T):
        g = [f32(r.standard_normal(N) * 10 ** r.uniform(-4, -2)) for _ in range(W)]
        cs.append(oracle.warmup_step(numels, g, x, m, v, c_sum, h).astype(np.float64))
    total = np.sum(cs, axis=0)
    assert len(set(map(tuple, cs))) == T and np.all(np.array(cs) > 1e-4)   # they vary, unclipped
    assert np.all(np.abs(c_sum - total) <= T * U * total)
    c_avg = np.zeros(3, np.float32)
    oracle.freeze(numels, v, v.copy(), [np.zeros(N, np.float32)] * W, np.zeros(N, np.float32),
                  c_sum, T, c_avg, np.zeros(3, np.float32), h)
    assert np.all(np.abs(c_avg - total / T) <= (T + 1) * U * total / T)


# P26 norm-ratio factor of a tensor whose sums vanish (eta = 0, zero
#     variances and momentum): the ratio is taken as 1, as for the trust
#     ratio, so f = 1 and c = c_avg; the other tensor is unaffected
def test_p26_norm_ratio_zero_sums():
    numels = [4096, 4096]
    N = sum(numels)
    r = rng(54)
    h = hp(rho_mode=1, eta=0.0)
    vfz = np.zeros(N, np.float32)
    vfz[4096:] = f32(r.uniform(1e-8, 1e-4, 4096))
    vf = vfz.copy()
    m = np.zeros(N, np.float32)
    m[4096:] = f32(r.standard_normal(4096) * 1e-3)
    x = f32(r.standard_normal(N) * 0.02)
    g = [np.zeros(N, np.float32)] * 2
    err_w = [np.zeros(N, np.float32) for _ in range(2)]
    c_avg = np.array([0.75, 0.75], np.float32)
    with np.errstate(invalid="ignore"):
        out = oracle.compressed_step(numels, 4096, g, err_w, np.zeros(N, np.float32), x, m, vfz, vf,
                                     c_avg, np.ones(2, np.float32), h)
    assert out["c"][0] == np.float32(0.75)
    assert np.isfinite(out["c"][1]) and np.all(np.isfinite(x[4096:]))
