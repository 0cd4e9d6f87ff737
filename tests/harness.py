"""Test harness: run the GPU library (DevRun, through the C ABI) and the CPU
oracle (HostRun) on the same seeded inputs, and compare their states.

HostRun can cover a window [lo, hi) of the flat buffer that starts on a
chunk boundary: every chunk-local quantity (signs, scales, errors, moments,
fresh variance) is then exact for the window, and per-tensor quantities
(c, f_prev, the parameters x) are exact for the tensors that lie wholly
inside it.  That lets the oracle check configurations too large for it to
run whole.
"""
import numpy as np

import oracle
from synth.workloads import HPARAMS

# parity bar for fp32 values that depend on per-tensor double sums
RTOL = 1e-5
ATOL = 1e-7


class DevRun:
    """Full-size state on the GPU, stepped through the C ABI."""

    def __init__(self, wl, store_worker_bits=True, carry_norm=False):
        """carry_norm: run the warmup through onebit_lamb_warmup_step_carry,
        which carries the per-segment sums of x^2 from one warmup step to the
        next (every step but the first then skips reading x for its norm)."""
        import torch
        import communication_compressed_optimizer_amd as ob
        self.ob = ob
        self.torch = torch
        self.wl = wl
        C, N, W, K, L = wl.chunk, wl.N, wl.W, wl.K, wl.L
        dev = "cuda"
        self.table = ob.LayerTable(wl.numels, C)
        assert (self.table.N, self.table.K) == (N, K)

        def f():
            return torch.empty(N, dtype=torch.float32, device=dev)

        self.x, self.m, self.v, self.vf = f(), f(), f(), f()
        self.err_s = torch.zeros(N, dtype=torch.float32, device=dev)
        self.g = [f() for _ in range(W)]
        self.e = [torch.zeros(N, dtype=torch.float32, device=dev) for _ in range(W)]
        words = K * C // 32
        if store_worker_bits:
            self.bits_w = [torch.zeros(words, dtype=torch.int32, device=dev) for _ in range(W)]
            self.scales_w = [torch.zeros(K, dtype=torch.float32, device=dev) for _ in range(W)]
        else:
            self.bits_w = self.scales_w = None
        self.bits_s = torch.zeros(words, dtype=torch.int32, device=dev)
        self.scales_s = torch.zeros(K, dtype=torch.float32, device=dev)
        self.c_sum = torch.zeros(L, dtype=torch.float32, device=dev)
        self.c_avg = torch.ones(L, dtype=torch.float32, device=dev)
        self.f_prev = torch.ones(L, dtype=torch.float32, device=dev)
        self.c_out = torch.zeros(L, dtype=torch.float32, device=dev)
        self.ws = torch.empty(self.table.workspace_size(W), dtype=torch.uint8, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.hp = ob.onebit_hparams(**HPARAMS)
        wl.fill("x", self.x)
        wl.fill("m", self.m)
        wl.fill("v", self.v)
        self.vf.copy_(self.v)
        self.carry_norm = carry_norm
        self.x_sq = torch.zeros(self.table.n_segments, dtype=torch.float64, device=dev)
        self.x_sq_valid = 0          # x_sq does not describe x until a carried step wrote it

    def fill_grads(self, step):
        for w in range(self.wl.W):
            self.wl.fill("g", self.g[w], 0, step, w)

    def warmup_step(self, step, fill=True):
        if fill:
            self.fill_grads(step)
        if self.carry_norm:
            self.ob.onebit_lamb_warmup_step_carry(self.table, self.wl.W, self.g, self.x, self.m,
                                                  self.v, self.c_sum, self.c_out, self.x_sq,
                                                  self.x_sq_valid, self.hp, self.ws, self.status)
            self.x_sq_valid = 1
        else:
            self.ob.onebit_lamb_warmup_step(self.table, self.wl.W, self.g, self.x, self.m, self.v,
                                            self.c_sum, self.c_out, self.hp, self.ws, self.status)

    def freeze(self, T_w):
        self.ob.onebit_lamb_freeze(self.table, self.wl.W, self.v, self.vf, self.e, self.err_s,
                                   self.c_sum, T_w, self.c_avg, self.f_prev, self.hp)

    def compressed_step(self, step, fill=True, packed=False):
        """packed: the momentum is the previous step's server output
        (bits_s, scales_s) and self.m is neither read nor written."""
        self.x_sq_valid = 0
        if fill:
            self.fill_grads(step)
        self.ob.onebit_lamb_compressed_step(
            self.table, self.wl.W, self.g, self.e, self.err_s, self.x,
            None if packed else self.m, self.v, self.vf,
            self.c_avg, self.f_prev, self.c_out, self.bits_w, self.scales_w, self.bits_s,
            self.scales_s, self.hp, self.ws, self.status)

    # -- 1-bit Adam mode: v is the (frozen) variance, vf is not used ------
    def adam_warmup_step(self, step, fill=True):
        self.x_sq_valid = 0
        if fill:
            self.fill_grads(step)
        self.ob.onebit_adam_warmup_step(self.wl.N, self.wl.W, self.g, self.x, self.m, self.v,
                                        self.hp)

    def adam_compressed_step(self, step, fill=True, chunk=None, packed=False):
        self.x_sq_valid = 0
        if fill:
            self.fill_grads(step)
        self.ob.onebit_adam_compressed_step(
            self.wl.N, chunk or self.wl.chunk, self.wl.W, self.g, self.e, self.err_s, self.x,
            None if packed else self.m, self.v, self.bits_w, self.scales_w, self.bits_s,
            self.scales_s, self.hp, self.status)

    def momentum_from_packed(self):
        """The packed momentum (the server's last output) as fp32."""
        out = self.torch.empty_like(self.m)
        self.ob.onebit_decompress(self.wl.N, self.wl.chunk, self.bits_s, self.scales_s, out)
        return out

    # -- SLAMB-style sparse stage ----------------------------------------
    def sparse_step(self, step, nsel, fill=True):
        self.x_sq_valid = 0
        torch = self.torch
        if fill:
            self.fill_grads(step)
        K, W = self.wl.K, self.wl.W
        if getattr(self, "_nsel", None) != nsel:
            self._nsel = nsel
            self.vals_s = torch.zeros(K * nsel * 64, dtype=torch.float32, device="cuda")
            self.vals_w = [torch.zeros(K * nsel * 64, dtype=torch.float32, device="cuda")
                           for _ in range(W)] if self.bits_w is not None else None
        self.sel = torch.from_numpy(self.wl.selection(step)).cuda()
        self.ob.onebit_sparse_compressed_step(
            self.table, W, nsel, self.sel, self.g, self.e, self.x, self.m, self.v, self.vf,
            self.c_avg, self.vals_w, self.vals_s, self.hp, self.status)

    def sparse_window(self, lo, hi):
        C, per = self.wl.chunk, self._nsel * 64
        k0, k1 = lo // C, -(-hi // C)
        d = self.window(lo, hi)
        d["vals_s"] = self.vals_s[k0 * per:k1 * per].cpu().numpy()
        if self.vals_w is not None:
            d["vals_w"] = [v[k0 * per:k1 * per].cpu().numpy() for v in self.vals_w]
        return d

    # -- window download -------------------------------------------------
    def window(self, lo, hi):
        C = self.wl.chunk
        k0, k1 = lo // C, -(-hi // C)
        f = lambda t: t[lo:hi].cpu().numpy()
        out = {"x": f(self.x), "m": f(self.m), "v": f(self.v), "vf": f(self.vf),
               "err_s": f(self.err_s), "e": [f(e) for e in self.e],
               "bits_s": self.bits_s[k0 * C // 32:k1 * C // 32].cpu().numpy().view(np.uint32),
               "scales_s": self.scales_s[k0:k1].cpu().numpy(),
               "c_sum": self.c_sum.cpu().numpy(), "c_avg": self.c_avg.cpu().numpy(),
               "f_prev": self.f_prev.cpu().numpy(), "c": self.c_out.cpu().numpy()}
        if self.bits_w is not None:
            out["bits_w"] = [b[k0 * C // 32:k1 * C // 32].cpu().numpy().view(np.uint32)
                             for b in self.bits_w]
            out["scales_w"] = [s[k0:k1].cpu().numpy() for s in self.scales_w]
        return out


class HostRun:
    """The oracle on the window [lo, hi) of the same workload."""

    def __init__(self, wl, lo=0, hi=None):
        C = wl.chunk
        hi = wl.N if hi is None else hi
        assert lo % C == 0 and (hi % C == 0 or hi == wl.N) and 0 <= lo < hi <= wl.N
        self.wl, self.lo, self.hi = wl, lo, hi
        self.numels, self.l_first, pieces = wl.window_table(lo, hi)
        off = wl.offsets
        # window-local indices of the tensors that lie wholly inside
        self.full = np.array([i for i, (l, a, b) in enumerate(pieces)
                              if a == off[l] and b == off[l + 1]], dtype=np.int64)
        self.layers = np.arange(self.l_first, self.l_first + len(self.numels))
        self.pieces = pieces
        n = hi - lo
        z = lambda: np.zeros(n, np.float32)
        self.x, self.m, self.v = z(), z(), z()
        wl.fill("x", self.x, lo)
        wl.fill("m", self.m, lo)
        wl.fill("v", self.v, lo)
        self.vf = self.v.copy()
        self.err_s = z()
        self.e = [z() for _ in range(wl.W)]
        self.g = [z() for _ in range(wl.W)]
        Lw = len(self.numels)
        self.c_sum = np.zeros(Lw, np.float32)
        self.c_avg = np.ones(Lw, np.float32)
        self.f_prev = np.ones(Lw, np.float32)
        self.c = np.zeros(Lw, np.float32)
        self.out = None
        self.hp = oracle.hparams(**HPARAMS)

    def fill_grads(self, step):
        for w in range(self.wl.W):
            self.wl.fill("g", self.g[w], self.lo, step, w)

    def warmup_step(self, step, fill=True):
        if fill:
            self.fill_grads(step)
        self.c = oracle.warmup_step(self.numels, self.g, self.x, self.m, self.v, self.c_sum, self.hp)

    def freeze(self, T_w):
        oracle.freeze(self.numels, self.v, self.vf, self.e, self.err_s, self.c_sum, T_w, self.c_avg,
                      self.f_prev, self.hp)

    def compressed_step(self, step, fill=True):
        if fill:
            self.fill_grads(step)
        self.out = oracle.compressed_step(self.numels, self.wl.chunk, self.g, self.e, self.err_s,
                                          self.x, self.m, self.v, self.vf, self.c_avg, self.f_prev,
                                          self.hp)
        self.c = self.out["c"]

    def adam_warmup_step(self, step, fill=True):
        if fill:
            self.fill_grads(step)
        oracle.adam_warmup_step(self.g, self.x, self.m, self.v, self.hp)

    def adam_compressed_step(self, step, fill=True):
        if fill:
            self.fill_grads(step)
        self.out = oracle.adam_compressed_step(self.wl.chunk, self.g, self.e, self.err_s, self.x,
                                               self.m, self.v, self.hp)

    def sparse_step(self, step, nsel, fill=True):
        if fill:
            self.fill_grads(step)
        C = self.wl.chunk
        sel = self.wl.selection(step, self.lo // C, -(-self.hi // C))
        self.out = oracle.sparse_step(self.numels, C, nsel, sel, self.g, self.e, self.x, self.m,
                                      self.v, self.vf, self.c_avg, self.hp)

    def load_from(self, d):
        """Adopt a downloaded GPU window (strict per-step parity)."""
        for k in ("x", "m", "v", "vf", "err_s"):
            getattr(self, k)[:] = d[k]
        for w in range(self.wl.W):
            self.e[w][:] = d["e"][w]
        sl = self.layers
        self.c_sum[:] = d["c_sum"][sl]
        self.c_avg[:] = d["c_avg"][sl]
        self.f_prev[:] = d["f_prev"][sl]


def _close(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    bad = ~(err <= ATOL + RTOL * np.abs(b))
    bad |= np.isnan(a) != np.isnan(b)
    return bad


def _entry(bad, a, b, exact):
    a = np.asarray(a)
    b = np.asarray(b)
    diff = np.abs(a.astype(np.float64) - b.astype(np.float64)) if a.size else np.zeros(0)
    return {"ok": not bool(np.any(bad)), "n_bad": int(np.sum(bad)), "n": int(a.size),
            "max_abs": float(diff.max()) if diff.size else 0.0, "exact": exact}


def compare_state(dev, host, d=None, stage="compression"):
    """Element-by-element comparison of the GPU window with the oracle.
    Bit-exact: signs, scales, errors, m, v, v_fresh.  Within tolerance:
    x (tensors wholly inside the window), c, c_sum, c_avg, f_prev."""
    if d is None:
        d = dev.window(host.lo, host.hi)
    rep = {}

    def exact(name, a, b):
        a = np.asarray(a)
        b = np.asarray(b)
        bad = a.view(np.uint32) != b.view(np.uint32) if a.dtype.itemsize == 4 else a != b
        rep[name] = _entry(bad, a, b, True)

    def close(name, a, b):
        rep[name] = _entry(_close(a, b), a, b, False)

    for k in ("m", "v", "vf", "err_s"):
        exact(k, d[k], getattr(host, k))
    for w in range(host.wl.W):
        exact(f"e{w}", d["e"][w], host.e[w])
    if host.out is not None and stage == "compression":
        exact("bits_s", d["bits_s"], host.out["bits_s"])
        exact("scales_s", d["scales_s"], host.out["scales_s"])
        if "bits_w" in d:
            for w in range(host.wl.W):
                exact(f"bits_w{w}", d["bits_w"][w], host.out["bits_w"][w])
                exact(f"scales_w{w}", d["scales_w"][w], host.out["scales_w"][w])
    # x on the tensors wholly inside the window
    off_w = np.concatenate([[0], np.cumsum(host.numels)])
    idx = np.concatenate([np.arange(off_w[i], off_w[i + 1]) for i in host.full]) \
        if host.full.size else np.zeros(0, np.int64)
    close("x", d["x"][idx], host.x[idx])
    gl = host.layers[host.full]
    for k, hk in (("c", host.c), ("c_sum", host.c_sum), ("c_avg", host.c_avg),
                  ("f_prev", host.f_prev)):
        close(k, d[k][gl], hk[host.full])
    return rep


def compare_adam(dev, host, d=None):
    """1-bit Adam: every array of the window bit for bit (there is no
    per-tensor quantity, so x is exact on every element too)."""
    if d is None:
        d = dev.window(host.lo, host.hi)
    rep = {}

    def exact(name, a, b):
        a = np.asarray(a)
        b = np.asarray(b)
        rep[name] = _entry(a.view(np.uint32) != b.view(np.uint32), a, b, True)

    for k in ("x", "m", "v", "err_s"):
        exact(k, d[k], getattr(host, k))
    for w in range(host.wl.W):
        exact(f"e{w}", d["e"][w], host.e[w])
    if host.out is not None:
        exact("bits_s", d["bits_s"], host.out["bits_s"])
        exact("scales_s", d["scales_s"], host.out["scales_s"])
        if "bits_w" in d:
            for w in range(host.wl.W):
                exact(f"bits_w{w}", d["bits_w"][w], host.out["bits_w"][w])
                exact(f"scales_w{w}", d["scales_w"][w], host.out["scales_w"][w])
    return rep


def compare_sparse(dev, host):
    """Sparse stage: every array of the window bit for bit (all of it is
    element-wise)."""
    d = dev.sparse_window(host.lo, host.hi)
    rep = {}

    def exact(name, a, b):
        a = np.asarray(a)
        b = np.asarray(b)
        rep[name] = _entry(a.view(np.uint32) != b.view(np.uint32), a, b, True)

    for k in ("m", "v", "vf"):
        exact(k, d[k], getattr(host, k))
    # x on the tensors wholly inside the window (c_avg is per tensor)
    off_w = np.concatenate([[0], np.cumsum(host.numels)])
    idx = np.concatenate([np.arange(off_w[i], off_w[i + 1]) for i in host.full]) \
        if host.full.size else np.zeros(0, np.int64)
    exact("x", d["x"][idx], host.x[idx])
    for w in range(host.wl.W):
        exact(f"e{w}", d["e"][w], host.e[w])
    exact("vals_s", d["vals_s"], host.out["vals_s"])
    if "vals_w" in d:
        for w in range(host.wl.W):
            exact(f"vals_w{w}", d["vals_w"][w], host.out["vals_w"][w])
    return rep


def assert_parity(rep, where=""):
    bad = {k: v for k, v in rep.items() if not v["ok"]}
    assert not bad, f"parity failed {where}: {bad}"
