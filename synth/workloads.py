"""Workload recipes: tensor tables, worker counts, step counts, initial
state and gradient distributions, and the optimizer's hyper-parameters.

No optimizer arithmetic lives here.  Each array is a pure function of
(seed, array id, step, worker, element index), so a window [lo, hi) of any
array can be filled on the host (for the oracle) or on the device (for the
GPU library) and the two agree bit for bit.

The shapes follow the paper's workload, BERT pre-training (BERT-Large:
hidden 1024, FFN 4096, 24 encoder blocks, 30522-token embedding; BERT-XL as
in SLAMB: 2.8B parameters, hidden 2560, FFN 10240, 36 blocks).  No weights or
data are used: parameters and gradients are synthetic.
"""
import dataclasses

import numpy as np

from . import G, M, SEL, V, X, index_host, layer_log_scales, normal_dev, normal_host, stream_id, \
    uniform_dev, uniform_host

HPARAMS = dict(beta1=0.9, beta2=0.999, eta=1e-8, lr=1e-3, weight_decay=0.0, c_min=0.01, c_max=10.0,
               f_min=0.5, f_max=4.0, kappa=0.1)


def encoder_block(h, ffn):
    """One BERT encoder block in tensor order: Wq bq Wk bk Wv bv Wo bo LN1g
    LN1b W1 b1 W2 b2 LN2g LN2b."""
    return [h * h, h, h * h, h, h * h, h, h * h, h, h, h, h * ffn, ffn, ffn * h, h, h, h]


def bert_large_table():
    return [30522 * 1024] + encoder_block(1024, 4096) * 24


def bert_xl_table():
    return encoder_block(2560, 10240) * 36


@dataclasses.dataclass
class Workload:
    name: str
    numels: list
    W: int
    chunk: int = 4096
    warmup_steps: int = 0
    compression_steps: int = 1
    init: str = "frozen"          # "fresh": m = v = 0, warmup first; "frozen": start in compression
    grad_std: float = 1e-3
    layer_scaled: bool = False    # gradient std times 10^U(-4,-1) per tensor
    x_std: float = 0.02
    m_std: float = 1e-3
    v_lo: float = 1e-8
    v_hi: float = 1e-4
    seed: int = 0

    @property
    def L(self):
        return len(self.numels)

    @property
    def N(self):
        return int(sum(self.numels))

    @property
    def K(self):
        return (self.N + self.chunk - 1) // self.chunk

    @property
    def offsets(self):
        return np.concatenate([[0], np.cumsum(np.asarray(self.numels, dtype=np.int64))])

    def grad_scales(self):
        if not self.layer_scaled:
            return np.ones(self.L, np.float64)
        return layer_log_scales(self.seed, self.L, -4.0, -1.0)

    # ---- window fills -------------------------------------------------
    def _segments(self, lo, hi):
        """(layer, a, b) pieces of [lo, hi) that lie in one tensor each."""
        off = self.offsets
        l = int(np.searchsorted(off, lo, side="right") - 1)
        while lo < hi:
            b = min(hi, int(off[l + 1]))
            yield l, lo, b
            lo = b
            l += 1

    def fill(self, array, out, lo=0, step=0, worker=0, cuda_stream=None):
        """Fill `out` (numpy float32 or a CUDA float32 tensor) with elements
        [lo, lo + len(out)) of `array` ("x", "m", "v", "g")."""
        on_dev = not isinstance(out, np.ndarray)
        n = out.numel() if on_dev else out.size
        nrm = (lambda o, s, a, mean, std: normal_dev(o, self.seed, s, a, mean, std, cuda_stream)) \
            if on_dev else (lambda o, s, a, mean, std: normal_host(o, self.seed, s, a, mean, std))
        uni = (lambda o, s, a, lo_, hi_: uniform_dev(o, self.seed, s, a, lo_, hi_, cuda_stream)) \
            if on_dev else (lambda o, s, a, lo_, hi_: uniform_host(o, self.seed, s, a, lo_, hi_))
        if n == 0:
            return out
        if array == "x":
            nrm(out, stream_id(X), lo, 0.0, self.x_std)
        elif array == "m":
            if self.init == "fresh":
                out[:] = 0
            else:
                nrm(out, stream_id(M), lo, 0.0, self.m_std)
        elif array == "v":
            if self.init == "fresh":
                out[:] = 0
            else:
                uni(out, stream_id(V), lo, self.v_lo, self.v_hi)
        elif array == "g":
            s = stream_id(G, step, worker)
            if not self.layer_scaled:
                nrm(out, s, lo, 0.0, self.grad_std)
            else:
                scales = self.grad_scales()
                for l, a, b in self._segments(lo, lo + n):
                    nrm(out[a - lo:b - lo], s, a, 0.0, self.grad_std * float(scales[l]))
        else:
            raise ValueError(array)
        return out

    def selection(self, step, k0=0, k1=None):
        """First transmitted 64-element block of chunks [k0, k1) for the
        sparse stage at `step`: uniform in [0, chunk/64), shared by all
        workers."""
        k1 = self.K if k1 is None else k1
        out = np.empty(k1 - k0, np.int32)
        return index_host(out, self.seed, stream_id(SEL, step), k0, self.chunk // 64)

    def window_table(self, lo, hi):
        """Tensor sizes of [lo, hi) clipped to the window, and the index of
        the first tensor; the first and last entries may be partial."""
        pieces = list(self._segments(lo, hi))
        return [b - a for _, a, b in pieces], (pieces[0][0] if pieces else 0), pieces


WORKLOADS = {
    "tiny": Workload("tiny", [256 * 256, 256, 1000 * 64], W=2, warmup_steps=5,
                     compression_steps=5, init="fresh", grad_std=0.02),
    "single": Workload("single", [16 * 1024 * 1024], W=4, compression_steps=1),
    "bert_large": Workload("bert_large", bert_large_table(), W=8, compression_steps=10),
    "mixed": Workload("mixed", bert_large_table(), W=8, warmup_steps=20, compression_steps=20,
                      init="fresh", layer_scaled=True),
    "bert_xl": Workload("bert_xl", bert_xl_table(), W=4, compression_steps=1),
}
