"""The host side of bench.py, on the CPU: the refusal of more than one GPU,
the algorithmic byte counts behind every GB/s it reports, and the gate that
drops the counter-measured traffic once the kernel sources have changed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stdout + res.stderr


def _per_array_bytes(N, K, C, W, arrays):
    """Sum of the bytes of the listed arrays: fp32 element arrays are 4N,
    a packed sign-and-scale array is K chunks of C/8 + 4 bytes."""
    packed = K * (C // 8 + 4)
    return sum(4 * N if kind == "f32" else packed for kind in arrays)


@pytest.mark.parametrize("name", ["tiny", "single", "bert_large", "bert_xl"])
def test_byte_counts_list_every_array_once(name):
    wl = WORKLOADS[name]
    N, K, C, W = wl.N, wl.K, wl.chunk, wl.W
    phase1 = (["f32"]                                   # m read
              + ["f32"] * W                             # gradients read
              + ["f32"] * (2 * W)                       # worker errors read and written
              + ["f32"] * 2                             # server error read and written
              + ["f32"] * 3                             # v_fresh read and written, v_frozen read
              + ["packed"] * (W + 1))                   # worker and server signs and scales
    assert bench.phase1_bytes(N, K, C, W) == _per_array_bytes(N, K, C, W, phase1)
    # the whole step adds x read and written and m written; v_frozen and the
    # server's packed output, read again by the update, count once
    step = phase1 + ["f32"] * 3
    assert bench.step_bytes(N, K, C, W) == _per_array_bytes(N, K, C, W, step)
    # packed momentum: m is read as the previous packed output, not written
    packed_step = phase1[1:] + ["packed"] + ["f32"] * 2
    assert bench.step_bytes_packed(N, K, C, W) == _per_array_bytes(N, K, C, W, packed_step)
    # 1-bit Adam, both kernels: the allreduce (phase 1 without the fresh and
    # frozen variances), then the update reading the server's packed output
    # back, x read and written, v_frozen read and m written
    adam = phase1[:-(W + 4)] + ["packed"] * (W + 1) + ["packed"] + ["f32"] * 4
    assert bench.adam_bytes(N, K, C, W) == _per_array_bytes(N, K, C, W, adam)


def test_phase1_bytes_match_the_committed_profile():
    """The BERT-Large phase-1 count equals the algorithmic bytes recorded in
    the committed counter summary that the bench line's traffic comes from."""
    wl = WORKLOADS["bert_large"]
    path = os.path.join(ROOT, "profiles", "traffic_compress_average_bert_large.txt")
    vals = dict(ln.split(":", 1) for ln in open(path) if ":" in ln and not ln.startswith("#"))
    assert int(vals["algorithmic_bytes_per_launch"]) == \
        bench.phase1_bytes(wl.N, wl.K, wl.chunk, wl.W) == 40_405_861_908


def test_traffic_is_dropped_when_the_kernels_change(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "t.txt").write_text("# a summary\nkernel: k\nkernel_source_sha: 0123456789abcdef\n"
                                "hbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_kernel_sha", lambda: "0123456789abcdef")
    assert bench._measured_traffic("t.txt") == 12345.0
    monkeypatch.setattr(bench, "_kernel_sha", lambda: "fedcba9876543210")
    assert bench._measured_traffic("t.txt") is None
    assert bench._measured_traffic("missing.txt") is None
