"""The C ABI from plain C on the GPU: tests/native/abi_c_check (built with
the library) runs two 1-bit LAMB compression steps and one 1-bit Adam step
through the C entry points on a ragged table and compares every output with
the CPU oracle bit for bit."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_c_check")


def test_c_caller_matches_oracle():
    assert os.path.exists(EXE), "tests/native/abi_c_check is not built; run __graft_entry__.build()"
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0 and "PASS" in res.stdout, res.stdout + res.stderr
