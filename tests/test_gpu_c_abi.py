"""The C boundary used from plain C: tests/c_abi/flarepp_c_check.c (built by
the package build with gcc against libflarepp.so and the HIP runtime, no
Python or torch in the process) allocates device memory, calls
flarepp_mixer_fwd on cases whose outputs follow in closed form (a single
token gives y = v; a closed gate with q_fixed = 0 gives y = mean_n v), and
checks an argument error."""

from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "flarepp_c_check")

pytestmark = pytest.mark.gpu


def test_c_client_closed_forms():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BIN):
        pytest.fail("tests/c_abi/flarepp_c_check is not built (run the package build)")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all passed" in r.stdout
    assert r.stdout.count("\nok ") + r.stdout.startswith("ok ") >= 3
