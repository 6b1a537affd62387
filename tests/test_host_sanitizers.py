"""Host sanitizers over the C boundary: the ABI's host code (argument
checks, launch plans, workspace and saved-buffer layouts) built with
AddressSanitizer and UndefinedBehaviorSanitizer
(tests/c_abi/build_host_sanitized.sh), then the CPU ABI tests
(tests/test_abi_cpu.py) run against that build in a child process with the
sanitizer runtime preloaded.  Any report fails the child, and this test.
No GPU is touched: every call in those tests returns before a launch."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = os.path.join(ROOT, "tests", "c_abi", "build_host_sanitized.sh")
OBJ = os.path.join(ROOT, "rank_latent_attention_mixer_amd", "_build")


def test_abi_under_address_and_undefined_sanitizers(tmp_path):
    if not (os.path.exists("/opt/rocm/bin/hipcc") and os.path.exists("/opt/rocm/llvm/bin/clang++")):
        pytest.skip("ROCm compilers not present")
    if not os.path.exists(os.path.join(OBJ, "encode_split.o")):
        pytest.skip("package objects not built (run the package build)")
    out = str(tmp_path / "hsan")
    r = subprocess.run(["bash", SCRIPT, out], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    runtime = open(os.path.join(out, "asan_runtime.txt")).read().strip()
    if not os.path.exists(runtime):
        pytest.skip("sanitizer runtime not present")
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, FLAREPP_LIBRARY=os.path.join(out, "libflarepp.so"),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-p", "no:cacheprovider", "-x"],
                       capture_output=True, text=True, timeout=900, env=env, cwd=str(tmp_path))
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in log
    shutil.rmtree(out, ignore_errors=True)
