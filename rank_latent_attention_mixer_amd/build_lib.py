"""Build libflarepp.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m rank_latent_attention_mixer_amd.build_lib [--jobs N] [--verbose]

Every call recompiles.  Objects go to rank_latent_attention_mixer_amd/_build/
(git-ignored); the shared library lands next to this file, where the Python
binding loads it from.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflarepp.so")
PROBE_LIB = os.path.join(PKG, "libflarepp_probe.so")
PROBE_SOURCES = ["probe/peak_probe.hip"]

SOURCES = ["encode_split.hip", "combine.hip", "decode.hip", "backward.hip", "backward_valu.hip",
           "flarepp_abi.cpp",
           "backward_abi.cpp", "frontend.hip", "frontend_abi.cpp"]

ARCH = "gfx950"
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: the compiler would otherwise form
    # v_pk_{add,mul,fma}_f32 from scalar float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libflarepp)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + HIPCC_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "flarepp_c_check.c")
C_CHECK = os.path.join(ROOT, "tests", "c_abi", "flarepp_c_check")


def _build_c_check(verbose: bool) -> None:
    """The plain-C client the C-ABI test runs: gcc, the HIP runtime, and
    libflarepp found next to the package through a relative rpath."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    tmp = C_CHECK + ".tmp"
    cmd = [shutil.which("gcc") or "gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(rocm, "include"),
           C_CHECK_SRC, "-o", tmp, "-L" + PKG, "-lflarepp", "-L" + os.path.join(rocm, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../../rank_latent_attention_mixer_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C client build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, C_CHECK)


def build(jobs: int = 4, verbose: bool = False) -> str:
    """Builds libflarepp.so, the measurement probe libflarepp_probe.so and
    the plain-C client of the ABI (tests/c_abi)."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    _build_c_check(verbose)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
