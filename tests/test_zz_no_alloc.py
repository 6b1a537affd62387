"""The allocation-free forward (flarepp_mixer_fwd_noalloc) against
flarepp_mixer_fwd through the C ABI: same kernels and token chunking, so
the outputs must agree bit for bit.  Two calls in a row, the second with a
smaller input, then the first shape again (the library's per-device array
keeps the previous call's contents; nothing in it may leak into a result),
and the first output also against the fp64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from flarepp_workloads import make_random_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
NAMES = ("q0", "q_fixed", "gate", "k0", "k", "v")


@pytest.fixture(scope="module")
def fp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_attention_mixer_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def _dev(x, dtype):
    out = {}
    for n in NAMES:
        t = torch.from_numpy(np.ascontiguousarray(x[n]))
        out[n] = (t if n == "gate" else t.to(TDT[dtype])).cuda()
    return out


def _both(fp, shape, dtype, seed, gate):
    B, H, N, M, D = shape
    print(f"[noalloc] case B{B} H{H} N{N} M{M} D{D} {dtype} seed {seed}", flush=True)
    x = make_random_inputs(B, H, N, M, D, dtype, seed=seed, gate=gate)
    d = _dev(x, dtype)
    args = [d[n] for n in NAMES]
    y_ref = fp.flarepp_mixer_fwd(*args)
    y = torch.full_like(y_ref, float("nan"))
    out = fp.flarepp_mixer_fwd_noalloc(*args, y=y)
    torch.cuda.synchronize()
    assert out is y
    return x, y_ref.float().cpu().numpy(), y.float().cpu().numpy()


def test_noalloc_matches_the_workspace_forward(fp):
    big = (2, 4, 3000, 64, 32)
    gate = np.array([-np.inf, 0.3, -1.2, 2.0])
    x, y_ref, y = _both(fp, big, "bf16", 11, gate)
    assert np.array_equal(y, y_ref)
    ref = oracle.flarepp_ref(*(np.asarray(x[n], np.float64) for n in NAMES))
    err = float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))
    print(f"[noalloc] first call vs oracle {err:.2e}", flush=True)
    assert err <= 2e-2
    # a smaller input next: other dtype, ragged N and M, D = 16
    _, y_ref2, y2 = _both(fp, (1, 2, 777, 40, 16), "fp16", 12, np.array([0.5, -0.5]))
    assert np.array_equal(y2, y_ref2)
    # and the first shape again, other inputs
    _, y_ref3, y3 = _both(fp, big, "bf16", 13, np.array([1.0, -np.inf, 0.0, -0.4]))
    assert np.array_equal(y3, y_ref3)
