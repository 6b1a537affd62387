"""GPU parity of the block front end (three head-split projections, k0 and
the seeds normalised head-wise) against the fp64 oracle
(oracle.frontend_ref / oracle.seed_norm_ref), through the C ABI.

Inputs are rounded to the operand type before both sides see them; the
kernel accumulates in fp32 and rounds its outputs to the operand type, so
the bar is max|out - ref| / max|ref| <= 1e-2 per tensor (the output rounding
alone is 2^-9 relative)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from flarepp_workloads import make_frontend_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}
TOL = 1e-2


@pytest.fixture(scope="module")
def fp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_attention_mixer_amd as m
    m.load_library()
    return m


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(TDT[dtype]).cuda()


def rel_err(g, ref):
    g = np.asarray(g, np.float64)
    return float(np.max(np.abs(g - ref)) / np.max(np.abs(ref)))


def run(fp, x, normalize=True, eps=1e-6):
    dt = x["dtype"]
    d = {n: dev(x[n], dt) for n in ("x", "w_k0", "w_k", "w_v", "b_k0", "b_k", "b_v", "g_k0")}
    k0, k, v = fp.flarepp_frontend_fwd(d["x"], d["w_k0"], d["w_k"], d["w_v"], x["H"],
                                       b_k0=d["b_k0"], b_k=d["b_k"], b_v=d["b_v"],
                                       g_k0=d["g_k0"], eps=eps, normalize_k0=normalize)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (k0, k, v)]


def ref_of(x, normalize=True, eps=1e-6, tokens=None):
    xx = x["x"] if tokens is None else x["x"][:, tokens]
    return oracle.frontend_ref(xx, x["w_k0"], x["w_k"], x["w_v"], x["H"], x["D"],
                               b_k0=x["b_k0"], b_k=x["b_k"], b_v=x["b_v"], g_k0=x["g_k0"],
                               eps=eps, normalize_k0=normalize)


CASES = [
    # (B, N, C, H, D, dtype, bias, gain)
    (2, 300, 64, 2, 32, "bf16", True, True),
    (1, 1000, 256, 8, 32, "bf16", True, True),     # the headline block width
    (2, 77, 48, 3, 16, "fp16", False, True),       # C not a multiple of the K step; F = 144
    (1, 513, 1024, 16, 64, "fp16", True, False),   # wide heads
    (3, 129, 32, 1, 64, "bf16", True, True),       # one head, F < one tile
    (1, 1, 16, 2, 16, "bf16", False, False),       # a single token
    # resident-weight kernel (C a multiple of 64 up to 256)
    (3, 50, 192, 4, 16, "fp16", True, True),       # C = 192; blocks straddle batches
    (1, 700, 128, 6, 64, "bf16", True, True),      # F = 1152: last feature group half used
    (2, 5, 256, 8, 32, "bf16", True, True),        # N < one block: one block over two batches
    (1, 4097, 64, 1, 16, "fp16", False, False),    # F = 48, one wave; ragged last block
    (2, 300, 256, 4, 64, "fp16", True, True),      # C = 256 at D = 64
]


@pytest.mark.parametrize("B,N,C,H,D,dtype,bias,gain", CASES)
def test_frontend_vs_oracle(fp, B, N, C, H, D, dtype, bias, gain):
    note(f"[frontend] B={B} N={N} C={C} H={H} D={D} {dtype} bias={bias} gain={gain}")
    x = make_frontend_inputs(B, N, C, H, D, dtype, seed=N + C, bias=bias, gain=gain)
    got = run(fp, x)
    ref = ref_of(x)
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    note(f"[frontend] errors k0 {errs[0]:.2e} k {errs[1]:.2e} v {errs[2]:.2e}")
    assert max(errs) <= TOL, errs
    # the head-wise normalisation: unit mean square over D (up to the gain and rounding)
    if not gain:
        ms = np.mean(got[0].astype(np.float64) ** 2, axis=-1)
        assert np.allclose(ms, 1.0, atol=2e-2)


def test_frontend_without_normalisation(fp):
    x = make_frontend_inputs(2, 200, 64, 4, 16, "bf16", seed=3)
    got = run(fp, x, normalize=False)
    ref = ref_of(x, normalize=False)
    assert max(rel_err(g, r) for g, r in zip(got, ref)) <= TOL


def test_frontend_million_tokens_sampled(fp):
    """Block width of the million-token workload (C = H D = 256, H = 8, D =
    32) at its full size; the oracle computes 4096 sampled tokens."""
    B, N, C, H, D = 1, 1 << 20, 256, 8, 32
    note(f"[frontend] B={B} N={N} C={C} H={H} D={D} bf16")
    x = make_frontend_inputs(B, N, C, H, D, "bf16", seed=11)
    got = run(fp, x)
    tok = np.sort(np.random.Generator(np.random.PCG64(12)).choice(N, 4096, replace=False))
    tok[-1] = N - 1
    ref = ref_of(x, tokens=tok)
    errs = [rel_err(g[:, :, tok], r) for g, r in zip(got, ref)]
    note(f"[frontend] sampled errors {errs}")
    assert max(errs) <= TOL


@pytest.mark.parametrize("dtype,D,gain", [("bf16", 32, True), ("fp16", 64, False), ("bf16", 8, True)])
def test_seed_norm(fp, dtype, D, gain):
    r = np.random.Generator(np.random.PCG64(D))
    H, M = 3, 77
    from flarepp_workloads import round_to_dtype
    q0 = round_to_dtype(r.standard_normal((H, M, D), dtype=np.float32), dtype)
    g = round_to_dtype(r.random((H, D), dtype=np.float32) + 0.5, dtype) if gain else None
    out = fp.flarepp_seed_norm_fwd(dev(q0, dtype), dev(g, dtype), eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.seed_norm_ref(q0, g, 1e-6)
    assert rel_err(out.float().cpu().numpy(), ref) <= TOL
    # in place gives the same values
    t = dev(q0, dtype)
    fp.flarepp_seed_norm_fwd(t, dev(g, dtype), eps=1e-6, out=t)
    torch.cuda.synchronize()
    assert torch.equal(t, out)
