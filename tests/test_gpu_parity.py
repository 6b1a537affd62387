"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max|y - y_ref| / max|y_ref| <= 1e-5 for fp32 inputs and <= 2e-2 for
bf16/fp16 inputs (fp32 accumulation), per workload and per run.  Every
workload runs at its full size; where the oracle cannot afford every head
(the million-token workload) it checks whole heads sampled from the run.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
from flarepp_workloads import WORKLOADS, make_inputs, make_random_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2, "fp16": 2e-2}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
NAMES = ("q0", "q_fixed", "gate", "k0", "k", "v")


@pytest.fixture(scope="module")
def fp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_attention_mixer_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    out = {}
    for n in NAMES:
        t = torch.from_numpy(np.ascontiguousarray(x[n]))
        out[n] = (t if n == "gate" else t.to(TDT[dtype])).cuda()
    return out


def f64(x):
    return {n: np.asarray(x[n], dtype=np.float64) for n in NAMES}


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def run_mixer(fp, x, dtype):
    d = to_dev(x, dtype)
    y = fp.flarepp_mixer_fwd(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"])
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def head_slice(x, b, h):
    return dict(q0=x["q0"][h:h + 1], q_fixed=x["q_fixed"][h:h + 1], gate=x["gate"][h:h + 1],
                k0=x["k0"][b:b + 1, h:h + 1], k=x["k"][b:b + 1, h:h + 1],
                v=x["v"][b:b + 1, h:h + 1])


@pytest.mark.parametrize("name", ["tiny_fp32", "small_mesh_bf16", "point_cloud_bf16",
                                  "wide_heads_fp16_gate_closed", "wide_heads_fp16"])
def test_workload_parity(fp, name):
    w = WORKLOADS[name]
    note(f"[parity] {name} {w.shape_dict} {w.dtype}")
    x = make_inputs(name)
    y = run_mixer(fp, x, w.dtype)
    assert np.all(np.isfinite(y))
    if w.B * w.H <= 32:
        ref = oracle.flarepp_ref(**f64(x))
        err = rel_err(y, ref)
    else:
        # every head of the first and last batch element
        errs = []
        for b in (0, w.B - 1):
            xs = {n: (x[n][b:b + 1] if n in ("k0", "k", "v") else x[n]) for n in NAMES}
            ref = oracle.flarepp_ref(**f64(xs))
            errs.append(rel_err(y[b:b + 1], ref))
        err = max(errs)
    note(f"[parity] {name} rel err {err:.3e} (tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype]


def test_million_token_parity_sampled_heads(fp):
    name = "million_token_bf16"
    w = WORKLOADS[name]
    note(f"[parity] {name} {w.shape_dict}")
    x = make_inputs(name)
    y = run_mixer(fp, x, w.dtype)
    assert np.all(np.isfinite(y))
    for h in (0, w.H - 1):
        ref = oracle.flarepp_ref(**f64(head_slice(x, 0, h)))
        err = rel_err(y[0:1, h:h + 1], ref)
        note(f"[parity] {name} head {h} rel err {err:.3e}")
        assert err <= TOL[w.dtype]


EDGE = [
    # (B, H, N, M, D, dtype)
    (1, 1, 1, 16, 8, "bf16"),        # a single token
    (1, 2, 37, 16, 8, "fp16"),       # fewer tokens than one tile
    (2, 1, 100, 100, 16, "bf16"),    # M not a multiple of 32, ragged tile
    (1, 3, 1000, 64, 32, "bf16"),
    (1, 2, 777, 200, 64, "fp16"),    # ragged everywhere, wide heads
    (2, 2, 4097, 512, 32, "bf16"),   # maximum M, one token past a tile
    (1, 1, 513, 1, 32, "bf16"),      # a single latent
    (1, 2, 300, 24, 8, "fp32"),
    (2, 1, 129, 70, 16, "fp32"),
    (1, 1, 1000, 512, 64, "fp32"),
    (1, 2, 65, 33, 64, "fp32"),
    (1, 2, 385, 512, 32, "bf16"),    # one token past a decoder tile, maximum M
    (1, 1, 257, 96, 16, "bf16"),     # two encoder tiles plus one token
    (3, 1, 128, 32, 32, "fp16"),     # exactly one encoder tile
    (1, 1, 2000, 512, 64, "bf16"),   # wide heads at maximum M
    (8, 64, 5, 16, 32, "bf16"),      # 512 heads of a few tokens each
    (4, 32, 70, 512, 16, "fp16"),    # 128 heads at maximum M
]


@pytest.mark.parametrize("B,H,N,M,D,dtype", EDGE)
def test_edge_shapes(fp, B, H, N, M, D, dtype):
    note(f"[edge] B{B} H{H} N{N} M{M} D{D} {dtype}")
    x = make_random_inputs(B, H, N, M, D, dtype, seed=1000 + N + M + D)
    y = run_mixer(fp, x, dtype)
    err = rel_err(y, oracle.flarepp_ref(**f64(x)))
    note(f"[edge] rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_head_count_past_grid_y_limit(fp, dtype):
    """67,584 (b, h) pairs, more than a grid's y extent holds: every launch
    keeps the head index on x. Whole batches sampled at the start, middle
    and end are checked against the oracle."""
    B, H, N, M, D = 2048, 33, 3, 5, 8
    note(f"[heads] B{B} H{H} N{N} M{M} D{D} {dtype}")
    x = make_random_inputs(B, H, N, M, D, dtype, seed=4242)
    y = run_mixer(fp, x, dtype)
    assert np.all(np.isfinite(y))
    for b in (0, B // 2 - 1, B - 1):
        xb = dict(x)
        for n in ("k0", "k", "v"):
            xb[n] = x[n][b:b + 1]
        err = rel_err(y[b:b + 1], oracle.flarepp_ref(**f64(xb)))
        note(f"[heads] batch {b} rel err {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_gate_special_values(fp, dtype):
    # per-head gates: closed, open, large positive, large negative finite
    x = make_random_inputs(2, 4, 300, 48, 16, dtype, seed=77,
                           gate=[-math.inf, math.inf, 30.0, -30.0])
    y = run_mixer(fp, x, dtype)
    err = rel_err(y, oracle.flarepp_ref(**f64(x)))
    note(f"[gate] {dtype} rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_gate_nan_propagates(fp, dtype):
    """A NaN gate logit makes its head's output NaN (sigma(NaN) times the
    synthesis); every other head matches the oracle."""
    x = make_random_inputs(2, 3, 300, 48, 16, dtype, seed=78, gate=[0.4, math.nan, -math.inf])
    y = run_mixer(fp, x, dtype)
    assert np.all(np.isnan(y[:, 1]))
    for h in (0, 2):
        ref = oracle.flarepp_ref(**f64({n: (x[n][h:h + 1] if n in ("q0", "q_fixed", "gate")
                                             else x[n][:, h:h + 1]) for n in NAMES}))
        err = rel_err(y[:, h:h + 1], ref)
        note(f"[gate-nan] {dtype} head {h} rel err {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_gate_closed_equals_flare_bitwise(fp, dtype):
    x = make_random_inputs(2, 3, 2000, 64, 32, dtype, seed=5, gate=-math.inf)
    d = to_dev(x, dtype)
    y1 = fp.flarepp_mixer_fwd(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"])
    y2 = fp.flare_mixer_fwd(d["q_fixed"], d["k"], d["v"], 1.0 / math.sqrt(32))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("dtype,scale", [("bf16", 1.0), ("fp16", 0.3), ("fp32", 1.0)])
def test_flare_mixer_vs_oracle(fp, dtype, scale):
    x = make_random_inputs(2, 2, 3000, 96, 32, dtype, seed=9)
    d = to_dev(x, dtype)
    y = fp.flare_mixer_fwd(d["q_fixed"], d["k"], d["v"], scale).float().cpu().numpy()
    ref = oracle.flare_ref(f64(x)["q_fixed"], f64(x)["k"], f64(x)["v"], scale)
    err = rel_err(y, ref)
    note(f"[flare] {dtype} scale {scale} rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_encode_seam_and_chunk_invariance(fp, dtype):
    x = make_random_inputs(2, 2, 5000, 128, 32, dtype, seed=11)
    d = to_dev(x, dtype)
    s = 1.0 / math.sqrt(32)
    ref = oracle.encode_ref(f64(x)["q_fixed"], f64(x)["k"], f64(x)["v"], s)
    zs = {}
    # 79, 27, 14, 8 and 2 chunks (plus the automatic choice): the merge
    # takes 8, 4, 2 and 1 lanes per latent slot
    for chunk in (0, 64, 192, 384, 640, 4992):
        z = fp.flare_encode_fwd(d["q_fixed"], d["k"], d["v"], s, chunk_tokens=chunk)
        torch.cuda.synchronize()
        zs[chunk] = z.cpu().numpy()
        err = rel_err(zs[chunk], ref)
        note(f"[encode] {dtype} chunk {chunk} rel err {err:.3e}")
        assert err <= TOL[dtype]
    # per-batch latents
    qb = np.stack([x["q_fixed"], x["q0"]])
    zb = fp.flare_encode_fwd(torch.from_numpy(qb).to(TDT[dtype]).cuda(), d["k"], d["v"], s)
    refb = oracle.encode_ref(qb.astype(np.float64), f64(x)["k"], f64(x)["v"], s)
    assert rel_err(zb.cpu().numpy(), refb) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_decode_seam(fp, dtype):
    x = make_random_inputs(1, 2, 3333, 160, 64, dtype, seed=12)
    rng = np.random.Generator(np.random.PCG64(3))
    z = rng.standard_normal((1, 2, 160, 64)).astype(np.float32)
    d = to_dev(x, dtype)
    s = 1.0 / math.sqrt(64)
    y = fp.flare_decode_fwd(d["q_fixed"], torch.from_numpy(z).cuda(), d["k"], s)
    ref = oracle.decode_ref(f64(x)["q_fixed"], z.astype(np.float64), f64(x)["k"], s)
    err = rel_err(y.float().cpu().numpy(), ref)
    note(f"[decode] {dtype} rel err {err:.3e}")
    assert err <= TOL[dtype]


def test_deterministic(fp):
    x = make_inputs("point_cloud_bf16")
    d = to_dev(x, "bf16")
    ys = [fp.flarepp_mixer_fwd(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"])
          for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


# ---------------------------------------------------------------------------
# The exact two-pass recompute.  The kernels sum 2^(S' - m) against a fixed
# reference m (m = 0 for bf16 probabilities, the first key group's maximum
# for fp16) and recompute a column exactly when its sums leave their range.
# These inputs force that path: every score carries a large component that
# is constant over the softmax axis (it cancels, so the exact result stays
# well conditioned in bf16), or later keys exceed the first group's maximum
# by more than the fp16 range.
# ---------------------------------------------------------------------------

FALLBACK = [
    ("bf16", "shift", 70.0),   # sums overflow: every 2^S' is beyond fp32
    ("bf16", "shift", -60.0),  # sums below the accepted range (2^-80)
    ("fp16", "ramp", 20.0),    # keys after the first group exceed it by > 2^15.9
]


def _fallback_inputs(dtype, kind, amount, decoder, B=1, H=2, N=3000, M=80, D=32, seed=21):
    from flarepp_workloads import round_to_dtype
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((H, M, D)).astype(np.float32)
    k = rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    if kind == "shift":
        k[..., 0] = 8.0
        q[..., 0] = amount
    elif decoder:  # latents after the first group score higher
        k[..., 0] = 4.0
        q[:, :, 0] = np.where(np.arange(M) >= 32, amount, 0.0)
    else:          # tokens after the first group score higher
        k[..., 0] = np.where(np.arange(N) >= 32, 4.0, 0.0)
        q[..., 0] = amount
    return [round_to_dtype(a, dtype) for a in (q, k, v)]


@pytest.mark.parametrize("dtype,kind,amount", FALLBACK)
def test_encode_exact_recompute(fp, dtype, kind, amount):
    q, k, v = _fallback_inputs(dtype, kind, amount, decoder=False)
    s = 1.0 / math.sqrt(q.shape[-1])
    dev = [torch.from_numpy(a).to(TDT[dtype]).cuda() for a in (q, k, v)]
    note(f"[encode recompute] {dtype} {kind} {amount}")
    z = fp.flare_encode_fwd(dev[0], dev[1], dev[2], s)
    torch.cuda.synchronize()
    ref = oracle.encode_ref(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), s)
    z = z.cpu().numpy()
    assert np.all(np.isfinite(z))
    err = rel_err(z, ref)
    note(f"[encode recompute] {dtype} {kind} {amount} rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("D", [32, 64])  # 64: rows and outputs pass the LDS staging tile
@pytest.mark.parametrize("dtype,kind,amount", FALLBACK)
def test_decode_exact_recompute(fp, dtype, kind, amount, D):
    # the same base-2 scores at every D: the product picks up s = 1/sqrt(D)
    q, k, _ = _fallback_inputs(dtype, kind, amount * math.sqrt(D / 32), decoder=True, D=D)
    B, H, N, D = k.shape
    M = q.shape[1]
    rng = np.random.Generator(np.random.PCG64(5))
    z = rng.standard_normal((B, H, M, D)).astype(np.float32)
    s = 1.0 / math.sqrt(D)
    note(f"[decode recompute] {dtype} {kind} {amount} D{D}")
    y = fp.flare_decode_fwd(torch.from_numpy(q).to(TDT[dtype]).cuda(), torch.from_numpy(z).cuda(),
                            torch.from_numpy(k).to(TDT[dtype]).cuda(), s)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    ref = oracle.decode_ref(q.astype(np.float64), z.astype(np.float64), k.astype(np.float64), s)
    assert np.all(np.isfinite(y))
    err = rel_err(y, ref)
    note(f"[decode recompute] {dtype} {kind} {amount} D{D} rel err {err:.3e}")
    assert err <= TOL[dtype]


def test_decode_accumulator_bound_triggers_exact_path(fp):
    """bf16 decoder: row sums finite and in range (~2^100) but values near
    2^30, so the accumulators (<= l max|z|) could pass the fp32 range; the
    bound l max|z| < 2^126 sends these tokens to the exact path, whose
    result is finite and matches the oracle."""
    q, k, _ = _fallback_inputs("bf16", "shift", 49.0, decoder=True)
    B, H, N, D = k.shape
    M = q.shape[1]
    rng = np.random.Generator(np.random.PCG64(6))
    z = (rng.standard_normal((B, H, M, D)) * 2.0 ** 30).astype(np.float32)
    s = 1.0 / math.sqrt(D)
    note("[decode bound] bf16 shift 49, |z| ~ 2^30")
    y = fp.flare_decode_fwd(torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(z).cuda(),
                            torch.from_numpy(k).to(torch.bfloat16).cuda(), s)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    ref = oracle.decode_ref(q.astype(np.float64), z.astype(np.float64), k.astype(np.float64), s)
    assert np.all(np.isfinite(y))
    err = rel_err(y, ref)
    note(f"[decode bound] rel err {err:.3e}")
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------------------
# Simplified FLARE++ (separate synthesis values, q = synthesized query)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,N,M,D,dtype", [
    (2, 4, 3000, 96, 32, "bf16"),
    (1, 2, 1500, 64, 64, "fp16"),
    (1, 2, 700, 40, 16, "fp32"),
])
def test_simplified_mixer_vs_oracle(fp, B, H, N, M, D, dtype):
    from flarepp_workloads import make_simplified_inputs
    note(f"[simplified] B{B} H{H} N{N} M{M} D{D} {dtype}")
    x = make_simplified_inputs(B, H, N, M, D, dtype, seed=300 + N)
    d = {n: torch.from_numpy(x[n]).to(TDT[dtype]).cuda() for n in ("q0", "k0", "v0", "k", "v")}
    y = fp.simplified_flarepp_mixer_fwd(d["q0"], d["k0"], d["v0"], d["k"], d["v"])
    torch.cuda.synchronize()
    ref = oracle.simplified_flarepp_ref(*(x[n].astype(np.float64) for n in ("q0", "k0", "v0", "k", "v")))
    err = rel_err(y.float().cpu().numpy(), ref)
    note(f"[simplified] rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_simplified_with_shared_values_equals_open_gate_flarepp(fp, dtype):
    x = make_random_inputs(2, 3, 2000, 64, 32, dtype, seed=8, gate=math.inf)
    d = to_dev(x, dtype)
    zeros = torch.zeros_like(d["q_fixed"])
    y1 = fp.flarepp_mixer_fwd(d["q0"], zeros, d["gate"], d["k0"], d["k"], d["v"])
    y2 = fp.simplified_flarepp_mixer_fwd(d["q0"], d["k0"], d["k0"], d["k"], d["v"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
