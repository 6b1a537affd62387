"""GPU parity of the backward pass: the HIP path (through the C ABI) against
the fp64 oracle gradients (oracle.flarepp_bwd_ref / oracle.flare_bwd_ref).

Inputs and the output gradient dy are seeded and rounded to the operand
type; the oracle takes those exact values in fp64.  Bar, per gradient
tensor: max|g - g_ref| / max|g_ref| <= 2e-2 for bf16/fp16 operands (fp32
accumulation, fp32 gradients out) and <= 1e-5 for fp32 inputs, the bars of
the forward pass.  fp32 inputs (every D) and D = 8 (every dtype) run the
VALU backward; the rest the matrix-core passes.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from flarepp_workloads import WORKLOADS, make_cotangent, make_inputs, make_random_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp16": 2e-2, "fp32": 1e-5}
TDT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
NAMES = ("q0", "q_fixed", "gate", "k0", "k", "v")
TOKEN_GRADS = ("dk0", "dk", "dv")
LATENT_GRADS = ("dq0", "dq_fixed")


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


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(TDT[dtype])).cuda()


def rel_err(g, ref):
    g = np.asarray(g, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(np.abs(g)))
    return float(np.max(np.abs(g - ref)) / scale)


def run_flarepp_bwd(fp, x, dy, dtype):
    d = {n: dev(x[n], None if n == "gate" else dtype) for n in NAMES}
    dyd = dev(dy, dtype)
    y, saved = fp.flarepp_mixer_fwd_train(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"],
                                          d["v"])
    g = fp.flarepp_mixer_bwd(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"], y,
                             dyd, saved)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}, y


def f64(x, names=NAMES):
    return {n: np.asarray(x[n], np.float64) for n in names}


def check_flarepp(name, got, ref, dtype, heads=None, batches=None):
    """Compare every gradient; heads/batches restrict to a sampled slice
    (the reference then holds only those heads and all batch elements)."""
    errs = {}
    for n in ("dq0", "dq_fixed", "dgate", "dk0", "dk", "dv"):
        g = got[n]
        if heads is not None:
            g = g[heads] if n in LATENT_GRADS or n == "dgate" else g[:, heads]
        errs[n] = rel_err(g, ref[n])
    note(f"[bwd] {name} " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
    return errs


SHAPES = [
    # (B, H, N, M, D, dtype, gate logits)
    (2, 3, 700, 80, 32, "bf16", [0.3, -np.inf, 1.2]),     # ragged; one closed head
    (1, 2, 1000, 64, 16, "fp16", [-0.5, 2.0]),
    (2, 2, 513, 100, 64, "bf16", [0.0, np.inf]),           # gate fully open on one head
    (1, 2, 300, 33, 64, "fp16", [1.0, -1.0]),
    (1, 1, 37, 1, 32, "bf16", [0.5]),                      # a single latent
    (1, 2, 129, 512, 32, "bf16", [0.2, -0.7]),             # maximum M
    (3, 1, 128, 32, 32, "fp16", [0.1]),                    # exactly one tile
    # D = 64 past the LDS of one token-pass workgroup: two latent ranges
    (1, 2, 700, 512, 64, "bf16", [-np.inf, 0.5]),          # closed head too
    (1, 1, 333, 450, 64, "fp16", [1.0]),                   # ranges 256 + 194
    (4, 32, 9, 24, 16, "bf16", list(np.linspace(-2.0, 2.0, 32))),  # 128 heads
]


@pytest.mark.parametrize("B,H,N,M,D,dtype,gate", SHAPES)
def test_flarepp_bwd_vs_oracle(fp, B, H, N, M, D, dtype, gate):
    note(f"[bwd] flarepp B={B} H={H} N={N} M={M} D={D} {dtype}")
    x = make_random_inputs(B, H, N, M, D, dtype, seed=31 + N, gate=np.array(gate, np.float32))
    dy = make_cotangent(B, H, N, D, dtype, seed=77 + N)
    got, _ = run_flarepp_bwd(fp, x, dy, dtype)
    for n, g in got.items():
        assert np.all(np.isfinite(g)), n
    ref = oracle.flarepp_bwd_ref(**f64(x), dy=np.asarray(dy, np.float64))
    check_flarepp(f"B={B} H={H} N={N} M={M} D={D} {dtype}", got, ref, dtype)
    closed = np.isneginf(np.asarray(gate))
    for h in np.nonzero(closed)[0]:
        assert np.all(got["dq0"][h] == 0) and np.all(got["dk0"][:, h] == 0)
        assert got["dgate"][h] == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_single_token_closed_form(fp, dtype):
    """N = 1: every latent encodes the one token (z_m = v), so y = v and the
    Jacobian terms cancel exactly: dv = dy and every other gradient is 0.
    The kernel's are zero up to operand rounding, measured against the
    natural size s |dy| |v| (|q| + |k|) of the terms that cancel."""
    B, H, N, M, D = 2, 2, 1, 40, 32
    x = make_random_inputs(B, H, N, M, D, dtype, seed=9)
    dy = make_cotangent(B, H, N, D, dtype, seed=10)
    got, _ = run_flarepp_bwd(fp, x, dy, dtype)
    assert rel_err(got["dv"], dy) <= 1e-2
    norm = lambda a: float(np.max(np.linalg.norm(np.asarray(a, np.float64), axis=-1)))
    s = 1.0 / np.sqrt(D)
    nat = s * norm(dy) * norm(x["v"]) * (norm(x["q_fixed"]) + norm(x["q0"]) + norm(x["k"]))
    for n in ("dk", "dq_fixed", "dq0", "dk0", "dgate"):
        assert float(np.max(np.abs(got[n]))) <= TOL[dtype] * nat, n


@pytest.mark.parametrize("B,H,N,M,D,dtype,scale", [
    (2, 2, 900, 96, 32, "bf16", 0.2),
    (1, 3, 500, 40, 16, "fp16", 0.5),
    (1, 1, 2000, 256, 64, "bf16", 0.125),
    (1, 2, 7, 20, 32, "fp16", 1.0),
    (1, 1, 1000, 512, 64, "bf16", 0.125),                  # two latent ranges
])
def test_flare_bwd_vs_oracle(fp, B, H, N, M, D, dtype, scale):
    note(f"[bwd] flare B={B} H={H} N={N} M={M} D={D} {dtype} scale={scale}")
    x = make_random_inputs(B, H, N, M, D, dtype, seed=5 + N)
    dy = make_cotangent(B, H, N, D, dtype, seed=6 + N)
    q, k, v = dev(x["q_fixed"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    y, saved = fp.flare_mixer_fwd_train(q, k, v, scale)
    g = fp.flare_mixer_bwd(q, k, v, scale, y, dev(dy, dtype), saved)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = oracle.flare_bwd_ref(
        np.asarray(x["q_fixed"], np.float64), np.asarray(x["k"], np.float64),
        np.asarray(x["v"], np.float64), scale, np.asarray(dy, np.float64))
    errs = {"dq": rel_err(g["dq"].cpu(), dq_ref), "dk": rel_err(g["dk"].cpu(), dk_ref),
            "dv": rel_err(g["dv"].cpu(), dv_ref)}
    note("[bwd] flare " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


def _scaled_operand(q, scale, dtype):
    """The latent operand the kernels multiply: c q rounded to the operand
    dtype (c = scale log2(e) is folded into the latents so that a score is
    one matrix product and p = 2^score), divided back by c.  The gradients
    are those of the mixer at this q; it differs from q by one rounding."""
    c32 = np.float32(scale * np.log2(np.e))
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    cq = torch.from_numpy(np.asarray(q, np.float32) * c32).to(tdt).double().numpy()
    return cq / np.float64(c32)


def test_flare_bwd_per_set_form_choice(fp):
    """Head 0 has a token whose scores against every latent sit ~120 below the
    rest (the token pass's one-exponential form would need a factor outside
    fp32 there, so that set takes the two-exponential form); head 1 is
    ordinary (one-exponential form).  dq, dk and dv of both heads are checked
    against the oracle's gradients at the latent operand the kernels use,
    q_eff = bf16(c q) / c.  For this input the gradients at q and at q_eff
    themselves differ by ~4e-2 in head 0's dq: the extreme token's key has
    norm 120, so the one bf16 rounding of c q moves its scores by up to
    ~0.2 (base 2) and its decoder weights by up to ~15%, and dq carries that
    key a second time.  Both figures are printed."""
    B, H, N, M, D, dtype = 1, 2, 300, 64, 32, "bf16"
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(77)
    q = rng.standard_normal((H, M, D)).astype(np.float32)
    u = rng.standard_normal(D).astype(np.float32)
    u = u / np.linalg.norm(u)
    # head 0: latents 4u plus noise orthogonal to u; token 17 = -120 u scores
    # about -122 (base 2) against every latent, the rest of order 1
    w = 0.3 * rng.standard_normal((M, D)).astype(np.float32)
    w -= np.outer(w @ u, u)
    q[0] = 4.0 * u + w
    k = rng.standard_normal((B, H, N, D)).astype(np.float32)
    k[0, 0, 17] = -120.0 * u
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    dy = rng.standard_normal((B, H, N, D)).astype(np.float32)
    rt = lambda a: torch.from_numpy(a).to(torch.bfloat16).float().numpy().astype(np.float64)
    q64, k64, v64, dy64 = rt(q), rt(k), rt(v), rt(dy)
    # the range that decides the form, from the definition (base-2 scores)
    c = scale / np.log(2.0)
    spread = []
    for hh in range(H):
        sc = c * q64[hh] @ k64[0, hh].T                       # [M, N]
        lse1 = np.log2(np.sum(np.exp2(sc - sc.max(1, keepdims=True)), 1)) + sc.max(1)
        lse2 = np.log2(np.sum(np.exp2(sc - sc.max(0, keepdims=True)), 0)) + sc.max(0)
        spread.append(float(lse1.max() - lse2.min()))
    note(f"[bwd] lse1 max - lse2 min per head: {spread}")
    assert spread[0] > 110.0 and spread[1] < 60.0
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    y, saved = fp.flare_mixer_fwd_train(qd, kd, vd, scale)
    g = fp.flare_mixer_bwd(qd, kd, vd, scale, y, dev(dy, dtype), saved)
    torch.cuda.synchronize()
    q_eff = _scaled_operand(q64, scale, dtype)
    ref_eff = oracle.flare_bwd_ref(q_eff, k64, v64, scale, dy64)
    ref_plain = oracle.flare_bwd_ref(q64, k64, v64, scale, dy64)
    for hh in range(H):
        errs = {"dq": rel_err(g["dq"].cpu()[hh], ref_eff[0][hh]),
                "dk": rel_err(g["dk"].cpu()[:, hh], ref_eff[1][:, hh]),
                "dv": rel_err(g["dv"].cpu()[:, hh], ref_eff[2][:, hh])}
        plain = {"dq": rel_err(g["dq"].cpu()[hh], ref_plain[0][hh]),
                 "dk": rel_err(g["dk"].cpu()[:, hh], ref_plain[1][:, hh]),
                 "dv": rel_err(g["dv"].cpu()[:, hh], ref_plain[2][:, hh])}
        note(f"[bwd] head {hh} vs oracle(q_eff) " + " ".join(f"{n} {e:.2e}" for n, e in errs.items())
             + "; vs oracle(q) " + " ".join(f"{n} {e:.2e}" for n, e in plain.items()))
        for n, e in errs.items():
            assert e <= TOL[dtype], (hh, n, e)
        # dk, dv (the token pass, where the form is chosen) also meet the bar
        # against the gradients at q itself
        assert plain["dk"] <= TOL[dtype] and plain["dv"] <= TOL[dtype], (hh, plain)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_closed_gate_bwd_equals_flare_bitwise(fp, dtype):
    """With every gate closed FLARE++ is FLARE with q = q_fixed: the token
    gradients and dq_fixed match the FLARE backward bit for bit, and the
    synthesis gradients are zero."""
    B, H, N, M, D = 2, 2, 600, 48, 32
    x = make_random_inputs(B, H, N, M, D, dtype, seed=3, gate=-np.inf)
    dy = make_cotangent(B, H, N, D, dtype, seed=4)
    got, _ = run_flarepp_bwd(fp, x, dy, dtype)
    q, k, v = dev(x["q_fixed"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    y, saved = fp.flare_mixer_fwd_train(q, k, v, 1.0 / np.sqrt(D))
    g = fp.flare_mixer_bwd(q, k, v, 1.0 / np.sqrt(D), y, dev(dy, dtype), saved)
    torch.cuda.synchronize()
    assert np.array_equal(got["dk"], g["dk"].cpu().numpy())
    assert np.array_equal(got["dv"], g["dv"].cpu().numpy())
    assert np.array_equal(got["dq_fixed"], g["dq"].cpu().numpy())
    assert not np.any(got["dq0"]) and not np.any(got["dk0"]) and not np.any(got["dgate"])


def _head_slice(x, dy, heads):
    xs = dict(q0=x["q0"][heads], q_fixed=x["q_fixed"][heads], gate=x["gate"][heads],
              k0=x["k0"][:, heads], k=x["k"][:, heads], v=x["v"][:, heads])
    return xs, dy[:, heads]


@pytest.mark.parametrize("name,heads", [
    ("small_mesh_bf16", None),
    ("point_cloud_bf16", [0, 7]),
    ("wide_heads_fp16", [0, 9]),
    ("wide_heads_fp16_gate_closed", [3]),
])
def test_workload_bwd(fp, name, heads):
    """Each workload at its full size; the oracle checks whole heads (every
    batch element of the sampled heads, so the latent gradients are whole)."""
    w = WORKLOADS[name]
    note(f"[bwd] workload {name} {w.shape_dict} {w.dtype} heads {heads}")
    x = make_inputs(name)
    dy = make_cotangent(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed + 100)
    got, _ = run_flarepp_bwd(fp, x, dy, w.dtype)
    for n, g in got.items():
        assert np.all(np.isfinite(g)), n
    if heads is None:
        xs, dys = x, dy
    else:
        xs, dys = _head_slice(x, dy, heads)
    ref = oracle.flarepp_bwd_ref(**f64(xs), dy=np.asarray(dys, np.float64))
    check_flarepp(name, got, ref, w.dtype, heads=heads)


@pytest.mark.timeout(600)
def test_million_token_bwd_sampled_head(fp):
    """The million-token workload at full size (the launch shapes the
    backward bench times); the oracle checks head 0 whole (about 40 s of
    fp64 CPU work)."""
    name = "million_token_bf16"
    w = WORKLOADS[name]
    note(f"[bwd] workload {name} {w.shape_dict}")
    x = make_inputs(name)
    dy = make_cotangent(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed + 100)
    got, _ = run_flarepp_bwd(fp, x, dy, w.dtype)
    for n, g in got.items():
        assert np.all(np.isfinite(g)), n
    xs, dys = _head_slice(x, dy, [0])
    ref = oracle.flarepp_bwd_ref(**f64(xs), dy=np.asarray(dys, np.float64))
    check_flarepp(name, got, ref, w.dtype, heads=[0])


def test_bwd_deterministic(fp):
    """Fixed reduction orders: two runs give identical gradients."""
    x = make_random_inputs(2, 2, 3000, 96, 32, "bf16", seed=12)
    dy = make_cotangent(2, 2, 3000, 32, "bf16", seed=13)
    a, _ = run_flarepp_bwd(fp, x, dy, "bf16")
    b, _ = run_flarepp_bwd(fp, x, dy, "bf16")
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_fwd_train_output_equals_forward(fp):
    """The training forward returns the same y as the plain forward."""
    x = make_random_inputs(1, 2, 2000, 64, 32, "bf16", seed=8)
    d = {n: dev(x[n], None if n == "gate" else "bf16") for n in NAMES}
    y0 = fp.flarepp_mixer_fwd(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"])
    y1, _ = fp.flarepp_mixer_fwd_train(d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("B,H,N,M,D,dtype", [
    (2, 2, 700, 80, 32, "bf16"),
    (1, 2, 1000, 64, 16, "fp16"),
    (1, 1, 513, 100, 64, "bf16"),
    (2, 1, 300, 33, 64, "fp16"),
    (1, 1, 513, 480, 64, "bf16"),                          # two latent ranges
])
def test_simplified_bwd_vs_oracle(fp, B, H, N, M, D, dtype):
    """Simplified mixer (separate synthesis values, q = q_dyn) against
    oracle.simplified_flarepp_bwd_ref."""
    from flarepp_workloads import make_simplified_inputs
    note(f"[bwd] simplified B={B} H={H} N={N} M={M} D={D} {dtype}")
    x = make_simplified_inputs(B, H, N, M, D, dtype, seed=40 + N)
    dy = make_cotangent(B, H, N, D, dtype, seed=41 + N)
    d = {n: dev(x[n], dtype) for n in ("q0", "k0", "v0", "k", "v")}
    y, saved = fp.simplified_flarepp_mixer_fwd_train(d["q0"], d["k0"], d["v0"], d["k"], d["v"])
    g = fp.simplified_flarepp_mixer_bwd(d["q0"], d["k0"], d["v0"], d["k"], d["v"], y,
                                        dev(dy, dtype), saved)
    torch.cuda.synchronize()
    ref = oracle.simplified_flarepp_bwd_ref(
        **{n: np.asarray(x[n], np.float64) for n in ("q0", "k0", "v0", "k", "v")},
        dy=np.asarray(dy, np.float64))
    errs = {n: rel_err(g[n].cpu().numpy(), ref[n]) for n in ("dq0", "dk0", "dv0", "dk", "dv")}
    note("[bwd] simplified " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


# ---------------------------------------------------------------- VALU backward
VALU_SHAPES = [
    # (B, H, N, M, D, dtype, gate logits)
    (2, 3, 700, 80, 32, "fp32", [0.3, -np.inf, 1.2]),     # ragged; one closed head
    (1, 2, 300, 33, 64, "fp32", [1.0, -1.0]),
    (1, 2, 1000, 64, 16, "fp32", [-0.5, 2.0]),
    (2, 2, 513, 100, 8, "fp32", [0.0, np.inf]),           # gate fully open on one head
    (1, 2, 1024, 16, 8, "fp32", [0.7, -0.2]),             # the tiny fp32 workload's shape
    (1, 1, 37, 1, 8, "fp32", [0.5]),                      # a single latent
    (1, 2, 129, 512, 16, "fp32", [0.2, -0.7]),            # maximum M
    (2, 3, 700, 80, 8, "bf16", [0.3, -np.inf, 1.2]),      # D = 8 below the matrix-core K
    (1, 2, 1000, 64, 8, "fp16", [-0.5, 2.0]),
    (1, 2, 129, 512, 8, "bf16", [0.2, -0.7]),
    (4, 32, 9, 24, 8, "fp16", list(np.linspace(-2.0, 2.0, 32))),  # 128 heads
]


@pytest.mark.parametrize("B,H,N,M,D,dtype,gate", VALU_SHAPES)
def test_valu_flarepp_bwd_vs_oracle(fp, B, H, N, M, D, dtype, gate):
    note(f"[bwd] valu flarepp B={B} H={H} N={N} M={M} D={D} {dtype}")
    x = make_random_inputs(B, H, N, M, D, dtype, seed=131 + N, gate=np.array(gate, np.float32))
    dy = make_cotangent(B, H, N, D, dtype, seed=177 + N)
    got, _ = run_flarepp_bwd(fp, x, dy, dtype)
    for n, g in got.items():
        assert np.all(np.isfinite(g)), n
    ref = oracle.flarepp_bwd_ref(**f64(x), dy=np.asarray(dy, np.float64))
    check_flarepp(f"valu B={B} H={H} N={N} M={M} D={D} {dtype}", got, ref, dtype)
    for h in np.nonzero(np.isneginf(np.asarray(gate)))[0]:
        assert np.all(got["dq0"][h] == 0) and np.all(got["dk0"][:, h] == 0)
        assert got["dgate"][h] == 0


@pytest.mark.parametrize("B,H,N,M,D,dtype,scale", [
    (2, 2, 900, 96, 32, "fp32", 0.2),
    (1, 3, 500, 40, 8, "fp32", 1.0),                      # the FLARE listing's scale
    (1, 1, 700, 256, 64, "fp32", 0.125),
    (1, 2, 7, 20, 8, "bf16", 0.5),
    (2, 2, 600, 48, 8, "fp16", 1.0 / np.sqrt(8.0)),
])
def test_valu_flare_bwd_vs_oracle(fp, B, H, N, M, D, dtype, scale):
    note(f"[bwd] valu flare B={B} H={H} N={N} M={M} D={D} {dtype} scale={scale}")
    x = make_random_inputs(B, H, N, M, D, dtype, seed=15 + N)
    dy = make_cotangent(B, H, N, D, dtype, seed=16 + N)
    q, k, v = dev(x["q_fixed"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    y, saved = fp.flare_mixer_fwd_train(q, k, v, scale)
    g = fp.flare_mixer_bwd(q, k, v, scale, y, dev(dy, dtype), saved)
    torch.cuda.synchronize()
    ref = oracle.flare_bwd_ref(np.asarray(x["q_fixed"], np.float64),
                               np.asarray(x["k"], np.float64), np.asarray(x["v"], np.float64),
                               scale, np.asarray(dy, np.float64))
    errs = {n: rel_err(g[n].cpu().numpy(), r) for n, r in zip(("dq", "dk", "dv"), ref)}
    note("[bwd] valu flare " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("B,H,N,M,D,dtype", [
    (2, 2, 700, 64, 32, "fp32"),
    (1, 2, 400, 40, 8, "fp32"),
    (1, 2, 500, 32, 8, "bf16"),
])
def test_valu_simplified_bwd_vs_oracle(fp, B, H, N, M, D, dtype):
    test_simplified_bwd_vs_oracle(fp, B, H, N, M, D, dtype)


def test_valu_bwd_deterministic(fp):
    B, H, N, M, D, dtype = 2, 2, 900, 72, 32, "fp32"
    x = make_random_inputs(B, H, N, M, D, dtype, seed=8, gate=np.array([0.4, -0.9], np.float32))
    dy = make_cotangent(B, H, N, D, dtype, seed=9)
    a, _ = run_flarepp_bwd(fp, x, dy, dtype)
    b, _ = run_flarepp_bwd(fp, x, dy, dtype)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
