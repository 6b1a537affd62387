"""Pins of the fp64 oracle against things other than itself.

The pages print no numeric worked example, so the oracle is pinned by:

* hand-worked closed-form cases (tests/golden/hand_cases.json);
* a pure-Python scalar brute force (math.exp / math.fsum) on tiny inputs;
* an independent library routine: torch's scaled_dot_product_attention in
  fp64 on the CPU, called once per attention step of the mixer;
* closed forms (N = 1, uniform keys, M = 1, constant values, zero queries);
* invariants the definition fixes: gate closed equals two-step FLARE, every
  softmax row sums to 1, outputs are convex combinations, permutation
  equivariance in the tokens, linearity in v, rank of the routing operator
  at most M, and exactness of the token-sharded (log-sum-exp) encoder.

A mutation check plants plausible mistakes in copies of the oracle (wrong
scale, gate sign, transposed softmax, wrong operand ...) and requires each
mistake to fail at least one pin.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from flarepp_workloads import (WORKLOADS, make_inputs, make_random_inputs,
                               round_to_dtype)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ---------------------------------------------------------------------------
# Independent references used as pins
# ---------------------------------------------------------------------------

def _brute_attention(Q, K, V, scale):
    """softmax(scale Q K^T) V with Python scalars (lists of lists)."""
    out = []
    for qr in Q:
        sc = [scale * math.fsum(a * b for a, b in zip(qr, kr)) for kr in K]
        top = max(sc)
        w = [math.exp(s - top) for s in sc]
        tot = math.fsum(w)
        out.append([math.fsum(wi * vr[d] for wi, vr in zip(w, V)) / tot
                    for d in range(len(V[0]))])
    return out


def _brute_flarepp(q0, q_fixed, gate, k0, k, v):
    B, H, N, D = np.shape(k)
    s = 1.0 / math.sqrt(D)
    y = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            g = float(gate[h])
            sig = 1.0 / (1.0 + math.exp(-g))
            qf = np.asarray(q_fixed[h], dtype=float).tolist()
            if sig == 0.0:
                q = qf
            else:
                qd = _brute_attention(np.asarray(q0[h], float).tolist(),
                                      np.asarray(k0[b, h], float).tolist(),
                                      np.asarray(k0[b, h], float).tolist(), s)
                q = [[a + sig * c for a, c in zip(ra, rc)] for ra, rc in zip(qf, qd)]
            kk = np.asarray(k[b, h], float).tolist()
            z = _brute_attention(q, kk, np.asarray(v[b, h], float).tolist(), s)
            y[b, h] = np.array(_brute_attention(kk, q, z, s))
    return y


def _torch_sdpa(q, k, v, scale=None):
    return F.scaled_dot_product_attention(q, k, v, scale=scale)


def _torch_flarepp(q0, q_fixed, gate, k0, k, v):
    """The mixer as three calls of torch's fp64 CPU attention routine."""
    T = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    k0t, kt, vt = T(k0), T(k), T(v)
    B = kt.shape[0]
    q0t = T(q0).unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    qft = T(q_fixed).unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    sig = torch.sigmoid(T(gate)).view(1, -1, 1, 1)
    qdyn = _torch_sdpa(q0t, k0t, k0t)
    # a closed gate contributes nothing (sigma = 0 exactly)
    q = qft + torch.where(sig == 0, torch.zeros_like(qdyn), sig * qdyn)
    z = _torch_sdpa(q, kt, vt)
    y = _torch_sdpa(kt, q, z)
    return y.numpy()


def _torch_flare(q, k, v, scale):
    T = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    kt, vt = T(k), T(v)
    qt = T(q).unsqueeze(0).expand(kt.shape[0], -1, -1, -1).contiguous()
    z = _torch_sdpa(qt, kt, vt, scale=scale)
    return _torch_sdpa(kt, qt, z, scale=scale).numpy()


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _load_golden():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    env = {"__builtins__": {}, "log": math.log, "sqrt": math.sqrt,
           "exp": math.exp, "inf": math.inf}

    def ev(x):
        if isinstance(x, list):
            return [ev(e) for e in x]
        return float(eval(x, env))  # expressions of our own committed file

    out = []
    for c in cases:
        out.append({k: (ev(v) if k not in ("name", "mixer", "derivation") else v)
                    for k, v in c.items()})
    return out


# ---------------------------------------------------------------------------
# The pin suite: each pin takes an implementation (an object with
# flarepp(q0, q_fixed, gate, k0, k, v) and flare(q, k, v, scale)) and
# returns a list of failure messages (empty when the pin holds).
# ---------------------------------------------------------------------------

class OracleImpl:
    flarepp = staticmethod(oracle.flarepp_ref)
    flare = staticmethod(oracle.flare_ref)


def _rand(B, H, N, M, D, seed, scale=1.0, gate=None):
    x = make_random_inputs(B, H, N, M, D, "fp32", seed, scale=scale, gate=gate)
    return {n: x[n].astype(np.float64) for n in ("q0", "q_fixed", "gate", "k0", "k", "v")}


def pin_golden(impl):
    fails = []
    for c in _load_golden():
        if c["mixer"] == "flare":
            y = impl.flare(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"])
        else:
            y = impl.flarepp(np.array(c["q0"]), np.array(c["q_fixed"]), np.array(c["gate"]),
                             np.array(c["k0"]), np.array(c["k"]), np.array(c["v"]))
        err = np.max(np.abs(np.asarray(y) - np.array(c["y"])))
        if not err <= 1e-13:
            fails.append(f"golden {c['name']}: max abs err {err:.3e}")
    return fails


def pin_brute(impl):
    fails = []
    for (B, H, N, M, D, seed, gate) in [(1, 1, 5, 2, 2, 11, None), (2, 2, 8, 3, 2, 12, None),
                                        (1, 2, 7, 3, 1, 13, [-math.inf, 0.7]),
                                        (2, 1, 4, 1, 2, 14, None)]:
        x = _rand(B, H, N, M, D, seed, gate=gate)
        y = impl.flarepp(**x)
        yb = _brute_flarepp(**x)
        if not _rel(y, yb) <= 1e-14:
            fails.append(f"brute B{B}H{H}N{N}M{M}D{D}: {_rel(y, yb):.2e}")
    return fails


def pin_torch(impl):
    fails = []
    for (B, H, N, M, D, seed, gate) in [(2, 3, 37, 5, 4, 21, None), (1, 2, 64, 8, 8, 22, [-math.inf, 1.5]),
                                        (3, 1, 19, 19, 3, 23, None)]:
        x = _rand(B, H, N, M, D, seed, gate=gate)
        y = impl.flarepp(**x)
        yt = _torch_flarepp(**x)
        if not _rel(y, yt) <= 1e-12:
            fails.append(f"torch flarepp B{B}H{H}N{N}M{M}D{D}: {_rel(y, yt):.2e}")
    x = _rand(2, 2, 33, 6, 4, 24)
    for scale in (1.0, 0.5, 1.0 / math.sqrt(4)):
        y = impl.flare(x["q_fixed"], x["k"], x["v"], scale)
        yt = _torch_flare(x["q_fixed"], x["k"], x["v"], scale)
        if not _rel(y, yt) <= 1e-12:
            fails.append(f"torch flare scale {scale}: {_rel(y, yt):.2e}")
    return fails


def pin_closed_forms(impl):
    fails = []
    # N = 1: every softmax over the single token is 1 and the decode gives
    # back z = v, for any latents and gate.
    x = _rand(2, 2, 1, 4, 3, 31)
    y = impl.flarepp(**x)
    if not _rel(y, x["v"]) <= 1e-14:
        fails.append("N=1 => y = v")
    # zero fixed queries and a closed gate: q = 0, encode weights are uniform
    # so every z_m = mean_n v_n, and then every y_n = mean_n v_n.
    x = _rand(1, 2, 23, 5, 4, 32, gate=-math.inf)
    x["q_fixed"][:] = 0.0
    y = impl.flarepp(**x)
    mean_v = x["v"].mean(axis=2, keepdims=True)
    if not _rel(y, np.broadcast_to(mean_v, y.shape)) <= 1e-13:
        fails.append("q=0 => y = mean(v)")
    # all keys equal: encode weights uniform -> z_m = mean(v) for every m,
    # and the decode averages identical rows -> y_n = mean(v).
    x = _rand(2, 1, 17, 4, 3, 33)
    x["k"][:] = x["k"][:, :, :1, :]
    y = impl.flarepp(**x)
    mean_v = x["v"].mean(axis=2, keepdims=True)
    if not _rel(y, np.broadcast_to(mean_v, y.shape)) <= 1e-13:
        fails.append("equal keys => y = mean(v)")
    # M = 1: the decode softmax over one latent is 1, so all y_n are equal
    # to z_1 = softmax(s q k^T) v.
    x = _rand(1, 2, 29, 1, 4, 34)
    y = impl.flarepp(**x)
    if not np.max(np.abs(y - y[:, :, :1, :])) <= 1e-13 * np.max(np.abs(y)):
        fails.append("M=1 => all y_n equal")
    # constant values: v = c gives y = c.
    x = _rand(1, 2, 31, 6, 4, 35)
    c = np.array([0.25, -3.0, 7.5, 1.0])
    x["v"][:] = c
    y = impl.flarepp(**x)
    if not _rel(y, np.broadcast_to(c, y.shape)) <= 1e-13:
        fails.append("v = c => y = c")
    return fails


def pin_gate_closed_is_flare(impl):
    x = _rand(2, 3, 41, 6, 4, 41, gate=-math.inf)
    y = impl.flarepp(**x)
    yf = impl.flare(x["q_fixed"], x["k"], x["v"], 1.0 / math.sqrt(4))
    return [] if np.array_equal(y, yf) else [f"gate closed != FLARE: {_rel(y, yf):.2e}"]


def pin_permutation(impl):
    x = _rand(2, 2, 27, 5, 4, 51)
    y = impl.flarepp(**x)
    perm = np.random.Generator(np.random.PCG64(7)).permutation(27)
    xp = dict(x)
    for n in ("k0", "k", "v"):
        xp[n] = x[n][:, :, perm, :]
    yp = impl.flarepp(**xp)
    return [] if _rel(yp, y[:, :, perm, :]) <= 1e-12 else ["permutation equivariance"]


def pin_linearity(impl):
    x = _rand(1, 2, 25, 4, 3, 61)
    v2 = _rand(1, 2, 25, 4, 3, 62)["v"]
    a, b = 0.75, -2.5
    y1 = impl.flarepp(**x)
    y2 = impl.flarepp(**{**x, "v": v2})
    y12 = impl.flarepp(**{**x, "v": a * x["v"] + b * v2})
    return [] if _rel(y12, a * y1 + b * y2) <= 1e-12 else ["linearity in v"]


PINS = [pin_golden, pin_brute, pin_torch, pin_closed_forms, pin_gate_closed_is_flare,
        pin_permutation, pin_linearity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(OracleImpl) == []


# ---------------------------------------------------------------------------
# Mutation check: mistakes planted in copies of the oracle must be caught.
# ---------------------------------------------------------------------------

def _softmax(L, axis):
    E = np.exp(L - L.max(axis=axis, keepdims=True))
    return E / E.sum(axis=axis, keepdims=True)


def _mutant_mixer(q0, q_fixed, gate, k0, k, v, bug):
    B, H, N, D = k.shape
    s = {"scale_1_over_D": 1.0 / D, "scale_one": 1.0}.get(bug, 1.0 / math.sqrt(D))
    y = np.empty((B, H, N, D))
    for b in range(B):
        for h in range(H):
            g = gate[h]
            with np.errstate(over="ignore"):
                sig = {"gate_sign": 1 / (1 + np.exp(g)), "gate_no_sigmoid": g}.get(
                    bug, 1 / (1 + np.exp(-g)))
            qf = q_fixed[b % H if bug == "latent_by_batch" else h]
            if sig == 0 or (bug == "gate_no_sigmoid" and not np.isfinite(g)):
                q = qf.copy()
            else:
                sv = v[b, h] if bug == "synth_value_v" else k0[b, h]
                A0 = _softmax(s * q0[h] @ k0[b, h].T, 0 if bug == "synth_softmax_axis" else 1)
                qd = A0 @ sv
                if bug == "drop_fixed":
                    q = sig * qd
                elif bug == "sigma_on_fixed":
                    q = sig * qf + qd
                else:
                    q = qf + sig * qd
            ke = k0[b, h] if bug == "encode_keys_k0" else k[b, h]
            z = _softmax(s * q @ ke.T, 1) @ v[b, h]
            if bug == "z_reversed":
                z = z[::-1]
            qk = qf if bug == "decode_keys_fixed" else q
            A2 = _softmax(s * k[b, h] @ qk.T, 0 if bug == "decode_softmax_tokens" else 1)
            y[b, h] = A2 @ z
    return y


MUTANTS = ["scale_1_over_D", "scale_one", "gate_sign", "gate_no_sigmoid", "synth_value_v",
           "synth_softmax_axis", "drop_fixed", "sigma_on_fixed", "encode_keys_k0",
           "z_reversed", "decode_keys_fixed", "decode_softmax_tokens", "latent_by_batch"]


def _mutant_impl(bug):
    def flarepp(q0, q_fixed, gate, k0, k, v):
        a = [np.asarray(t, np.float64) for t in (q0, q_fixed, gate, k0, k, v)]
        return _mutant_mixer(*a, bug=bug)

    class Impl:
        pass
    Impl.flarepp = staticmethod(flarepp)
    Impl.flare = staticmethod(oracle.flare_ref)
    return Impl


def test_unmutated_copy_passes_pins():
    Impl = _mutant_impl(None)
    for pin in PINS:
        assert pin(Impl) == [], pin.__name__


@pytest.mark.parametrize("bug", MUTANTS)
def test_planted_mistake_is_caught(bug):
    Impl = _mutant_impl(bug)
    failed = [p.__name__ for p in PINS if p(Impl)]
    assert failed, f"mutant {bug} passed every pin"


# ---------------------------------------------------------------------------
# Invariants on the oracle's intermediates
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_convexity():
    x = _rand(2, 2, 50, 7, 4, 71)
    for b in range(2):
        for h in range(2):
            it = oracle.flarepp_head_intermediates(x["q0"], x["q_fixed"], x["gate"],
                                                   x["k0"], x["k"], x["v"], b, h)
            for A in (it["A0"], it["A1"], it["A2"]):
                assert np.all(A >= 0)
                assert np.max(np.abs(A.sum(axis=1) - 1)) <= 1e-12
            kk0, vv = x["k0"][b, h], x["v"][b, h]
            eps = 1e-13
            assert np.all(it["q_dyn"] >= kk0.min(axis=0) - eps)
            assert np.all(it["q_dyn"] <= kk0.max(axis=0) + eps)
            assert np.all(it["z"] >= vv.min(axis=0) - eps)
            assert np.all(it["z"] <= vv.max(axis=0) + eps)
            assert np.all(it["y"] >= it["z"].min(axis=0) - eps)
            assert np.all(it["y"] <= it["z"].max(axis=0) + eps)


def test_intermediates_match_mixer():
    x = _rand(2, 3, 40, 6, 4, 72, gate=[-math.inf, 0.3, -1.1])
    y, inter = oracle.flarepp_ref(**x, return_intermediates=True)
    for b in range(2):
        for h in range(3):
            it = oracle.flarepp_head_intermediates(x["q0"], x["q_fixed"], x["gate"],
                                                   x["k0"], x["k"], x["v"], b, h)
            assert _rel(it["y"], y[b, h]) <= 1e-13
            assert _rel(it["q"], inter["q"][b, h]) <= 1e-14
            assert _rel(it["z"], inter["z"][b, h]) <= 1e-13
            if h == 0:
                assert it["A0"] is None and np.array_equal(it["q"], x["q_fixed"][h])


def test_routing_operator_rank_at_most_M():
    # R = A2 A1 maps values v to outputs y = R v; it is N x N, row-stochastic
    # and of rank at most M (explicit low-rank factorisation).
    M = 4
    x = _rand(1, 1, 24, M, 3, 81)
    it = oracle.flarepp_head_intermediates(x["q0"], x["q_fixed"], x["gate"], x["k0"],
                                           x["k"], x["v"], 0, 0)
    R = it["A2"] @ it["A1"]
    assert R.shape == (24, 24)
    assert np.max(np.abs(R.sum(axis=1) - 1)) <= 1e-12
    sv = np.linalg.svd(R, compute_uv=False)
    assert sv[M - 1] > 1e-6 * sv[0]
    assert sv[M] < 1e-12 * sv[0]
    assert _rel(R @ x["v"][0, 0], it["y"]) <= 1e-12


@pytest.mark.parametrize("shards", [1, 2, 3, 7, 64, 97])
def test_sharded_encoder_is_exact(shards):
    x = _rand(2, 2, 97, 6, 4, 91)
    s = 0.5
    z = oracle.encode_ref(x["q_fixed"], x["k"], x["v"], s)
    zs = oracle.encode_sharded_ref(x["q_fixed"], x["k"], x["v"], s, shards)
    assert _rel(zs, z) <= 1e-13


def test_sharded_encoder_large_score_spread():
    # shards whose maxima differ by hundreds must still merge without
    # overflow or underflow of the final result
    x = _rand(1, 1, 40, 3, 2, 92, scale=6.0)
    z = oracle.encode_ref(x["q_fixed"], x["k"], x["v"], 4.0)
    zs = oracle.encode_sharded_ref(x["q_fixed"], x["k"], x["v"], 4.0, 5)
    assert np.all(np.isfinite(zs)) and _rel(zs, z) <= 1e-12


def test_gate_sigma_special_values():
    s = oracle.gate_sigma(np.array([-np.inf, 0.0, np.inf, math.log(3.0)]))
    assert s[0] == 0.0 and s[1] == 0.5 and s[2] == 1.0
    assert abs(s[3] - 0.75) <= 1e-16


def test_flare_listing_scale_one_vs_torch():
    # FLARE.py README "FLARE" listing passes scale 1.0 to both calls
    x = _rand(2, 2, 30, 5, 3, 93)
    y = oracle.flare_ref(x["q_fixed"], x["k"], x["v"], 1.0)
    assert _rel(y, _torch_flare(x["q_fixed"], x["k"], x["v"], 1.0)) <= 1e-12


# ---------------------------------------------------------------------------
# The seeded input generators (shared by both sides)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_rounding_matches_torch(dtype, tdt):
    rng = np.random.Generator(np.random.PCG64(5))
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    if dtype == "fp16":
        x = np.clip(x, -60000, 60000)
    r = round_to_dtype(x, dtype)
    t = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    assert np.array_equal(r, t)


def test_workloads_are_deterministic_and_shaped():
    for name in ("tiny_fp32", "small_mesh_bf16"):
        a = make_inputs(name)
        b = make_inputs(name)
        w = WORKLOADS[name]
        for n in ("q0", "q_fixed", "gate", "k0", "k", "v"):
            assert np.array_equal(a[n], b[n])
        assert a["q0"].shape == (w.H, w.M, w.D)
        assert a["k"].shape == (w.B, w.H, w.N, w.D)
        assert a["gate"].shape == (w.H,)
    c = make_inputs("wide_heads_fp16_gate_closed")
    assert np.all(np.isneginf(c["gate"]))


def test_tiny_workload_oracle_against_torch():
    x = make_inputs("tiny_fp32")
    xs = {n: x[n].astype(np.float64) for n in ("q0", "q_fixed", "gate", "k0", "k", "v")}
    assert _rel(oracle.flarepp_ref(**xs), _torch_flarepp(**xs)) <= 1e-12


# ---------------------------------------------------------------------------
# Simplified FLARE++ (separate synthesis values, q = synthesized query)
# ---------------------------------------------------------------------------

def _srand(B, H, N, M, D, seed):
    from flarepp_workloads import make_simplified_inputs
    x = make_simplified_inputs(B, H, N, M, D, "fp32", seed)
    return {n: x[n].astype(np.float64) for n in ("q0", "k0", "v0", "k", "v")}


def _torch_simplified(q0, k0, v0, k, v):
    T = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    kt, vt = T(k), T(v)
    q0t = T(q0).unsqueeze(0).expand(kt.shape[0], -1, -1, -1).contiguous()
    q = _torch_sdpa(q0t, T(k0), T(v0))
    z = _torch_sdpa(q, kt, vt)
    return _torch_sdpa(kt, q, z).numpy()


def _brute_simplified(q0, k0, v0, k, v):
    B, H, N, D = np.shape(k)
    s = 1.0 / math.sqrt(D)
    y = np.zeros((B, H, N, D))
    L = lambda a: np.asarray(a, float).tolist()
    for b in range(B):
        for h in range(H):
            q = _brute_attention(L(q0[h]), L(k0[b, h]), L(v0[b, h]), s)
            z = _brute_attention(q, L(k[b, h]), L(v[b, h]), s)
            y[b, h] = np.array(_brute_attention(L(k[b, h]), q, z, s))
    return y


def test_simplified_with_shared_values_is_open_gate_flarepp():
    # v0 = k0, q_fixed = 0 and g = +inf (sigma = 1) give the same operations
    x = _srand(2, 2, 40, 6, 4, 61)
    y = oracle.simplified_flarepp_ref(x["q0"], x["k0"], x["k0"], x["k"], x["v"])
    yp = oracle.flarepp_ref(x["q0"], np.zeros_like(x["q0"]), np.full(2, np.inf), x["k0"],
                            x["k"], x["v"])
    assert _rel(y, yp) <= 1e-15


@pytest.mark.parametrize("shape", [(2, 3, 37, 5, 4), (1, 2, 64, 8, 8), (3, 1, 19, 19, 3)])
def test_simplified_vs_torch(shape):
    x = _srand(*shape, seed=62)
    assert _rel(oracle.simplified_flarepp_ref(**x), _torch_simplified(**x)) <= 1e-12


def test_simplified_vs_brute_force():
    for shape, seed in (((1, 1, 6, 2, 2), 63), ((2, 2, 5, 3, 1), 64)):
        x = _srand(*shape, seed=seed)
        assert _rel(oracle.simplified_flarepp_ref(**x), _brute_simplified(**x)) <= 1e-14


def test_simplified_closed_forms():
    x = _srand(2, 2, 1, 4, 3, 65)   # one token: every softmax is 1, y = v
    assert _rel(oracle.simplified_flarepp_ref(**x), x["v"]) <= 1e-14
    x = _srand(1, 2, 30, 5, 4, 66)  # constant values: y is that constant
    x["v"] = np.full_like(x["v"], -2.5)
    assert _rel(oracle.simplified_flarepp_ref(**x), x["v"]) <= 1e-14


def test_simplified_synthesis_value_matters():
    # a copy that ignores v0 (uses k0 as the synthesis value) must fail the
    # library pin: the pins above see the separate synthesis values
    x = _srand(2, 2, 30, 5, 4, 67)
    wrong = oracle.simplified_flarepp_ref(x["q0"], x["k0"], x["k0"], x["k"], x["v"])
    assert _rel(wrong, _torch_simplified(**x)) > 1e-6
