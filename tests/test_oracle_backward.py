"""Pins of the fp64 gradient oracle (oracle/flarepp_backward.py).

The pages give no gradient values, so the analytic gradients are pinned by
torch's fp64 autograd through its scaled_dot_product_attention (an
independent library routine), by central finite differences of the forward
oracle, by the closed-gate special case, and by planted mistakes that must
fail those pins.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from flarepp_workloads import make_random_inputs, make_simplified_inputs

NAMES = ("q0", "q_fixed", "gate", "k0", "k", "v")


def _x(B, H, N, M, D, seed, gate=None):
    x = make_random_inputs(B, H, N, M, D, "fp32", seed, gate=gate)
    return {n: x[n].astype(np.float64) for n in NAMES}


def _dy(B, H, N, D, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal((B, H, N, D))


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _torch_grads(x, dy):
    """Gradients by torch autograd through three SDPA calls (fp64, CPU)."""
    t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    B = t["k"].shape[0]
    q0 = t["q0"].unsqueeze(0).expand(B, -1, -1, -1)
    qf = t["q_fixed"].unsqueeze(0).expand(B, -1, -1, -1)
    sig = torch.sigmoid(t["gate"]).view(1, -1, 1, 1)
    qd = F.scaled_dot_product_attention(q0, t["k0"], t["k0"])
    q = qf + sig * qd
    z = F.scaled_dot_product_attention(q, t["k"], t["v"])
    y = F.scaled_dot_product_attention(t["k"], q, z)
    y.backward(torch.tensor(dy))
    return {"d" + n: t[n].grad.numpy() for n in ("q0", "q_fixed", "gate", "k0", "k", "v")}


@pytest.mark.parametrize("shape,seed", [((2, 3, 37, 5, 4), 1), ((1, 2, 64, 8, 8), 2),
                                        ((3, 1, 19, 19, 3), 3)])
def test_flarepp_gradients_vs_torch_autograd(shape, seed):
    B, H, N, M, D = shape
    x = _x(B, H, N, M, D, seed)
    dy = _dy(B, H, N, D, seed + 100)
    g = oracle.flarepp_bwd_ref(**x, dy=dy)
    gt = _torch_grads(x, dy)
    for n in ("dq0", "dq_fixed", "dgate", "dk0", "dk", "dv"):
        assert _rel(g[n], gt[n]) <= 1e-10, n


def test_flare_gradients_vs_torch_autograd():
    x = _x(2, 2, 33, 6, 4, 4)
    dy = _dy(2, 2, 33, 4, 5)
    for scale in (1.0, 0.37):
        dq, dk, dv = oracle.flare_bwd_ref(x["q_fixed"], x["k"], x["v"], scale, dy)
        t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True)
             for n in ("q_fixed", "k", "v")}
        q = t["q_fixed"].unsqueeze(0).expand(2, -1, -1, -1)
        z = F.scaled_dot_product_attention(q, t["k"], t["v"], scale=scale)
        y = F.scaled_dot_product_attention(t["k"], q, z, scale=scale)
        y.backward(torch.tensor(dy))
        assert _rel(dq, t["q_fixed"].grad.numpy()) <= 1e-10
        assert _rel(dk, t["k"].grad.numpy()) <= 1e-10
        assert _rel(dv, t["v"].grad.numpy()) <= 1e-10


def test_flarepp_gradients_vs_finite_differences():
    x = _x(1, 2, 7, 3, 2, 6, gate=[0.4, -1.1])
    dy = _dy(1, 2, 7, 2, 7)
    g = oracle.flarepp_bwd_ref(**x, dy=dy)
    eps = 1e-6
    rng = np.random.Generator(np.random.PCG64(8))
    for n in NAMES:
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in x[n].shape)
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[n][idx] += eps
            xm[n][idx] -= eps
            fd = (np.sum(oracle.flarepp_ref(**xp) * dy) - np.sum(oracle.flarepp_ref(**xm) * dy)) / (2 * eps)
            an = g["d" + n][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, idx, fd, an)


def test_closed_gate_has_no_synthesis_gradient():
    x = _x(2, 2, 20, 4, 4, 9, gate=-math.inf)
    dy = _dy(2, 2, 20, 4, 10)
    g = oracle.flarepp_bwd_ref(**x, dy=dy)
    assert np.all(g["dq0"] == 0) and np.all(g["dk0"] == 0) and np.all(g["dgate"] == 0)
    dq, dk, dv = oracle.flare_bwd_ref(x["q_fixed"], x["k"], x["v"], 0.5, dy)
    assert _rel(g["dq_fixed"], dq) <= 1e-14
    assert _rel(g["dk"], dk) <= 1e-14 and _rel(g["dv"], dv) <= 1e-14


def test_simplified_gradients_vs_torch_autograd():
    xs = make_simplified_inputs(2, 2, 30, 5, 4, "fp32", 11)
    x = {n: xs[n].astype(np.float64) for n in ("q0", "k0", "v0", "k", "v")}
    dy = _dy(2, 2, 30, 4, 12)
    g = oracle.simplified_flarepp_bwd_ref(**x, dy=dy)
    t = {n: torch.tensor(x[n], requires_grad=True) for n in x}
    q0 = t["q0"].unsqueeze(0).expand(2, -1, -1, -1)
    q = F.scaled_dot_product_attention(q0, t["k0"], t["v0"])
    z = F.scaled_dot_product_attention(q, t["k"], t["v"])
    y = F.scaled_dot_product_attention(t["k"], q, z)
    y.backward(torch.tensor(dy))
    for n in x:
        assert _rel(g["d" + n], t[n].grad.numpy()) <= 1e-10, n


def _attention_backward_no_delta(qh, kh, vh, scale, dout):
    A = oracle.attention_matrix(qh, kh, scale)
    dS = A * (np.asarray(dout) @ np.asarray(vh).T)   # the row-sum term dropped
    return scale * dS @ kh, scale * dS.T @ qh, A.T @ dout


@pytest.mark.parametrize("bug", ["no_delta", "transposed_ds", "no_sigma_chain", "dk0_key_only"])
def test_planted_gradient_mistakes_fail(bug, monkeypatch):
    import oracle.flarepp_backward as fb
    x = _x(1, 2, 17, 4, 4, 13, gate=[0.3, 1.2])
    dy = _dy(1, 2, 17, 4, 14)
    gt = _torch_grads(x, dy)
    if bug == "no_delta":
        monkeypatch.setattr(fb, "attention_backward", _attention_backward_no_delta)
    elif bug == "transposed_ds":
        orig = fb.attention_backward

        def wrong(qh, kh, vh, scale, dout):
            dq, dk, dv = orig(qh, kh, vh, scale, dout)
            return dq, dk[::-1].copy(), dv
        monkeypatch.setattr(fb, "attention_backward", wrong)
    elif bug == "no_sigma_chain":
        monkeypatch.setattr(fb, "gate_sigma", lambda g: np.ones_like(np.asarray(g, float)))
    elif bug == "dk0_key_only":
        orig = fb.attention_backward

        def key_only(qh, kh, vh, scale, dout):
            dq, dk, dv = orig(qh, kh, vh, scale, dout)
            if np.shares_memory(kh, vh):  # the synthesis call: k0 is key and value
                dv = np.zeros_like(dv)
            return dq, dk, dv
        monkeypatch.setattr(fb, "attention_backward", key_only)
    g = fb.flarepp_bwd_ref(**x, dy=dy)
    failed = [n for n in ("dq0", "dq_fixed", "dgate", "dk0", "dk", "dv") if _rel(g[n], gt[n]) > 1e-6]
    assert failed, bug
