"""Pins of the front-end oracle (oracle/flarepp_frontend.py): input
projections and head-wise RMS normalisation, checked against torch fp64
library routines (linear, rms_norm), closed forms and invariants; planted
mistakes in a copy of the oracle must each fail at least one pin."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.flarepp_frontend as fe

torch = pytest.importorskip("torch")
F = torch.nn.functional


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _case(B=2, N=37, C=24, H=3, D=8, seed=0, bias=True, gain=True):
    r = _rng(seed)
    x = r.standard_normal((B, N, C))
    w = [r.standard_normal((H * D, C)) / np.sqrt(C) for _ in range(3)]
    b = [r.standard_normal(H * D) if bias else None for _ in range(3)]
    g = r.uniform(0.5, 1.5, (H, D)) if gain else None
    return dict(x=x, w_k0=w[0], w_k=w[1], w_v=w[2], b_k0=b[0], b_k=b[1], b_v=b[2], g_k0=g,
                H=H, D=D)


def _torch_frontend(c, eps):
    x = torch.tensor(c["x"])
    B, N, _ = x.shape
    H, D = c["H"], c["D"]

    def proj(w, b):
        y = F.linear(x, torch.tensor(w), None if b is None else torch.tensor(b))
        return y.view(B, N, H, D).permute(0, 2, 1, 3)
    k0 = proj(c["w_k0"], c["b_k0"])
    k0 = torch.stack([F.rms_norm(k0[:, h], (D,), None if c["g_k0"] is None
                                 else torch.tensor(c["g_k0"][h]), eps) for h in range(H)], 1)
    return k0.numpy(), proj(c["w_k"], c["b_k"]).numpy(), proj(c["w_v"], c["b_v"]).numpy()


def _pins(mod):
    """Every pin as (name, passed) for the module `mod` (the oracle or a
    mutated copy); raises nothing."""
    out = []
    for seed, bias, gain in ((0, True, True), (1, False, False)):
        c = _case(seed=seed, bias=bias, gain=gain)
        got = mod.frontend_ref(**c, eps=1e-5)
        ref = _torch_frontend(c, 1e-5)
        out.append((f"torch-{seed}", all(np.allclose(a, b, rtol=1e-12, atol=1e-12)
                                          for a, b in zip(got, ref))))
    # identity weights: the projection is the head-major split of the features
    r = _rng(5)
    B, N, H, D = 2, 9, 3, 4
    x = r.standard_normal((B, N, H * D))
    eye = np.eye(H * D)
    k0, k, v = mod.frontend_ref(x, eye, eye, eye, H, D, normalize_k0=False)
    split = x.reshape(B, N, H, D).transpose(0, 2, 1, 3)
    out.append(("identity", np.array_equal(k, split) and np.array_equal(v, split)
                and np.array_equal(k0, split)))
    # a non-symmetric weight: row o of W picks feature perm[o]
    perm = r.permutation(H * D)
    P = np.zeros((H * D, H * D))
    P[np.arange(H * D), perm] = 1.0
    _, k, _ = mod.frontend_ref(x, eye, P, eye, H, D, normalize_k0=False)
    out.append(("permutation", np.array_equal(k, x[..., perm].reshape(B, N, H, D)
                                              .transpose(0, 2, 1, 3))))
    # unit mean square over each head's D features (gain 1, eps 0), and
    # invariance to the scale of the tokens
    c = _case(seed=3, bias=False, gain=False)
    k0 = mod.frontend_ref(**c, eps=0.0)[0]
    out.append(("unit-ms", np.allclose(np.mean(k0 ** 2, axis=-1), 1.0, rtol=1e-12)))
    c2 = dict(c, x=7.5 * c["x"])
    out.append(("scale-inv", np.allclose(mod.frontend_ref(**c2, eps=0.0)[0], k0, rtol=1e-12)))
    # gain per head: doubling the gain of head 1 doubles only head 1 of k0
    c = _case(seed=4)
    g2 = c["g_k0"].copy()
    g2[1] *= 2.0
    a = mod.frontend_ref(**c)[0]
    b = mod.frontend_ref(**dict(c, g_k0=g2))[0]
    out.append(("gain-head", np.allclose(b[:, 1], 2 * a[:, 1]) and np.array_equal(b[:, 0], a[:, 0])))
    # seeds
    q0 = r.standard_normal((H, 11, D))
    g = r.uniform(0.5, 1.5, (H, D))
    ref = torch.stack([F.rms_norm(torch.tensor(q0[h]), (D,), torch.tensor(g[h]), 1e-6)
                       for h in range(H)]).numpy()
    out.append(("seeds-torch", np.allclose(mod.seed_norm_ref(q0, g, 1e-6), ref, rtol=1e-12)))
    return out


def test_oracle_passes_every_pin():
    failed = [n for n, ok in _pins(fe) if not ok]
    assert not failed, failed


def test_exported_from_package():
    assert oracle.frontend_ref is fe.frontend_ref and oracle.seed_norm_ref is fe.seed_norm_ref


class _Mutant:
    """A copy of the oracle with one planted mistake."""

    def __init__(self, bug):
        self.bug = bug

    def rms_norm_ref(self, u, gain=None, eps=1e-6):
        u = np.asarray(u, np.float64)
        if self.bug == "eps_outside":
            out = u / (np.sqrt(np.mean(u * u, axis=-1, keepdims=True)) + eps)
        elif self.bug == "sum_not_mean":
            out = u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + eps)
        elif self.bug == "norm_over_tokens":
            out = u / np.sqrt(np.mean(u * u, axis=-2, keepdims=True) + eps)
        else:
            out = u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
        if gain is not None:
            g = np.asarray(gain, np.float64)
            if self.bug == "gain_head0":
                g = np.broadcast_to(g[:, :1] if g.shape[1] > 1 else g, g.shape)
            out = out * g
        return out

    def projection_ref(self, x, w, b, H, D):
        x = np.asarray(x, np.float64)
        w = np.asarray(w, np.float64)
        p = x @ (w if self.bug == "untransposed" else w.T)
        if b is not None:
            p = p + b
        B, N, _ = x.shape
        if self.bug == "token_major_split":
            return p.reshape(B, N, D, H).transpose(0, 3, 1, 2)
        return p.reshape(B, N, H, D).transpose(0, 2, 1, 3)

    def frontend_ref(self, x, w_k0, w_k, w_v, H, D, b_k0=None, b_k=None, b_v=None, g_k0=None,
                     eps=1e-6, normalize_k0=True):
        k0 = self.projection_ref(x, w_k0, b_k0, H, D)
        if normalize_k0:
            gain = None if g_k0 is None else np.asarray(g_k0)[None, :, None, :]
            k0 = self.rms_norm_ref(k0, gain, eps)
        if self.bug == "normalise_k":
            k = self.rms_norm_ref(self.projection_ref(x, w_k, b_k, H, D), None, eps)
        else:
            k = self.projection_ref(x, w_k, b_k, H, D)
        return k0, k, self.projection_ref(x, w_v, b_v, H, D)

    def seed_norm_ref(self, q0, gain=None, eps=1e-6):
        g = None if gain is None else np.asarray(gain)[:, None, :]
        return self.rms_norm_ref(q0, g, eps)


@pytest.mark.parametrize("bug", ["eps_outside", "sum_not_mean", "norm_over_tokens", "gain_head0",
                                 "untransposed", "token_major_split", "normalise_k"])
def test_planted_mistakes_fail(bug):
    failed = [n for n, ok in _pins(_Mutant(bug)) if not ok]
    assert failed, bug
