"""Plain fp64 CPU oracle for the FLARE++ front end: the input projections
and the head-wise normalisation that feed the mixer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as flarepp_oracle.py).

What the pages state:

* Issue #2024, "[FEA]: Update FLARE++ to the v2 reference design ...",
  section "Changes from v1 to v2": FLARE++ uses three input projections
  instead of four (the synthesis keys and values are shared, so one C -> C
  projection is saved), and it normalises the synthesis call head by head:
  the seeds and the synthesis keys/values.
* FLARE.py README, section "FLARE++": the core mixer itself has no
  projections or normalisation; its listing takes k0, k, v already
  projected, [B, H, N, D].
* The exact form of the normalisation is in the paper's Appendix A, which is
  not on the pages.

Readings taken (each listed in the design notes):

* a projection is an affine map of the token features, x @ W^T + b, with W
  in the [out_features, in_features] = [H*D, C] layout of a linear layer, b
  optional; the H*D outputs split into H heads of D features, head-major;
* the head-wise normalisation is a root-mean-square normalisation over the D
  features of one head of one token (or one seed), with an optional per-head
  gain g[H, D] and a caller-given eps inside the square root:
  u / sqrt(mean_d(u_d^2) + eps) * g;
* it applies to k0 (the shared synthesis keys and values) and to the seeds
  q0; k and v are not normalised.

Pinned by tests/test_oracle_frontend.py (torch fp64 linear and rms_norm,
identity and permutation weights, scale invariance, unit mean square,
planted mistakes).
"""

from __future__ import annotations

import numpy as np

__all__ = ["rms_norm_ref", "projection_ref", "frontend_ref", "seed_norm_ref"]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def rms_norm_ref(u, gain=None, eps=1e-6):
    """u / sqrt(mean(u^2 over the last axis) + eps) * gain, in fp64.

    u: [..., D]; gain: broadcastable to u (e.g. [H, 1, D] for [B,H,N,D]) or None.
    """
    u = _f64(u)
    ms = np.mean(u * u, axis=-1, keepdims=True)
    out = u / np.sqrt(ms + float(eps))
    if gain is not None:
        out = out * _f64(gain)
    return out


def projection_ref(x, w, b, H, D):
    """Head-split projection of the tokens: [B, N, C] -> [B, H, N, D].

    x: [B, N, C]; w: [H*D, C] (linear-layer layout); b: [H*D] or None.
    """
    x = _f64(x)
    w = _f64(w)
    p = x @ w.T                                   # [B, N, H*D]
    if b is not None:
        p = p + _f64(b)
    B, N, _ = x.shape
    return p.reshape(B, N, H, D).transpose(0, 2, 1, 3)


def frontend_ref(x, w_k0, w_k, w_v, H, D, b_k0=None, b_k=None, b_v=None, g_k0=None,
                 eps=1e-6, normalize_k0=True):
    """The three projections of the FLARE++ block input, k0 normalised head-wise.

    Returns (k0, k, v), each [B, H, N, D] fp64.
    """
    k0 = projection_ref(x, w_k0, b_k0, H, D)
    if normalize_k0:
        gain = None if g_k0 is None else _f64(g_k0)[None, :, None, :]
        k0 = rms_norm_ref(k0, gain, eps)
    return k0, projection_ref(x, w_k, b_k, H, D), projection_ref(x, w_v, b_v, H, D)


def seed_norm_ref(q0, gain=None, eps=1e-6):
    """Head-wise normalisation of the seeds q0 [H, M, D]; gain [H, D] or None."""
    g = None if gain is None else _f64(gain)[:, None, :]
    return rms_norm_ref(q0, g, eps)
