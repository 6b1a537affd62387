"""Plain fp64 CPU gradients of the FLARE++ and FLARE mixers.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as flarepp_oracle.py).

The pages define the forward pass (FLARE.py README, "FLARE++" and "FLARE"
listings; issue #2024, "Changes from v1 to v2") and state that the
token-sharded encoder has a custom backward (issue #2024, "Multi-GPU context
parallelism"), whose derivation (Appendix B of the paper) is not on the
pages.  The gradients here are therefore derived from the forward definition
by the chain rule, with every attention matrix materialised:

For one attention O = A V, A = softmax_rows(s Q K^T), given dO:
  dV = A^T dO
  dA = dO V^T
  dS = A * (dA - rowsum(dA * A))          (softmax Jacobian, row by row)
  dQ = s dS K ,   dK = s dS^T Q

FLARE++ per (b, h):  q_dyn = att(q0, k0, k0), q = q_fixed + sigma q_dyn,
z = att(q, k, v), y = att(k, q, z).  Backward: the decoder gives dk, dq and
dz; the encoder adds to dq and dk and gives dv; the gate step gives
dq_fixed = sum_b dq, d(q_dyn) = sigma dq, dsigma = sum dq * q_dyn and
dgate = dsigma sigma (1 - sigma); the synthesis (k0 as key and value) gives
dq0 and dk0.  Latents q0 and q_fixed are shared over the batch, so their
gradients sum over b.
"""

from __future__ import annotations

import numpy as np

from .flarepp_oracle import attention_matrix, gate_sigma

__all__ = ["attention_backward", "flare_bwd_ref", "flarepp_bwd_ref",
           "simplified_flarepp_bwd_ref"]


def attention_backward(qh, kh, vh, scale, dout):
    """Gradients of softmax(scale qh kh^T) vh for one head.

    qh: [R, D], kh: [S, D], vh: [S, Dv], dout: [R, Dv].
    Returns (dq [R, D], dk [S, D], dv [S, Dv]) in fp64.
    """
    qh = np.asarray(qh, np.float64)
    kh = np.asarray(kh, np.float64)
    vh = np.asarray(vh, np.float64)
    dout = np.asarray(dout, np.float64)
    A = attention_matrix(qh, kh, scale)            # [R, S]
    dv = A.T @ dout
    dA = dout @ vh.T
    dS = A * (dA - np.sum(dA * A, axis=1, keepdims=True))
    dq = scale * (dS @ kh)
    dk = scale * (dS.T @ qh)
    return dq, dk, dv


def _flare_head_bwd(q, k, v, scale, dy):
    """FLARE for one (b, h): z = att(q, k, v), y = att(k, q, z).
    Returns (dq, dk, dv) with dq the latent gradient of this (b, h)."""
    A1 = attention_matrix(q, k, scale)
    z = A1 @ np.asarray(v, np.float64)
    # decoder: queries k, keys q, values z
    dk_dec, dq_dec, dz = attention_backward(k, q, z, scale, dy)
    # encoder: queries q, keys k, values v
    dq_enc, dk_enc, dv = attention_backward(q, k, v, scale, dz)
    return dq_dec + dq_enc, dk_dec + dk_enc, dv


def flare_bwd_ref(q, k, v, scale, dy):
    """Gradients of the two-step FLARE mixer (FLARE.py README, "FLARE").

    q: [H,M,D] (shared over the batch); k, v, dy: [B,H,N,D].
    Returns dq [H,M,D] (summed over b), dk, dv [B,H,N,D].
    """
    B, H, N, D = np.shape(k)
    dq = np.zeros(np.shape(q), np.float64)
    dk = np.empty((B, H, N, D), np.float64)
    dv = np.empty((B, H, N, D), np.float64)
    for b in range(B):
        for h in range(H):
            g = _flare_head_bwd(q[h], k[b, h], v[b, h], scale, dy[b, h])
            dq[h] += g[0]
            dk[b, h] = g[1]
            dv[b, h] = g[2]
    return dq, dk, dv


def flarepp_bwd_ref(q0, q_fixed, gate, k0, k, v, dy):
    """Gradients of the FLARE++ mixer (flarepp_oracle.flarepp_ref).

    Returns dict(dq0 [H,M,D], dq_fixed [H,M,D], dgate [H], dk0, dk, dv
    [B,H,N,D]).  A closed gate (sigma = 0) gives dq0 = 0, dk0 = 0 and
    dgate = 0 (the synthesis does not reach the output).
    """
    B, H, N, D = np.shape(k)
    s = 1.0 / np.sqrt(D)
    sig = gate_sigma(gate)
    out = dict(dq0=np.zeros(np.shape(q0), np.float64),
               dq_fixed=np.zeros(np.shape(q_fixed), np.float64),
               dgate=np.zeros(H, np.float64),
               dk0=np.zeros((B, H, N, D), np.float64),
               dk=np.empty((B, H, N, D), np.float64),
               dv=np.empty((B, H, N, D), np.float64))
    for b in range(B):
        for h in range(H):
            qf = np.asarray(q_fixed[h], np.float64)
            if sig[h] == 0.0:
                qd = np.zeros_like(qf)
            else:
                qd = attention_matrix(q0[h], k0[b, h], s) @ np.asarray(k0[b, h], np.float64)
            q = qf + sig[h] * qd
            dq, dk, dv = _flare_head_bwd(q, k[b, h], v[b, h], s, dy[b, h])
            out["dk"][b, h] = dk
            out["dv"][b, h] = dv
            out["dq_fixed"][h] += dq
            if sig[h] == 0.0:
                continue
            out["dgate"][h] += np.sum(dq * qd) * sig[h] * (1.0 - sig[h])
            dq0, dk0_key, dk0_val = attention_backward(q0[h], k0[b, h], k0[b, h], s, sig[h] * dq)
            out["dq0"][h] += dq0
            out["dk0"][b, h] = dk0_key + dk0_val
    return out


def simplified_flarepp_bwd_ref(q0, k0, v0, k, v, dy):
    """Gradients of the simplified mixer (flarepp_oracle.simplified_flarepp_ref):
    q = att(q0, k0, v0), then FLARE with q.  Returns dict(dq0, dk0, dv0, dk, dv)."""
    B, H, N, D = np.shape(k)
    s = 1.0 / np.sqrt(D)
    out = dict(dq0=np.zeros(np.shape(q0), np.float64),
               dk0=np.empty((B, H, N, D), np.float64), dv0=np.empty((B, H, N, D), np.float64),
               dk=np.empty((B, H, N, D), np.float64), dv=np.empty((B, H, N, D), np.float64))
    for b in range(B):
        for h in range(H):
            q = attention_matrix(q0[h], k0[b, h], s) @ np.asarray(v0[b, h], np.float64)
            dq, dk, dv = _flare_head_bwd(q, k[b, h], v[b, h], s, dy[b, h])
            out["dk"][b, h] = dk
            out["dv"][b, h] = dv
            dq0, dk0, dv0 = attention_backward(q0[h], k0[b, h], v0[b, h], s, dq)
            out["dq0"][h] += dq0
            out["dk0"][b, h] = dk0
            out["dv0"][b, h] = dv0
    return out
