"""Seeded synthetic inputs for the FLARE++ mixer workloads.

This module holds only random-number generation and dtype rounding: none of
the mixer's arithmetic.  It is the one piece shared by the GPU-side callers
(tests, bench, smoke) and the oracle-side callers, which each receive the
same host arrays.

Workloads (shapes from the pages' settings, values synthetic):

* ``tiny_fp32``          B=1  H=2  N=1024      M=16  D=8   fp32
* ``small_mesh_bf16``    B=4  H=8  N=4096      M=64  D=16  bf16, tensors
  scaled by 1/sqrt(D)
* ``point_cloud_bf16``   B=2  H=8  N=40000     M=256 D=32  bf16, k0/k/v are
  noise plus a smooth rank-8 field over random 3-D points, tokens shuffled
* ``million_token_bf16`` B=1  H=8  N=1048576   M=512 D=32  bf16 (headline)
* ``wide_heads_fp16_gate_closed`` / ``wide_heads_fp16``
                         B=8  H=16 N=16384     M=128 D=64  fp16; identical
  tensors, the first with every gate logit = -inf (two-step FLARE).

Recipe: NumPy ``Generator(PCG64(seed))``; draws in fp32 in the order q0,
q_fixed, gate, k0, k, v (then the point-cloud extras, see ``_point_cloud``);
every tensor except the gate is rounded to the workload dtype with
round-to-nearest-even.  Arrays come back as float32 holding exactly
representable values of that dtype, so the GPU side converts them to its
dtype losslessly and the oracle upcasts them to fp64 exactly.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get_workload", "make_inputs",
           "make_random_inputs", "make_simplified_inputs", "round_to_dtype", "DTYPES"]

DTYPES = ("fp32", "bf16", "fp16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    M: int
    D: int
    dtype: str
    seed: int
    kind: str = "iid"          # "iid" | "iid_scaled" | "point_cloud"
    gate: str = "random"       # "random" | "closed"
    description: str = ""

    @property
    def shape_dict(self):
        return dict(B=self.B, H=self.H, N=self.N, M=self.M, D=self.D)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 1, 2, 1024, 16, 8, "fp32", seed=1,
                 description="tiny fp32 mixer, iid N(0,1)"),
        Workload("small_mesh_bf16", 4, 8, 4096, 64, 16, "bf16", seed=2,
                 kind="iid_scaled",
                 description="small-mesh bf16 mixer, iid N(0,1)/sqrt(D)"),
        Workload("point_cloud_bf16", 2, 8, 40000, 256, 32, "bf16", seed=3,
                 kind="point_cloud",
                 description="irregular 3-D point cloud, noise + rank-8 "
                             "smooth field, shuffled tokens"),
        Workload("million_token_bf16", 1, 8, 1048576, 512, 32, "bf16", seed=4,
                 description="million-token bf16 mixer, iid N(0,1)"),
        Workload("wide_heads_fp16_gate_closed", 8, 16, 16384, 128, 64, "fp16",
                 seed=5, gate="closed",
                 description="wide heads fp16, gate logits -inf (FLARE)"),
        Workload("wide_heads_fp16", 8, 16, 16384, 128, 64, "fp16", seed=5,
                 description="wide heads fp16, gate logits iid N(0,1)"),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp32 values to ``dtype`` (round to nearest, ties to even) and
    return them as float32 (exact for every dtype handled here)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # RNE on the upper 16 bits; inputs here are finite
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
        return r.view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng, shape, scale=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def _point_cloud(rng, B, H, N, D, base):
    """Add a smooth rank-8 field over random 3-D points to the noise tensors.

    Per sample b: points p_n ~ U[0,1]^3 and random Fourier features
    phi_r(p) = sqrt(2) cos(2 pi <omega_r, p> + beta_r), r = 1..8, with
    omega_r ~ N(0, I_3), beta_r ~ U[0, 2 pi).  Per tensor and head a mixing
    matrix W [8, D] ~ N(0, 1/8) adds Phi W to that head's noise (rank 8,
    about unit variance).  Finally one random token permutation per sample
    is applied to k0, k and v alike (tokens stored in shuffled order).
    """
    R = 8
    for b in range(B):
        pts = rng.random(size=(N, 3), dtype=np.float32)
        omega = rng.standard_normal(size=(3, R), dtype=np.float32)
        beta = rng.random(size=(R,), dtype=np.float32) * np.float32(2 * math.pi)
        phi = np.float32(math.sqrt(2.0)) * np.cos(
            np.float32(2 * math.pi) * (pts @ omega) + beta)          # [N, R]
        for t in base:                                               # k0, k, v
            W = _normal(rng, (H, R, D), scale=1.0 / math.sqrt(R))
            for h in range(H):
                t[b, h] += phi @ W[h]
        perm = rng.permutation(N)
        for t in base:
            t[b] = t[b][:, perm, :]


def make_inputs(workload, seed: int | None = None):
    """Generate the seeded inputs of a workload.

    Returns a dict with q0, q_fixed [H,M,D], gate [H] (fp32 logits, not
    rounded), k0, k, v [B,H,N,D] as float32 arrays holding dtype-exact
    values, plus 'dtype' and the shape entries.
    """
    w = workload if isinstance(workload, Workload) else get_workload(workload)
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, H, N, M, D = w.B, w.H, w.N, w.M, w.D
    sc = 1.0 / math.sqrt(D) if w.kind == "iid_scaled" else 1.0
    q0 = _normal(rng, (H, M, D), sc)
    q_fixed = _normal(rng, (H, M, D), sc)
    gate = _normal(rng, (H,))
    k0 = _normal(rng, (B, H, N, D), sc)
    k = _normal(rng, (B, H, N, D), sc)
    v = _normal(rng, (B, H, N, D), sc)
    if w.kind == "point_cloud":
        _point_cloud(rng, B, H, N, D, [k0, k, v])
    if w.gate == "closed":
        gate = np.full((H,), -np.inf, dtype=np.float32)
    out = dict(q0=q0, q_fixed=q_fixed, gate=gate.astype(np.float32), k0=k0, k=k, v=v)
    for name in ("q0", "q_fixed", "k0", "k", "v"):
        out[name] = round_to_dtype(out[name], w.dtype)
    out.update(dtype=w.dtype, B=B, H=H, N=N, M=M, D=D)
    return out


def make_random_inputs(B, H, N, M, D, dtype, seed, scale=1.0, gate=None):
    """Seeded iid N(0, scale^2) inputs of arbitrary shape (edge-case tests).

    ``gate``: None for iid N(0,1) logits, a float for a constant logit, or an
    array of H logits.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q0 = _normal(rng, (H, M, D), scale)
    q_fixed = _normal(rng, (H, M, D), scale)
    g = _normal(rng, (H,))
    k0 = _normal(rng, (B, H, N, D), scale)
    k = _normal(rng, (B, H, N, D), scale)
    v = _normal(rng, (B, H, N, D), scale)
    if gate is not None:
        g = np.broadcast_to(np.asarray(gate, dtype=np.float32), (H,)).copy()
    out = dict(q0=q0, q_fixed=q_fixed, gate=g.astype(np.float32), k0=k0, k=k, v=v)
    for name in ("q0", "q_fixed", "k0", "k", "v"):
        out[name] = round_to_dtype(out[name], dtype)
    out.update(dtype=dtype, B=B, H=H, N=N, M=M, D=D)
    return out


def make_simplified_inputs(B, H, N, M, D, dtype, seed, scale=1.0):
    """Seeded iid N(0, scale^2) inputs of the simplified mixer: q0 [H,M,D] and
    k0, v0, k, v [B,H,N,D], drawn in that order and rounded to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(q0=_normal(rng, (H, M, D), scale))
    for name in ("k0", "v0", "k", "v"):
        out[name] = _normal(rng, (B, H, N, D), scale)
    for name in ("q0", "k0", "v0", "k", "v"):
        out[name] = round_to_dtype(out[name], dtype)
    out.update(dtype=dtype, B=B, H=H, N=N, M=M, D=D)
    return out


def make_cotangent(B, H, N, D, dtype, seed, scale=1.0):
    """Seeded output gradient dy ~ iid N(0, scale^2) [B,H,N,D], rounded to
    ``dtype`` (float32 array holding dtype-exact values)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return round_to_dtype(_normal(rng, (B, H, N, D), scale), dtype)


def make_frontend_inputs(B, N, C, H, D, dtype, seed, bias=True, gain=True):
    """Seeded inputs of the block front end: x [B,N,C] ~ N(0,1), the three
    linear-layer weights [H*D, C] ~ N(0, 1/C), biases [H*D] ~ N(0, 0.1^2)
    (or None), the k0 normalisation gain [H, D] ~ U[0.5, 1.5) (or None);
    drawn in that order and rounded to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(x=_normal(rng, (B, N, C)))
    for name in ("w_k0", "w_k", "w_v"):
        out[name] = _normal(rng, (H * D, C), 1.0 / math.sqrt(C))
    for name in ("b_k0", "b_k", "b_v"):
        out[name] = _normal(rng, (H * D,), 0.1) if bias else None
    out["g_k0"] = (rng.random(size=(H, D), dtype=np.float32) + np.float32(0.5)) if gain else None
    for name, a in list(out.items()):
        if a is not None:
            out[name] = round_to_dtype(a, dtype)
    out.update(dtype=dtype, B=B, N=N, C=C, H=H, D=D)
    return out
