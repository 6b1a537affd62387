"""Plain fp64 CPU oracle for the FLARE++ token-mixer forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The GPU library never routes through it and shares no code with it.

What is computed (and where the pages define it):

* "FLARE++ and FLARE: Low-rank attention routing for PDE surrogates"
  (FLARE.py README), section "FLARE++", core token-mixer listing: the mixer is
  three scaled-dot-product attention calls plus a gate.  The first call lets
  the learned seeds q0 [H,M,D] attend over k0, with k0 serving as both key and
  value; the gated routing query is q_fixed + gate * q_dyn; the second call
  encodes the N tokens into M latents (queries q, keys k, values v); the third
  decodes back to the N tokens (queries k, keys q, values z).  All calls use
  the attention default scale 1/sqrt(D).
* "[FEA]: Update FLARE++ to the v2 reference design and add token-sharded
  context parallelism for FLARE/FLARE++ #2024", section "Changes from v1 to
  v2", item "Fixed reference and gate": the gate is sigma(g) of a per-head
  logit g, and with the gate closed the mixer is FLARE.  Item "Three input
  projections instead of four": synthesis keys and values are shared (k0).
* Same issue, section "Multi-GPU context parallelism": the token-sharded
  encoder is exact; shards exchange latent-sized partial outputs and
  log-sum-exp statistics and rebuild the globally normalised attention.
  ``encode_sharded_ref`` is that merge, written from the definition.
* FLARE.py README, section "FLARE": two-step FLARE, encode then decode with a
  caller-chosen scale (the listing there passes 1.0).

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

* scale is 1/sqrt(D) for all three FLARE++ calls; ``flare_ref`` takes it;
* the gate arrives as fp32 logits g[H]; sigma is applied here in fp64, with
  g = -inf giving exactly 0 (synthesis skipped) and g = +inf giving 1;
* the [H,M,D] latents are shared by every batch element b;
* inputs are the dtype-rounded values upcast exactly to fp64; all arithmetic
  here is fp64 and every attention matrix is materialised;
* no mask: every query attends to every key.

Pinned by tests/test_oracle_pins.py (closed forms, invariants, brute force,
hand-worked golden cases and an independent library attention routine) and,
function by function, by tests/test_oracle_units.py (every public function
here against torch's fp64 attention or autograd, scalar brute force or a
closed form, including latents given per batch element).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "gate_sigma",
    "attention",
    "attention_matrix",
    "encode_ref",
    "decode_ref",
    "flare_ref",
    "flarepp_ref",
    "simplified_flarepp_ref",
    "flarepp_head_intermediates",
    "synthesis_ref",
    "encode_partials_ref",
    "merge_partials_ref",
    "encode_sharded_ref",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def gate_sigma(g):
    """Logistic gate sigma(g) = 1 / (1 + exp(-g)) in fp64.

    Issue #2024, "Changes from v1 to v2", "Fixed reference and gate".
    exp(+inf) = inf gives sigma(-inf) = 0 exactly; exp(-inf) = 0 gives 1.
    """
    g = _f64(g)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def attention_matrix(qh, kh, scale):
    """A = softmax_rows(scale * qh @ kh^T) for one head.

    qh: [R, D] queries, kh: [S, D] keys.  Returns A: [R, S]; every row of A
    is a probability vector over the S keys.
    """
    qh = _f64(qh)
    kh = _f64(kh)
    L = qh @ kh.T
    L *= float(scale)
    L -= L.max(axis=1, keepdims=True)
    np.exp(L, out=L)
    L /= L.sum(axis=1, keepdims=True)
    return L


def attention(qh, kh, vh, scale):
    """Scaled-dot-product attention for one head: softmax(scale q k^T) v.

    qh: [R, D], kh: [S, D], vh: [S, Dv] -> [R, Dv].
    """
    A = attention_matrix(qh, kh, scale)
    return A @ _f64(vh)


def _per_batch_latent(q, b, h):
    """Latents may be shared over the batch ([H, M, D]) or per batch
    ([B, H, M, D]); pick the [M, D] slice for (b, h)."""
    q = np.asarray(q)
    return q[h] if q.ndim == 3 else q[b, h]


def encode_ref(q, k, v, scale):
    """Encode N tokens into M latents: z[b,h] = softmax(scale q k^T) v.

    FLARE.py README, "FLARE++" listing (second attention call) and "FLARE"
    listing (gather step).  q: [H,M,D] or [B,H,M,D]; k, v: [B,H,N,D].
    Returns z: [B,H,M,D] fp64.
    """
    B, H, _, _ = np.shape(k)
    M = np.shape(q)[-2]
    Dv = np.shape(v)[-1]
    z = np.empty((B, H, M, Dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            z[b, h] = attention(_per_batch_latent(q, b, h), k[b, h], v[b, h], scale)
    return z


def decode_ref(q, z, k, scale):
    """Decode M latents back to N tokens: y[b,h] = softmax(scale k q^T) z.

    The softmax runs over the M latents for each token (the tokens are the
    queries, the routing queries q are the keys and z the values).
    FLARE.py README, "FLARE++" listing (third call), "FLARE" listing
    (scatter step).  q: [H,M,D] or [B,H,M,D]; z: [B,H,M,Dv]; k: [B,H,N,D].
    """
    B, H, N, _ = np.shape(k)
    Dv = np.shape(z)[-1]
    y = np.empty((B, H, N, Dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            y[b, h] = attention(k[b, h], _per_batch_latent(q, b, h), z[b, h], scale)
    return y


def flare_ref(q, k, v, scale):
    """Two-step FLARE mixer: encode with latents q, then decode.

    FLARE.py README, section "FLARE", listing; the scale is the caller's.
    q: [H,M,D]; k, v: [B,H,N,D] -> y [B,H,N,D].
    """
    z = encode_ref(q, k, v, scale)
    return decode_ref(q, z, k, scale)


def synthesis_ref(q0, k0, scale):
    """Query synthesis: q_dyn[b,h] = softmax(scale q0 k0^T) k0.

    FLARE.py README, "FLARE++" listing (first call, keys = values = k0);
    issue #2024 "Sharing synthesis keys and values".  Returns [B,H,M,D].
    """
    return encode_ref(q0, k0, k0, scale)


def flarepp_head_intermediates(q0, q_fixed, gate, k0, k, v, b, h):
    """All intermediates of the FLARE++ mixer for one (b, h), in fp64.

    Returns a dict with sigma, q_dyn (None when the gate is closed), q, z, y
    and the three attention matrices A0 (synthesis, M x N), A1 (encode,
    M x N) and A2 (decode, N x M; A0 is None when the gate is closed).
    Scale is 1/sqrt(D) in all three calls (attention default scale, FLARE++
    listing of the FLARE.py README).
    """
    D = np.shape(k)[-1]
    s = 1.0 / np.sqrt(D)
    sig = float(gate_sigma(np.asarray(gate)[h]))
    qf = _f64(q_fixed[h])
    if sig == 0.0:
        # closed gate: q is the fixed reference alone, FLARE exactly
        A0 = None
        q_dyn = None
        q = qf.copy()
    else:
        A0 = attention_matrix(q0[h], k0[b, h], s)
        q_dyn = A0 @ _f64(k0[b, h])
        q = qf + sig * q_dyn
    A1 = attention_matrix(q, k[b, h], s)
    z = A1 @ _f64(v[b, h])
    A2 = attention_matrix(k[b, h], q, s)
    y = A2 @ z
    return dict(sigma=sig, q_dyn=q_dyn, q=q, z=z, y=y, A0=A0, A1=A1, A2=A2)


def flarepp_ref(q0, q_fixed, gate, k0, k, v, return_intermediates=False):
    """FLARE++ token mixer y = mixer(q0, q_fixed, gate, k0, k, v) in fp64.

    q0, q_fixed: [H,M,D]; gate: [H] logits; k0, k, v: [B,H,N,D].
    Steps per (b, h), scale s = 1/sqrt(D):
      sigma = 1/(1+exp(-g_h));
      q_dyn = softmax(s q0 k0^T) k0          (skipped when sigma == 0);
      q     = q_fixed + sigma q_dyn;
      z     = softmax(s q k^T) v;
      y     = softmax(s k q^T) z.
    With return_intermediates, also returns dict(q=[B,H,M,D], z=[B,H,M,D]).
    """
    B, H, N, D = np.shape(k)
    M = np.shape(q0)[-2]
    s = 1.0 / np.sqrt(D)
    y = np.empty((B, H, N, D), dtype=np.float64)
    qs = np.empty((B, H, M, D), dtype=np.float64)
    zs = np.empty((B, H, M, D), dtype=np.float64)
    sig = gate_sigma(gate)
    for b in range(B):
        for h in range(H):
            qf = _f64(q_fixed[h])
            if sig[h] == 0.0:
                q = qf.copy()
            else:
                q = qf + sig[h] * attention(q0[h], k0[b, h], k0[b, h], s)
            z = attention(q, k[b, h], v[b, h], s)
            y[b, h] = attention(k[b, h], q, z, s)
            qs[b, h] = q
            zs[b, h] = z
    if return_intermediates:
        return y, dict(q=qs, z=zs)
    return y


def simplified_flarepp_ref(q0, k0, v0, k, v):
    """Simplified FLARE++ (what the first preprint called FLARE++) in fp64.

    Issue #2024, "v1 vs. v2" and "Changes from v1 to v2": four input
    projections (the synthesis has its own values v0) and no fixed reference
    or gate (the routing queries are the synthesized ones); the paper summary
    "FLARE++: Low-rank attention with dynamic attention routing",
    "Dynamic Query Synthesis": the seeds attend over the input tokens and the
    M results serve as the routing queries of the FLARE encode-decode pair.
    Per (b, h), s = 1/sqrt(D):
      q = softmax(s q0 k0^T) v0;  z = softmax(s q k^T) v;  y = softmax(s k q^T) z.
    q0: [H,M,D]; k0, v0, k, v: [B,H,N,D].
    """
    B, H, N, D = np.shape(k)
    s = 1.0 / np.sqrt(D)
    y = np.empty((B, H, N, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            q = attention(q0[h], k0[b, h], v0[b, h], s)
            z = attention(q, k[b, h], v[b, h], s)
            y[b, h] = attention(k[b, h], q, z, s)
    return y


# --------------------------------------------------------------------------
# Token-sharded (split-N) encoder with log-sum-exp statistics.
# Issue #2024, "Multi-GPU context parallelism for FLARE and FLARE++": each
# shard contributes latent-sized outputs plus softmax statistics, and the
# merge rebuilds the globally normalised encoder output exactly.
# --------------------------------------------------------------------------

def encode_partials_ref(qh, kh, vh, scale, bounds):
    """Per-shard statistics for one head.

    qh [M,D], kh/vh [N,D]; bounds: list of (start, stop) token ranges.
    For each shard c with scores L_c = scale qh kh_c^T:
      m_c = row max of L_c, l_c = row sum of exp(L_c - m_c),
      O_c = exp(L_c - m_c) vh_c (unnormalised).
    Returns (m [C,M], l [C,M], O [C,M,Dv]).
    """
    qh = _f64(qh)
    kh = _f64(kh)
    vh = _f64(vh)
    ms, ls, Os = [], [], []
    for (a, e) in bounds:
        L = scale * (qh @ kh[a:e].T)
        m = L.max(axis=1)
        E = np.exp(L - m[:, None])
        ms.append(m)
        ls.append(E.sum(axis=1))
        Os.append(E @ vh[a:e])
    return np.stack(ms), np.stack(ls), np.stack(Os)


def merge_partials_ref(m, l, O):
    """Log-sum-exp merge of shard statistics into the normalised output.

    m* = max_c m_c; w_c = exp(m_c - m*); z = sum_c w_c O_c / sum_c w_c l_c.
    """
    m = _f64(m)
    mstar = m.max(axis=0)
    w = np.exp(m - mstar[None, :])
    num = (w[:, :, None] * _f64(O)).sum(axis=0)
    den = (w * _f64(l)).sum(axis=0)
    return num / den[:, None]


def encode_sharded_ref(q, k, v, scale, num_shards):
    """Encoder output computed shard by shard and merged (see above).

    Splits the N tokens into ``num_shards`` contiguous ranges of nearly equal
    length.  Equal to ``encode_ref`` up to fp64 rounding.
    """
    B, H, N, _ = np.shape(k)
    M = np.shape(q)[-2]
    Dv = np.shape(v)[-1]
    edges = np.linspace(0, N, num_shards + 1).round().astype(int)
    bounds = [(int(edges[i]), int(edges[i + 1])) for i in range(num_shards)
              if edges[i + 1] > edges[i]]
    z = np.empty((B, H, M, Dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            m, l, O = encode_partials_ref(_per_batch_latent(q, b, h), k[b, h],
                                          v[b, h], scale, bounds)
            z[b, h] = merge_partials_ref(m, l, O)
    return z
