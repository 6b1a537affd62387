"""Function-by-function pins of the fp64 oracle.

Every public function of ``oracle`` is checked here, by name, against
something other than itself: torch's fp64 CPU attention routine
(``scaled_dot_product_attention``, math path) or autograd, a pure-Python
scalar brute force, or a closed form.  ``test_every_public_function_is_pinned``
keeps the list complete: a new public oracle function without an entry in
``PINNED_BY`` fails it.

The latents of the encoder and decoder may be shared by the batch
([H, M, D]) or given per batch element ([B, H, M, D]); both layouts are
pinned, with batch elements whose latents differ, and a copy of the oracle
that ignores the batch index of per-batch latents must fail those pins.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.flarepp_oracle as fwd_oracle


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _brute_attention(Q, K, V, scale):
    """softmax(scale Q K^T) V with Python scalars."""
    out = []
    for qr in Q:
        sc = [scale * math.fsum(a * b for a, b in zip(qr, kr)) for kr in K]
        top = max(sc)
        w = [math.exp(s - top) for s in sc]
        tot = math.fsum(w)
        out.append([math.fsum(wi * vr[d] for wi, vr in zip(w, V)) / tot
                    for d in range(len(V[0]))])
    return np.array(out)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# single-head building blocks
# ---------------------------------------------------------------------------

def test_gate_sigma_pin():
    g = np.array([-np.inf, -30.0, -1.5, 0.0, 0.7, 30.0, np.inf])
    want = torch.sigmoid(_t(g)).numpy()
    got = oracle.gate_sigma(g)
    assert got[0] == 0.0 and got[-1] == 1.0
    assert _rel(got, want) <= 1e-15


def test_nan_gate_propagates_to_its_head_only():
    """A NaN gate logit gives a NaN routing query for its head, so that
    head's output is NaN; the other heads are the ones of a finite gate."""
    r = _rng(31)
    B, H, N, M, D = 1, 3, 40, 6, 4
    x = dict(q0=r.standard_normal((H, M, D)), q_fixed=r.standard_normal((H, M, D)),
             gate=np.array([0.4, np.nan, -np.inf]), k0=r.standard_normal((B, H, N, D)),
             k=r.standard_normal((B, H, N, D)), v=r.standard_normal((B, H, N, D)))
    y = oracle.flarepp_ref(**x)
    assert np.all(np.isnan(y[:, 1]))
    finite = dict(x, gate=np.array([0.4, 0.0, -np.inf]))
    y_ok = oracle.flarepp_ref(**finite)
    assert np.array_equal(y[:, 0], y_ok[:, 0]) and np.array_equal(y[:, 2], y_ok[:, 2])


def test_attention_matrix_pin():
    r = _rng(11)
    q, k = r.standard_normal((7, 5)), r.standard_normal((13, 5))
    for scale in (1.0, 1 / math.sqrt(5), 3.0):
        A = oracle.attention_matrix(q, k, scale)
        want = torch.softmax(scale * (_t(q) @ _t(k).T), dim=1).numpy()
        assert A.shape == (7, 13)
        assert _rel(A, want) <= 1e-13
        assert np.max(np.abs(A.sum(axis=1) - 1.0)) <= 1e-14
    # a large score spread stays finite (the row maximum is subtracted)
    A = oracle.attention_matrix(100.0 * q, k, 10.0)
    assert np.all(np.isfinite(A))


def test_attention_pin_torch_and_brute():
    r = _rng(12)
    q, k, v = r.standard_normal((4, 3)), r.standard_normal((6, 3)), r.standard_normal((6, 2))
    got = oracle.attention(q, k, v, 0.8)
    want = F.scaled_dot_product_attention(_t(q)[None], _t(k)[None], _t(v)[None],
                                          scale=0.8)[0].numpy()
    assert _rel(got, want) <= 1e-13
    assert _rel(got, _brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.8)) <= 1e-13


def test_attention_backward_pin_autograd():
    r = _rng(13)
    q, k, v = r.standard_normal((5, 4)), r.standard_normal((9, 4)), r.standard_normal((9, 3))
    dout = r.standard_normal((5, 3))
    scale = 0.6
    dq, dk, dv = oracle.attention_backward(q, k, v, scale, dout)
    qt, kt, vt = (_t(a).requires_grad_(True) for a in (q, k, v))
    o = torch.softmax(scale * qt @ kt.T, dim=1) @ vt
    o.backward(_t(dout))
    assert _rel(dq, qt.grad.numpy()) <= 1e-12
    assert _rel(dk, kt.grad.numpy()) <= 1e-12
    assert _rel(dv, vt.grad.numpy()) <= 1e-12


# ---------------------------------------------------------------------------
# encoder / decoder with shared and per-batch latents
# ---------------------------------------------------------------------------

def _enc_inputs(seed, B=3, H=2, N=23, M=5, D=4):
    r = _rng(seed)
    return dict(q_shared=r.standard_normal((H, M, D)),
                q_batch=r.standard_normal((B, H, M, D)),
                k=r.standard_normal((B, H, N, D)),
                v=r.standard_normal((B, H, N, D)),
                z=r.standard_normal((B, H, M, D)))


def _torch_encode(q, k, v, scale):
    qt = _t(q)
    if qt.dim() == 3:
        qt = qt.unsqueeze(0).expand(np.shape(k)[0], -1, -1, -1).contiguous()
    return F.scaled_dot_product_attention(qt, _t(k), _t(v), scale=scale).numpy()


def _torch_decode(q, z, k, scale):
    qt = _t(q)
    if qt.dim() == 3:
        qt = qt.unsqueeze(0).expand(np.shape(k)[0], -1, -1, -1).contiguous()
    return F.scaled_dot_product_attention(_t(k), qt, _t(z), scale=scale).numpy()


@pytest.mark.parametrize("layout", ["shared", "per_batch"])
def test_encode_ref_pin(layout):
    x = _enc_inputs(21)
    q = x["q_shared"] if layout == "shared" else x["q_batch"]
    for scale in (0.5, 1.0):
        got = oracle.encode_ref(q, x["k"], x["v"], scale)
        assert _rel(got, _torch_encode(q, x["k"], x["v"], scale)) <= 1e-13


@pytest.mark.parametrize("layout", ["shared", "per_batch"])
def test_decode_ref_pin(layout):
    x = _enc_inputs(22)
    q = x["q_shared"] if layout == "shared" else x["q_batch"]
    for scale in (0.5, 1.0):
        got = oracle.decode_ref(q, x["z"], x["k"], scale)
        assert _rel(got, _torch_decode(q, x["z"], x["k"], scale)) <= 1e-13


def test_per_batch_latents_brute_force():
    """Scalar brute force of one (b, h) with per-batch latents, b != 0."""
    x = _enc_inputs(23, B=2, H=2, N=6, M=3, D=2)
    b, h, s = 1, 1, 0.9
    qbh = x["q_batch"][b, h]
    z = oracle.encode_ref(x["q_batch"], x["k"], x["v"], s)
    want_z = _brute_attention(qbh.tolist(), x["k"][b, h].tolist(), x["v"][b, h].tolist(), s)
    assert _rel(z[b, h], want_z) <= 1e-13
    y = oracle.decode_ref(x["q_batch"], x["z"], x["k"], s)
    want_y = _brute_attention(x["k"][b, h].tolist(), qbh.tolist(), x["z"][b, h].tolist(), s)
    assert _rel(y[b, h], want_y) <= 1e-13


def test_per_batch_equal_latents_match_shared():
    x = _enc_inputs(24)
    B = x["k"].shape[0]
    qb = np.broadcast_to(x["q_shared"], (B,) + x["q_shared"].shape).copy()
    assert np.array_equal(oracle.encode_ref(qb, x["k"], x["v"], 0.7),
                          oracle.encode_ref(x["q_shared"], x["k"], x["v"], 0.7))
    assert np.array_equal(oracle.decode_ref(qb, x["z"], x["k"], 0.7),
                          oracle.decode_ref(x["q_shared"], x["z"], x["k"], 0.7))


def test_ignoring_the_batch_index_fails_the_per_batch_pins(monkeypatch):
    """Planted mistake: per-batch latents read from batch element 0 only."""
    monkeypatch.setattr(fwd_oracle, "_per_batch_latent",
                        lambda q, b, h: np.asarray(q)[h] if np.ndim(q) == 3 else np.asarray(q)[0, h])
    x = _enc_inputs(25)
    got = oracle.encode_ref(x["q_batch"], x["k"], x["v"], 1.0)
    assert _rel(got, _torch_encode(x["q_batch"], x["k"], x["v"], 1.0)) > 1e-3
    got = oracle.decode_ref(x["q_batch"], x["z"], x["k"], 1.0)
    assert _rel(got, _torch_decode(x["q_batch"], x["z"], x["k"], 1.0)) > 1e-3


# ---------------------------------------------------------------------------
# synthesis
# ---------------------------------------------------------------------------

def test_synthesis_ref_pin():
    """q_dyn = softmax(s q0 k0^T) k0: the first call of the FLARE++ listing,
    keys and values both k0 (issue #2024, three input projections)."""
    r = _rng(31)
    B, H, N, M, D = 2, 3, 17, 4, 8
    q0, k0 = r.standard_normal((H, M, D)), r.standard_normal((B, H, N, D))
    s = 1 / math.sqrt(D)
    got = oracle.synthesis_ref(q0, k0, s)
    q0t = _t(q0).unsqueeze(0).expand(B, -1, -1, -1).contiguous()
    want = F.scaled_dot_product_attention(q0t, _t(k0), _t(k0), scale=s).numpy()
    assert got.shape == (B, H, M, D)
    assert _rel(got, want) <= 1e-13


def test_synthesis_ref_closed_forms():
    r = _rng(32)
    H, M, D = 2, 5, 4
    q0 = r.standard_normal((H, M, D))
    # one token: every seed synthesizes that token's key
    k0 = r.standard_normal((1, H, 1, D))
    got = oracle.synthesis_ref(q0, k0, 0.5)
    assert np.array_equal(got, np.broadcast_to(k0, (1, H, M, D)))
    # identical keys: the result is that key whatever the seeds
    row = r.standard_normal(D)
    k0 = np.broadcast_to(row, (2, H, 9, D)).copy()
    got = oracle.synthesis_ref(q0, k0, 0.5)
    assert np.max(np.abs(got - row)) <= 1e-14


def test_head_intermediates_pin_torch():
    """q, q_dyn, z, y of one (b, h) against torch's attention, gate open and
    closed (the closed gate has no synthesis: q_dyn is None, q = q_fixed)."""
    r = _rng(33)
    B, H, N, M, D = 2, 2, 19, 4, 8
    q0, qf = r.standard_normal((H, M, D)), r.standard_normal((H, M, D))
    k0, k, v = (r.standard_normal((B, H, N, D)) for _ in range(3))
    gate = np.array([0.4, -np.inf])
    s = 1 / math.sqrt(D)
    for h in range(H):
        it = oracle.flarepp_head_intermediates(q0, qf, gate, k0, k, v, 1, h)
        T = lambda a: _t(a)[None]
        if h == 1:
            assert it["q_dyn"] is None and it["A0"] is None
            q = qf[h]
        else:
            qd = F.scaled_dot_product_attention(T(q0[h]), T(k0[1, h]), T(k0[1, h]), scale=s)[0]
            assert _rel(it["q_dyn"], qd.numpy()) <= 1e-13
            q = qf[h] + torch.sigmoid(torch.tensor(0.4, dtype=torch.float64)).item() * qd.numpy()
        assert _rel(it["q"], q) <= 1e-13
        z = F.scaled_dot_product_attention(T(q), T(k[1, h]), T(v[1, h]), scale=s)[0].numpy()
        y = F.scaled_dot_product_attention(T(k[1, h]), T(q), T(z), scale=s)[0].numpy()
        assert _rel(it["z"], z) <= 1e-13
        assert _rel(it["y"], y) <= 1e-13


# ---------------------------------------------------------------------------
# token-sharded encoder statistics (issue #2024, "Multi-GPU context
# parallelism"): per-shard (m, l, O) and their log-sum-exp merge
# ---------------------------------------------------------------------------

def test_encode_partials_ref_brute_force():
    r = _rng(41)
    q, k, v = r.standard_normal((3, 2)), r.standard_normal((7, 2)), r.standard_normal((7, 2))
    bounds = [(0, 3), (3, 4), (4, 7)]
    m, l, O = oracle.encode_partials_ref(q, k, v, 0.7, bounds)
    for c, (a, e) in enumerate(bounds):
        for i in range(3):
            sc = [0.7 * math.fsum(x * y for x, y in zip(q[i], k[j])) for j in range(a, e)]
            mc = max(sc)
            w = [math.exp(t - mc) for t in sc]
            assert abs(m[c, i] - mc) <= 1e-15
            assert abs(l[c, i] - math.fsum(w)) <= 1e-14
            for d in range(2):
                want = math.fsum(wj * v[j, d] for wj, j in zip(w, range(a, e)))
                assert abs(O[c, i, d] - want) <= 1e-14 * max(1.0, abs(want))


def test_merge_partials_ref_pin():
    r = _rng(42)
    q, k, v = r.standard_normal((4, 3)), r.standard_normal((11, 3)), r.standard_normal((11, 2))
    want = oracle.attention(q, k, v, 1.3)
    # one shard: the merge is O / l
    m, l, O = oracle.encode_partials_ref(q, k, v, 1.3, [(0, 11)])
    assert _rel(oracle.merge_partials_ref(m, l, O), O[0] / l[0][:, None]) <= 1e-15
    # several shards, given in any order, rebuild the full attention
    m, l, O = oracle.encode_partials_ref(q, k, v, 1.3, [(0, 2), (2, 9), (9, 11)])
    assert _rel(oracle.merge_partials_ref(m, l, O), want) <= 1e-14
    perm = [2, 0, 1]
    assert _rel(oracle.merge_partials_ref(m[perm], l[perm], O[perm]), want) <= 1e-14


@pytest.mark.parametrize("layout", ["shared", "per_batch"])
def test_encode_sharded_ref_pin(layout):
    x = _enc_inputs(43, N=31)
    q = x["q_shared"] if layout == "shared" else x["q_batch"]
    for shards in (1, 4, 31):
        got = oracle.encode_sharded_ref(q, x["k"], x["v"], 0.9, shards)
        assert _rel(got, _torch_encode(q, x["k"], x["v"], 0.9)) <= 1e-13


# ---------------------------------------------------------------------------
# coverage of the public surface
# ---------------------------------------------------------------------------

PINNED_BY = {
    # forward (this file and tests/test_oracle_pins.py)
    "gate_sigma": "test_gate_sigma_pin",
    "attention": "test_attention_pin_torch_and_brute",
    "attention_matrix": "test_attention_matrix_pin",
    "encode_ref": "test_encode_ref_pin",
    "decode_ref": "test_decode_ref_pin",
    "flare_ref": "test_oracle_pins.py::test_flare_listing_scale_one_vs_torch",
    "flarepp_ref": "test_oracle_pins.py::test_oracle_pin",
    "simplified_flarepp_ref": "test_oracle_pins.py::test_simplified_vs_torch",
    "flarepp_head_intermediates": "test_head_intermediates_pin_torch",
    "synthesis_ref": "test_synthesis_ref_pin",
    "encode_partials_ref": "test_encode_partials_ref_brute_force",
    "merge_partials_ref": "test_merge_partials_ref_pin",
    "encode_sharded_ref": "test_encode_sharded_ref_pin",
    # gradients (tests/test_oracle_backward.py)
    "attention_backward": "test_attention_backward_pin_autograd",
    "flare_bwd_ref": "test_oracle_backward.py",
    "flarepp_bwd_ref": "test_oracle_backward.py",
    "simplified_flarepp_bwd_ref": "test_oracle_backward.py",
    # front end (tests/test_oracle_frontend.py)
    "rms_norm_ref": "test_oracle_frontend.py",
    "projection_ref": "test_oracle_frontend.py",
    "frontend_ref": "test_oracle_frontend.py",
    "seed_norm_ref": "test_oracle_frontend.py",
}


def test_every_public_function_is_pinned():
    import os
    here = os.path.dirname(__file__)
    missing = sorted(set(oracle.__all__) - set(PINNED_BY))
    assert not missing, f"public oracle functions without a pin: {missing}"
    stale = sorted(set(PINNED_BY) - set(oracle.__all__))
    assert not stale, f"pins of functions that are gone: {stale}"
    for name, where in PINNED_BY.items():
        fname, _, test = where.partition("::")
        if fname.startswith("test_") and fname.endswith(".py"):
            with open(os.path.join(here, fname)) as f:
                text = f.read()
            assert name in text, f"{fname} never calls {name}"
            if test:
                assert f"def {test}" in text, f"{where} does not exist"
        else:
            assert f"def {where}" in open(__file__).read(), f"{where} does not exist"
