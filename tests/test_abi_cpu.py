"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/flarepp.h, sizes workspaces, and rejects every invalid
argument before touching the device.  A valid call on a machine without a
device returns FLAREPP_ERR_HIP instead of crashing.  No compute runs here."""

from __future__ import annotations

import ctypes
import os

import pytest

import rank_latent_attention_mixer_amd as fp

pytestmark = pytest.mark.skipif(not os.path.exists(fp.library_path()),
                                reason="libflarepp.so not built")

OK, INV, UNS, WS, HIP = (fp.FLAREPP_OK, fp.FLAREPP_ERR_INVALID_ARGUMENT,
                         fp.FLAREPP_ERR_UNSUPPORTED, fp.FLAREPP_ERR_WORKSPACE,
                         fp.FLAREPP_ERR_HIP)

# fake, distinct, 256-aligned addresses: never dereferenced because every
# call below fails validation (or the device check) before any launch
FAKE = {name: ctypes.c_void_p(0x10000000 * (i + 1)) for i, name in
        enumerate(["q0", "qf", "gate", "k0", "k", "v", "y", "ws", "z", "v0"])}


def lib():
    return fp.load_library()


def test_every_declared_function_is_exported():
    names = fp.declared_functions()
    assert {"flarepp_mixer_fwd", "flare_mixer_fwd", "flare_encode_fwd", "flare_decode_fwd",
            "flarepp_workspace_size", "flarepp_status_string"} <= set(names)
    L = lib()
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_status_strings_and_version():
    for code, name in [(OK, "FLAREPP_OK"), (INV, "FLAREPP_ERR_INVALID_ARGUMENT"),
                       (UNS, "FLAREPP_ERR_UNSUPPORTED"), (WS, "FLAREPP_ERR_WORKSPACE"),
                       (HIP, "FLAREPP_ERR_HIP")]:
        assert fp.flarepp_status_string(code) == name
    assert fp.flarepp_status_string(99) == "FLAREPP_UNKNOWN_STATUS"
    assert fp.flarepp_version().count(".") == 2


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_workspace_sizes(dtype):
    s = fp.flarepp_workspace_size(1, 8, 1 << 20, 512, 32, dtype)
    assert s > 0 and s % 256 == 0
    # grows with N only through the chunk count (partials are latent-sized)
    assert fp.flarepp_workspace_size(1, 8, 1 << 21, 512, 32, dtype) == s
    assert fp.flare_decode_workspace_size(1, 8, 1 << 20, 512, 32, dtype) == s
    assert fp.flare_encode_workspace_size(1, 8, 1 << 20, 512, 32, dtype, 0) == s
    # a finer chunking needs more partial storage
    assert fp.flare_encode_workspace_size(1, 8, 1 << 20, 512, 32, dtype, 64) > s


@pytest.mark.parametrize("args,code", [
    ((0, 8, 1024, 64, 32, 1), 0), ((1, 0, 1024, 64, 32, 1), 0), ((1, 8, 0, 64, 32, 1), 0),
    ((1, 8, 1024, 0, 32, 1), 0), ((1, 8, 1024, 64, 0, 1), 0), ((1, 8, 1024, 64, 32, 3), 0),
    ((1, 8, 1024, 64, 48, 1), 0), ((1, 8, 1024, 513, 32, 1), 0),
    ((1 << 40, 1 << 20, 1 << 20, 64, 32, 1), 0),
])
def test_workspace_size_rejects(args, code):
    assert fp.flarepp_workspace_size(*args) == code


def test_encode_workspace_rejects_bad_chunk():
    assert fp.flare_encode_workspace_size(1, 2, 1000, 16, 8, 0, 100) == 0
    assert fp.flare_encode_workspace_size(1, 2, 1000, 16, 8, 0, -64) == 0
    assert fp.flare_encode_workspace_size(1, 2, 1000, 16, 8, 0, 128) > 0


def _mixer(B=1, H=2, N=1024, M=16, D=8, dt=1, q0="q0", qf="qf", gate="gate", k0="k0",
           k="k", v="v", y="y", ws="ws", wsb=None):
    ptr = lambda n: None if n is None else (n if isinstance(n, ctypes.c_void_p) else FAKE[n])
    if wsb is None:
        wsb = fp.flarepp_workspace_size(B, H, N, M, D, dt) or 1 << 30
    return lib().flarepp_mixer_fwd(B, H, N, M, D, dt, ptr(q0), ptr(qf), ptr(gate), ptr(k0),
                                   ptr(k), ptr(v), ptr(y), ptr(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q0=None), INV), (dict(qf=None), INV), (dict(gate=None), INV), (dict(k0=None), INV),
    (dict(k=None), INV), (dict(v=None), INV), (dict(y=None), INV),
    (dict(B=0), INV), (dict(H=-1), INV), (dict(N=0), INV), (dict(M=0), INV), (dict(D=0), INV),
    (dict(dt=7), INV), (dict(D=12), UNS), (dict(D=128), UNS), (dict(M=600), UNS),
    (dict(B=1 << 40, N=1 << 40), INV),
    (dict(ws=None), WS), (dict(wsb=1), WS),
    (dict(ws=ctypes.c_void_p(0x10000000 * 8 + 64)), WS),     # misaligned workspace
    (dict(y="k"), INV), (dict(y="v"), INV), (dict(y="k0"), INV), (dict(y="q0"), INV),
    (dict(y=ctypes.c_void_p(0x10000000 * 5 + 8)), INV),         # y overlaps k
    (dict(y="ws"), INV),                                         # y overlaps the workspace
    (dict(k="ws"), INV), (dict(q0="ws"), INV),                   # an input overlaps the workspace
    (dict(k=ctypes.c_void_p(0x10000000 * 5 + 8)), INV),          # misaligned k
    (dict(y=ctypes.c_void_p(0x10000000 * 7 + 2)), INV),          # misaligned y
    (dict(qf=ctypes.c_void_p(0x10000000 * 2 + 4)), INV),         # misaligned q_fixed
])
def test_mixer_rejects_before_any_launch(kw, code):
    assert _mixer(**kw) == code


def test_valid_call_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert _mixer() == HIP


def test_flare_rejects_bad_scale():
    L = lib()
    ws = fp.flarepp_workspace_size(1, 2, 64, 16, 8, 0)
    for scale in (0.0, -1.0, float("inf"), float("nan")):
        st = L.flare_mixer_fwd(1, 2, 64, 16, 8, 0, scale, FAKE["q0"], FAKE["k"], FAKE["v"],
                               FAKE["y"], FAKE["ws"], ws, None)
        assert st == INV


def test_encode_and_decode_seams_validate():
    L = lib()
    ws = fp.flare_encode_workspace_size(2, 2, 128, 16, 8, 1, 64)
    # q_batch_stride must be 0 or H*M*D
    assert L.flare_encode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 5, FAKE["k"], FAKE["v"],
                              FAKE["z"], 64, FAKE["ws"], ws, None) == INV
    # chunk not a multiple of 64
    assert L.flare_encode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, FAKE["k"], FAKE["v"],
                              FAKE["z"], 96, FAKE["ws"], ws, None) == INV
    # z aliasing k
    assert L.flare_encode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, FAKE["k"], FAKE["v"],
                              FAKE["k"], 64, FAKE["ws"], ws, None) == INV
    wsd = fp.flare_decode_workspace_size(2, 2, 128, 16, 8, 1)
    assert L.flare_decode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, FAKE["z"], FAKE["k"],
                              FAKE["k"], FAKE["ws"], wsd, None) == INV
    assert L.flare_decode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, None, FAKE["k"],
                              FAKE["y"], FAKE["ws"], wsd, None) == INV
    # inputs overlapping the workspace (which the kernels write) and misaligned pointers
    assert L.flare_encode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, FAKE["ws"], FAKE["v"],
                              FAKE["z"], 64, FAKE["ws"], ws, None) == INV
    assert L.flare_encode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, FAKE["k"], FAKE["v"],
                              ctypes.c_void_p(FAKE["z"].value + 4), 64, FAKE["ws"], ws, None) == INV
    assert L.flare_decode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["ws"], 0, FAKE["z"], FAKE["k"],
                              FAKE["y"], FAKE["ws"], wsd, None) == INV
    assert L.flare_decode_fwd(2, 2, 128, 16, 8, 1, 0.5, FAKE["q0"], 0, FAKE["z"],
                              ctypes.c_void_p(FAKE["k"].value + 8), FAKE["y"], FAKE["ws"], wsd,
                              None) == INV
    ws_flare = fp.flarepp_workspace_size(1, 2, 64, 16, 8, 1)
    assert L.flare_mixer_fwd(1, 2, 64, 16, 8, 1, 0.5, FAKE["q0"], FAKE["ws"], FAKE["v"],
                             FAKE["y"], FAKE["ws"], ws_flare, None) == INV
    assert L.flare_mixer_fwd(1, 2, 64, 16, 8, 1, 0.5, FAKE["q0"], FAKE["k"],
                             ctypes.c_void_p(FAKE["v"].value + 2), FAKE["y"], FAKE["ws"],
                             ws_flare, None) == INV


def _simplified(B=1, H=2, N=1024, M=16, D=8, dt=1, q0="q0", k0="k0", v0="v0", k="k", v="v",
                y="y", ws="ws", wsb=None):
    ptr = lambda n: None if n is None else FAKE[n]
    if wsb is None:
        wsb = fp.flarepp_workspace_size(B, H, N, M, D, dt) or 1 << 30
    return lib().simplified_flarepp_mixer_fwd(B, H, N, M, D, dt, ptr(q0), ptr(k0), ptr(v0),
                                              ptr(k), ptr(v), ptr(y), ptr(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q0=None), INV), (dict(k0=None), INV), (dict(v0=None), INV), (dict(k=None), INV),
    (dict(v=None), INV), (dict(y=None), INV), (dict(M=0), INV), (dict(D=12), UNS),
    (dict(ws=None), WS), (dict(wsb=1), WS), (dict(y="v0"), INV), (dict(y="k0"), INV),
])
def test_simplified_rejects_before_any_launch(kw, code):
    assert _simplified(**kw) == code


def test_flarepp_still_requires_fixed_queries_and_gate():
    # null q_fixed or gate is an error for FLARE++ (not a silent switch to
    # the simplified mixer)
    assert _mixer(qf=None) == INV and _mixer(gate=None) == INV


def test_simplified_valid_call_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert _simplified() == HIP


# ---------------------------------------------------------------- backward
GRADS = {name: ctypes.c_void_p(0x10000000 * (i + 20)) for i, name in
         enumerate(["dq0", "dqf", "dgate", "dk0", "dk", "dv", "saved", "dy", "bws"])}


def test_saved_size_formula():
    B, H, N, M, D = 2, 3, 1000, 40, 32
    assert lib().flarepp_saved_size(B, H, N, M, D) == 4 * (3 * B * H * M * D + 2 * B * H * M + B * H * N)
    assert lib().flarepp_saved_size(0, 1, 1, 1, 16) == 0


@pytest.mark.parametrize("args,ok", [
    ((1, 8, 1 << 20, 512, 32, 1), True),
    ((2, 2, 700, 80, 16, 2), True),
    ((1, 1, 100, 416, 64, 1), True),
    ((1, 1, 100, 512, 64, 2), True),     # token pass over two latent ranges
    ((1, 1, 100, 513, 64, 1), False),    # M above the library's maximum
    ((1, 1, 100, 64, 8, 1), True),       # D = 8: the VALU backward
    ((1, 1, 100, 64, 32, 0), True),      # fp32: the VALU backward
    ((1, 1, 100, 64, 12, 0), False),     # D outside {8, 16, 32, 64}
    ((1, 1, 0, 64, 32, 1), False),
])
def test_bwd_workspace_size(args, ok):
    assert (fp.load_library().flarepp_bwd_workspace_size(*args) > 0) == ok


def _bwd(B=1, H=2, N=1024, M=16, D=32, dt=1, saved_bytes=None, wsb=None, **kw):
    names = dict(q0="q0", qf="qf", gate="gate", k0="k0", k="k", v="v", y="y", dy="dy",
                 saved="saved", dq0="dq0", dqf="dqf", dgate="dgate", dk0="dk0", dk="dk",
                 dv="dv", ws="bws")
    names.update(kw)
    ptr = lambda n: None if n is None else (n if isinstance(n, ctypes.c_void_p)
                                            else FAKE.get(n) or GRADS[n])
    if saved_bytes is None:
        saved_bytes = lib().flarepp_saved_size(B, H, N, M, D)
    if wsb is None:
        wsb = fp.load_library().flarepp_bwd_workspace_size(B, H, N, M, D, dt) or 1 << 30
    n = names
    return lib().flarepp_mixer_bwd(B, H, N, M, D, dt, ptr(n["q0"]), ptr(n["qf"]), ptr(n["gate"]),
                                   ptr(n["k0"]), ptr(n["k"]), ptr(n["v"]), ptr(n["y"]),
                                   ptr(n["dy"]), ptr(n["saved"]), saved_bytes, ptr(n["dq0"]),
                                   ptr(n["dqf"]), ptr(n["dgate"]), ptr(n["dk0"]), ptr(n["dk"]),
                                   ptr(n["dv"]), ptr(n["ws"]), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q0=None), INV), (dict(gate=None), INV), (dict(k0=None), INV), (dict(k=None), INV),
    (dict(y=None), INV), (dict(dy=None), INV), (dict(saved=None), INV), (dict(dq0=None), INV),
    (dict(dqf=None), INV), (dict(dgate=None), INV), (dict(dk0=None), INV), (dict(dk=None), INV),
    (dict(dv=None), INV), (dict(D=12), UNS), (dict(dt=5), INV), (dict(M=513), UNS),
    (dict(saved_bytes=64), WS), (dict(ws=None), WS), (dict(wsb=1), WS),
    (dict(dk="k"), INV), (dict(dv="dy"), INV), (dict(dk0="saved"), INV),
    (dict(dy=ctypes.c_void_p(0x10000000 * 27 + 8)), INV),       # misaligned dy
    (dict(dk=ctypes.c_void_p(0x10000000 * 24 + 4)), INV),       # misaligned dk
    (dict(dk="bws"), INV),                                        # gradient over the workspace
    (dict(k="bws"), INV), (dict(saved="bws"), INV),               # input over the workspace
    (dict(dq0="dk"), INV), (dict(dgate="dq0"), INV), (dict(dv="dk0"), INV),  # gradients alias
    (dict(dqf="q0"), INV),                                        # latent gradient over an input
])
def test_bwd_rejects_before_any_launch(kw, code):
    assert _bwd(**kw) == code


def test_bwd_valid_call_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert _bwd() == HIP


def test_fwd_train_rejects_small_saved_buffer():
    B, H, N, M, D, dt = 1, 2, 1024, 16, 32, 1
    L = lib()
    ws = fp.flarepp_workspace_size(B, H, N, M, D, dt)
    args = [FAKE[n] for n in ("q0", "qf", "gate", "k0", "k", "v", "y")]
    assert L.flarepp_mixer_fwd_train(B, H, N, M, D, dt, *args, GRADS["saved"], 64, FAKE["ws"],
                                     ws, None) == WS
    assert L.flare_mixer_fwd_train(B, H, N, M, D, dt, 0.5, FAKE["q0"], FAKE["k"], FAKE["v"],
                                   FAKE["y"], GRADS["saved"], 64, FAKE["ws"], ws, None) == WS


def test_simplified_bwd_validates():
    B, H, N, M, D, dt = 1, 2, 1024, 16, 32, 1
    L = lib()
    sb = L.flarepp_saved_size(B, H, N, M, D)
    wsb = L.flarepp_bwd_workspace_size(B, H, N, M, D, dt)
    P = lambda n: FAKE.get(n) or GRADS[n]

    def call(v0="v0", dv0="dv", dk0="dk0", dk="dq0"):
        return L.simplified_flarepp_mixer_bwd(
            B, H, N, M, D, dt, P("q0"), P("k0"), None if v0 is None else P(v0), P("k"), P("v"),
            P("y"), P("dy"), P("saved"), sb, P("dqf"), P(dk0),
            None if dv0 is None else P(dv0), P(dk), P("dgate"), P("bws"), wsb, None)
    assert call(v0="k0") == INV          # v0 == k0 belongs to flarepp_mixer_bwd
    assert call(v0=None) == INV
    assert call(dv0=None) == INV
    assert call(dv0="v0") == INV         # gradient overlaps an input
    import torch
    if not torch.cuda.is_available():
        assert call() == HIP


# ---------------------------------------------------------------- front end
FE = {name: ctypes.c_void_p(0x10000000 * (i + 40)) for i, name in
      enumerate(["x", "w0", "w1", "w2", "b0", "b1", "b2", "g", "o0", "o1", "o2"])}


def _fe(B=1, N=100, C=64, H=2, D=32, dt=1, eps=1e-6, norm=1, **kw):
    n = dict(x="x", w0="w0", w1="w1", w2="w2", b0="b0", b1="b1", b2="b2", g="g", o0="o0",
             o1="o1", o2="o2")
    n.update(kw)
    P = lambda k: None if n[k] is None else (n[k] if isinstance(n[k], ctypes.c_void_p) else FE[n[k]])
    return lib().flarepp_frontend_fwd(B, N, C, H, D, dt, P("x"), P("w0"), P("w1"), P("w2"),
                                      P("b0"), P("b1"), P("b2"), P("g"), eps, norm, P("o0"),
                                      P("o1"), P("o2"), None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INV), (dict(w1=None), INV), (dict(o2=None), INV), (dict(dt=0), UNS),
    (dict(dt=5), INV), (dict(D=8), UNS), (dict(C=24), UNS), (dict(N=0), INV),
    (dict(eps=0.0), INV), (dict(eps=float("nan")), INV), (dict(o1="o0"), INV),
    (dict(o0="x"), INV), (dict(o2="w1"), INV),
    (dict(x=ctypes.c_void_p(0x10000000 * 40 + 8)), INV),     # misaligned x
])
def test_frontend_rejects_before_any_launch(kw, code):
    assert _fe(**kw) == code


def test_frontend_optional_arguments_and_device():
    import torch
    # biases, gain and eps are optional without normalisation
    st = _fe(b0=None, b1=None, b2=None, g=None, eps=0.0, norm=0)
    assert st == (HIP if not torch.cuda.is_available() else st)
    L = lib()
    assert L.flarepp_seed_norm_fwd(2, 10, 65, 1, FE["x"], None, 1e-6, FE["o0"], None) == UNS
    assert L.flarepp_seed_norm_fwd(2, 10, 32, 1, FE["x"], None, 0.0, FE["o0"], None) == INV
    assert L.flarepp_seed_norm_fwd(2, 10, 32, 0, FE["x"], None, 1e-6, FE["o0"], None) == UNS
    if not torch.cuda.is_available():
        assert L.flarepp_seed_norm_fwd(2, 10, 32, 1, FE["x"], None, 1e-6, FE["x"], None) == HIP


def test_probe_library_exports_its_header():
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "include", "flarepp_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(flarepp_probe\w*)\s*\(", text)))
    assert names == ["flarepp_probe_launch", "flarepp_probe_work"]
    path = os.path.join(os.path.dirname(fp.library_path()), "libflarepp_probe.so")
    if not os.path.exists(path):
        pytest.skip("libflarepp_probe.so not built")
    P = ctypes.CDLL(path)
    for n in names:
        assert hasattr(P, n), n
    P.flarepp_probe_work.restype = ctypes.c_double
    P.flarepp_probe_work.argtypes = [ctypes.c_int] * 3
    # 1 workgroup of 4 waves, 1 iteration: 4 x 8 products of 2*32*32*16 flops
    assert P.flarepp_probe_work(0, 1, 1) == 4 * 8 * 2 * 32 * 32 * 16
    assert P.flarepp_probe_work(1, 2, 3) == 2 * 256 * 3 * 8
    P.flarepp_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    assert P.flarepp_probe_launch(0, 0, 1, None, None) == 1   # rejected before any launch
    assert P.flarepp_probe_launch(7, 1, 1, ctypes.c_void_p(0x1000), None) == 1


def test_noalloc_validates_before_any_device_call():
    """The allocation-free forward: shape errors and shapes whose workspace
    exceeds the library's array are rejected before any HIP call."""
    L = lib()
    P = lambda n: FAKE[n]
    args = [P(n) for n in ("q0", "qf", "gate", "k0", "k", "v", "y")]
    import torch
    if not torch.cuda.is_available():
        assert L.flarepp_mixer_fwd_noalloc(1, 2, 1024, 16, 8, 1, *args, None) == HIP
    assert L.flarepp_mixer_fwd_noalloc(1, 2, 0, 16, 8, 1, *args, None) == INV
    assert L.flarepp_mixer_fwd_noalloc(1, 2, 1024, 16, 12, 1, *args, None) == UNS
    big = (32, 16, 1 << 20, 512, 64)
    assert L.flarepp_workspace_size(*big, 1) > fp.FLAREPP_NOALLOC_SCRATCH_BYTES
    far = [ctypes.c_void_p((i + 1) << 40) for i in range(7)]   # 69 GB tensors, disjoint
    assert L.flarepp_mixer_fwd_noalloc(*big, 1, *far, None) == WS
    a = list(args)
    a[1] = None                                     # q_fixed
    assert L.flarepp_mixer_fwd_noalloc(1, 2, 1024, 16, 8, 1, *a, None) == INV
    a = list(args)
    a[6] = FAKE["k"]                                # y over k
    assert L.flarepp_mixer_fwd_noalloc(1, 2, 1024, 16, 8, 1, *a, None) == INV
    a = list(args)
    a[4] = ctypes.c_void_p(FAKE["k"].value + 8)     # misaligned k
    assert L.flarepp_mixer_fwd_noalloc(1, 2, 1024, 16, 8, 1, *a, None) == INV


def test_bwd_fp32_and_d8_are_supported():
    """fp32 (every D) and D = 8 (every dtype) run on the VALU backward: a
    workspace size is reported and a valid call only fails for want of a
    device."""
    L = fp.load_library()
    for dt in (0, 1, 2):
        for D in (8, 16, 32, 64):
            assert L.flarepp_bwd_workspace_size(2, 3, 1000, 40, D, dt) > 0, (dt, D)
    import torch
    if not torch.cuda.is_available():
        assert _bwd(dt=0) == HIP
        assert _bwd(D=8) == HIP
