"""The library's calls under HIP graph capture: a forward, a training
forward and a backward are captured once (on torch's capture stream, with
preallocated outputs and workspaces) and replayed several times, with
eager work and synchronisations between the replays; every replay must
equal the eager result bit for bit.  Nothing in these paths allocates,
synchronises or records a memset node."""

from __future__ import annotations

import numpy as np
import pytest

from flarepp_workloads import make_cotangent, make_random_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_attention_mixer_amd as m
    m.load_library()
    return m


def _inputs(B=2, H=3, N=3000, M=96, D=32):
    x = make_random_inputs(B, H, N, M, D, "bf16", seed=77, gate=[0.4, -np.inf, 1.1])
    t = {n: torch.from_numpy(x[n]).cuda() for n in ("q0", "q_fixed", "gate", "k0", "k", "v")}
    for n in ("q0", "q_fixed", "k0", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    return [t[n] for n in ("q0", "q_fixed", "gate", "k0", "k", "v")]


def test_forward_graph_replays_equal_eager(fp):
    args = _inputs()
    B, H, N, D = args[4].shape
    M = args[0].shape[1]
    code = fp.dtype_code(args[4])
    ws = torch.empty(fp.flarepp_workspace_size(B, H, N, M, D, code), dtype=torch.uint8, device="cuda")
    y_eager = fp.flarepp_mixer_fwd(*args, workspace=ws).clone()
    y = torch.empty_like(y_eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up on the capture stream
        fp.flarepp_mixer_fwd(*args, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp.flarepp_mixer_fwd(*args, y=y, workspace=ws)
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), i
        fp.flarepp_mixer_fwd(*args, workspace=torch.empty_like(ws))  # eager work between
        torch.cuda.synchronize()


def test_backward_graph_replays_equal_eager(fp):
    args = _inputs(N=1500, M=64)
    B, H, N, D = args[4].shape
    M = args[0].shape[1]
    dy = torch.from_numpy(make_cotangent(B, H, N, D, "bf16", seed=78)).cuda().to(torch.bfloat16)
    code = fp.dtype_code(args[4])
    lib = fp.load_library()
    ws = torch.empty(fp.flarepp_workspace_size(B, H, N, M, D, code), dtype=torch.uint8, device="cuda")
    bws = torch.empty(lib.flarepp_bwd_workspace_size(B, H, N, M, D, code), dtype=torch.uint8,
                      device="cuda")
    y, saved = fp.flarepp_mixer_fwd_train(*args, workspace=ws)
    g_eager = {n: t.clone() for n, t in fp.flarepp_mixer_bwd(*args, y, dy, saved, workspace=bws).items()}
    y2 = torch.empty_like(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _, saved2 = fp.flarepp_mixer_fwd_train(*args, y=y2, workspace=ws)
        out = fp.flarepp_mixer_bwd(*args, y2, dy, saved2, workspace=bws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        # the backward writes into gradient tensors allocated at capture
        _cap = fp.flarepp_mixer_bwd(*args, y2, dy, saved2, workspace=bws)
    for i in range(3):
        for t in _cap.values():
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for n in g_eager:
            assert torch.equal(_cap[n], g_eager[n]), (i, n)
        fp.flarepp_mixer_fwd(*args, workspace=torch.empty_like(ws))
        torch.cuda.synchronize()
