"""Host logic of bench.py that needs no GPU: the one-GPU guard, the source
digest that ties the committed HBM-traffic counters to the kernel sources,
the parsing of that counter summary, and the algorithmic work per launch."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from flarepp_workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_digest_is_stable_and_skips_non_forward_files(tmp_path, monkeypatch):
    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert bench.source_digest() == d
    # a copy of the forward sources gives the same digest; backward, front-end
    # files and sub-directories do not enter it
    csrc = os.path.join(ROOT, "rank_latent_attention_mixer_amd", "csrc")
    fake_root = tmp_path / "r"
    fake = fake_root / "rank_latent_attention_mixer_amd" / "csrc"
    fake.mkdir(parents=True)
    for f in os.listdir(csrc):
        p = os.path.join(csrc, f)
        if os.path.isfile(p) and not f.startswith(("backward", "frontend")):
            (fake / f).write_bytes(open(p, "rb").read())
    (fake / "backward_extra.hip").write_text("// not part of the forward")
    (fake / "probe").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    assert bench.source_digest() == d
    (fake / "decode.hip").write_bytes(b"changed")
    assert bench.source_digest() != d


def test_read_traffic(tmp_path):
    path = tmp_path / "t.txt"
    path.write_text("# comment\nsource_digest %s\nworkload million_token_bf16\n"
                    "hbm_bytes_per_launch.decode 1078149679\n" % bench.source_digest())
    assert bench.read_traffic(str(path), "million_token_bf16", "decode") == 1078149679
    assert bench.read_traffic(str(path), "million_token_bf16", "encode") is None
    assert bench.read_traffic(str(path), "point_cloud_bf16", "decode") is None
    path.write_text("source_digest 0000000000000000\nworkload million_token_bf16\n"
                    "hbm_bytes_per_launch.decode 5\n")
    assert bench.read_traffic(str(path), "million_token_bf16", "decode") is None
    assert bench.read_traffic(str(tmp_path / "missing.txt"), "million_token_bf16", "decode") is None


def test_algorithmic_work_at_the_million_token_workload():
    w = WORKLOADS["million_token_bf16"]
    work = bench.algorithmic_work(w, [True] * w.H)
    per_launch_flops = 4 * w.B * w.N * w.M * w.D * w.H
    assert work["decode"][0] == work["encode"][0] == work["encode_synthesis"][0] == per_launch_flops
    assert work["decode"][1] == 2 * w.B * w.N * w.D * 2 * w.H       # k in, y out
    assert work["encode_synthesis"][1] == w.B * w.N * w.D * 2 * w.H  # k0 once
    closed = bench.algorithmic_work(w, [False] * w.H)
    assert closed["encode_synthesis"] == (0, 0)


@pytest.mark.parametrize("args", [["--backward"], ["--frontend"], ["--probe"]])
def test_modes_need_a_device(args):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and r.stdout == ""


def test_frontend_traffic_follows_the_front_end_sources(tmp_path):
    """The committed front-end counter summary is read while the front end's
    sources are the ones it was taken on, and a summary carrying another
    digest (sources changed since) reads as None."""
    committed = os.path.join(ROOT, "profiles", "hbm_traffic_frontend_million_token_bf16.txt")
    d = bench.frontend_digest()
    assert d != bench.source_digest()
    got = bench.read_traffic(committed, "million_token_bf16", "frontend_wres", d)
    if f"source_digest {d}\n" in open(committed).read():
        assert got is not None and got > 2147876864  # at least the algorithmic bytes
    else:  # sources edited since the counters were taken
        assert got is None
    stale = tmp_path / "t.txt"
    stale.write_text(open(committed).read().replace(f"source_digest {d}", "source_digest 0000000000000000"))
    assert bench.read_traffic(str(stale), "million_token_bf16", "frontend_wres", d) is None


def test_bench_line_carries_the_pages_context_claim():
    """The result line quotes the pages' scale claim as context, with the
    hardware the pages name for it (none) and no target attached."""
    import bench
    src = open(bench.__file__).read()
    assert '"context": PAGES_CONTEXT' in src
    c = bench.PAGES_CONTEXT
    assert "1e6 tokens on a single GPU" in c["claim"] and "FLARE" in c["claim"]
    assert c["hardware"] == "not named by the pages"
    assert c["role"] == "context, not a target"
    assert "#1150" in c["source"] and "FLARE.py README" in c["source"]
