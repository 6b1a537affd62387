#!/usr/bin/env python3
"""FLARE++ mixer forward throughput on one MI355X.

A step is one flarepp_mixer_fwd call (synthesis, gated query, encode,
decode) over one batch of the million-token workload (B=1, H=8, N=1,048,576,
M=512, D=32, bf16, seeded synthetic inputs already resident in HBM).  The
timed region is exactly K plain calls; the per-kernel split comes from K
further calls with HIP events between the launches.
Prints one JSON line on stdout; progress goes to stderr.
Without --warmup the warm-up runs for at least WARMUP_SECONDS (and at
least 5 steps), so that the GPU has reached the clock it sustains under the
work before the timed region: a few milliseconds of warm-up measure a
still-ramping clock, up to 20% slower at the smaller workloads.  The JSON
line reports the number of warm-up steps run.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--cpu-seconds S | --no-cpu-baseline]
  python bench.py --copy-calibration-mib S   (plain device copy of S MiB, for
                                              scaling the HBM byte counters;
                                              then 20 more copies timed)
  python bench.py --backward [--steps K] [--warmup W] [--workload NAME]
                  (times flarepp_mixer_bwd alone: one training forward fills
                   the saved tensors, then K backward calls are timed)
  python bench.py --frontend [--steps K] [--warmup W] [--workload NAME]
                  (times flarepp_frontend_fwd, the three projections of the
                   block input x [B, N, H*D] with k0 normalised head-wise)
  python bench.py --probe   (measured dense bf16 MFMA and v_exp_f32 rates of
                             this device, beside the published peak)
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FLARE++ mixer fwd tokens/s & TFLOP/s (%bf16 MFMA peak), 1 GPU, N=1M M=512"

# The pages' own statement of scale, restated (context, not a target).
# FLARE.py README, section "FLARE" ("Scale" bullet): two-step FLARE trains end
# to end on meshes of about one million points on one GPU; physicsnemo issue
# #1150, opening description (one million tokens on a single GPU) and reply
# item 3 (that study used mixed precision, fp16 forward and fp32 backward).
# No GPU model is named for this claim on the pages.
PAGES_CONTEXT = {
    "claim": "FLARE (two-step, not FLARE++) trained end to end at about 1e6 tokens on a single GPU",
    "hardware": "not named by the pages",
    "precision": "mixed: fp16 forward, fp32 backward",
    "throughput": "none printed by the pages",
    "source": ('FLARE.py README, section "FLARE" (Scale bullet); physicsnemo issue #1150, '
               "opening description and reply item 3"),
    "role": "context, not a target",
}
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
# fp32 vector, published: 256 CUs x 4 SIMDs x 16 lanes x 2 flops per FMA x 2
# (packed two-wide FMA) x 2.4 GHz; kernels built without packed fp32
# instructions issue at most half of it
PEAK_FP32_VECTOR_TFLOPS = 157.3
# kernel i of a forward runs between timing events i + 1 and i + 2 (events 0
# and 1 are recorded back to back: the seeds need no launch of their own)
KERNELS = ["encode_synthesis", "combine_query", "encode", "combine_value", "decode"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_million_token_bf16.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e: int):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def source_digest() -> str:
    """Digest of the mixer forward's sources (kernels, shared headers, the
    forward launch plan); the backward's and the front end's own files are
    left out."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_latent_attention_mixer_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith(("backward", "frontend")) or not os.path.isfile(os.path.join(csrc, f)):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


FRONTEND_SOURCES = ("frontend.hip", "frontend.hpp", "frontend_abi.cpp", "flarepp_device.hpp",
                    "kernels.hpp", "abi_common.hpp")


def frontend_digest() -> str:
    """Digest of the front end's kernel sources and the headers they include."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_latent_attention_mixer_amd", "csrc")
    for f in FRONTEND_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(path, workload, kernel, digest=None):
    """HBM bytes per launch of `kernel` from a counter summary made of lines
    'key value...'; None unless it was taken on the current kernel sources
    (`digest`, by default the forward's)."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) >= 2 and not line.startswith("#"):
                kv[f[0]] = f[1:]
    if kv.get("source_digest", [None])[0] != (digest or source_digest()):
        return None
    if kv.get("workload", [None])[0] != workload:
        return None
    v = kv.get(f"hbm_bytes_per_launch.{kernel}")
    return int(float(v[0])) if v else None


def copy_calibration(mib):
    """Issues 5 plain device-to-device copies of `mib` MiB so that a counter
    run can relate FETCH_SIZE / WRITE_SIZE to known bytes (every copy of the
    run moves the same bytes), then times 20 more."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.rand(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    # then the same copy timed on its own (after a time-based warm-up), as
    # the HBM rate a plain read-and-write stream reaches on this device
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARMUP_SECONDS:
        dst.copy_(src)
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(20):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / 20
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "copies": 5,
                      "timed_copy_ms": round(ms, 4),
                      "timed_copy_GBs": round(2 * n * 4 / (ms / 1e3) / 1e9, 1)}), flush=True)
    return 0


def algorithmic_work(w, sig_open):
    """Per-launch algorithmic flops and HBM bytes of the three attention
    kernels (exp and normalisation not counted; partials not counted)."""
    e = 2 if w.dtype in ("bf16", "fp16") else 4
    tok = w.B * w.N
    per_head_flops = 4 * tok * w.M * w.D          # QK^T and PV, 2 flops per MAC
    per_head_bytes = tok * w.D * e                # one pass over one [N, D] tensor
    hopen = int(sum(sig_open))
    return {
        "encode_synthesis": (per_head_flops * hopen, per_head_bytes * hopen),       # k0 once
        "encode": (per_head_flops * w.H, 2 * per_head_bytes * w.H),                # k, v
        "decode": (per_head_flops * w.H, 2 * per_head_bytes * w.H),                # k in, y out
    }


WARMUP_SECONDS = 0.5


def warm_up(a, torch, step):
    """Untimed warm-up: exactly a.warmup steps if given, else at least 5
    steps and WARMUP_SECONDS of them (a.warmup is then set to the count)."""
    if a.warmup is not None:
        for _ in range(a.warmup):
            step()
        torch.cuda.synchronize()
        return
    n, t0 = 0, time.perf_counter()
    while n < 5 or time.perf_counter() - t0 < WARMUP_SECONDS:
        for _ in range(5):
            step()
        n += 5
        torch.cuda.synchronize()
    a.warmup = n


def cpu_baseline(x, w, seconds):
    """The fp64 oracle, timed on whole heads of the same workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()
                if i.get("user_api") == "blas"]
    except Exception:  # noqa: BLE001
        blas = []
    threads = max([n for _, n in blas] + [1])
    heads = 0
    t_total = 0.0
    for b in range(w.B):
        for h in range(w.H):
            sl = dict(q0=x["q0"][h:h + 1], q_fixed=x["q_fixed"][h:h + 1],
                      gate=x["gate"][h:h + 1], k0=x["k0"][b:b + 1, h:h + 1],
                      k=x["k"][b:b + 1, h:h + 1], v=x["v"][b:b + 1, h:h + 1])
            sl = {n: np.asarray(a, dtype=np.float64) for n, a in sl.items()}
            t0 = time.perf_counter()
            oracle.flarepp_ref(**sl)
            t_total += time.perf_counter() - t0
            heads += 1
            log(f"[cpu] oracle head (b={b}, h={h}) done, {t_total:.1f}s so far")
            if t_total >= seconds:
                break
        if t_total >= seconds:
            break
    t_head = t_total / heads
    tokens_per_s = (w.B * w.N) / (t_head * w.B * w.H)
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads (full N={w.N}) of {w.name}, fp64 NumPy, "
                      f"{t_total:.1f}s; rate scaled to all heads",
            "blas": blas}


def bench_backward(a, fp, torch, np, w, x, args, y, ws):
    """Times K flarepp_mixer_bwd calls on the saved tensors of one training
    forward; prints one JSON line."""
    from flarepp_workloads import make_cotangent
    dev = y.device
    tdt = y.dtype
    dy = torch.from_numpy(make_cotangent(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed + 100))
    dy = dy.to(dev).to(tdt)
    y, saved = fp.flarepp_mixer_fwd_train(*args, y=y, workspace=ws)
    code = fp.dtype_code(y)
    nbytes = fp.load_library().flarepp_bwd_workspace_size(w.B, w.H, w.N, w.M, w.D, code)
    bws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] backward: saved {saved.numel() * 4 / 2**20:.1f} MiB, "
        f"workspace {nbytes / 2**20:.1f} MiB")
    warm_up(a, torch, lambda: fp.flarepp_mixer_bwd(*args, y, dy, saved, workspace=bws))
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(a.steps):
        g = fp.flarepp_mixer_bwd(*args, y, dy, saved, workspace=bws)
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / a.steps
    for n, t in g.items():
        if not bool(torch.isfinite(t).all()):
            log(f"[bench] non-finite gradient {n}")
            return 1
    sig = 1.0 / (1.0 + np.exp(-x["gate"].astype(np.float64)))
    # five products per attention backward (S, dP, dV, dQ, dK), 2 flops per
    # multiply-add; the synthesis only where the gate is open
    attn = sum((3 if s > 0 else 2) for s in sig)
    flops = 5 * 2 * attn * w.B * w.N * w.M * w.D
    t = ms_per_step / 1e3
    result = {
        "metric": "FLARE++ mixer bwd tokens/s & TFLOP/s (%bf16 MFMA peak), 1 GPU",
        "value": round(w.B * w.N / t, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D,
                   "dtype": w.dtype, "global_batch": w.B, "seq_len": w.N,
                   "parallelism": "single-gpu", "pass": "backward"},
        "tflops": round(flops / t / 1e12, 2),
        "frac_bf16_peak": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
        # the whole backward pass against the matrix-core peak (its kernels
        # are listed with their times in the backward kernel-time profile)
        "roofline": {"bound": "mfma", "achieved": round(flops / t / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "whole backward", "algorithmic_flops_per_call": int(flops)},
        "source_digest": source_digest(),
    }
    print(json.dumps(result), flush=True)
    return 0


def probe_peaks():
    """Measured matrix-core and exponential rates (libflarepp_probe.so):
    1024 workgroups of 4 waves (four per SIMD), long independent chains."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "rank_latent_attention_mixer_amd", "libflarepp_probe.so"))
    lib.flarepp_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.flarepp_probe_work.restype = ctypes.c_double
    lib.flarepp_probe_work.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    blocks, iters = 1024, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for which, name in ((0, "mfma_bf16"), (1, "exp_f32")):
        for _ in range(2):
            if lib.flarepp_probe_launch(which, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream):
                raise RuntimeError("probe launch failed")
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(10):
            lib.flarepp_probe_launch(which, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)
        stop.record()
        torch.cuda.synchronize()
        t = start.elapsed_time(stop) / 10 / 1e3
        res[name] = lib.flarepp_probe_work(which, blocks, iters) / t
        log(f"[probe] {name}: {t * 1e3:.3f} ms per launch")
    # sustained (about a second each): the same products on random-bit and
    # on all-ones operands; the ratio is the clock the power limit takes away
    # when operand bits toggle
    for which, name in ((2, "mfma_bf16_random_sustained"), (3, "mfma_bf16_ones_sustained")):
        launches, t_total = 0, 0.0
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        while t_total < 1.0:
            start.record()
            for _ in range(20):
                lib.flarepp_probe_launch(which, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)
            stop.record()
            torch.cuda.synchronize()
            t_total += start.elapsed_time(stop) / 1e3
            launches += 20
        # the rate of the last 20 launches, after the clock has settled
        t = start.elapsed_time(stop) / 20 / 1e3
        res[name] = lib.flarepp_probe_work(which, blocks, iters) / t
        log(f"[probe] {name}: {t * 1e3:.3f} ms per launch after {t_total:.2f} s")
    # co-issue on one SIMD (four waves per SIMD): time per wave-iteration of
    # 4 products alone, 32 three-source FMAs alone, and both interleaved
    co = {}
    for which, name in ((4, "mfma"), (5, "fma"), (6, "mix")):
        for _ in range(2):
            lib.flarepp_probe_launch(which, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(10):
            lib.flarepp_probe_launch(which, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)
        stop.record()
        torch.cuda.synchronize()
        t = start.elapsed_time(stop) / 10 / 1e3
        # ns per wave-iteration on one SIMD (1024 SIMDs share the launch)
        co[name] = t * 1e9 * 1024 / lib.flarepp_probe_work(which, blocks, iters)
        log(f"[probe] co-issue {name}: {co[name]:.2f} ns per wave-iteration per SIMD")
    hidden = (co["mfma"] + co["fma"] - co["mix"]) / co["fma"]
    from flarepp_workloads import WORKLOADS
    w = WORKLOADS["million_token_bf16"]
    exps = 3 * w.B * w.H * w.N * w.M  # one forward, every gate open
    print(json.dumps({
        "probe": "dense bf16 v_mfma_f32_32x32x16 and v_exp_f32 throughput, 1 GPU",
        "mfma_bf16_tflops_measured": round(res["mfma_bf16"] / 1e12, 1),
        "mfma_bf16_tflops_published": PEAK_BF16_TFLOPS,
        "exp_f32_per_s_measured": float(f"{res['exp_f32']:.4g}"),
        "exp_ms_per_million_token_forward": float(f"{exps / res['exp_f32'] * 1e3:.4g}"),
        "mfma_bf16_tflops_sustained_random_operands": round(res["mfma_bf16_random_sustained"] / 1e12, 1),
        "mfma_bf16_tflops_sustained_ones_operands": round(res["mfma_bf16_ones_sustained"] / 1e12, 1),
        "coissue_ns_per_wave_iteration": {k: round(v, 2) for k, v in co.items()},
        "coissue_fma_share_hidden_by_mfma": round(hidden, 3),
    }), flush=True)
    return 0


def bench_frontend(a, fp, torch, w):
    """Times K flarepp_frontend_fwd calls at the workload's block width
    (C = H D); prints one JSON line with the HBM roofline."""
    from flarepp_workloads import make_frontend_inputs
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
    C = w.H * w.D
    log(f"[bench] front end: B={w.B} N={w.N} C={C} H={w.H} D={w.D} {w.dtype}")
    x = make_frontend_inputs(w.B, w.N, C, w.H, w.D, w.dtype, seed=w.seed + 200)
    d = {n: torch.from_numpy(x[n]).to(dev).to(tdt) for n in
         ("x", "w_k0", "w_k", "w_v", "b_k0", "b_k", "b_v", "g_k0")}
    out = tuple(torch.empty((w.B, w.H, w.N, w.D), dtype=tdt, device=dev) for _ in range(3))
    call = lambda: fp.flarepp_frontend_fwd(d["x"], d["w_k0"], d["w_k"], d["w_v"], w.H,
                                           b_k0=d["b_k0"], b_k=d["b_k"], b_v=d["b_v"],
                                           g_k0=d["g_k0"], eps=1e-6, out=out)
    warm_up(a, torch, call)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(a.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / a.steps
    T = w.B * w.N
    e = 2
    nbytes = T * C * e + 3 * w.H * w.D * C * e + 3 * T * w.H * w.D * e
    flops = 2 * T * C * 3 * w.H * w.D
    t = ms / 1e3
    result = {
        "metric": "FLARE++ block front end (3 projections + head-wise norm) tokens/s, 1 GPU",
        "value": round(T / t, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "C": C, "H": w.H, "D": w.D,
                   "dtype": w.dtype, "pass": "frontend"},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(os.path.join(ROOT, "profiles",
                                                          f"hbm_traffic_frontend_{w.name}.txt"),
                                             w.name, "frontend_wres", frontend_digest()),
                     "kernel": "frontend_wres", "algorithmic_bytes_per_launch": nbytes},
        "source_digest": frontend_digest(),
        "tflops": round(flops / t / 1e12, 2),
    }
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="warm-up steps (default: as many as fill WARMUP_SECONDS)")
    ap.add_argument("--workload", default="million_token_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--frontend", action="store_true")
    ap.add_argument("--probe", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="launch each timed forward as one replay of a captured HIP graph")
    a = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}, WORLD_SIZE {world}); "
              "the mixer is built and measured on a single MI355X", file=sys.stderr)
        return 2

    if a.copy_calibration_mib > 0:
        return copy_calibration(a.copy_calibration_mib)
    if a.probe:
        return probe_peaks()

    import numpy as np
    import torch

    import rank_latent_attention_mixer_amd as fp
    from flarepp_workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        log("no GPU available")
        return 1
    fp.load_library()
    w = WORKLOADS[a.workload]
    if a.frontend:
        return bench_frontend(a, fp, torch, w)
    dev = torch.device("cuda:0")
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
    log(f"[bench] generating {w.name} {w.shape_dict} {w.dtype}")
    t0 = time.perf_counter()
    x = make_inputs(w)
    d = {}
    for n in ("q0", "q_fixed", "k0", "k", "v"):
        d[n] = torch.from_numpy(x[n]).to(dev).to(tdt)
    d["gate"] = torch.from_numpy(x["gate"]).to(dev)
    y = torch.empty_like(d["k"])
    code = fp.dtype_code(d["k"])
    ws = torch.empty(fp.flarepp_workspace_size(w.B, w.H, w.N, w.M, w.D, code), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident ({time.perf_counter() - t0:.1f}s)")

    args = (d["q0"], d["q_fixed"], d["gate"], d["k0"], d["k"], d["v"])
    if a.backward:
        return bench_backward(a, fp, torch, np, w, x, args, y, ws)
    if not a.graph:
        warm_up(a, torch, lambda: fp.flarepp_mixer_fwd(*args, y=y, workspace=ws))

    # the timed region: exactly K forwards (plain calls, or replays of one
    # forward captured as a HIP graph)
    graph = None
    if a.graph:
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            fp.flarepp_mixer_fwd(*args, y=y, workspace=ws)
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fp.flarepp_mixer_fwd(*args, y=y, workspace=ws)
        warm_up(a, torch, graph.replay)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(a.steps):
        if graph is not None:
            graph.replay()
        else:
            fp.flarepp_mixer_fwd(*args, y=y, workspace=ws)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / a.steps
    # per-kernel split: K more forwards with HIP events recorded between the
    # launches on the library's stream (outside the timed region)
    hip = HipEvents()
    evs = [[hip.create() for _ in range(fp.FLAREPP_TIMED_EVENTS)] for _ in range(a.steps)]
    for i in range(a.steps):
        fp.flarepp_mixer_fwd_timed(*args, events=evs[i], y=y, workspace=ws)
    torch.cuda.synchronize()
    per_kernel = {}
    for j, name in enumerate(KERNELS):
        per_kernel[name] = sum(hip.elapsed_ms(e[j + 1], e[j + 2]) for e in evs) / a.steps
    for e in evs:
        for h in e:
            hip.destroy(h)
    log("[bench] per-kernel ms: " + ", ".join(f"{k} {v:.4f}" for k, v in per_kernel.items()))

    sig = 1.0 / (1.0 + np.exp(-x["gate"].astype(np.float64)))
    sig_open = [s > 0 for s in sig]
    flops = sum((12 if o else 8) for o in sig_open) * w.B * w.N * w.M * w.D
    t = ms_per_step / 1e3
    tokens_per_s = w.B * w.N / t
    tflops = flops / t / 1e12

    work = algorithmic_work(w, sig_open)
    dom = max(work, key=lambda k: per_kernel[k])
    f_launch, b_launch = work[dom]
    dur = per_kernel[dom] / 1e3
    achieved = f_launch / dur / 1e12
    traffic = read_traffic(TRAFFIC_FILE, w.name, dom)
    # fp32 runs the vector-ALU kernels: their bound is the fp32 vector rate
    bound, peak = ("alu", PEAK_FP32_VECTOR_TFLOPS) if w.dtype == "fp32" else ("mfma", PEAK_BF16_TFLOPS)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "kernel": dom,
                "algorithmic_flops_per_launch": f_launch,
                "algorithmic_bytes_per_launch": b_launch,
                "avg_launch_ms": round(per_kernel[dom], 4),
                "achieved_algorithmic_GBs": round(b_launch / dur / 1e9, 1)}

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D,
                   "dtype": w.dtype, "global_batch": w.B, "seq_len": w.N,
                   "parallelism": "single-gpu", "launch": "hip-graph" if a.graph else "stream"},
        "tflops": round(tflops, 2),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "per_kernel_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "roofline": roofline,
        "cpu_baseline": None,
        "context": PAGES_CONTEXT,
        "source_digest": source_digest(),
    }
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, w, a.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
