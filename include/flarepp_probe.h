/*
 * libflarepp_probe: throughput probes used by bench.py to measure, on the
 * device at hand, the two rates that bound the mixer's kernels -- dense bf16
 * matrix-core flops and v_exp_f32 exponentials -- next to the published
 * peaks.  Measurement infrastructure only; not part of the mixer's API.
 */
#ifndef FLAREPP_PROBE_H
#define FLAREPP_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

enum { FLAREPP_PROBE_MFMA_BF16 = 0, FLAREPP_PROBE_EXP_F32 = 1 };

/* Launches probe `which` with `blocks` workgroups of 256 threads, each lane
 * running `iters` iterations; writes one float per thread to `out` (device,
 * blocks*256 floats, caller-owned).  Returns 0, 1 for invalid arguments, 4
 * for a launch error.  Asynchronous on `stream`. */
int flarepp_probe_launch(int which, int blocks, int iters, float* out, void* stream);

/* Work done by one such launch: flops (MFMA probe) or exponentials. */
double flarepp_probe_work(int which, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif
