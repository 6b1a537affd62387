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

/* MFMA_BF16: eight accumulator chains, near-constant operands;
 * EXP_F32: eight exponential chains per lane;
 * MFMA_BF16_RANDOM / MFMA_BF16_ONES: the same products with operands of
 * random sign and mantissa, or all 1.0 -- run for a second or more, the
 * pair shows how far the power limit lowers the clock when operand bits
 * toggle as real data does.
 * COISSUE_MFMA / COISSUE_FMA / COISSUE_MIX: per iteration four independent
 * 32x32x16 products, 32 independent three-source fp32 FMAs, or both
 * interleaved (eight FMAs after each product) -- the three times give the
 * share of vector-ALU time the matrix cores hide on one SIMD. */
enum {
  FLAREPP_PROBE_MFMA_BF16 = 0,
  FLAREPP_PROBE_EXP_F32 = 1,
  FLAREPP_PROBE_MFMA_BF16_RANDOM = 2,
  FLAREPP_PROBE_MFMA_BF16_ONES = 3,
  FLAREPP_PROBE_COISSUE_MFMA = 4,
  FLAREPP_PROBE_COISSUE_FMA = 5,
  FLAREPP_PROBE_COISSUE_MIX = 6
};

/* Launches probe `which` with `blocks` workgroups of 256 threads, each lane
 * running `iters` iterations; writes one float per thread to `out` (device,
 * blocks*256 floats, caller-owned).  Returns 0, 1 for invalid arguments, 4
 * for a launch error.  Asynchronous on `stream`. */
int flarepp_probe_launch(int which, int blocks, int iters, float* out, void* stream);

/* Work done by one such launch: flops (MFMA probes), exponentials, or
 * wave-iterations (co-issue probes). */
double flarepp_probe_work(int which, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif
