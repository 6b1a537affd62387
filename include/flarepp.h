/*
 * libflarepp: forward pass of the FLARE++ token mixer (and two-step FLARE)
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed, for every batch element b and head h, with s = 1/sqrt(D):
 *
 *   sigma = 1 / (1 + exp(-g_h))                                   (gate)
 *   q_dyn = softmax_rows(s q0_h k0_bh^T) k0_bh                    (synthesis)
 *   q     = q_fixed_h + sigma q_dyn                               (routing query)
 *   z     = softmax_rows(s q k_bh^T) v_bh                         (encode, N -> M)
 *   y_bh  = softmax_rows(s k_bh q^T) z                            (decode, M -> N)
 *
 * Sources: "FLARE++ and FLARE: Low-rank attention routing for PDE
 * surrogates" (FLARE.py README), section "FLARE++" (core mixer listing: three
 * scaled-dot-product attention calls with the default 1/sqrt(D) scale, k0 as
 * both synthesis key and value) and section "FLARE" (two-step mixer); issue
 * "[FEA]: Update FLARE++ to the v2 reference design and add token-sharded
 * context parallelism for FLARE/FLARE++ #2024", section "Changes from v1 to
 * v2" (q = q_fixed + sigma(g) q_dynamic; gate closed gives FLARE; shared
 * synthesis keys and values) and section "Multi-GPU context parallelism"
 * (exact split encoder with log-sum-exp statistics, used here across
 * token chunks of one GPU).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *   Token tensors are [B, H, N, D]; latent tensors [H, M, D] are shared by
 *   all batch elements.  Element type is given by `dtype` (flarepp_dtype);
 *   the gate is always fp32.
 * - Alignment: every token, latent, output and saved-tensor pointer must be
 *   16-byte aligned (the kernels move them in 16-byte vectors); the
 *   workspace needs 256 bytes.  A misaligned pointer is
 *   FLAREPP_ERR_INVALID_ARGUMENT (workspace: FLAREPP_ERR_WORKSPACE).
 * - Aliasing: outputs (y, z, saved tensors, gradients) and the workspace are
 *   written by the kernels; none of them may overlap each other or any
 *   input, else FLAREPP_ERR_INVALID_ARGUMENT.
 * - Arithmetic: products accumulate in fp32; softmax statistics are fp32;
 *   intermediates q, z are kept in fp32 and rounded to the input dtype only
 *   where they feed a matrix-core product.  The output is rounded to the
 *   input dtype (round to nearest even).  fp32 inputs use an fp32 path with
 *   no reduced-precision step.
 * - Ownership: the caller owns every buffer (inputs, output, workspace).
 *   The library allocates nothing per call and keeps no pointer after the
 *   call returns.
 * - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *   default stream) and nothing is synchronised; results are valid once the
 *   caller synchronises that stream, and inputs must stay alive until then.
 *   One workspace must not be used by two calls in flight on different
 *   streams at the same time.
 * - Errors: the return value is a flarepp_status.  All argument checks run
 *   before any launch; on error nothing is enqueued.  Errors raised inside
 *   kernels surface at the caller's next synchronisation.  Non-finite values
 *   in the token or latent tensors propagate (NaN in, NaN out); the gate
 *   may be +/-inf.
 * - Results are deterministic: the token chunking depends only on the
 *   shape, and no atomics are used.
 */
#ifndef FLAREPP_H
#define FLAREPP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLAREPP_F32 = 0,
  FLAREPP_BF16 = 1,
  FLAREPP_F16 = 2
} flarepp_dtype;

typedef enum {
  FLAREPP_OK = 0,
  FLAREPP_ERR_INVALID_ARGUMENT = 1, /* null pointer, size < 1, overflow, bad dtype,
                                       non-finite or non-positive scale, output
                                       or workspace aliasing an input, pointer
                                       not 16-byte aligned */
  FLAREPP_ERR_UNSUPPORTED = 2,      /* D not in {8,16,32,64}, M > 512, or the
                                       current device is not gfx950 */
  FLAREPP_ERR_WORKSPACE = 3,        /* workspace NULL, too small or not 256-byte
                                       aligned */
  FLAREPP_ERR_HIP = 4               /* a HIP runtime call or launch failed, or no
                                       device is present */
} flarepp_status;

/* Largest number of latents M the kernels accept (the decode keeps the
 * routing queries and the encoded latents of one head resident in LDS). */
#define FLAREPP_MAX_M 512

/* Human-readable name of a status code (static storage, never NULL). */
const char* flarepp_status_string(int status);

/* Library version as "major.minor.patch" (static storage). */
const char* flarepp_version(void);

/*
 * Workspace bytes needed by flarepp_mixer_fwd / flare_mixer_fwd for this
 * shape and dtype.  Returns 0 if the arguments are invalid or unsupported
 * (same checks as the compute calls, minus pointers and device).
 * The workspace holds the per-chunk softmax partials of the split encoder
 * and the operand copies of q and z; it needs 256-byte alignment.
 */
size_t flarepp_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                              int dtype);

/*
 * FLARE++ mixer forward: y = mixer(q0, q_fixed, gate, k0, k, v), scale
 * 1/sqrt(D) in all three attention steps ("FLARE++" listing, FLARE.py
 * README; gate from issue #2024 "Fixed reference and gate").
 *
 *   q0, q_fixed : [H, M, D] dtype   learned seeds and fixed routing queries
 *   gate        : [H] fp32          gate LOGITS g; sigma(g) is applied inside.
 *                                   g = -inf closes the gate: the synthesis
 *                                   step is skipped on the device for that head
 *                                   and the head computes FLARE exactly.
 *   k0          : [B, H, N, D]      synthesis keys, also the synthesis values
 *   k, v        : [B, H, N, D]      keys and values of the input tokens
 *   y           : [B, H, N, D]      output, written; must not overlap any input
 *   workspace   : >= flarepp_workspace_size(B,H,N,M,D,dtype) bytes, 256-aligned
 *   stream      : hipStream_t (NULL = default stream)
 */
int flarepp_mixer_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                      const void* q0, const void* q_fixed, const float* gate,
                      const void* k0, const void* k, const void* v, void* y,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * flarepp_mixer_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call allocates nothing; its
 * kernels use a device array owned by the library, FLAREPP_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per device, held from the first such call on a device until the
 * process ends.  Every call on one device shares that array: calls that
 * overlap in time on one device (two streams, or two host threads) race and
 * must be serialised by the caller.  The kernels need no part of the array
 * cleared between calls.
 *   Arguments and results as for flarepp_mixer_fwd (same kernels, same
 *   token chunking, so the same bits).
 *   FLAREPP_ERR_WORKSPACE: flarepp_workspace_size(B,H,N,M,D,dtype) exceeds
 *   FLAREPP_NOALLOC_SCRATCH_BYTES (checked before any HIP call); use
 *   flarepp_mixer_fwd with a caller workspace for such shapes.
 */
#define FLAREPP_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int flarepp_mixer_fwd_noalloc(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                              const void* q0, const void* q_fixed, const float* gate,
                              const void* k0, const void* k, const void* v, void* y,
                              void* stream);

/*
 * Same computation as flarepp_mixer_fwd, with timing marks for profiling.
 * `events` points to FLAREPP_TIMED_EVENTS hipEvent_t handles created by the
 * caller; the call records them on `stream` around its launches:
 *   events[0] start                      events[1] = events[0] (no launch: the
 *                                         synthesis encoder scales the seeds itself)
 *   events[2] after the synthesis encoder events[3] after the gated combine
 *   events[4] after the encoder          events[5] after the value combine
 *   events[6] after the decoder
 * so that elapsed(events[i], events[i+1]) is the duration of one kernel.
 * Errors as for flarepp_mixer_fwd; events == NULL is INVALID_ARGUMENT.
 */
#define FLAREPP_TIMED_EVENTS 7
int flarepp_mixer_fwd_timed(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                            const void* q0, const void* q_fixed, const float* gate,
                            const void* k0, const void* k, const void* v, void* y,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events);

/*
 * Simplified FLARE++ mixer forward (what the first preprint called FLARE++;
 * issue #2024, "v1 vs. v2" and "Changes from v1 to v2": four input
 * projections, so the synthesis has its own values v0, and no fixed
 * reference or gate, so the routing queries are the synthesized ones;
 * paper summary "FLARE++: Low-rank attention with dynamic attention
 * routing", "Dynamic Query Synthesis"), scale 1/sqrt(D) throughout:
 *   q    = softmax_rows(s q0 k0^T) v0          per (b, h)
 *   z    = softmax_rows(s q k^T) v ;  y = softmax_rows(s k q^T) z.
 *
 *   q0      : [H, M, D] dtype  learned seeds
 *   k0, v0  : [B, H, N, D]     synthesis keys and values (v0 == k0 is allowed
 *                              and gives flarepp_mixer_fwd with q_fixed = 0
 *                              and an open gate, g = +inf)
 *   k, v    : [B, H, N, D]     keys and values of the input tokens
 *   y       : [B, H, N, D]     output, written; must not overlap any input
 *   workspace as for flarepp_mixer_fwd (the same size function applies).
 * Errors as for flarepp_mixer_fwd.
 */
int simplified_flarepp_mixer_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 int dtype, const void* q0, const void* k0, const void* v0,
                                 const void* k, const void* v, void* y, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Two-step FLARE mixer forward (FLARE.py README, section "FLARE"):
 *   z = softmax_rows(scale q k^T) v ;  y = softmax_rows(scale k q^T) z.
 * The listing on that page uses scale = 1.0; a closed-gate FLARE++ head
 * equals this call with scale = 1/sqrt(D).
 *
 *   q     : [H, M, D] dtype  latent queries
 *   k, v  : [B, H, N, D]     keys and values
 *   y     : [B, H, N, D]     output, written; must not overlap any input
 *   scale : finite and > 0
 *   workspace as for flarepp_mixer_fwd (the same size function applies).
 */
int flare_mixer_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                    float scale, const void* q, const void* k, const void* v, void* y,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes for flare_encode_fwd with a given token chunk length
 * (chunk_tokens = 0 selects the same chunking as the mixer calls).
 */
size_t flare_encode_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                   int dtype, int64_t chunk_tokens);

/*
 * Encoder alone (the "flare_encode" step named in issue #2024, "Multi-GPU
 * context parallelism"): z = softmax_rows(scale q k^T) v, computed as
 * per-chunk partials (row max, row sum, unnormalised output) over token
 * chunks of `chunk_tokens` tokens and merged with log-sum-exp weights.
 *
 *   q              : [H, M, D] dtype if q_batch_stride == 0, else [B, H, M, D]
 *                    with q_batch_stride == H*M*D elements
 *   k, v           : [B, H, N, D] dtype (v may equal k)
 *   z              : [B, H, M, D] fp32, written
 *   chunk_tokens   : 0 = default chunking; otherwise a positive multiple of 64
 *   workspace      : >= flare_encode_workspace_size(..., chunk_tokens)
 */
int flare_encode_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                     float scale, const void* q, int64_t q_batch_stride,
                     const void* k, const void* v, float* z, int64_t chunk_tokens,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for flare_decode_fwd. */
size_t flare_decode_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                   int dtype);

/*
 * Decoder alone: y = softmax_rows(scale k q^T) z, the softmax running over
 * the M latents of each token (third call of the FLARE++ listing, second
 * call of the FLARE listing).
 *
 *   q  : [H, M, D] dtype if q_batch_stride == 0, else [B, H, M, D] with
 *        q_batch_stride == H*M*D
 *   z  : [B, H, M, D] fp32 latent values
 *   k  : [B, H, N, D] dtype token keys (the queries of this step)
 *   y  : [B, H, N, D] dtype, written; must not overlap any input
 */
int flare_decode_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                     float scale, const void* q, int64_t q_batch_stride, const float* z,
                     const void* k, void* y, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Training: forward with saved tensors, and the backward pass.
 *
 * The gradients follow from the forward definition by the chain rule (the
 * pages state that the token-sharded encoder has a custom backward, issue
 * #2024 "Multi-GPU context parallelism", but do not print it).  For one
 * attention O = softmax_rows(s Q K^T) V with output gradient dO:
 *   dV = A^T dO,  dS = A * (dO V^T - rowsum(dO * O)),  dQ = s dS K,
 *   dK = s dS^T Q.
 * The backward supports every dtype with D in {8, 16, 32, 64} and M <= 512.
 * bf16 and fp16 with D >= 16 run on the matrix cores (the token pass holds
 * a head's latents in one workgroup's 160 KiB LDS; at D = 64 with M > 384 it
 * runs over two latent ranges, the second adding into the gradients the
 * first stored); fp32 inputs (every D) and D = 8 (below the matrix-core
 * contraction length) run on VALU kernels in fp32 arithmetic, one thread per
 * latent row or token.  Other cases return FLAREPP_ERR_UNSUPPORTED.  The token
 * tensors k, v, k0, y, dy and every gradient output (fp32) must be 16-byte
 * aligned, else FLAREPP_ERR_INVALID_ARGUMENT.  Gradient outputs must not
 * overlap any input or `saved`.  Results are deterministic (fixed reduction
 * orders).  Calls run asynchronously on `stream`.
 * ---------------------------------------------------------------------- */

/* Bytes of the `saved` buffer a training forward fills (fp32): the routing
 * query q [B,H,M,D], z [B,H,M,D], q_dyn [B,H,M,D], the base-2 log-sum-exp of
 * the synthesis and encoder rows [B,H,M] each and of the decoder rows
 * [B,H,N].  0 for invalid sizes. */
size_t flarepp_saved_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D);

/* flarepp_mixer_fwd that also fills `saved` (>= flarepp_saved_size bytes,
 * 16-byte aligned, caller-owned, must not overlap y or the workspace). */
int flarepp_mixer_fwd_train(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                            const void* q0, const void* q_fixed, const float* gate,
                            const void* k0, const void* k, const void* v, void* y, float* saved,
                            size_t saved_bytes, void* workspace, size_t workspace_bytes,
                            void* stream);

/* flare_mixer_fwd that also fills `saved` (z and the encoder and decoder
 * log-sum-exp rows; the q and q_dyn slots are left untouched). */
int flare_mixer_fwd_train(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                          float scale, const void* q, const void* k, const void* v, void* y,
                          float* saved, size_t saved_bytes, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes of flarepp_mixer_bwd / flare_mixer_bwd (256-byte aligned);
 * 0 for unsupported or invalid arguments. */
size_t flarepp_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                  int dtype);

/*
 * FLARE++ backward.  Inputs as for flarepp_mixer_fwd plus the forward's
 * output y and the output gradient dy [B,H,N,D] (dtype), and `saved` from
 * flarepp_mixer_fwd_train on the same inputs.  Writes (fp32):
 *   dq0, dq_fixed : [H, M, D]   (summed over the batch)
 *   dgate         : [H]         (gradient w.r.t. the gate LOGITS)
 *   dk0, dk, dv   : [B, H, N, D]
 * A closed gate (g = -inf) gives zero dq0, dk0 and dgate for its head.
 */
int flarepp_mixer_bwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                      const void* q0, const void* q_fixed, const float* gate, const void* k0,
                      const void* k, const void* v, const void* y, const void* dy,
                      const float* saved, size_t saved_bytes, float* dq0, float* dq_fixed,
                      float* dgate, float* dk0, float* dk, float* dv, void* workspace,
                      size_t workspace_bytes, void* stream);

/* FLARE backward with the caller's scale; `saved` from flare_mixer_fwd_train.
 * Writes dq [H, M, D] (summed over the batch), dk, dv [B, H, N, D] (fp32). */
int flare_mixer_bwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                    float scale, const void* q, const void* k, const void* v, const void* y,
                    const void* dy, const float* saved, size_t saved_bytes, float* dq, float* dk,
                    float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* simplified_flarepp_mixer_fwd that also fills `saved` (the q slot holds
 * the synthesized query q = q_dyn). */
int simplified_flarepp_mixer_fwd_train(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                       int dtype, const void* q0, const void* k0, const void* v0,
                                       const void* k, const void* v, void* y, float* saved,
                                       size_t saved_bytes, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Backward of the simplified mixer (issue #2024, "Changes from v1 to v2":
 * the v1 form, q = softmax(s q0 k0^T) v0 with its own synthesis values).
 * `saved` from simplified_flarepp_mixer_fwd_train on the same inputs.
 * Writes (fp32): dq0 [H, M, D] (summed over the batch), dk0, dv0, dk, dv
 * [B, H, N, D].  v0 == k0 is rejected (that is FLARE++ with an open gate and
 * no fixed queries; use flarepp_mixer_bwd).  Other rules as flarepp_mixer_bwd.
 */
int simplified_flarepp_mixer_bwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 int dtype, const void* q0, const void* k0, const void* v0,
                                 const void* k, const void* v, const void* y, const void* dy,
                                 const float* saved, size_t saved_bytes, float* dq0, float* dk0,
                                 float* dv0, float* dk, float* dv, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Front end of the block (issue #2024, "Changes from v1 to v2": three input
 * projections, the synthesis keys and values shared; the synthesis call
 * normalised head by head -- its exact form is in the paper's Appendix A,
 * which the pages do not include; the core mixer of the FLARE.py README,
 * section "FLARE++", has neither projections nor normalisation).  Reading taken: a projection is
 * x @ W^T + b with W in the [H*D, C] layout of a linear layer, split into H
 * heads of D features (head-major); the head-wise normalisation is
 * u / sqrt(mean_d(u_d^2) + eps) * g over the D features of one head, applied
 * to k0 and to the seeds q0, not to k or v.
 * ---------------------------------------------------------------------- */

/*
 * k0, k, v = the three projections of the block input x, k0 normalised.
 *   x                 : [B, N, C] dtype (C a multiple of 16)
 *   w_k0, w_k, w_v    : [H*D, C] dtype;  b_k0, b_k, b_v : [H*D] dtype or NULL
 *   g_k0              : [H, D] dtype gain, or NULL (gain 1)
 *   eps               : > 0 (checked when normalize_k0 != 0)
 *   k0, k, v          : [B, H, N, D] dtype, written; must not overlap any
 *                       input or each other
 * bf16/fp16, D in {16, 32, 64}; all tensors 16-byte aligned.  fp32 and other
 * D return FLAREPP_ERR_UNSUPPORTED.  One launch on `stream`, no workspace.
 */
int flarepp_frontend_fwd(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D, int dtype,
                         const void* x, const void* w_k0, const void* w_k, const void* w_v,
                         const void* b_k0, const void* b_k, const void* b_v, const void* g_k0,
                         float eps, int normalize_k0, void* k0, void* k, void* v, void* stream);

/* Head-wise normalisation of the seeds: q0_out = q0 / sqrt(mean_d(q0^2) +
 * eps) * g per (h, m); q0 [H, M, D] dtype, g [H, D] or NULL, D <= 64;
 * q0_out may be q0 itself (in place) but must not overlap it otherwise. */
int flarepp_seed_norm_fwd(int64_t H, int64_t M, int64_t D, int dtype, const void* q0,
                          const void* g_q0, float eps, void* q0_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLAREPP_H */
