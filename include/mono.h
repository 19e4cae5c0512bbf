/*
 * libmonolayer: the small-batch decode step of a DeepSeek-V4.1-style MoE
 * layer half on one MI355X (gfx950), as hand-written HIP kernels.
 *
 * The step (one "layer half", the FFN side of a decoder layer):
 *   mHC mix of the 4-stream hyper-connection row -> split / Sinkhorn into
 *   pre, post and comb -> pre-weighted collapse + weighted RMSNorm -> router
 *   (f32 logits, sqrt(softplus), bias, canonical top-k, normalise, clamp,
 *   scale) -> shared and routed SwiGLU experts (weights f32, bf16, Q8_0 or
 *   MXFP4, dequantised in the inner loop) -> block = routed + shared ->
 *   post/comb expand into the new 4-stream row, with an optional carry of the
 *   next layer half's mix sums.
 * Sources: the ds4 page "v41: fuse the single-box decode glue (HC, MoE,
 * attention)" ("What" section and commit messages) for the step list and its
 * rounding points; the SGLang page "[DeepSeek-V4] Add mhc_fused_post_pre
 * kernel" ("Motivation") for the post -> next-pre carry; the SGLang page
 * "[AMD][V4.1] Mono kernel framework ... and DeepSeek-V4.1 decode layers"
 * (figure "DeepSeek-V4.1 layer on mono", kernel K2) and the lm-sys page "Add
 * the AMD low-latency kernels section" ("Layer diagram") for the fused
 * persistent launch.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no pointer after the call returns. Weights
 *    are borrowed views.
 *  - Layouts are dense row-major. "act" tensors (state, x, norm, hidden rows,
 *    shared, block, new state) are stored as shape->act: f32 or bf16.
 *  - stream is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work: no host synchronisation, no allocation, no device-wide sync, so a
 *    sequence of calls can be captured in a HIP graph.
 *  - Arguments are checked on the host before anything is enqueued. A failing
 *    call returns a negative mono_status, enqueues nothing, and
 *    mono_last_error() lists EVERY failed check (thread-local string).
 *  - rows == 0 is valid: the call checks its arguments and returns MONO_OK
 *    without enqueueing anything.
 *  - ws is a workspace of mono_workspace_bytes(shape) bytes, initialised once
 *    with mono_workspace_init. Calls that share a workspace must be ordered
 *    (one stream); concurrent calls on one workspace race.
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    orders; repeated calls on the same device give identical bytes.
 */
#ifndef MONOLAYER_MONO_H
#define MONOLAYER_MONO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MONO_F32 = 0,   /* 4 bytes per value */
  MONO_BF16 = 1,  /* 2 bytes per value */
  MONO_Q8_0 = 2,  /* int8 values, one fp16 scale per 32 consecutive values of a row */
  MONO_MXFP4 = 3  /* e2m1 values two per byte (low nibble = even element), one e8m0 scale
                     (2^(e-127)) per 32 consecutive values of a row */
} mono_fmt;

typedef enum {
  MONO_OK = 0,
  MONO_E_INVAL = -1,       /* a bad argument (see mono_last_error) */
  MONO_E_UNSUPPORTED = -2, /* a valid but unsupported combination */
  MONO_E_DEVICE = -3,      /* a HIP runtime error while enqueueing */
  MONO_E_TIMEOUT = -4      /* a device-side bounded wait expired (mono_workspace_poll) */
} mono_status;

/* Activation quantisation of the expert matrix-vector products [vLLM "[ROCm][Perf][GLM-5] Fused
 * sparse-layer decode via AITER MonoKernel", Details, Numerics: the activations entering the
 * MXFP4 experts are quantised to MXFP8]. With MONO_AQ_MXFP8 the input of every matrix stored in
 * MXFP4 (the norm row for gate and up, the hidden row for down) is replaced by its MXFP8 round
 * trip, the OCP MX v1.0 conversion: per block of 32 values along the contraction, the shared
 * exponent X = floor(log2 max|v|) - 8 clamped to [-127, 127], each value the E4M3 number nearest
 * to v / 2^X (ties to even, magnitudes above 448 clamped to 448), times 2^X. Matrices in other
 * formats see the unquantised activations; the norm and hidden rows written out are unchanged.
 * Used by mono_moe_experts, mono_ffn_layer and mono_ffn_layer_static; the other calls ignore it. */
typedef enum { MONO_AQ_NONE = 0, MONO_AQ_MXFP8 = 1 } mono_act_quant;

/* Shape of one layer-half step. Limits (checked on the host, every failure listed):
 *   0 <= rows <= 8; n_streams == 4; hidden a positive multiple of 64; inter a positive multiple
 *   of 32 and shared_inter a non-negative multiple of 32; 1 <= top_k <= 16 and
 *   top_k <= n_experts <= 512; act MONO_F32 or MONO_BF16; 0 <= sinkhorn_iters <= 1000;
 *   routed_scale finite; eps_hc, eps_norm >= 0; act_quant MONO_AQ_NONE or MONO_AQ_MXFP8, the
 *   latter with routed.fmt MONO_MXFP4 (checked by the calls that take the layer).
 *   On-chip buffers (ab = 4 for f32, 2 for bf16 activations): (rows + 1) * hidden * ab <=
 *   114688 bytes, rows * max(inter, shared_inter) * ab <= 81920 bytes and
 *   max(inter, shared_inter) * ab <= 16384 bytes, and the slice of hidden positions one
 *   workgroup expands must fit its LDS on the current device (MONO_E_UNSUPPORTED otherwise). */
typedef struct {
  int rows;         /* R: decode rows (tokens) in the step */
  int hidden;       /* H */
  int n_streams;    /* hyper-connection streams, must be 4 */
  int n_experts;    /* E routed experts */
  int top_k;        /* k */
  int inter;        /* I: routed expert intermediate width */
  int shared_inter; /* Is: shared expert intermediate width (0 = no shared expert) */
  mono_fmt act;     /* MONO_F32 or MONO_BF16 */
  float routed_scale; /* rho, applied to the normalised routing weights */
  int sinkhorn_iters; /* Sinkhorn iterations for comb (20 in the workloads) */
  float eps_hc;       /* epsilon inside the mix RMS (1e-6) */
  float eps_norm;     /* epsilon inside the collapse RMSNorm (1e-6) */
  int act_quant;      /* mono_act_quant: MONO_AQ_MXFP8 quantises the activations entering the
                         MXFP4 experts (routed.fmt must be MONO_MXFP4) */
} mono_shape;

/* One expert set: n experts (n = E routed, n = 1 shared), each gate [inter][H], up [inter][H],
 * down [H][inter], experts stacked along the first axis. *_s are the block scales:
 * NULL for f32/bf16, fp16 [n][rows][cols/32] for Q8_0, e8m0 bytes [n][rows][cols/32] for MXFP4.
 * Value and scale arrays must be 16-byte aligned. */
typedef struct {
  mono_fmt fmt;
  const void* gate;
  const void* up;
  const void* down;
  const void* gate_s;
  const void* up_s;
  const void* down_s;
} mono_experts;

/* One layer half's weights. */
typedef struct {
  const float* w_mix;    /* [24][4H] f32: mix rows 0..3 pre, 4..7 post, 8..23 comb (i, j) */
  const float* hc_scale; /* [3] f32: gate scales of pre, post, comb */
  const float* hc_base;  /* [24] f32: gate biases */
  const void* w_norm;    /* [H] act: RMSNorm weight */
  const float* w_router; /* [E][H] f32 */
  const float* bias;     /* [E] f32: selection bias */
  mono_experts routed;   /* E experts, inter I */
  mono_experts shared;   /* 1 expert, inter Is (ignored when shared_inter == 0) */
} mono_layer;

/* ---------------------------------------------------------------------------------------------
 * Workspace and diagnostics */

/* Bytes of workspace a step of this shape needs (0 if the shape is invalid). */
size_t mono_workspace_bytes(const mono_shape* shape);

/* Enqueues the initialisation of ws (counters, error word, debug fields, tagged regions) as a
 * kernel (no memset node, so it can be captured). Needed once before first use and when the
 * workspace is used for a different shape (the fused launch tags the values it exchanges between
 * workgroups with a launch count; the init clears the tags); it also clears the error word
 * after a MONO_E_TIMEOUT. */
mono_status mono_workspace_init(void* ws, const mono_shape* shape, void* stream);

/* Synchronises `stream`, then copies the workspace error word to err[4] (host memory):
 * err[0] = 0 or 1 (a bounded wait expired in some launch since the last init), err[1] = phase,
 * err[2] = workgroup, err[3] = number of expired waits. Returns MONO_E_TIMEOUT when err[0] != 0.
 * Not for the hot path. */
mono_status mono_workspace_poll(const void* ws, uint32_t err[4], void* stream);

/* Test hooks (enqueued on `stream`): spin_limit_ticks bounds every device-side wait in units of
 * the 100 MHz real-time counter (0 = default, 2 s); fault_wg / fault_phase make that workgroup
 * withhold the values it publishes for the other workgroups at that point (-1 = off): 1 its mix
 * partial sums, 2 its router logits, 3 its hidden rows. */
mono_status mono_workspace_set_debug(void* ws, uint32_t spin_limit_ticks, int32_t fault_wg,
                                     int32_t fault_phase, void* stream);

/* Test hook: when enable != 0, later mono_ffn_layer launches on this workspace record, per
 * workgroup, the 100 MHz real-time counter at phase boundaries (MONO_T_TRACE): 0 start,
 * 1 mix partials, 2 pre-side inputs ready, 3 pre side, 4 router, 5 shared gate/up, 6 select
 * rows, 7 select finished, 8 plan, 9 routed gate/up, 10 routed down (several rows), 11 down +
 * block, 12 expand, 13 carry;
 * 14-18 inside the pre side (raw sums, mixes, gates, collapse, sum of squares), 19 select
 * scores, 20 shared down (several rows), 21 first down group staged, 22 router start (first
 * router wave), 23 router logits stored, 24 logits gathered,
 * 25-31 routed gate/up done in waves 1-7 (slot 9 is wave 0).
 * Enqueued on `stream`. */
mono_status mono_workspace_set_trace(void* ws, int enable, void* stream);

/* Debug mode (race shaker): when max_ticks != 0, mono_ffn_layer launches on this workspace
 * issued after the call make every wave wait, at each phase boundary, a pseudo-random time in
 * [0, max_ticks) ticks of the 100 MHz real-time counter, drawn from (seed, launch epoch,
 * workgroup, wave, boundary). The results do not depend on timing, so they must stay
 * byte-identical to a launch without delays; a difference or an expired wait points at a race. max_ticks above MONO_JITTER_MAX_TICKS (a delay of 0.1 ms) is
 * refused with MONO_E_INVAL; 0 turns it off, as does mono_workspace_init. A host-side setting
 * (kept per workspace address, thread-safe); nothing is enqueued. Not for the hot path. */
#define MONO_JITTER_MAX_TICKS 10000u
mono_status mono_workspace_set_jitter(void* ws, uint32_t max_ticks, uint32_t seed);

/* Intermediate tensors kept in the workspace by mono_ffn_layer (and by the unfused calls, for
 * the tensors they produce internally), for inspection after the stream has synchronised. */
typedef enum {
  MONO_T_MIXES = 0,    /* [R][24] f32 */
  MONO_T_PRE = 1,      /* [R][4] f32 */
  MONO_T_POST = 2,     /* [R][4] f32 */
  MONO_T_COMB = 3,     /* [R][4][4] f32 */
  MONO_T_X = 4,        /* [R][H] act */
  MONO_T_NORM = 5,     /* [R][H] act */
  MONO_T_LOGITS = 6,   /* [R][E] f32 */
  MONO_T_IDX = 7,      /* [R][k] int32 */
  MONO_T_WEIGHTS = 8,  /* [R][k] f32 */
  MONO_T_H_ROUTED = 9, /* [R][k][I] SwiGLU hidden rows of the selected experts, each value tagged:
                          bf16 act: uint32 = bf16 bits | tag << 16; f32 act: uint64 = f32 bits |
                          tag << 32 (the tag orders the fused launch's workgroups) */
  MONO_T_H_SHARED = 10,/* [R][Is], tagged as MONO_T_H_ROUTED */
  MONO_T_SHARED = 11,  /* [R][H] act */
  MONO_T_ROUTED = 12,  /* [R][H] f32 */
  MONO_T_BLOCK = 13,   /* [R][H] act */
  MONO_T_CARRY = 14,   /* [R][25] f32 */
  MONO_T_TRACE = 15    /* [grid][32] uint64: per-workgroup phase timestamps of the last traced
                          mono_ffn_layer (100 MHz real-time counter), see mono_workspace_set_trace */
} mono_tensor;

/* Device address and size of one intermediate inside ws (host-side arithmetic only). */
mono_status mono_workspace_tensor(const mono_shape* shape, void* ws, mono_tensor which,
                                  void** ptr, size_t* bytes);

/* Every failed check of the last failing call on this thread ("" if none). */
const char* mono_last_error(void);

/* Number of workgroups of the persistent launch on the current device (0 if no device). */
int mono_grid_size(void);

/* ---------------------------------------------------------------------------------------------
 * The step, as four unfused calls and one fused persistent launch. The fused launch computes
 * exactly the same bytes as the four calls in sequence on the same device. */

/* mHC pre side [ds4 page, HC fusion commit: "rms_norm_mix" over the 4-stream row, then
 * split/sinkhorn + pre-weighted collapse + BF16 + weighted RMSNorm + BF16].
 *   state    [R][4][H] act (read)
 *   carry_in [R][25] f32 or NULL: raw mix sums and sum of squares of `state` computed by the
 *            previous layer half's expand (the mix matvec is then skipped)
 *   outputs  mixes [R][24], pre [R][4], post [R][4], comb [R][4][4] (f32); x, norm [R][H] act.
 *            mixes and x may be NULL. */
mono_status mono_hc_mix_collapse(const mono_shape* shape, const void* state,
                                 const mono_layer* layer, const float* carry_in, float* mixes,
                                 float* pre, float* post, float* comb, void* x, void* norm,
                                 void* ws, void* stream);

/* Router [ds4 page, router commit: F32 logits matvec, then sqrt(softplus), the bias, the
 * canonical (score descending, index ascending) top-k, the normalised weights, the clamp, the
 * division and the scale, each rounded separately].
 *   norm [R][H] act (read); logits [R][E] f32 (may be NULL); idx [R][k] int32 in selection
 *   order; weights [R][k] f32 (sum to routed_scale). */
mono_status mono_router_select(const mono_shape* shape, const void* norm,
                               const mono_layer* layer, float* logits, int32_t* idx,
                               float* weights, void* ws, void* stream);

/* Experts [ds4 page, router/shared commit: gate/up rounded to BF16 before SwiGLU and the product
 * after it, the down projection rounded on its store, the routed + shared sum and its rounding;
 * SGLang mono page, K2: shared + routed experts]. Each distinct selected expert is streamed
 * once for all rows that chose it.
 *   norm [R][H] act, idx [R][k] int32 (each in [0, E), distinct within a row), weights [R][k]
 *   f32 (read). shared_out [R][H] act (may be NULL), routed_out [R][H] f32 (may be NULL),
 *   block [R][H] act = bf16(routed + shared). The hidden rows stay in ws (MONO_T_H_*). */
mono_status mono_moe_experts(const mono_shape* shape, const void* norm, const int32_t* idx,
                             const float* weights, const mono_layer* layer, void* shared_out,
                             float* routed_out, void* block, void* ws, void* stream);

/* mHC post side [ds4 page, HC fusion commit: post/comb expand + BF16; SGLang fused post/pre
 * page, Motivation: post + bf16 residual + next pre-norm GEMM partials + RMS square-sum
 * partials].
 *   state [R][4][H], block [R][H] act, post [R][4], comb [R][4][4] f32 (read)
 *   new_state [R][4][H] act (must not alias state)
 *   w_mix_next [24][4H] f32 or NULL; carry_out [R][25] f32 (required iff w_mix_next): raw next
 *   mix sums over the bf16 new state, then its sum of squares. */
mono_status mono_hc_expand(const mono_shape* shape, const void* state, const void* block,
                           const float* post, const float* comb, const float* w_mix_next,
                           void* new_state, float* carry_out, void* ws, void* stream);

/* The model tail's head weights: its own 4-row mix, one scale, four biases and the output norm
 * weight. All device pointers, caller-owned. */
typedef struct {
  const float* w_head;     /* [4][4H] f32 */
  const float* head_scale; /* [1] f32 */
  const float* head_base;  /* [4] f32 */
  const void* w_norm;      /* [H] act: the output norm weight */
} mono_head;

/* Model tail [ds4 page, single-box commit: the logits' collapse and the output norm reuse the
 * collapse without a split; SGLang fused post/pre page, Modifications: the last FFN post is
 * deferred and closed at the model tail]. From the new state of the last layer half:
 *   m[i] = (w_head[i] . s) / sqrt(mean(s^2) + eps_hc) over the flattened row s (4H values),
 *   pre[i] = sigmoid(head_scale m[i] + head_base[i]) (the split's pre half; no post, comb or
 *   Sinkhorn), x = act(sum_i pre[i] state_i), norm = act(x / sqrt(mean(x^2) + eps_norm) w_norm).
 *   state [R][4][H] act (read); pre [R][4] f32 and x [R][H] act may be NULL; norm [R][H] act.
 * Uses shape's rows, hidden, act, eps_hc and eps_norm (the rest must still be a valid shape).
 * One launch of R workgroups on `stream`; no workspace. */
mono_status mono_hc_head(const mono_shape* shape, const void* state, const mono_head* head,
                         float* pre, void* x, void* norm, void* stream);

/* The whole layer half as ONE persistent launch [SGLang mono page, K2; lm-sys page, Layer
 * diagram: mix weights and the shared expert load early, routed weights after routing; vLLM
 * GLM-5 page, Details: residual stream carried across per-layer launches, the epoch advanced
 * once per step]. One workgroup per compute unit, all resident at once (refused with
 * MONO_E_UNSUPPORTED when the device cannot hold them). There is no grid barrier: a workgroup
 * hands each value to others with the launch's epoch tag beside it and the reader polls until
 * the tag is current. The epoch comes from start counters in ws that every workgroup advances
 * first, so each launch has its own, also after a launch that ended early. Every wait is
 * bounded: on expiry the launch ends early, its outputs are invalid, and the error word is set
 * (mono_workspace_poll reports MONO_E_TIMEOUT from then on, until mono_workspace_init clears
 * it); later launches on the same workspace compute correct results.
 *   state_in [R][4][H] act; carry_in [R][25] or NULL (as in mono_hc_mix_collapse)
 *   state_out [R][4][H] act (may alias state_in); w_mix_next / carry_out as in mono_hc_expand.
 *   All intermediates are kept in ws (mono_workspace_tensor). */
mono_status mono_ffn_layer(const mono_shape* shape, const mono_layer* layer,
                           const float* w_mix_next, const void* state_in, const float* carry_in,
                           void* state_out, float* carry_out, void* ws, void* stream);

/* ---------------------------------------------------------------------------------------------
 * For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): mono_ffn_layer with its workspace in a static device array of
 * MONO_STATIC_WS_BYTES on each GPU, held from the first call on that GPU until the process
 * ends. The caller still passes inputs and outputs (as for mono_ffn_layer); the call itself
 * allocates nothing. The first call on a device, and a call whose shape differs from the previous
 * call's on that device, first enqueues the workspace initialisation (a kernel) on `stream`.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race. Device-side wait timeouts are recorded in the array's error word, which
 * this variant does not report. Returns MONO_E_UNSUPPORTED (before any device work) when the
 * shape's workspace (mono_workspace_bytes) exceeds MONO_STATIC_WS_BYTES. */
#define MONO_STATIC_WS_BYTES (8u << 20)
mono_status mono_ffn_layer_static(const mono_shape* shape, const mono_layer* layer,
                                  const float* w_mix_next, const void* state_in,
                                  const float* carry_in, void* state_out, float* carry_out,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MONOLAYER_MONO_H */
