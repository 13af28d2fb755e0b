/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention decode step.
 *
 * One call advances M independent streams of one KDA layer by one token:
 *
 *   1. short causal convolution (kernel 4, three cached taps) + SiLU over the
 *      q, k and v channels ("GLM-5.3 deep dive", 8.2.4 step 2; "At the 262k
 *      cap the DSA indexer costs 12x the sparse MLA it selects for",
 *      "Geometry": depthwise, kernel 4, 3 taps, 3 tensors);
 *   2. per-head L2 normalisation of q and k, and the q scale (8.2.4 step 6;
 *      8.2.6 implementation notes: epsilon 1e-6, q scaled after the norm);
 *   3. the gated delta rule on the per-head [D x D] state and the readout
 *      (8.2.3 Eq. 1:  S' = (I - b k k^T) Diag(a) S + b k v^T,  o = S'^T q,
 *      evaluated as fade, predict, correct, read: 8.2.6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers to memory the caller owns.  The
 *   library never allocates, frees, synchronises, or keeps state between
 *   calls (kda_prefill_gated_ws takes its scratch memory as a caller
 *   workspace).  Every pointer must be 16-byte aligned.
 * - Arrays are dense, row-major, last index fastest.  "bf16" is the 16-bit
 *   bfloat16 bit pattern (uint16); "f32" is IEEE binary32.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *   and runs asynchronously.  KDA_OK means the work was enqueued; faults
 *   during execution surface at the caller's next synchronisation.
 * - Every argument check happens on the host before any HIP call, so an
 *   invalid call returns its status without touching the GPU.
 * - M == 0 is an empty batch: KDA_OK, nothing is read or written.
 * - Results are bitwise deterministic for a given input, shape, work split
 *   and device.
 * - Values outside the stated ranges (alpha, beta not in [0, 1], NaN) are the
 *   caller's contract and are not checked on the device.
 * - Rounding to bf16 is round-to-nearest-even; all arithmetic is f32.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,   /* a required pointer is NULL                         */
    KDA_ERR_SHAPE = 2,  /* H < 1, or D not one of the supported head widths   */
    KDA_ERR_DTYPE = 3,  /* state_dtype is not a kda_state_dtype               */
    KDA_ERR_ALIGN = 4,  /* a pointer is not 16-byte aligned                   */
    KDA_ERR_ALIAS = 5,  /* an output overlaps an input it may not overlap     */
    KDA_ERR_ARG = 6,    /* M < 0, C < 1, non-finite scale, sizes overflow     */
    KDA_ERR_HIP = 7     /* the HIP runtime refused the launch                 */
};

/* Largest token count per stream of one kda_decode_multi or
 * kda_prefill_gated call (2^30): keeps every token index of the kernels'
 * chunk loops inside int. */
#define KDA_MAX_TOKENS (1 << 30)

/* Storage type of the recurrent state.  Arithmetic is f32 either way. */
typedef enum { KDA_STATE_F32 = 0, KDA_STATE_BF16 = 1 } kda_state_dtype;

/* Forget-gate forms ("GLM-5.3 deep dive", 8.2.3, the gate as fla computes
 * it), per head h and key channel c, from the raw gate projection f:
 *   KDA_GATE_BOUNDED:  g = lower_bound * sigmoid(exp(A_log[h]) * (f + dt_bias))
 *                      (GLM-5.3-Flash: lower_bound = -5, so alpha > e^-5)
 *   KDA_GATE_SOFTPLUS: g = -exp(A_log[h]) * softplus(f + dt_bias)  (fla's default)
 *   alpha = exp(g). */
typedef enum { KDA_GATE_BOUNDED = 0, KDA_GATE_SOFTPLUS = 1 } kda_gate_kind;

/* epsilon inside the L2 norm: x * 1/sqrt(sum x^2 + eps) */
#define KDA_L2NORM_EPS 1e-6f

/* Supported head widths D (= dk = dv): 16, 32, 64, 128. */

/*
 * kda_decode_step -- the fused step: conv + SiLU, L2 norm, gated delta
 * update and readout, for M streams x H heads of width D.
 *
 *  state   [M][H][D][D]  f32 or bf16 (state_dtype), updated in place.
 *                        Row i is key channel i (faded by alpha_i), column j
 *                        is value channel j.
 *  x_qkv   [M][3][H*D]   bf16: this token's pre-conv q, k, v (projections).
 *  conv_w  [3*H*D][4]    bf16: depthwise conv weights, q channels then k then
 *                        v; tap 3 multiplies the current token, tap 0 the
 *                        oldest cached one.  No bias.
 *  conv_in [M][3][3*H*D] bf16: the last three raw inputs per channel,
 *                        tap 0 oldest (the channel index runs over q|k|v).
 *  conv_out same shape:  receives (tap1, tap2, x).  May be the SAME pointer
 *                        as conv_in (in-place); must not partially overlap.
 *                        Distinct buffers let the library split a head over
 *                        several workgroups when M*H is small.
 *  alpha   [M][H][D]     f32 per key-channel decay, in [0, 1] (linear, not log).
 *  beta    [M][H]        f32 write strength, in [0, 1].
 *  scale   q scale applied after the norm (1/sqrt(D) as in fla's decode; 1
 *          for Eq. 1 as printed).  Must be finite.
 *  o       [M][H][D]     bf16 output, o = S'^T q^ computed from the unrounded
 *                        f32 new state and rounded once.
 *
 * state, o and conv_out must not overlap each other or any input (except
 * conv_out == conv_in exactly).  Returns a KDA_* status.
 */
int kda_decode_step(int M, int H, int D, int state_dtype,
                    void *state, const void *x_qkv, const void *conv_w,
                    const void *conv_in, void *conv_out,
                    const float *alpha, const float *beta, float scale,
                    void *o, void *stream);

/*
 * kda_decode_step_split -- kda_decode_step with an explicit work split:
 * `nsplit` workgroups per head, each owning D/nsplit value columns.  nsplit
 * is 1, 2 or 4; values above 1 need D == 128 and conv_out != conv_in (the
 * workgroups of a head all read the head's q/k conv taps).  The split
 * changes the order of the f32 sums over key rows, so results for different
 * nsplit agree to f32 rounding, not bit for bit (each one is deterministic).
 * The conv state is bit-identical for every nsplit.  kda_decode_step picks nsplit itself
 * from M*H and the device's compute-unit count.  Returns a KDA_* status
 * (KDA_ERR_ARG for an nsplit it cannot honour).
 */
int kda_decode_step_split(int M, int H, int D, int state_dtype,
                          void *state, const void *x_qkv, const void *conv_w,
                          const void *conv_in, void *conv_out,
                          const float *alpha, const float *beta, float scale,
                          void *o, void *stream, int nsplit);

/*
 * kda_decode_step_gated -- kda_decode_step with the step's gate inputs in
 * raw form, computed in the kernel's prologue ("GLM-5.3 deep dive", 8.2.4
 * steps 4 and 5; 8.2.3 for the gate): alpha from the forget gate, beta =
 * sigmoid(beta_logit).  In place of alpha and beta it takes
 *
 *  f_gate      [M][H*D]  bf16: raw forget-gate projection of this token.
 *  A_log       [H]       f32: per-head A_log.
 *  dt_bias     [H*D]     f32: per-head, per-channel bias (shared by streams).
 *  beta_logit  [M][H]    bf16: write-strength logits.
 *  gate_kind   a kda_gate_kind; gate_lower_bound must be finite and < 0 for
 *              KDA_GATE_BOUNDED and is ignored for KDA_GATE_SOFTPLUS.
 *
 * Everything else, the splits the library may choose, and the aliasing rules
 * (the new inputs count as inputs) are those of kda_decode_step.  alpha and
 * beta are formed in f32 and never written to memory.  Returns a KDA_*
 * status (KDA_ERR_ARG for a bad gate_kind or lower bound).
 */
int kda_decode_step_gated(int M, int H, int D, int state_dtype,
                          void *state, const void *x_qkv, const void *conv_w,
                          const void *conv_in, void *conv_out,
                          const void *f_gate, const float *A_log,
                          const float *dt_bias, const void *beta_logit,
                          int gate_kind, float gate_lower_bound, float scale,
                          void *o, void *stream);

/*
 * kda_decode_layer_step -- the KDA layer's core for one token, between the
 * input projections and the output projection ("GLM-5.3 deep dive", 8.2.4
 * steps 2-7): kda_decode_step_gated followed by the gated RMSNorm of each
 * head's outputs (8.2.4 step 7 and implementation notes:
 * FusedRMSNormGated over the head's D outputs, sigmoid gate):
 *
 *   y_j = o_j / sqrt((1/D) sum_i o_i^2 + norm_eps) * norm_weight[j] * sigmoid(out_gate_j)
 *
 * computed from the unrounded f32 o (o itself is not written).
 *
 *  out_gate     [M][H*D]  bf16: output-gate projection of this token.
 *  norm_weight  [D]       f32: RMSNorm weight, shared by the heads.
 *  norm_eps     finite, >= 0 (1e-5 in GLM-5.3-Flash).
 *  y            [M][H][D] bf16 output (rounded once, RNE).
 *
 * One workgroup always owns a whole head here (no column split).  Other
 * arguments and rules as kda_decode_step_gated.  Returns a KDA_* status.
 */
int kda_decode_layer_step(int M, int H, int D, int state_dtype,
                          void *state, const void *x_qkv, const void *conv_w,
                          const void *conv_in, void *conv_out,
                          const void *f_gate, const float *A_log,
                          const float *dt_bias, const void *beta_logit,
                          int gate_kind, float gate_lower_bound, float scale,
                          const void *out_gate, const float *norm_weight,
                          float norm_eps, void *y, void *stream);

/*
 * kda_decode_multi -- T consecutive tokens of each of M streams in one call
 * (fla's decode mode runs inputs of up to 64 tokens through the recurrent
 * form, "GLM-5.3 deep dive" 8.2.6): token t of a stream is the step of
 * kda_decode_step applied to the state and conv state left by token t - 1.
 * One workgroup keeps a head's state on chip for all T tokens, so the state
 * is read and written once per call instead of once per token (with bf16
 * storage it is also rounded once per call).  For speculative/MTP
 * verification and short prefill.
 *
 *  T       tokens per stream, 0 <= T <= KDA_MAX_TOKENS (T == 0 or M == 0:
 *          nothing is touched; above the cap: KDA_ERR_ARG).
 *  x_qkv   [M][T][3][H*D]  bf16 pre-conv q|k|v of each token.
 *  alpha   [M][T][H][D]    f32.
 *  beta    [M][T][H]       f32.
 *  o       [M][T][H][D]    bf16 output of every token.
 *  state, conv_w, conv_in, conv_out, scale as kda_decode_step (conv_out may
 *  be conv_in; it receives the last three raw inputs after token T - 1).
 *
 * Aliasing rules as kda_decode_step.  Returns a KDA_* status.
 */
int kda_decode_multi(int T, int M, int H, int D, int state_dtype,
                     void *state, const void *x_qkv, const void *conv_w,
                     const void *conv_in, void *conv_out,
                     const float *alpha, const float *beta, float scale,
                     void *o, void *stream);

/*
 * kda_prefill_gated -- L consecutive tokens of each of M streams (a prompt
 * or a long continuation), computed chunk by chunk in the WY / UT form of
 * "GLM-5.3 deep dive" 8.2.5 on matrix cores: the same recurrence as L calls
 * of kda_decode_step_gated (conv + SiLU, L2 norms, bounded forget gate,
 * beta = sigmoid(logit), gated delta rule, readout), reordered into matrix
 * products over chunks of 16 tokens.
 *
 *  L          tokens per stream, 0 <= L <= KDA_MAX_TOKENS (L == 0 or M == 0:
 *             nothing is touched; above the cap: KDA_ERR_ARG).
 *  D          must be 128.
 *  x_qkv      [M][L][3][H*D]  bf16 pre-conv q|k|v.
 *  f_gate     [M][L][H*D]     bf16 raw forget-gate projection.
 *  A_log [H], dt_bias [H*D]   f32, as kda_decode_step_gated.
 *  beta_logit [M][L][H]       bf16.
 *  gate_lower_bound           in [-5, 0): the bounded gate only.  Within a
 *             16-token chunk the cumulative log-decay is then >= -80, so the
 *             chunk's decay products and their inverses stay inside f32's
 *             range (8.2.3 implementation notes on the -5 bound).
 *  o          [M][L][H][D]    bf16 output of every token.
 *  state, conv_w, conv_in, conv_out, scale as kda_decode_step (conv_out may
 *  be conv_in; it receives the last three raw inputs).
 *
 * One workgroup per (stream, head) sweeps its chunks in order, so M*H
 * should be at least the device's compute-unit count for a full device.
 * When 2*M*H is at most that count and conv_out is not conv_in, two
 * workgroups share each head, each owning half of the value columns (the
 * columns of the state evolve independently); the results are bit-identical
 * to the one-workgroup form.  In place (conv_out == conv_in) the kernel
 * always runs one workgroup per head, as the second one would read cached
 * taps the first has overwritten.
 * Results agree with the token-by-token recurrence to the rounding of the
 * reordered f32 arithmetic (see the tests), not bit for bit.  Returns a
 * KDA_* status (KDA_ERR_SHAPE for D != 128, KDA_ERR_ARG for a lower bound
 * outside [-5, 0)).
 */
int kda_prefill_gated(int L, int M, int H, int D, int state_dtype,
                      void *state, const void *x_qkv, const void *conv_w,
                      const void *conv_in, void *conv_out,
                      const void *f_gate, const float *A_log,
                      const float *dt_bias, const void *beta_logit,
                      float gate_lower_bound, float scale, void *o,
                      void *stream);

/* Bytes of one (stream, head, 16-token chunk) record of the two-pass prefill. */
#define KDA_PREFILL_RECORD_BYTES 42496

/*
 * kda_prefill_workspace_bytes -- workspace that lets kda_prefill_gated_ws run
 * an L-token call in one segment: ceil(L / 16) * M * H *
 * KDA_PREFILL_RECORD_BYTES.  0 for an invalid shape (L, M or H < 1, D != 128)
 * or a size above 2^40.  Smaller workspaces also work (see below).
 */
size_t kda_prefill_workspace_bytes(int L, int M, int H, int D);

/*
 * kda_prefill_gated_ws -- kda_prefill_gated in the two-pass chunk form of
 * "GLM-5.3 deep dive" 8.2.5 (the intra-chunk work is parallel over chunks;
 * only the state is carried from chunk to chunk):
 *   pass 1, one workgroup per (stream, head, chunk): conv + SiLU, gate, beta,
 *     L2 norms, A = StrictTril(Diag(beta)(Gamma . K)(K / Gamma)^T), the
 *     output mask P and the solves (I + A) W = Diag(beta)(Gamma . K),
 *     (I + A) U = Diag(beta) V, written to the workspace as one record per
 *     chunk;
 *   pass 2, per (stream, head) and in chunk order: Delta = U - W S,
 *     O = (Gamma . Q) S + P Delta, S' = Diag(gamma_C) S + ((gamma_C / Gamma)
 *     . K)^T Delta, with 16 value columns per wave.
 * A single long prompt (few streams) then occupies the whole device in pass
 * 1, where kda_prefill_gated's one workgroup per head would leave most CUs
 * idle.
 *
 *  Arguments before `workspace` are those of kda_prefill_gated, with the same
 *  meaning, layouts, ranges and aliasing rules.
 *  workspace        DEVICE scratch memory the caller owns, 16-byte aligned,
 *                   overlapping no other argument; its contents on entry are
 *                   ignored and on exit unspecified.  Calls that share one
 *                   workspace must be ordered (same stream).
 *  workspace_bytes  its size.  With kda_prefill_workspace_bytes(L, M, H, D)
 *                   or more the call runs as one segment (two launches); a
 *                   smaller workspace runs the sequence in segments of as
 *                   many chunks as fit (two launches each), down to
 *                   M * H * KDA_PREFILL_RECORD_BYTES, plus M * H * 65536
 *                   bytes for bf16 state (an f32 copy of the state carried
 *                   between segments, so the state is rounded to bf16 once,
 *                   at the end).  Below that: KDA_ERR_ARG.
 *  passes           0: the library chooses (two passes while 2 * M * H is at
 *                   most the compute-unit count of the stream's device, else
 *                   the one-pass kernel of kda_prefill_gated, which then
 *                   fills the device and leaves the workspace untouched);
 *                   1: one pass (workspace unused, may be NULL, not
 *                   checked); 2: two passes.  For 0 and 2 the workspace is
 *                   checked (NULL, alignment, size, overlap) whichever form
 *                   runs.
 *
 * Results agree with the token-by-token recurrence to the rounding of the
 * reordered f32 arithmetic, as kda_prefill_gated's; the one- and two-pass
 * forms perform the same operations per chunk and column in the same order
 * but are not guaranteed bit-identical to each other.  Returns a KDA_* status.
 */
int kda_prefill_gated_ws(int L, int M, int H, int D, int state_dtype,
                         void *state, const void *x_qkv, const void *conv_w,
                         const void *conv_in, void *conv_out,
                         const void *f_gate, const float *A_log,
                         const float *dt_bias, const void *beta_logit,
                         float gate_lower_bound, float scale, void *o,
                         void *workspace, size_t workspace_bytes, int passes,
                         void *stream);

/*
 * kda_prefill_gated_noalloc -- kda_prefill_gated_ws for callers that cannot
 * allocate device memory or own a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the two-pass
 * form's workspace is a 64 MiB array in the library's device memory, one
 * per GPU, held until the process ends.  The call itself allocates nothing
 * (no hipMalloc / hipFree / allocating library routine).
 *
 *  Arguments, layouts, ranges and aliasing rules as kda_prefill_gated.  The
 *  form is chosen as kda_prefill_gated_ws with passes = 0; the two passes
 *  run in segments of as many chunks as the array holds records for.
 *  Above the array's capacity (M * H * KDA_PREFILL_RECORD_BYTES, plus
 *  M * H * 65536 for bf16 state when the sequence takes more than one
 *  segment, over 64 MiB -- only reachable where 2 * M * H is at most the
 *  device's CU count, i.e. on devices of more than ~3000 CUs): KDA_ERR_ARG.
 *  The array keeps whatever the last call left; nothing in it needs to
 *  start at any value.  Calls on one GPU share its array: calls that may
 *  overlap in time on one GPU (different streams) race and must not be made.
 *  On the first call on a device the library looks up the array's device
 *  address (KDA_ERR_HIP if the runtime cannot).  Returns a KDA_* status.
 */
int kda_prefill_gated_noalloc(int L, int M, int H, int D, int state_dtype,
                              void *state, const void *x_qkv, const void *conv_w,
                              const void *conv_in, void *conv_out,
                              const void *f_gate, const float *A_log,
                              const float *dt_bias, const void *beta_logit,
                              float gate_lower_bound, float scale, void *o,
                              void *stream);

/*
 * kda_conv_step -- the conv stage alone, over C independent channels
 * ("GLM-5.3 deep dive", 8.2.4 step 2; one launch over all q|k|v channels).
 *
 *  x        [M][C]     bf16 current token.
 *  conv_w   [C][4]     bf16 weights (tap 3 = current token).
 *  conv_in  [M][3][C]  bf16 cached taps, tap 0 oldest.
 *  conv_out [M][3][C]  bf16 shifted taps (tap1, tap2, x); may equal conv_in.
 *  y        [M][C]     f32 SiLU(conv) output.
 *
 * C must be a multiple of 8.  Returns a KDA_* status.
 */
int kda_conv_step(int M, int C, const void *x, const void *conv_w,
                  const void *conv_in, void *conv_out, float *y, void *stream);

/*
 * kda_recurrent_step -- steps 2 and 3 alone, from post-conv (post-SiLU) f32
 * q|k|v: L2 norm, q scale, gated delta update and readout ("GLM-5.3 deep
 * dive", 8.2.3 Eq. 1 and 8.2.6).  kda_conv_step followed by this call
 * computes what kda_decode_step computes.
 *
 *  qkv [M][3][H*D] f32; state, alpha, beta, scale, o as kda_decode_step.
 *  Returns a KDA_* status.
 */
int kda_recurrent_step(int M, int H, int D, int state_dtype, void *state,
                       const float *qkv, const float *alpha, const float *beta,
                       float scale, void *o, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
