/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective state-space scan library.
 *
 * The library computes, per channel d and state index n of a diagonal SSM,
 *   zero-order hold:  Abar = exp(delta_t * A),  Bbar = (Abar - 1) / A * B_t
 *   recurrence:       h_t  = Abar * h_{t-1} + Bbar * x_t          (state first)
 *   readout + gate:   y_t  = (C_t . h_t + D * x_t) * SiLU(z_t)
 * with delta, B and C given per token and A fixed per (channel, state).
 * Sources (web pages, cited by title and section):
 *   - ultralytics glossary "State Space Models (SSM)", section "SSMの仕組み":
 *     ZOH formulas, the recurrence, and the recurrent/convolution equivalence;
 *   - paperlens tutorial "Mamba と状態空間モデル": eq.(1)/(2) (continuous
 *     system and its discretisation), section "Mamba: 状態を「選択的」にする"
 *     (per-token delta, B, C with fixed A) and the practice notes (state
 *     snapshot/restore, no silent slow fallback);
 *   - ihouse article on Mamba-3: the state and output equations with the D
 *     term, and the decode step being a memory-bound outer-product update;
 *   - agenticai-flow guide, section "アーキテクチャ図解": the S6 output is
 *     multiplied by SiLU of the z branch.
 * Also: the scan's variants (A per channel, Euler rule), its fused prologue
 * (causal conv1d, softplus of delta), its backward (all input gradients) and
 * its masked-matrix form for a step and decay shared per head, forward and
 * backward (ssm_ssd_fwd, ssm_ssd_bwd).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major memory,
 *     16-byte aligned (misaligned pointers return SSM_ERR_INVALID_ARG).
 *   - The caller owns every buffer, including the workspace; the library
 *     allocates no device memory and keeps no mutable global state, so
 *     concurrent calls on different streams are safe.
 *   - Calls only enqueue work on `stream` (a hipStream_t, NULL = the null
 *     stream) and never synchronise the host.  Argument errors are returned
 *     before anything is enqueued; launch failures return SSM_ERR_HIP;
 *     asynchronous device faults surface at the caller's next synchronisation.
 *   - There is no fallback: a shape, dtype or state size without a kernel
 *     returns SSM_ERR_UNSUPPORTED instead of running a slow path.
 *   - io_dtype selects the type of x, delta, z, B, C and y (all the same).
 *     A, D and every state tensor are always fp32; arithmetic is fp32.
 *   - dstate: 16 everywhere; 32, 64 and 128 also for the forward scan (not
 *     fused), the decode step and the backward; 64 or 128 for the
 *     masked-matrix forward; other values return SSM_ERR_UNSUPPORTED.
 *   - NaN/Inf in inputs propagate by IEEE rules; nothing is checked on device.
 */
#ifndef SSM_H_
#define SSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 3

/* Values of the io_dtype arguments. */
#define SSM_DTYPE_F32 0
#define SSM_DTYPE_BF16 1

/* Values of the discretization argument of ssm_scan_fwd_ex. */
#define SSM_DISC_ZOH 0   /* Bbar = (exp(delta*A) - 1) / A * B  (zero-order hold) */
#define SSM_DISC_EULER 1 /* Bbar = delta * B                                      */

/* Status codes returned by every entry point. */
#define SSM_OK 0
#define SSM_ERR_INVALID_ARG 1 /* NULL required pointer, negative size, aliasing */
#define SSM_ERR_UNSUPPORTED 2 /* valid request with no kernel (e.g. dstate != 16) */
#define SSM_ERR_WORKSPACE 3   /* workspace missing or smaller than required */
#define SSM_ERR_HIP 4         /* a HIP runtime call or kernel launch failed */

/* Capacity of the device scratch array of ssm_scan_fwd_noalloc (64 MiB, held
 * by every GPU the library runs on until the process ends). */
#define SSM_NOALLOC_SCRATCH_BYTES 67108864

/* Version of this ABI (SSM_ABI_VERSION). */
int ssm_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *ssm_status_str(int status);

/*
 * Execution plan of a scan: `waves_per_group` (2, 4, 8 or 16) wavefronts
 * share one group of 64 channels (with 4, the automatic choice, each wave
 * owns 16 of the channels with all 16 states; otherwise each wave owns
 * 16/waves_per_group state indices of all 64 channels); the sequence is cut
 * into `nchunks` chunks that run in parallel and are stitched by a
 * cross-chunk carry.  The plan changes only the schedule and the rounding
 * order of the readout's sum, never the definition of the result.
 *
 * ssm_scan_plan() fills in the plan ssm_scan_fwd() uses for these sizes and,
 * when `phase` is not NULL, the phase value of the schedule it runs in (3:
 * two-launch, 7: three-pass; see ssm_scan_fwd_phase).  The chunk count and
 * the schedule come from a cost model of the launches on MI355X's 256 CUs
 * (blocks per CU, resident blocks, the pre-pass's cost per step).
 * Returns SSM_ERR_INVALID_ARG for negative sizes or NULL plan outputs.
 */
int ssm_scan_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                  int io_dtype, int *waves_per_group, int *nchunks, int *phase);

/*
 * Device workspace, in bytes, that ssm_scan_fwd_planned() needs for a scan
 * cut into `nchunks` chunks (nchunks <= 0: the automatic plan's count, i.e.
 * what ssm_scan_fwd() needs).  It holds the per-chunk carry state.
 * Returns -1 for invalid sizes.  A result of 0 means no workspace is needed.
 */
int64_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim,
                                 int64_t dstate, int io_dtype, int nchunks);

/*
 * Selective scan over a whole sequence (forward).
 *   x, delta, z, y : [batch, seqlen, dim]  io_dtype.  delta is the step size
 *                    after any softplus, i.e. used as given.
 *   A              : [dim, dstate] fp32 (real diagonal; A == 0 uses the limit
 *                    Bbar = delta * B).
 *   B, C           : [batch, seqlen, dstate] io_dtype, shared by all channels.
 *   Dskip          : [dim] fp32, NULL => D = 0.
 *   z              : NULL => no gate (y = C.h + D x).
 *   h0             : [batch, dim, dstate] fp32 initial state, NULL => zeros.
 *   y              : output.  h_last: [batch, dim, dstate] fp32 final state,
 *                    NULL => not written.
 *   workspace      : device buffer of at least ssm_scan_workspace_bytes(...)
 *                    bytes (may be NULL when that is 0).
 * dstate: 16 runs the chunked kernels (plan of ssm_scan_fwd_planned); 32,
 * 64 and 128 (the larger states of the paperlens tutorial's d_state setting
 * and of Mamba-3, ihouse article "推論効率") run one pass per sequence with
 * more waves per channel group: their workspace size is 0, waves_per_group
 * and nchunks are ignored, ssm_scan_fwd_phase accepts only phase 3 (or 7) and the
 * fused prologue is not available (SSM_ERR_UNSUPPORTED).  Other dstate:
 * SSM_ERR_UNSUPPORTED.
 * Outputs must not alias inputs (exact pointer equality is rejected).
 * seqlen == 0 writes h_last (= h0, or zeros) when given and nothing else;
 * batch == 0 or dim == 0 is a no-op.  More than 65535 batch rows run as
 * consecutive launches of at most 65528 rows on the stream (ssm_scan_fwd_phase
 * then accepts only phase 3 or 7).  Returns an SSM_* status.
 */
int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                 int io_dtype, const void *x, const void *delta, const float *A,
                 const void *B, const void *C, const float *Dskip, const void *z,
                 const float *h0, void *y, float *h_last, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd with an explicit plan (for tests and tuning).  A value <= 0
 * for waves_per_group or nchunks takes the automatic choice for that field.
 * nchunks is clamped to [1, seqlen].  The schedule (two-launch or
 * three-pass, ssm_scan_fwd_phase) is the one the cost model prefers for the
 * resulting chunk count.  Unsupported waves_per_group values return
 * SSM_ERR_UNSUPPORTED.  The workspace must be sized with the same nchunks.
 */
int ssm_scan_fwd_planned(int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int io_dtype, const void *x,
                         const void *delta, const float *A, const void *B,
                         const void *C, const float *Dskip, const void *z,
                         const float *h0, void *y, float *h_last,
                         void *workspace, size_t workspace_bytes,
                         int waves_per_group, int nchunks, void *stream);

/*
 * The launches of a chunked scan, for callers that enqueue them apart (e.g.
 * to time or overlap them).  The update composes associatively over chunks
 * (paperlens tutorial, section "代償と、それを払う方法（並列スキャン）"), so
 * every chunk but the first can start from a state that a cheaper pass has
 * computed.  Two-launch schedule, phase bits:
 *   1 -- chunk 0's main pass (its part of y, and the state entering chunk 1)
 *        in one launch with the pre-pass of chunks 1 .. nchunks-2 (each run
 *        from a zero state, end state recorded), then the composition of
 *        those chunk maps into the state entering every chunk, written to
 *        the workspace;
 *   2 -- the main pass of chunks 1 .. nchunks-1 from their entering states,
 *        writing the rest of y and h_last (reads the workspace phase 1 wrote);
 *   3 -- both, in order.
 * Adding 4 selects the three-pass schedule instead:
 *   5 -- the pre-pass of chunks 0 .. nchunks-2 and the composition (nothing
 *        but the workspace written);  6 -- the main pass of every chunk;
 *   7 -- both.
 * With nchunks == 1 phase bit 1 is a no-op and bit 2 runs the whole scan.
 * Arguments, plan and workspace are those of ssm_scan_fwd_planned and must be
 * identical for the launches of one scan.  Other phase values return
 * SSM_ERR_INVALID_ARG.
 */
int ssm_scan_fwd_phase(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int io_dtype, const void *x, const void *delta,
                       const float *A, const void *B, const void *C,
                       const float *Dskip, const void *z, const float *h0, void *y,
                       float *h_last, void *workspace, size_t workspace_bytes,
                       int waves_per_group, int nchunks, int phase, void *stream);

/*
 * ssm_scan_fwd_planned for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace argument: the chunk-carry workspace
 * (per-chunk end states, entering states and delta sums) lives in a
 * file-scope device array of SSM_NOALLOC_SCRATCH_BYTES bytes, which each GPU
 * holds from the first call on it until the process ends.  The call makes no
 * hipMalloc, hipFree or other allocating call.  The caller still passes
 * inputs and outputs, with the meaning, layout and checks of ssm_scan_fwd.
 * waves_per_group and nchunks: as ssm_scan_fwd_planned (<= 0 = automatic).
 * A plan whose workspace (ssm_scan_workspace_bytes with the same nchunks)
 * exceeds SSM_NOALLOC_SCRATCH_BYTES returns SSM_ERR_WORKSPACE before
 * anything is enqueued (the single L = 262144, D = 4096 sequence, for
 * instance, fits with at most 120 chunks; its automatic plan takes 128); such
 * callers pass a smaller nchunks.  The first call on a device looks up that device's copy of the
 * array (SSM_ERR_HIP if that fails).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; a call writes every scratch value before reading it, so nothing
 * needs clearing, but calls that overlap on one GPU (on different streams, or
 * from several threads) race on the array and must be serialised by the
 * caller.
 */
int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int io_dtype, const void *x,
                         const void *delta, const float *A, const void *B,
                         const void *C, const float *Dskip, const void *z,
                         const float *h0, void *y, float *h_last,
                         int waves_per_group, int nchunks, void *stream);

/*
 * ssm_scan_fwd_planned with two variants of the per-element formula:
 *   a_per_channel = 1 -- A is [dim]: one real value per channel shared by its
 *                        dstate states (the scalar-A structure of Mamba-2:
 *                        ihouse article, "Mambaの進化の道のり"; ultralytics
 *                        glossary, "S4からMambaへ").  0: A is [dim, dstate]
 *                        as in ssm_scan_fwd.
 *   discretization    -- SSM_DISC_ZOH, or SSM_DISC_EULER for Bbar = delta * B
 *                        (paperlens tutorial, pseudo-code of the selection
 *                        section; ihouse article: Mamba-2 used this form).
 *                        Abar = exp(delta * A) in both.
 * The result equals ssm_scan_fwd on A broadcast to [dim, dstate] (ZOH) or on
 * the Euler recurrence.  Other arguments, plan and workspace as in
 * ssm_scan_fwd_planned; waves_per_group 16 returns SSM_ERR_UNSUPPORTED.
 * Other flag values return SSM_ERR_INVALID_ARG.
 */
int ssm_scan_fwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    int io_dtype, const void *x, const void *delta, const float *A,
                    int a_per_channel, int discretization, const void *B, const void *C,
                    const float *Dskip, const void *z, const float *h0, void *y,
                    float *h_last, void *workspace, size_t workspace_bytes,
                    int waves_per_group, int nchunks, void *stream);

/*
 * Workspace of ssm_scan_bwd in bytes for these sizes (-1 for invalid sizes,
 * 0 when nothing is needed).
 */
int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim,
                                     int64_t dstate, int io_dtype);

/*
 * Backward of the selective scan: the gradients of a loss with respect to
 * every input of ssm_scan_fwd_ex, given dy = dL/dy and dh_last = dL/dh_last.
 * The states are recomputed from the inputs, not read from the forward pass
 * (paperlens tutorial, section on the hardware-aware algorithm: the backward
 * recomputes what the forward kept on chip).  The derivative is the chain
 * rule on the recurrence of ssm_scan_fwd (ultralytics glossary, "SSMの仕組み";
 * paperlens tutorial, eq. (2) and the selection section).
 *   inputs      : as ssm_scan_fwd_ex (a_per_channel, discretization select
 *                 the variant; h0 NULL => zeros).
 *   dy          : [batch, seqlen, dim] io_dtype.
 *   dh_last     : [batch, dim, dstate] fp32, NULL => 0.
 *   dx, ddelta  : [batch, seqlen, dim] io_dtype outputs.
 *   dz          : [batch, seqlen, dim] io_dtype; required when z is given,
 *                 must be NULL when it is not.
 *   dA          : fp32, shape of A ([dim, dstate], or [dim] when
 *                 a_per_channel), summed over batch and time.
 *   dB, dC      : [batch, seqlen, dstate] io_dtype, summed over channels.
 *   dD          : [dim] fp32, NULL => not written (computed with D = 0 when
 *                 Dskip is NULL).
 *   dh0         : [batch, dim, dstate] fp32, NULL => not written.
 *   workspace   : at least ssm_scan_bwd_workspace_bytes(...) bytes.
 * Results are deterministic: every sum runs in a fixed order.  Outputs must
 * not alias inputs, each other or the workspace.  seqlen == 0 writes dA = 0,
 * dD = 0 and dh0 = dh_last (or 0).  dstate 16 runs the backward kernels
 * directly; 32, 64 and 128 run them on each 16-state slice in turn (the
 * states of a channel evolve independently and meet only in sums over n),
 * with the per-(t, d) sums accumulated in fp32 in the workspace.  Other
 * dstate, and more than 65535 batch rows: SSM_ERR_UNSUPPORTED.  Returns an
 * SSM_* status.
 */
int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void *x, const void *delta, const float *A, int a_per_channel,
                 int discretization, const void *B, const void *C, const float *Dskip,
                 const void *z, const float *h0, const void *dy, const float *dh_last,
                 void *dx, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
                 float *dh0, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Selective scan with its prologue fused in: the two steps that come right
 * before the scan in a Mamba block are computed on the way into the kernel
 * instead of in a separate pass over HBM.
 *   x[b,t,d]     = act( sum_k conv_w[d,k] * x_raw[b, t-(d_conv-1)+k, d] + conv_b[d] )
 *                  -- causal depthwise convolution over time, width d_conv
 *                  (paperlens tutorial, section "現場ではこう使う": the short
 *                  1-D convolution in front of the SSM; agenticai-flow guide,
 *                  implementation example: d_conv = 4).  Steps before the
 *                  start of the sequence count as zero; act is SiLU when
 *                  conv_silu == 1 and the identity when 0 (the pages do not
 *                  say which follows the convolution).
 *   delta[b,t,d] = softplus(delta_raw[b,t,d] + delta_bias[d])
 *                  -- paperlens tutorial, section "Mamba: 状態を「選択的」にする".
 * followed by the scan of ssm_scan_fwd on (x, delta).
 *   x_raw, delta_raw : [batch, seqlen, dim] io_dtype.
 *   conv_w           : [dim, d_conv] fp32; conv_w[d, d_conv-1] multiplies the
 *                      current step.  1 <= d_conv <= 4 (larger:
 *                      SSM_ERR_UNSUPPORTED).
 *   conv_b, delta_bias : [dim] fp32, NULL => 0.
 *   Every other argument, the plan (waves_per_group 2, 4 or 8; 16 returns
 *   SSM_ERR_UNSUPPORTED) and the workspace are those of ssm_scan_fwd_planned.
 * D multiplies the convolution output x (the scan's input).  Returns an SSM_*
 * status.
 */
int ssm_scan_fwd_fused(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int io_dtype, const void *x_raw, const float *conv_w,
                       const float *conv_b, int d_conv, int conv_silu,
                       const void *delta_raw, const float *delta_bias, const float *A,
                       const void *B, const void *C, const float *Dskip, const void *z,
                       const float *h0, void *y, float *h_last, void *workspace,
                       size_t workspace_bytes, int waves_per_group, int nchunks,
                       void *stream);

/*
 * One recurrent decode step for one new token per sequence (paperlens
 * tutorial, S4 section and practice notes: constant time and memory per
 * token; ihouse article, decode arithmetic intensity).
 *   h        : [batch, dim, dstate] fp32, read and updated IN PLACE.
 *   x, delta, z, y : [batch, dim] io_dtype.  B, C : [batch, dstate] io_dtype.
 *   A [dim, dstate] fp32; Dskip [dim] fp32 (NULL => 0); z NULL => no gate.
 * dstate 16, 32, 64 or 128 (other: SSM_ERR_UNSUPPORTED).
 * The result equals one step of ssm_scan_fwd with h0 = h.  y must not alias
 * an input.  batch == 0 or dim == 0 is a no-op.  Returns an SSM_* status.
 */
int ssm_decode_step(int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
                    float *h, const void *x, const void *delta, const float *A,
                    const void *B, const void *C, const float *Dskip,
                    const void *z, void *y, void *stream);

/*
 * ssm_decode_step with the variants of ssm_scan_fwd_ex: a_per_channel = 1
 * takes A as [dim] (one value per channel shared by its states; the scalar A
 * of Mamba-2, ihouse article "Mambaの進化の道のり"), discretization
 * SSM_DISC_EULER uses Bbar = delta * B (paperlens tutorial, selection
 * pseudo-code).  The result equals one step of ssm_scan_fwd_ex with the same
 * flags and h0 = h.  For a step shared by a head of channels (as in
 * ssm_ssd_fwd), pass delta and A repeated over the head's channels.  Other
 * arguments and errors as ssm_decode_step; invalid flags return
 * SSM_ERR_INVALID_ARG.
 */
int ssm_decode_step_ex(int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
                       float *h, const void *x, const void *delta, const float *A,
                       int a_per_channel, int discretization, const void *B,
                       const void *C, const float *Dskip, const void *z, void *y,
                       void *stream);

/*
 * Selective scan whose step size and decay rate are shared by each head of
 * `headdim` consecutive channels, computed in the masked-matrix form on the
 * matrix cores (ihouse article, "Mambaの進化の道のり": with A reduced to a
 * scalar, most of the SSM's work is a masked matrix multiplication; paperlens
 * tutorial, "代償と、それを払う方法（並列スキャン）": the recurrence composes
 * chunk by chunk).  Channel d = h * headdim + p of head h uses
 *   delta[b,t,d] = dt[b,t,h]  and  A[d, n] = A[h]  for every state n,
 * and otherwise the recurrence, readout, skip and gate of ssm_scan_fwd:
 *   h_t = exp(dt_t A) h_{t-1} + coef_t x_t B_t,   y_t = (C_t . h_t + D x_t) SiLU(z_t),
 * with coef_t = (exp(dt_t A) - 1) / A (SSM_DISC_ZOH; dt_t at A = 0) or dt_t
 * (SSM_DISC_EULER).  The result equals ssm_scan_fwd_ex with A per channel on
 * dt repeated over each head's channels.
 *   x, z, y : [batch, seqlen, nheads * headdim] bf16.  dt : [batch, seqlen,
 *             nheads] bf16, >= 0 (already through softplus).  B, C : [batch,
 *             seqlen, dstate] bf16, shared by every head.  A : [nheads] fp32.
 *   Dskip   : [nheads * headdim] fp32, NULL => 0.  z NULL => no gate.
 *   h0, h_last : [batch, nheads * headdim, dstate] fp32, NULL => zeros / not
 *             written.
 * Supported: io_dtype SSM_DTYPE_BF16, headdim 64, dstate 64 or 128; other
 * values return SSM_ERR_UNSUPPORTED (the fp32 path of the same arithmetic is
 * ssm_scan_fwd_ex).  Products run on bf16 matrix cores with fp32
 * accumulation; operands that are not bf16 inputs (masked weights, state,
 * weighted inputs) are split into two bf16 parts, so results carry fp32-level
 * accuracy (relative error ~1e-5).
 *   workspace : device memory of at least ssm_ssd_fwd_workspace_bytes(...,
 *               nsplit = 1) bytes, owned by the caller: per 64-step chunk of
 *               each batch row, the lower-triangular tiles of C B^T and B^T
 *               (which every head reads), written before the scan; its
 *               contents on entry do not matter.  NULL or too small (with
 *               seqlen > 0) => SSM_ERR_WORKSPACE.
 * Outputs must not alias inputs (nor each other, nor the workspace); seqlen
 * == 0 sets h_last to h0 (or zeros); batch == 0 or nheads == 0 is a no-op.
 * Returns an SSM_* status.
 */
int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                int64_t dstate, int io_dtype, int discretization, const void *x,
                const void *dt, const float *A, const void *B, const void *C,
                const float *Dskip, const void *z, const float *h0, void *y,
                float *h_last, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * ssm_ssd_fwd with the sequence cut into segments that separate blocks run:
 * a state-only pass gives each segment's end state from a zero state and its
 * decay, a carry composes them in order (the recurrence composes segment by
 * segment: paperlens tutorial, "代償と、それを払う方法（並列スキャン）"), and the main
 * pass starts every segment from its entering state.  This gives a few
 * (batch row, head) pairs, e.g. one long sequence, enough blocks to fill the
 * chip, at the price of the state-only pass over all segments but the last.
 *   nsplit    : number of segments; 0 => automatic (none when there are at
 *               least 640 blocks of (half head, batch row), else about 1280
 *               blocks, no segment shorter than 256 steps); 1 => ssm_ssd_fwd.
 *   workspace : at least ssm_ssd_fwd_workspace_bytes(..., nsplit) bytes: the
 *               per-chunk products of ssm_ssd_fwd plus, with segments, each
 *               segment's end state, entering state and decay.
 * Other arguments, results and errors as ssm_ssd_fwd.
 */
int64_t ssm_ssd_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                    int64_t headdim, int64_t dstate, int nsplit);
int ssm_ssd_fwd_planned(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int io_dtype, int discretization, const void *x,
                        const void *dt, const float *A, const void *B, const void *C,
                        const float *Dskip, const void *z, const float *h0, void *y,
                        float *h_last, int nsplit, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * Workspace of ssm_ssd_bwd in bytes for these sizes (-1 for invalid sizes,
 * 0 when nothing is needed).
 */
int64_t ssm_ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                    int64_t headdim, int64_t dstate, int io_dtype);

/*
 * Backward of ssm_ssd_fwd (step and decay shared per head): the gradients of
 * a loss with respect to every input, given dy and dh_last -- the chain rule
 * through the recurrence the forward computes (a parameter shared by a
 * head's channels gets the sum of their gradients).  Two implementations,
 * chosen by shape:
 *   - bf16 I/O, headdim 64, dstate 64 or 128, at most 65535 32-step chunks:
 *     the masked-matrix form on the matrix cores, every 32-step chunk
 *     independent (ihouse article on Mamba-3, section on Mamba's evolution:
 *     the scalar-decay SSM as masked matrix products).  One launch runs two
 *     walks over the chunks per (half head, batch row): forward from h0,
 *     storing the state entering every chunk, and backward from dh_last,
 *     storing the adjoint leaving every chunk (what reaches the start is
 *     dh0).  Then one kernel per (group of 16 heads, chunk, batch row) forms
 *     all gradients of the chunk from them, and small passes sum dB, dC over
 *     the head groups and dA, dD over (batch row, chunk);
 *     the gradient of each step's log-decay is assembled inside its chunk
 *     from the chunk's masked matrices and its two boundary states (no
 *     prefix over the sequence).  Workspace: two fp32 states per chunk,
 *     2 * batch * ceil(seqlen / 32) * nheads * 64 * dstate * 4 bytes, plus
 *     about batch * seqlen * dstate * 8 * ceil(nheads / 16) bytes of partial
 *     sums (2.79 GB at batch 4, L 4096, 80 heads, 128 states).
 *   - otherwise: ssm_scan_bwd's recurrence kernels on the per-channel
 *     problem the per-head one stands for (dt and A repeated over each
 *     head's channels), the per-channel gradients of dt and A summed over
 *     each head's channels in fp32 in a fixed order.
 *   inputs      : as ssm_ssd_fwd (dt [batch, seqlen, nheads], A [nheads]).
 *   dy          : [batch, seqlen, nheads * headdim] io_dtype; dh_last as
 *                 h_last, NULL => 0.
 *   dx, dz      : [batch, seqlen, nheads * headdim] io_dtype (dz required
 *                 when z is given, NULL otherwise).
 *   ddt         : [batch, seqlen, nheads] io_dtype.  dA : [nheads] fp32.
 *   dB, dC      : [batch, seqlen, dstate] io_dtype.  dD : [nheads * headdim]
 *                 fp32, NULL => not written.  dh0 : as h0, NULL => not written.
 *   workspace   : at least ssm_ssd_bwd_workspace_bytes(...) bytes.
 * io_dtype fp32 or bf16, any headdim, dstate 16, 32, 64 or 128 (other:
 * SSM_ERR_UNSUPPORTED).  Batches of more than 65535 rows, and more than 65535
 * chunks of the per-channel path, return SSM_ERR_UNSUPPORTED (the forward
 * splits such batches into launches; the backward does not).  Deterministic.
 * Outputs must not alias inputs, each other or the workspace.  Returns an
 * SSM_* status.
 */
int ssm_ssd_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                int64_t dstate, int io_dtype, int discretization, const void *x,
                const void *dt, const float *A, const void *B, const void *C,
                const float *Dskip, const void *z, const float *h0, const void *dy,
                const float *dh_last, void *dx, void *ddt, float *dA, void *dB, void *dC,
                float *dD, void *dz, float *dh0, void *workspace, size_t workspace_bytes,
                void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_H_ */
