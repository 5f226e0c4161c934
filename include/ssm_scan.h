/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan (S6) library, libssm_scan.so.
 *
 * What is computed.  For every batch row b, channel d and state index n:
 *
 *     Delta_t = softplus(delta_t + dt_bias_d)
 *     Abar_t  = exp(Delta_t * A_dn)                     zero-order hold of a diagonal A
 *     h_t     = Abar_t * h_{t-1} + Delta_t * B_tn * x_t  first-order input term Bbar = Delta * B
 *     y_t     = sum_n C_tn * h_tn + Dskip_d * x_t        readout of the updated state
 *     out_t   = y_t * silu(z_t)                          (out_t = y_t when z is NULL)
 *
 * The recurrence and readout are the selective state-space layer of the pages
 * "Mamba" (sections "Main Claim", "Scan View"), "Mamba Selective State-Space
 * Module" ("Math Or Compute Schema") and "DL0170 Mamba Selective SSM vs
 * Attention" ("Mathematical Formulation": zero-order hold of a negative
 * diagonal A, simplified input term, Delta as an input-dependent forget gate).
 * The pages leave the step-size map, the skip term and the gate function
 * open; softplus(delta + dt_bias), Dskip * x and silu are the readings this
 * library implements.
 *
 * Layout.  All tensors are dense, row-major, with no strides:
 *     x, delta, z, y : (batch, L, D), D fastest              io dtype
 *     B, C           : (batch, L, N), shared by all channels io dtype
 *     A              : (D, N)                                 float32
 *     Dskip, dt_bias : (D)                                    float32
 *     h0, h_last, h  : (batch, D, N), N fastest               float32
 * N must be 16.  io dtype is SSM_F32 (float) or SSM_BF16 (bfloat16 bit
 * patterns, 16 bits each); bf16 outputs are rounded to nearest even.
 *
 * Memory and execution.  Every pointer is a DEVICE pointer on the current HIP
 * device.  The caller owns every buffer, including the workspace; the
 * library allocates no device memory and keeps no pointer after a call
 * returns.  Calls only enqueue kernels on `stream` (a hipStream_t; NULL is the
 * null stream) and never synchronise; buffers must stay alive until the
 * stream has run them.
 *
 * Errors.  Every entry point validates all of its arguments before it enqueues
 * anything; on error nothing is enqueued, no output is touched, the return
 * value is a negative ssm_status and ssm_last_error() describes it.  A failed
 * kernel launch returns SSM_ERR_HIP.  Non-finite inputs are not errors: they
 * propagate through the arithmetic.  A positive A is accepted and may
 * overflow (the pages' A is negative).
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 2

typedef enum {
    SSM_F32 = 0,   /* float32 */
    SSM_BF16 = 1   /* bfloat16 bit patterns */
} ssm_dtype;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = -1,       /* a required pointer is NULL */
    SSM_ERR_SHAPE = -2,      /* batch, L or D < 1, a size overflows, or a bad chunk length */
    SSM_ERR_N = -3,          /* N != 16 */
    SSM_ERR_DTYPE = -4,      /* unknown io dtype */
    SSM_ERR_ALIGN = -5,      /* a pointer is not aligned as required below */
    SSM_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than the query returns */
    SSM_ERR_ALIAS = -7,      /* an output overlaps an input or another output, or the workspace overlaps any argument */
    SSM_ERR_HIP = -8         /* a HIP call or kernel launch failed */
} ssm_status;

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

/* Text of the last error on the calling thread ("" if none).  Valid until the
 * next ssm_* call on the same thread. */
const char* ssm_last_error(void);

/*
 * Workspace bytes that ssm_scan_fwd needs for this shape (0 when the sequence
 * is processed in one chunk).  chunk_len as for ssm_scan_fwd.  Returns a
 * negative ssm_status for an invalid shape.  Host-only; touches no device.
 */
int64_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N,
                                     int io_dtype, int64_t chunk_len);

/*
 * Chunk plan used for this shape: writes the chunk length and chunk count
 * (either pointer may be NULL).  Host-only.  Returns SSM_OK or a negative
 * ssm_status.
 */
int ssm_scan_fwd_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                      int64_t chunk_len, int64_t* chunk_len_out, int64_t* n_chunks_out);

/*
 * Whole-sequence selective scan: out (into y) and the final state h_L.
 *
 * The sequence is cut into chunks of chunk_len tokens ("Mamba", "Scan View":
 * the recurrence is associative, so chunks can be scanned in parallel and
 * joined).  Each chunk first runs a local scan from a zero state to get its
 * carry (summed step size, end state); the carries are then folded in order
 * from h0 with (S1, H1) then (S2, H2) = (S1 + S2, exp(A * S2) * H1 + H2); a
 * final pass rescans every chunk from its true starting state and writes y.
 * The (batch, L, D, N) states never reach memory.
 *
 *   x, delta, B, C  required; z NULL = ungated; h0 NULL = zero initial state.
 *   A, Dskip, dt_bias required.
 *   y               required output, (batch, L, D) io dtype.
 *   h_last          NULL = not wanted, else (batch, D, N) float32 output.
 *   chunk_len       0 = the library's plan for the MI355X; else a positive
 *                   multiple of 32 (a smaller, ragged last chunk is allowed)
 *                   of at most (2^31 - 1) / (4 D) tokens, so that a chunk's
 *                   rows stay within 32-bit byte offsets (SSM_ERR_SHAPE
 *                   otherwise; the library's plan respects the same cap).
 *   workspace       at least ssm_scan_fwd_workspace_bytes(...) bytes, 16-byte
 *                   aligned; may be NULL when that size is 0.
 * Alignment: io tensors to their element size; B and C to 16 bytes; float32
 * tensors to 4 bytes.  y and h_last must not overlap any input, each other or
 * the workspace; the workspace must not overlap any input either (the carry
 * pass writes it while other workgroups still read the inputs).  Any such
 * overlap is SSM_ERR_ALIAS.
 */
int ssm_scan_fwd(const void* x, const void* delta, const void* z,
                 const void* B, const void* C,
                 const float* A, const float* Dskip, const float* dt_bias,
                 const float* h0,
                 void* y, float* h_last,
                 int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                 int64_t chunk_len, void* workspace, int64_t workspace_bytes,
                 void* stream);

/*
 * ssm_scan_fwd for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation while running.
 * The same computation and kernels as ssm_scan_fwd, with no workspace
 * argument: the chunk carries go to a fixed scratch array inside the library
 * (64 MiB, 2^26 bytes, one copy per GPU, held until the process ends), and
 * the call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  The first call on a device looks up that device's address of
 * the array once.
 *
 *   Arguments, layout, alignment and errors as ssm_scan_fwd.
 *   chunk_len       0 = the library's plan among the chunk lengths whose
 *                   carries, batch * (chunks - 1) * D * (N + 1) * 4 bytes,
 *                   fit the scratch (SSM_ERR_WORKSPACE if none does); an
 *                   explicit chunk_len whose carries do not fit is
 *                   SSM_ERR_WORKSPACE.  With the same chunk_len the results are
 *                   bit-identical to ssm_scan_fwd's.
 * Every call on one GPU shares that GPU's scratch: calls that can overlap in
 * time on one GPU (on different streams, or from different threads without
 * ordering between their streams) race and give wrong results.  Order them
 * on one stream.  Nothing in the scratch needs to start at any value; it
 * holds the last call's carries afterwards.
 */
int ssm_scan_fwd_noalloc(const void* x, const void* delta, const void* z,
                         const void* B, const void* C,
                         const float* A, const float* Dskip, const float* dt_bias,
                         const float* h0,
                         void* y, float* h_last,
                         int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                         int64_t chunk_len, void* stream);

/*
 * The scan fed by the block's local convolution, fused: the scan input is
 *
 *     x_t = silu(conv_b_d + sum_{k<K} conv_w_dk * xin_{t-K+1+k})
 *
 * a causal depthwise convolution of width K = conv_k (1..4) along time,
 * then silu, computed inside the scan kernels from xin, so x never goes
 * through memory ("Mamba", "Block Structure": a local convolution adds
 * short-range context before the selective SSM; "Mamba: State Space
 * Models", "What a Mamba Block Contains": a short convolution for local
 * mixing.  The pages give neither the width nor an activation: width <= 4
 * and silu are the readings this library implements).  Everything else is
 * ssm_scan_fwd with x replaced by the convolved input (Dskip multiplies the
 * convolved x as well).
 *
 *   xin             (batch, L, D) io dtype, required.
 *   conv_w          (D, conv_k) float32, tap k weighting xin_{t-K+1+k}; conv_b (D) float32.
 *   conv_init       (batch, conv_k - 1, D) io dtype: the inputs just before the
 *                   sequence (a stream continued), NULL = zeros.
 *   conv_last       (batch, conv_k - 1, D) io dtype output: the last conv_k - 1
 *                   inputs of [conv_init, xin], to pass as conv_init of the
 *                   next segment; NULL = not wanted.
 *   workspace       sized by ssm_scan_fwd_workspace_bytes for the same shape.
 * Errors as ssm_scan_fwd; conv_k outside 1..4 is SSM_ERR_SHAPE.  conv_last
 * must not overlap any input or other output.
 */
int ssm_conv_scan_fwd(const void* xin, const float* conv_w, const float* conv_b, int64_t conv_k,
                      const void* conv_init,
                      const void* delta, const void* z, const void* B, const void* C,
                      const float* A, const float* Dskip, const float* dt_bias,
                      const float* h0,
                      void* y, float* h_last, void* conv_last,
                      int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                      int64_t chunk_len, void* workspace, int64_t workspace_bytes,
                      void* stream);

/*
 * Single-token decode step against a cached float32 state, in place.
 *
 * The recurrence advanced by one token ("Mamba & State-Space Sequence
 * Models", "Core mechanics": inference runs the recurrence one step at a
 * time with a state whose size does not grow): h <- Abar * h + Delta * B * x,
 * then out = (C . h + Dskip * x) * silu(z).
 *
 *   h               (batch, D, N) float32, read and overwritten.
 *   x, delta, z     (batch, D) io dtype; z NULL = ungated.
 *   B, C            (batch, N) io dtype.
 *   y               (batch, D) io dtype output; must not overlap h or any input.
 */
int ssm_state_update(float* h,
                     const void* x, const void* delta, const void* z,
                     const void* B, const void* C,
                     const float* A, const float* Dskip, const float* dt_bias,
                     void* y,
                     int64_t batch, int64_t D, int64_t N, int io_dtype,
                     void* stream);

/*
 * Single-token decode step through the local convolution: the step input is
 * silu(conv_b + conv_w . [conv_state, xin]) as in ssm_conv_scan_fwd, then
 * ssm_state_update's step.  conv_state (batch, conv_k - 1, D) io dtype holds
 * the last conv_k - 1 inputs and is shifted in place (oldest row dropped,
 * xin appended); NULL allowed only for conv_k = 1.  Serving a stream: start
 * from the conv_last and h_last of ssm_conv_scan_fwd over the prompt.  h,
 * y and conv_state must not overlap each other or any input.
 */
int ssm_conv_state_update(float* h, void* conv_state,
                          const void* xin, const float* conv_w, const float* conv_b, int64_t conv_k,
                          const void* delta, const void* z,
                          const void* B, const void* C,
                          const float* A, const float* Dskip, const float* dt_bias,
                          void* y,
                          int64_t batch, int64_t D, int64_t N, int io_dtype,
                          void* stream);

/*
 * Workspace bytes and chunk plan of ssm_scan_bwd for this shape (the
 * backward always needs a workspace).  chunk_len as for ssm_scan_bwd.
 * Host-only; negative ssm_status for an invalid shape.
 */
int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N,
                                     int io_dtype, int64_t chunk_len);
int ssm_scan_bwd_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                      int64_t chunk_len, int64_t* chunk_len_out, int64_t* n_chunks_out);

/*
 * Backward of ssm_scan_fwd: gradients of J = sum(dout * out) + sum(dh_last * h_L)
 * with respect to every input.
 *
 * Training differentiates through the scan, and the pages' kernel recomputes
 * the states for it rather than storing them ("DL0170 Mamba Selective SSM vs
 * Attention", point (3) and the paragraph after Figure 1).  So does this
 * call: it takes the forward's inputs, not its activations.  The adjoint
 * mu_t = dJ/dh_t runs backward in time, mu_t = C_t dy_t + Abar_{t+1} mu_{t+1}
 * with dy_t = dout_t * silu(z_t), and is chunked with the same carry algebra
 * as the forward state; within a chunk the states are recomputed a few tokens
 * at a time from stored sub-chunk starting states.
 *
 *   x, delta, z, B, C, A, Dskip, dt_bias, h0   as passed to ssm_scan_fwd
 *                   (z NULL = ungated, h0 NULL = zero initial state).
 *   dout            (batch, L, D) io dtype, required.
 *   dh_last         (batch, D, N) float32 gradient of h_L; NULL = zero.
 *   dx, ddelta      (batch, L, D) io dtype outputs, required.
 *   dz              (batch, L, D) io dtype output; required when z is given,
 *                   NULL when z is NULL.
 *   dB, dC          (batch, L, N) float32 outputs (summed over channels).
 *   dA              (D, N) float32 output; dDskip, ddt_bias (D) float32
 *                   outputs (summed over batch rows and tokens).  Outputs are
 *                   overwritten, not accumulated into.
 *   dh0             (batch, D, N) float32 output or NULL (not wanted); the
 *                   gradient with respect to the starting state, also when
 *                   h0 is NULL.
 *   chunk_len       0 = the library's plan; else a positive multiple of 32,
 *                   capped as for ssm_scan_fwd.
 *   workspace       at least ssm_scan_bwd_workspace_bytes(...) bytes,
 *                   256-byte aligned, required.
 * Alignment as for ssm_scan_fwd (dout, dx, ddelta, dz like x).  No output may
 * overlap an input, another output or the workspace, and the workspace may
 * not overlap an input (SSM_ERR_ALIAS).  The sums over channels,
 * tokens and batch rows are taken in a fixed order: results are bitwise
 * reproducible for a given shape and chunk_len.
 */
int ssm_scan_bwd(const void* x, const void* delta, const void* z,
                 const void* B, const void* C,
                 const float* A, const float* Dskip, const float* dt_bias,
                 const float* h0,
                 const void* dout, const float* dh_last,
                 void* dx, void* ddelta, void* dz, float* dB, float* dC,
                 float* dA, float* dDskip, float* ddt_bias, float* dh0,
                 int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                 int64_t chunk_len, void* workspace, int64_t workspace_bytes,
                 void* stream);

/*
 * SSD (Mamba-2 style) layer: the selective SSM with a scalar decay per head.
 *
 * "Mamba", "Relation to Mamba-2" writes the layer as a causal matrix mixer
 * and credits Mamba-2 with a faster chunk algorithm for it; "Mamba &
 * State-Space Sequence Models", "Core mechanics" names the duality with a
 * class of linear attention; "DL0170 Mamba Selective SSM vs Attention" has
 * Mamba-2 raise N beyond 16.  The reading implemented: per head h (P = 64
 * channels), Abar_t = exp(Delta_t,h * A_h) times the identity on the P x N
 * state, Delta_t,h = softplus(delta_t,h + dt_bias_h), B_t and C_t shared by
 * all heads,
 *     h_t = Abar_t h_{t-1} + Delta_t,h x_t,h B_t^T,  y_t,h = h_t C_t + Dskip_h x_t,h,
 * out = y * silu(z) when z is given.  Evaluated in chunks of 64 tokens with
 * bf16 matrix-core products (fp32 accumulation, fp32 carried state).
 *
 *   x, z, y   (batch, L, H, 64) bf16, 16-byte aligned; z NULL = ungated.
 *   delta     (batch, L, H) bf16.
 *   B, C      (batch, L, N) bf16, N = 64, 128 or 256, 16-byte aligned.
 *   A, Dskip, dt_bias (H) float32.
 *   h0, h_last (batch, H, 64, N) float32, 16-byte aligned; NULL = zeros / not wanted.
 *   workspace at least ssm_ssd_fwd_workspace_bytes(...) bytes of device
 *             memory, 16-byte aligned, owned by the caller, contents ignored;
 *             it receives C_t . B_i of every chunk (bf16, no head in it), which
 *             all heads of a batch row share, and, when the sequences are cut
 *             into segments (see ssm_ssd_fwd_plan), each segment's fp32 end
 *             state and starting state.  It must not overlap any argument and
 *             must not be used by another call until this one's work on the
 *             stream is done.
 * When batch * H sequences are too few to fill the GPU, each sequence is cut
 * into segments of whole chunks walked in parallel: a first pass leaves each
 * segment's end state from zero and its total decay, an in-order fold turns
 * them into every segment's starting state (the combine of "Mamba", "Scan
 * View", with a scalar decay per head), and the layer then runs per segment.
 * The result is the same function up to rounding order.
 * io_dtype must be SSM_BF16 (SSM_ERR_DTYPE otherwise); N other than 64, 128
 * or 256 is SSM_ERR_N; P other than 64 is SSM_ERR_SHAPE; a missing or small
 * workspace is SSM_ERR_WORKSPACE.
 */
int ssm_ssd_fwd(const void* x, const void* delta, const void* z,
                const void* B, const void* C,
                const float* A, const float* Dskip, const float* dt_bias,
                const float* h0,
                void* y, float* h_last,
                int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype,
                void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes ssm_ssd_fwd needs: batch * ceil(L / 64) * 8192, plus
 * batch * H * (n_segments - 1) * (64 * N + 1) * 4 when the plan below cuts the
 * sequences into n_segments > 1 segments.  Negative ssm_status for an invalid
 * shape.  Host-only; touches no device. */
int64_t ssm_ssd_fwd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype);

/* The segments ssm_ssd_fwd cuts each sequence into (1 = walked whole) and the
 * chunks of 64 tokens per segment (the last segment may be shorter).  Errors
 * as ssm_ssd_fwd_workspace_bytes; NULL outputs are SSM_ERR_NULL.  Host-only. */
int ssm_ssd_fwd_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype,
                     int64_t* n_segments, int64_t* segment_chunks);

/*
 * Per-kernel timing, for measurement tools; not needed to compute anything.
 *
 * The switch is PROCESS-WIDE state (the only mutable state of the library
 * besides each thread's error text and the no-allocation scratch address of
 * each device): while it is on, launches from every thread record events, so
 * turn it on only in a measurement run, not in a library shared with other work.
 * Not for use inside graph capture.
 *
 * ssm_timing_enable(1, kernel) makes every later launch of the named kernel
 * of this library (every kernel when kernel is NULL), on any thread,
 * bracketed by two hipEvents recorded on the launch's own stream;
 * ssm_timing_enable(0, NULL) stops recording.  Each pair spans the kernel plus
 * a few microseconds of dispatch around it, which matters only for kernels of
 * tens of microseconds; recording events between kernels also costs time, so
 * time whole calls with recording off.  Kernel names:
 * "s6_chunk_carry", "s6_carry_scan", "s6_chunk_out", "s6_step", and for the
 * backward "s6_bwd_carries", "s6_carry_scan2", "s6_chunk_bwd",
 * "s6_bwd_reduce", and for the SSD layer "ssd_gram", "ssd_seg_local",
 * "ssd_seg_fold", "ssd_chunked".  Returns SSM_OK.
 *
 * ssm_timing_collect waits for every recorded event, then writes for up to
 * max_kernels distinct kernels their name (static strings owned by the
 * library), launch count and summed duration in milliseconds, clears the
 * record and returns the number of distinct kernels (negative ssm_status on a
 * HIP error).  Any output pointer may be NULL.
 */
int ssm_timing_enable(int on, const char* kernel);
int ssm_timing_collect(int max_kernels, const char** names, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
