/*
 * libmambascan — selective state space hot path for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a device pointer (HBM) owned by the
 * caller unless stated otherwise; sizes are element counts.  Every compute
 * entry point enqueues its kernels on `hip_stream` (NULL = the default
 * stream) and returns without synchronising.  The library never allocates,
 * frees or retains caller memory; scratch space comes only from the caller's
 * `workspace` buffer, sized by the matching *_workspace_size() query.
 *
 * Validation happens on the host before any HIP call: on any error nothing
 * is enqueued and no output is written.  Status codes:
 *   MSS_ERR_NULL        a required pointer is NULL
 *   MSS_ERR_SHAPE       a size is not positive, or too large for 32-bit
 *                       in-kernel indexing of one row/plane
 *   MSS_ERR_DTYPE       unknown dtype code
 *   MSS_ERR_ALIGN       a pointer is not 16-byte aligned
 *   MSS_ERR_UNSUPPORTED a shape the library does not implement (see each call)
 *   MSS_ERR_WORKSPACE   workspace NULL or smaller than the query returned
 *   MSS_ERR_ALIAS       an output buffer overlaps an input buffer
 *   MSS_ERR_HIP         a HIP launch failed (mss_last_hip_error() has the code)
 *   MSS_ERR_WAIT        (mss_workspace_status only) a bounded wait between
 *                       workgroups gave up during the call: its outputs are
 *                       not valid
 *
 * The same inputs, shapes and flags give bitwise-identical outputs: no
 * floating-point atomics are used and reduction orders are fixed.
 *
 * Thread safety: the library holds no mutable global state other than the
 * thread-local last HIP error and, for mss_selective_scan_fwd_noalloc, one
 * fixed scratch buffer per GPU (see there); concurrent calls on different
 * streams with disjoint outputs and workspaces are safe.
 */
#ifndef MAMBASCAN_H_
#define MAMBASCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSS_ABI_VERSION 2

typedef enum {
  MSS_OK = 0,
  MSS_ERR_NULL = 1,
  MSS_ERR_SHAPE = 2,
  MSS_ERR_DTYPE = 3,
  MSS_ERR_ALIGN = 4,
  MSS_ERR_UNSUPPORTED = 5,
  MSS_ERR_WORKSPACE = 6,
  MSS_ERR_ALIAS = 7,
  MSS_ERR_HIP = 8,
  MSS_ERR_WAIT = 9
} mss_status;

/* Storage type of the streamed tensors (u, delta, B, C, z, y; x for SSD).
 * A, D and every state tensor are always fp32.  bf16 inputs are widened
 * exactly to fp32; bf16 outputs are rounded to nearest even. */
typedef enum { MSS_FP32 = 0, MSS_BF16 = 1 } mss_dtype;

/* Force the per-state exp(delta*A[d,n]) decay path of the selective scan.
 * Without this flag the scan checks on the device, per block of 64 channels,
 * whether A[d,n] == A[d,0] holds exactly for every channel in the block (A
 * constant over the states, the Mamba-2 form), else whether
 * A[d,n] == (n+1)*A[d,0] does (the S4D-real structure); where one holds it
 * computes the same decays from r = exp(delta*A[d,0]) alone, as r or as
 * r^(n+1) (equal in exact arithmetic).                                     */
#define MSS_FLAG_DECAY_GENERAL 0x1u

/* ------------------------------------------------------------------------ */
/* Selective scan (Mamba-1 selective SSM layer, forward).                    */
/*                                                                          */
/* Defined by the discretised state-space recurrence: decay                  */
/*   Abar = exp(delta*A)  ("Mamba (deep learning)", state-space paragraph)   */
/* and h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = C_t h_t ("Mamba-1/2/3 visual */
/* guide", blog.yecov.com, section 1 SSM equation), with delta, B, C varying */
/* with t (same blog, section 2 selectivity table) and the output multiplied */
/* by a gate branch (section 2 block diagram).  Per (b, d):                  */
/*   h[n] = h0[b,d,n] (or 0)                                                */
/*   for l in 0..L-1:                                                        */
/*     h[n]  = exp(delta[b,d,l]*A[d,n]) * h[n] + delta[b,d,l]*B[b,n,l]*u[b,d,l] */
/*     out   = sum_n C[b,n,l]*h[n] + D[d]*u[b,d,l]                          */
/*     y[b,d,l] = out * z/(1+exp(-z)),  z = z[b,d,l]   (out if z == NULL)    */
/*   h_last[b,d,:] = h                                                       */
/* The expanded state (b x d x L x N) is never written to memory.            */
/*                                                                          */
/* Layouts (dense, row-major, last index fastest):                           */
/*   u, delta, z, y : [batch, dim, seqlen]     io_dtype                     */
/*   B, C           : [batch, dstate, seqlen]  io_dtype (shared by all d)   */
/*   A              : [dim, dstate] fp32;  D : [dim] fp32 (NULL = no skip)  */
/*   h0, h_last     : [batch, dim, dstate] fp32 (each may be NULL)          */
/* delta is used as given (no softplus or bias inside).                     */
/* Supported: 1 <= dstate <= 128; seqlen < 2^24; dim*seqlen < 2^31;        */
/* batch <= 65535.                                                          */
/* Outputs y and h_last must not overlap any input or each other.           */
/* ------------------------------------------------------------------------ */
mss_status mss_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                                  const void* C, const float* D, const void* z, const float* h0,
                                  void* y, float* h_last, int64_t batch, int64_t dim,
                                  int64_t dstate, int64_t seqlen, mss_dtype io_dtype,
                                  uint32_t flags, void* workspace, size_t workspace_bytes,
                                  void* hip_stream);

/* ------------------------------------------------------------------------ */
/* mss_selective_scan_fwd without a workspace, for callers that cannot       */
/* allocate device memory (code under HIP graph capture, tight serving       */
/* loops, harnesses that forbid allocation).  The same computation, limits   */
/* and errors as mss_selective_scan_fwd; its scratch is instead a fixed      */
/* 64 MiB buffer inside the library, one per GPU, set up on the first call   */
/* on that GPU (the stream's device must be current) and held until the      */
/* process ends.  The call allocates nothing.  Shapes whose                  */
/* mss_selective_scan_workspace_size() exceeds 64 MiB return                 */
/* MSS_ERR_WORKSPACE, with nothing enqueued.  All calls on one GPU share that */
/* buffer: calls that overlap in time on one GPU (different streams, or      */
/* threads) race and give wrong results; calls in one stream are ordered.    */
/* wait_status (nullable, 4-byte aligned device int, must not overlap any    */
/* input or output): set to 0 by the call, to nonzero if a bounded wait      */
/* between workgroups gave up (the outputs are then not valid).              */
/* ------------------------------------------------------------------------ */
mss_status mss_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A,
                                          const void* B, const void* C, const float* D,
                                          const void* z, const float* h0, void* y, float* h_last,
                                          int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                          mss_dtype io_dtype, uint32_t flags, int* wait_status,
                                          void* hip_stream);

/* Bytes of device workspace mss_selective_scan_fwd needs for this shape
 * (0 when the shape is unsupported).  The workspace need not be zeroed. */
size_t mss_selective_scan_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                         int64_t seqlen, mss_dtype io_dtype, uint32_t flags);

/* Flags of mss_selective_scan_fwd_fused (with MSS_FLAG_DECAY_GENERAL).     */
#define MSS_FLAG_CONV_SILU 0x2u      /* u = silu(convolution) instead of u = convolution */
#define MSS_FLAG_DELTA_SOFTPLUS 0x4u /* delta = softplus(delta_raw + bias) instead of delta_raw + bias */

/* ------------------------------------------------------------------------ */
/* Selective scan fed by its prologue, in one pass.                          */
/*                                                                          */
/* The block around the layer has an input projection, a short convolution, */
/* the selective state space layer and a gate ("Mamba (deep learning)",      */
/* paragraph on the block); the convolution's kernel size is 4 ("Mamba       */
/* State-Space Models", usage example, d_conv).  This entry point computes   */
/* the layer's u from the convolution and delta from its raw value inside    */
/* the scan, so neither is written to or read from memory:                   */
/*   c[b,d,l] = conv_b[d] + sum_{k=0..3} conv_w[d,k] * x[b,d,l-3+k]          */
/*              (x = 0 before the first step: causal, one filter per channel) */
/*   u[b,d,l] = c  (or silu(c) = c/(1+exp(-c)) with MSS_FLAG_CONV_SILU)      */
/*   v        = delta_raw[b,d,l] + delta_bias[d]                             */
/*   delta[b,d,l] = v  (or softplus(v) = log(1+exp(v)) with                  */
/*              MSS_FLAG_DELTA_SOFTPLUS)                                     */
/* then exactly mss_selective_scan_fwd(u, delta, A, B, C, D, z, h0, ...).    */
/* The pages name the convolution but not its activation, nor any transform */
/* of delta: both are options (softplus is the form of the workload's       */
/* delta).                                                                   */
/*                                                                          */
/* Layouts: x, delta_raw : [batch, dim, seqlen] io_dtype;  conv_w : [dim, 4] */
/*   fp32 (tap 3 multiplies the current step);  conv_b, delta_bias : [dim]   */
/*   fp32 (each may be NULL = 0);  everything else as in                      */
/*   mss_selective_scan_fwd.  Limits, workspace (the size                    */
/*   mss_selective_scan_workspace_size returns), stream and errors as there; */
/*   y and h_last must not overlap any input or each other.                  */
/* ------------------------------------------------------------------------ */
mss_status mss_selective_scan_fwd_fused(const void* x, const float* conv_w, const float* conv_b,
                                        const void* delta_raw, const float* delta_bias, const float* A,
                                        const void* B, const void* C, const float* D, const void* z,
                                        const float* h0, void* y, float* h_last, int64_t batch,
                                        int64_t dim, int64_t dstate, int64_t seqlen, mss_dtype io_dtype,
                                        uint32_t flags, void* workspace, size_t workspace_bytes,
                                        void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Selective scan, backward (training).                                      */
/*                                                                          */
/* The gradient of a scalar loss through mss_selective_scan_fwd, given       */
/* dy = dloss/dy and optionally dh_last = dloss/dh_last.  Training runs the  */
/* layer over whole sequences ("Mamba (deep learning)", paragraph on how the */
/* model trains and generates; "Mamba-1/2/3 visual guide", section 2 figure: */
/* training and prefill use the parallel scan); the gradient is the chain    */
/* rule through the forward recurrence in reverse time.  Per (b, d), with dh */
/* the gradient of the state after step t and a = exp(delta*A):             */
/*   dout = dy*silu(z), dz = dy*out*silu'(z)   (out = C.h + D*u)            */
/*   dh += C*dout;  dC += dout*h;  dA += dh*h_prev*a*delta                   */
/*   ddelta = sum_n dh*(h_prev*a*A + B*u);  du = sum_n dh*delta*B + D*dout   */
/*   dB += dh*delta*u;  dh *= a   (then the previous step); dh0 = final dh   */
/* dB and dC are summed over the channels, dA over batch and time, dD over   */
/* batch and time.  The states are recomputed (a forward pass writes the     */
/* state entering every 16-step tile into the workspace), not taken from the */
/* caller.                                                                   */
/*                                                                          */
/* Inputs: as mss_selective_scan_fwd (u, delta, A, B, C, D, z, h0 with the   */
/* same layouts and dtypes), dy [batch, dim, seqlen] io_dtype, dh_last       */
/* [batch, dim, dstate] fp32 (NULL = zero).                                  */
/* Outputs (written, not accumulated): du, ddelta [batch, dim, seqlen] and   */
/* dB, dC [batch, dstate, seqlen] in io_dtype; dA [dim, dstate] fp32;        */
/* dD [dim] fp32 (NULL = not computed; with D NULL it is the gradient at     */
/* D = 0); dz [batch, dim, seqlen] io_dtype, given exactly when z is (else    */
/* MSS_ERR_NULL); dh0 [batch, dim, dstate] fp32 (NULL = not computed; the     */
/* gradient of the initial state, h0 or zero).                              */
/* Supported: 1 <= dstate <= 128 (else MSS_ERR_UNSUPPORTED) and the scan's   */
/* other limits (else MSS_ERR_SHAPE).  Above 32 states the gradient is taken */
/* by slices of 32 states (each state's recurrence is independent; du,       */
/* ddelta and dz are sums over the slices, the skip term taken once), in     */
/* fp32, rounded to io_dtype once at the end; the workspace then also holds */
/* fp32 copies of the [batch, dim, seqlen] tensors.  flags: 0 or             */
/* MSS_FLAG_DECAY_GENERAL (as in the forward).  Outputs must not overlap any  */
/* input or each other.  The workspace (size from                            */
/* mss_selective_scan_bwd_workspace_size) need not be zeroed.                */
/* ------------------------------------------------------------------------ */
mss_status mss_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                                  const void* C, const float* D, const void* z, const float* h0,
                                  const void* dy, const float* dh_last, void* du, void* ddelta,
                                  float* dA, void* dB, void* dC, float* dD, void* dz, float* dh0,
                                  int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                  mss_dtype io_dtype, uint32_t flags, void* workspace,
                                  size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace mss_selective_scan_bwd needs (0 when the shape  */
/* is unsupported).                                                          */
size_t mss_selective_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                             int64_t seqlen, mss_dtype io_dtype, uint32_t flags);

/* ------------------------------------------------------------------------ */
/* Backward of the scan fed by its prologue (mss_selective_scan_fwd_fused). */
/*                                                                          */
/* The gradient of a scalar loss through the fused forward exactly as      */
/* defined there ("Mamba (deep learning)", paragraph on the block: the      */
/* convolution in front of the SSM; "Mamba State-Space Models", usage       */
/* example, kernel size 4): the scan's gradient (as mss_selective_scan_bwd) */
/* at u and delta formed in fp32 from x and delta_raw, taken back through   */
/* the prologue.  With c = conv_b + sum_k conv_w[d,k] x[t-3+k] and          */
/* v = delta_raw + delta_bias:                                              */
/*   dc = du * silu'(c) (MSS_FLAG_CONV_SILU; else du),                       */
/*   ddelta_raw = ddelta * sigmoid(v) (MSS_FLAG_DELTA_SOFTPLUS; else ddelta),*/
/*   dx[s] = sum_k conv_w[d,k] dc[s+3-k],  dconv_w[d,k] = sum dc[t] x[t-3+k],*/
/*   dconv_b = sum dc,  ddelta_bias = sum ddelta_raw (sums over batch, time).*/
/* Inputs: as mss_selective_scan_fwd_fused, plus dy [batch, dim, seqlen]    */
/* io_dtype and dh_last [batch, dim, dstate] fp32 (NULL = zero).            */
/* Outputs (written): dx, ddelta_raw [batch, dim, seqlen] io_dtype;         */
/* dconv_w [dim, 4] fp32; dconv_b, ddelta_bias [dim] fp32 (NULL = not       */
/* computed); dA, dB, dC, dD, dz, dh0 as mss_selective_scan_bwd.  Internally */
/* fp32 throughout (the workspace holds fp32 copies of the [batch, dim,      */
/* seqlen] and [batch, dstate, seqlen] tensors); gradients in io_dtype are  */
/* rounded once.  Supported shapes as mss_selective_scan_bwd; flags: any of */
/* MSS_FLAG_DECAY_GENERAL, MSS_FLAG_CONV_SILU, MSS_FLAG_DELTA_SOFTPLUS (the */
/* forward's).  Outputs must not overlap any input or each other; the       */
/* workspace (size from mss_selective_scan_fused_bwd_workspace_size) need    */
/* not be zeroed; its first word is the call's status word.                 */
/* ------------------------------------------------------------------------ */
mss_status mss_selective_scan_fused_bwd(const void* x, const float* conv_w, const float* conv_b,
                                        const void* delta_raw, const float* delta_bias, const float* A,
                                        const void* B, const void* C, const float* D, const void* z,
                                        const float* h0, const void* dy, const float* dh_last, void* dx,
                                        void* ddelta_raw, float* dconv_w, float* dconv_b, float* ddelta_bias,
                                        float* dA, void* dB, void* dC, float* dD, void* dz, float* dh0,
                                        int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                        mss_dtype io_dtype, uint32_t flags, void* workspace,
                                        size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace mss_selective_scan_fused_bwd needs (0 when the */
/* shape is unsupported).                                                    */
size_t mss_selective_scan_fused_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                                   int64_t seqlen, mss_dtype io_dtype, uint32_t flags);

/* ------------------------------------------------------------------------ */
/* Single-token state update (generation step).                             */
/*                                                                          */
/* One step of the same recurrence, with the state carried between calls     */
/* ("Mamba-1/2/3 visual guide", section 2 figure: prefill uses the parallel */
/* scan, one-token generation the recurrent update of the same model;       */
/* section 1: generation carries only the fixed-size state).  Per (b, d):    */
/*   h[b,d,n] = exp(delta[b,d]*A[d,n]) * h[b,d,n] + delta[b,d]*B[b,n]*u[b,d] */
/*   y[b,d]   = (sum_n C[b,n]*h[b,d,n] + D[d]*u[b,d]) * silu(z[b,d])         */
/* h is read and written in place.                                           */
/*                                                                          */
/* Layouts: h [batch, dim, dstate] fp32;  u, delta, z, y [batch, dim];       */
/*          B, C [batch, dstate];  A [dim, dstate] fp32;  D [dim] fp32.      */
/* D and z may be NULL.  Supported: 1 <= dstate <= 128 (else                */
/* MSS_ERR_UNSUPPORTED) and batch*dim <= 2^28 (else MSS_ERR_SHAPE).  `flags` */
/* must be 0.  y must not overlap h or any input; h must not overlap any     */
/* input.                                                                    */
/* ------------------------------------------------------------------------ */
mss_status mss_state_update(float* h, const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z, void* y,
                            int64_t batch, int64_t dim, int64_t dstate, mss_dtype io_dtype,
                            uint32_t flags, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Mamba-3 state update (one generation step).                               */
/*                                                                          */
/* "Mamba-1/2/3 visual guide", section 4, gives Mamba-3's recurrence three   */
/* changes over Mamba-2's: an exponential-trapezoidal discretisation (the   */
/* step's input taken at both its ends, with an exponential transition), a  */
/* complex state that decays while it rotates, and MIMO (several inputs and */
/* outputs per state update as a small matrix product, raising the work per */
/* byte of the state that decode streams).  The page gives no formulas; the */
/* readings implemented (each an option):                                    */
/*   alpha = exp(delta A_h), times e^{i delta theta[h,n]} with               */
/*           MSS_FLAG_COMPLEX_STATE (the rotation angle grows with delta);   */
/*   u = sum_r x[b,h,r,p] B[b,g,r,n],  u' likewise from x_prev and B_prev    */
/*   h[p,n] <- alpha h[p,n] + (delta/2)(alpha u' + u)  (x_prev, B_prev given: */
/*           the trapezoid rule on the step's input integral)                */
/*   h[p,n] <- alpha h[p,n] + delta u                  (otherwise)           */
/*   y[b,h,r,p] = (sum_n C[b,g,r,n] Re h[p,n] + D_h x[b,h,r,p]) * silu(z)    */
/* per batch b, head h (group g = h / (nheads/ngroups)), state row p and     */
/* state n; R = rank inputs and outputs per head (R = 1: the SISO update of  */
/* the Mamba-2 head).  For a sequence of steps, x_prev and B_prev are the    */
/* previous step's x and B (zero before the first step).                     */
/*                                                                          */
/* Layouts: h [batch, nheads, headdim, dstate] fp32, in place, or with       */
/*   MSS_FLAG_COMPLEX_STATE [batch, nheads, headdim, dstate, 2] (re, im);    */
/*   x, x_prev, z, y [batch, nheads, rank, headdim] io_dtype;                */
/*   B, B_prev, C [batch, ngroups, rank, dstate] io_dtype; delta [batch,     */
/*   nheads] fp32; A, D [nheads] fp32; theta [nheads, dstate] fp32.          */
/* x_prev and B_prev are both given or both NULL; theta is required with    */
/* MSS_FLAG_COMPLEX_STATE (else ignored); D and z may be NULL.               */
/* Supported: headdim a multiple of 16 up to 4096, dstate 64, 128 or 256,    */
/* rank 1..8, nheads % ngroups == 0 (else MSS_ERR_UNSUPPORTED); batch and    */
/* nheads at most 65535 and batch*nheads*headdim at most 2^28 (else          */
/* MSS_ERR_SHAPE).  h, delta, A, theta and D 16-byte aligned.  y and h must  */
/* not overlap any input or each other.                                      */
/* ------------------------------------------------------------------------ */
#define MSS_FLAG_COMPLEX_STATE 0x10u
mss_status mss_mamba3_state_update(float* h, const void* x, const void* x_prev, const float* delta,
                                   const float* A, const float* theta, const void* B,
                                   const void* B_prev, const void* C, const float* D, const void* z,
                                   void* y, int64_t batch, int64_t nheads, int64_t headdim,
                                   int64_t ngroups, int64_t dstate, int64_t rank, mss_dtype io_dtype,
                                   uint32_t flags, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Mamba-2 SSD layer, chunked.                                               */
/*                                                                          */
/* The same recurrence with A restricted to a scalar per head ("Mamba-1/2/3 */
/* visual guide", section 3 comparison table: scalar times identity within a */
/* head), heads of one group sharing B and C.  Per (b, head h, group g):     */
/*   S[p,n] = h0[b,h,p,n] (or 0)                                            */
/*   for t: S = exp(delta[b,t,h]*A[h]) * S + delta[b,t,h]*x[b,t,h,:] B[b,t,g,:]^T */
/*          y[b,t,h,p] = (sum_n C[b,t,g,n]*S[p,n] + D[h]*x[b,t,h,p]) * silu(z) */
/* computed chunk by chunk (section 3 figures: dense products inside a       */
/* chunk, the state passed between chunks):                                  */
/*   inside a chunk  Y_diag = (Lmask o C B^T)(delta x) on the matrix cores,  */
/*   Y_off = diag(exp(s)) C S_prev^T,  S_next = exp(s_last) S_prev + local.  */
/*                                                                          */
/* Layouts: x, z [batch, seqlen, nheads, headdim] in_dtype;                  */
/*          delta [batch, seqlen, nheads] fp32;  A, D [nheads] fp32;         */
/*          B, C [batch, seqlen, ngroups, dstate] in_dtype;                  */
/*          y [batch, seqlen, nheads, headdim] fp32;                          */
/*          h0, h_last [batch, nheads, headdim, dstate] fp32;                */
/*          chunk_states [batch, nchunks, nheads, headdim, dstate] fp32, the */
/*          state after the last step of each chunk, nchunks = ceil(L/chunk). */
/* D, z, h0, chunk_states and h_last may be NULL.                           */
/* Supported: in_dtype MSS_BF16; headdim 64 or 128; dstate a multiple of 16 */
/* up to 256; chunk 64, 128 or 256; nheads % ngroups == 0 (else            */
/* MSS_ERR_UNSUPPORTED); seqlen*nheads*headdim below 2^30 - 64,             */
/* seqlen*ngroups*dstate below 2^30 and ceil(seqlen/chunk) * nheads *       */
/* (headdim/64) * batch below 2^22 (else MSS_ERR_SHAPE).  seqlen need not   */
/* be a multiple of chunk.                                                  */
/* `flags` must be 0.  Outputs must not overlap inputs or each other.        */
/* Tuning: the environment variable MSS_SSD_CHUNKS_PER_PIECE, when it holds */
/* a positive count, sets how many chunks one piece of the sequence takes   */
/* (else chosen from the sizes; at most 64 pieces either way).  The         */
/* workspace query and the call read it; a value that needs more workspace  */
/* than was queried gives MSS_ERR_WORKSPACE.  mss_ssd_chunk_bwd's forward  */
/* pass (chunk 64) reads it too.                                            */
/* ------------------------------------------------------------------------ */
mss_status mss_ssd_chunk_fwd(const void* x, const float* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const float* h0,
                             float* y, float* chunk_states, float* h_last, int64_t batch,
                             int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                             int64_t dstate, int64_t chunk, mss_dtype in_dtype, uint32_t flags,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace mss_ssd_chunk_fwd needs (0 when unsupported). */
size_t mss_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t ngroups, int64_t dstate, int64_t chunk, mss_dtype in_dtype);

/* ------------------------------------------------------------------------ */
/* Mamba-2 SSD layer, backward (training).                                   */
/*                                                                          */
/* The gradient of a scalar loss through mss_ssd_chunk_fwd, given dy =       */
/* dloss/dy and optionally dh_last = dloss/dh_last.  Training runs the SSD   */
/* over whole sequences with the chunked algorithm ("Mamba-1/2/3 visual      */
/* guide", section 3 comparison table, training row); the gradient is the    */
/* chain rule through the forward recurrence in reverse time.  Per (b, h),   */
/* with dout = dy*silu(z) (dy without z), G the gradient of the state after  */
/* step t (G = dout_t C_t^T + exp(delta_{t+1} A) G_{t+1}, G after the last   */
/* step = dout C^T + dh_last) and S the state:                               */
/*   dx_t = delta_t G B_t + D dout_t;   dz_t = dy_t y_t silu'(z_t)           */
/*          (y_t = C_t S_t + D x_t, the output before the gate)              */
/*   ddelta_t = x_t^T G B_t + A <G, exp(delta_t A) S_{t-1}>                  */
/*   dB_t, dC_t = sums over the heads of the group of delta_t G^T x_t and    */
/*          S_t^T dout_t;  dA, dD = sums over batch and time of              */
/*          delta_t <G, exp(delta_t A) S_{t-1}> and dout_t . x_t;            */
/*   dh0 = exp(delta_0 A) G_0.                                               */
/* The states are recomputed (a forward pass with 64-step chunks keeps the   */
/* state after every 64 steps in the workspace), not taken from the caller. */
/* Sums run in a fixed order: the results are bitwise repeatable.           */
/*                                                                          */
/* Inputs: as mss_ssd_chunk_fwd (x, delta, A, B, C, D, z, h0; same layouts  */
/* and dtypes), dy [batch, seqlen, nheads, headdim] fp32 (the forward's y    */
/* dtype), dh_last [batch, nheads, headdim, dstate] fp32 (NULL = zero).      */
/* Outputs (fp32, written, not accumulated): dx, dz [batch, seqlen, nheads,  */
/* headdim]; ddelta [batch, seqlen, nheads]; dA [nheads]; dB, dC [batch,     */
/* seqlen, ngroups, dstate]; dD [nheads] (NULL = not computed; with D NULL   */
/* it is the gradient at D = 0); dz given exactly when z is (else            */
/* MSS_ERR_NULL); dh0 [batch, nheads, headdim, dstate] (NULL = not computed; */
/* the gradient of h0, or of a zero initial state).                          */
/* Supported: in_dtype MSS_BF16; headdim 64 or 128; dstate a multiple of 16 */
/* up to 256; nheads % ngroups == 0 (else MSS_ERR_UNSUPPORTED); the         */
/* forward's size limits with chunk 64 (else MSS_ERR_SHAPE).  Above 128     */
/* states the gradient is taken by two halves of the states (each state     */
/* column evolves on its own; dx, ddelta, dA and dz are sums over the       */
/* halves, the skip term taken once); the workspace then also holds the     */
/* halves' B/C and state columns and the second half's sums.  `flags` must  */
/* be 0.  Outputs must not overlap any input or each other.  The workspace  */
/* (size from mss_ssd_bwd_workspace_size) need not be zeroed.               */
/* Tuning: the environment variable MSS_SSD_BWD_HEADS_PER_WG, when it holds */
/* a divisor of a group's nheads/ngroups * headdim/64 64-row head slices,   */
/* sets how many of them one gradient workgroup takes, and                  */
/* MSS_SSD_BWD_BLOCKS_PER_PIECE (a positive count) how many 64-step blocks  */
/* one piece of the adjoint passes takes (else both are chosen from the     */
/* sizes); both functions read them, so they must not change between them.  */
/* ------------------------------------------------------------------------ */
mss_status mss_ssd_chunk_bwd(const void* x, const float* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const float* h0,
                             const float* dy, const float* dh_last, float* dx, float* ddelta,
                             float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0,
                             int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t ngroups, int64_t dstate, mss_dtype in_dtype, uint32_t flags,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace mss_ssd_chunk_bwd needs (0 when unsupported). */
size_t mss_ssd_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                  int64_t ngroups, int64_t dstate, mss_dtype in_dtype);

/* ------------------------------------------------------------------------ */
/* Status of a call that used `workspace`.                                   */
/*                                                                          */
/* The selective scan (forward, fused, backward) hands states between        */
/* workgroups through flags in its workspace; each wait for such a flag is   */
/* bounded, and a wait that gives up (never expected) leaves the call's      */
/* outputs invalid and sets the status word, the workspace's first 4 bytes, */
/* which every call of the library clears in its first kernel (the SSD      */
/* workspace has the word too and never sets it).  This waits for           */
/* `hip_stream` (NULL = the default stream) to finish, reads the word and    */
/* returns MSS_OK, or MSS_ERR_WAIT when the last call that used the         */
/* workspace gave up a wait; MSS_ERR_NULL for a NULL workspace, MSS_ERR_HIP  */
/* when the synchronisation or the read fails.                              */
/* ------------------------------------------------------------------------ */
mss_status mss_workspace_status(const void* workspace, void* hip_stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* mss_status_string(mss_status status);

/* hipError_t of the last MSS_ERR_HIP returned on the calling thread. */
int mss_last_hip_error(void);

/* MSS_ABI_VERSION of the loaded library. */
int mss_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MAMBASCAN_H_ */
