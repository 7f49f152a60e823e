/*
 * ssm.h -- C ABI of libssm: the selective state-space scan (S6) on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (one independent channel per (b, d); all tensors row-major):
 *
 *   Delta_t  = softplus(delta[b,d,t] + delta_bias[d])  (flags & SSM_DELTA_SOFTPLUS)
 *            =          delta[b,d,t] + delta_bias[d]   (otherwise)
 *   Abar_t,n = exp(Delta_t * A[d,n])
 *   Bbar_t,n = Delta_t                                 (Euler, the default)
 *            = (Abar_t,n - 1) / A[d,n]                 (flags & SSM_BBAR_ZOH)
 *   h_t,n    = Abar_t,n * h_{t-1},n + Bbar_t,n * B[b,n,t] * u[b,d,t]
 *   y[b,d,t] = (sum_n C[b,n,t] * h_t,n + D_skip[d] * u[b,d,t]) * silu(z[b,d,t])
 *
 * Sources, cited by page title and section:
 *  - "Mamba" paper review (wiki.alexanderbaur.de), "SSM": the continuous
 *    system h' = Ah + Bx, y = Ch; zero-order hold Abar = exp(Delta A);
 *    the recurrence h_t = Abar h_{t-1} + Bbar x_t; diagonal A used SISO per
 *    channel.  "Selection Mechanism": Delta, B, C vary per token.
 *    "Optimization": one fused kernel for discretisation, scan and readout,
 *    the state never stored in HBM; parallel scan of the associative step.
 *  - "Paper: Mamba" course module (konke.bhala.ai/m/F12), "Math & data
 *    structures": zero-order hold Abar = exp(Delta A) and
 *    Bbar = (exp(Delta A) - 1)/A B, with Euler (Bbar = Delta B) as the
 *    alternative; the associative composition of affine steps.  Euler is the
 *    default input term, SSM_BBAR_ZOH selects the zero-order-hold one.
 *  - NN LAB "Mamba" page (khchao.com), "Derivation of the Discrete
 *    Transition Matrices": the input held constant over each step, and
 *    each state of a diagonal A discretised on its own.
 *  - "Exercises -- State-space models (Mamba, S4)" (brentwoodlivery.com):
 *    readout y_k = C h_k after the update; zero initial state; softplus as
 *    the positive time step; decoding one token at a time with a
 *    constant-size state (O(1) work, O(N) memory per token).
 *  - The D_skip term and the silu(z) output gate are not written out on the
 *    pages; the "Mamba" review's block description only mentions a gate on
 *    a residual branch.  They are applied as in the formula above.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library allocates nothing and keeps no state between calls.
 *  - dtype selects the storage of u, delta, B, C, z and y: SSM_F32 (float)
 *    or SSM_BF16 (bfloat16 bit patterns, 2 bytes).  A, delta_bias, D_skip,
 *    h0, last_state and the decode state are always float32.
 *  - Layouts, L fastest: u, delta, z, y: (batch, dim, seqlen); B, C:
 *    (batch, dstate, seqlen); A: (dim, dstate); delta_bias, D_skip: (dim);
 *    h0, last_state, state: (batch, dim, dstate).  Contiguous, no strides.
 *  - Pointers must be aligned to their element size (SSM_ERR_ALIGN
 *    otherwise).  16-byte aligned pointers with rows of a multiple of 16
 *    bytes take the vectorised path of the scans (when 64 rows span less
 *    than 2^31 bytes: up to 16M bf16 or 8M float32 steps); any other legal
 *    alignment or length works, slower.
 *  - stream is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work and return; they never synchronise.  Two calls that write the same
 *    outputs or workspace on different streams race.
 *  - Arguments are validated before any HIP call; on an error nothing is
 *    enqueued.  A launch failure returns SSM_ERR_HIP.
 *  - NaN and Inf inputs propagate as in the formula: a non-finite u, delta
 *    or z of channel (b, d) at step t makes that channel's outputs from t
 *    on non-finite where the formula does (NaN where it gives NaN, Inf of
 *    the same sign where it gives Inf) and leaves other channels alone; a
 *    non-finite B or C reaches every channel of its batch row.  (ssm_ssd_
 *    scan_fwd differs: see there.)  Exception, float32 range: where one
 *    step's decay exp(Delta*A) underflows to 0 in float32 (Delta*A below
 *    about -87) an infinite state meets it as 0 * Inf = NaN; the decay of a
 *    whole segment of a split sequence is kept at or above the smallest
 *    normal float for that reason.  A is not checked for sign (A > 0 is an
 *    unstable system and its state grows, as the pages note).
 *  - Buffers the call writes (y, last_state, conv_state_out, the decode
 *    state and conv_state, the gradients, the workspace) must not overlap
 *    each other or any buffer the call reads, judged on their byte ranges
 *    (SSM_ERR_ALIAS otherwise); buffers that are only read may overlap.  In
 *    particular last_state must not be h0.
 *  - With SSM_BBAR_ZOH the coefficient (Abar - 1)/A is taken from the Taylor
 *    series Delta (1 + x/2 + x^2/6 + x^3/24), x = Delta A, where |x| < 0.1,
 *    and from (Abar - 1)/A elsewhere, so its float32 relative error stays
 *    near 1e-6 for every Delta A; A = 0 gives Delta, the limit.
 *  - Results are deterministic: the same inputs on the same device give the
 *    same bits, run after run.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = -1,      /* a required pointer is NULL                          */
  SSM_ERR_SHAPE = -2,     /* negative size, dstate not in {1,2,4,8,16}, too large
                             (seqlen above 2^31 - 4097: steps are 32-bit in the kernels) */
  SSM_ERR_DTYPE = -3,     /* dtype not an ssm_dtype_t value                      */
  SSM_ERR_ALIGN = -4,     /* a pointer not aligned to its element size           */
  SSM_ERR_WORKSPACE = -5, /* workspace NULL or smaller than the query's answer   */
  SSM_ERR_HIP = -6,       /* the HIP runtime reported an error at launch         */
  SSM_ERR_ALIAS = -7,     /* a buffer the call writes overlaps another of its buffers */
  SSM_ERR_FLAGS = -8,     /* flags holds a bit that is not an ssm_flag_t value   */
  SSM_ERR_SCRATCH = -9    /* ssm_scan_fwd_noalloc: needs more than its static scratch */
} ssm_status_t;

/* Bits of the `flags` argument (0 and 1 keep the meaning of the plain
 * softplus switch). */
typedef enum {
  SSM_DELTA_SOFTPLUS = 1, /* Delta = softplus(delta + bias), else delta + bias   */
  SSM_BBAR_ZOH = 2        /* zero-order-hold input term, else Euler (Delta)      */
} ssm_flag_t;

/*
 * ssm_scan_fwd_workspace_bytes -- bytes of device workspace that
 * ssm_scan_fwd needs for this problem: B and C interleaved per step for the
 * kernel, in the input dtype (batch * seqlen * 2 * dstate elements), plus,
 * when the sequence is split across workgroups, each segment's end state
 * and Delta sum.  Pure host function: no HIP call.  Returns 0 for an empty
 * problem and for arguments that ssm_scan_fwd would reject.
 */
size_t ssm_scan_fwd_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen,
                                    int dtype);

/*
 * ssm_scan_fwd -- the selective scan over a whole sequence (prefill or the
 * training forward pass), formula above.
 *
 *   u, delta     in   (batch, dim, seqlen), dtype           required
 *   A            in   (dim, dstate) float32                  required
 *   B, C         in   (batch, dstate, seqlen), dtype         required
 *   D_skip       in   (dim) float32                          NULL -> 0
 *   z            in   (batch, dim, seqlen), dtype            NULL -> no gate
 *   delta_bias   in   (dim) float32                          NULL -> 0
 *   flags        bits of ssm_flag_t: SSM_DELTA_SOFTPLUS, SSM_BBAR_ZOH
 *   h0           in   (batch, dim, dstate) float32           NULL -> zero state
 *   y            out  (batch, dim, seqlen), dtype            required; must not
 *                     be u, delta or z
 *   last_state   out  (batch, dim, dstate) float32           NULL -> not written
 *   workspace    scratch of at least ssm_scan_fwd_workspace_bytes(...) bytes,
 *                256-byte aligned device memory owned by the caller (NULL only
 *                when the query returns 0).  Its contents on entry do not
 *                matter; calls sharing one workspace must not overlap.
 *   batch, dim >= 0; dstate in {1,2,4,8,16}; seqlen >= 0.  seqlen == 0 only
 *   writes last_state (= h0, or zeros).
 */
int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                 const void* C, const float* D_skip, const void* z,
                 const float* delta_bias, int flags, const float* h0, void* y,
                 float* last_state, int batch, int dim, int dstate, int64_t seqlen,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static per-device scratch of ssm_scan_fwd_noalloc. */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * ssm_scan_fwd_noalloc -- ssm_scan_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Instead of a caller's workspace it uses a static
 * device array of the library, SSM_NOALLOC_SCRATCH_BYTES on each device the
 * library runs on, held from the library's load on that device until the
 * process ends.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first use on a device looks up the
 * array's device address once (hipGetSymbolAddress).  The caller passes every
 * input and output.
 *
 *   Arguments, layouts, results and errors as ssm_scan_fwd, without the
 *   workspace arguments.
 *   Problems whose ssm_scan_fwd_workspace_bytes(...) exceeds
 *   SSM_NOALLOC_SCRATCH_BYTES return SSM_ERR_SCRATCH before any HIP call
 *   (the 2.8B-shaped layer, batch 16, D 5120, N 16, L 2048 bf16, needs 2 MiB).
 *   Every call on one device shares that device's scratch, which keeps the
 *   last call's contents (no part of it needs to be zero on entry).  Calls
 *   that can run at the same time on one device -- on different streams, or
 *   from host threads whose streams run concurrently -- race on it; the
 *   caller must order them (one stream, or events).
 */
int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D_skip, const void* z,
                         const float* delta_bias, int flags, const float* h0, void* y,
                         float* last_state, int batch, int dim, int dstate, int64_t seqlen,
                         int dtype, void* stream);

/*
 * ssm_state_update -- one decode step for a single new token per sequence:
 * the formula above with seqlen = 1, starting from and writing back `state`.
 *
 *   state        in/out (batch, dim, dstate) float32, updated in place  required
 *   u, delta     in   (batch, dim), dtype                               required
 *   A            in   (dim, dstate) float32                             required
 *   B, C         in   (batch, dstate), dtype                            required
 *   D_skip       in   (dim) float32                                     NULL -> 0
 *   z            in   (batch, dim), dtype                               NULL -> no gate
 *   delta_bias   in   (dim) float32                                     NULL -> 0
 *   flags        bits of ssm_flag_t, as for ssm_scan_fwd
 *   y            out  (batch, dim), dtype                               required
 *   batch, dim >= 0; dstate in {1,2,4,8,16}.
 */
int ssm_state_update(float* state, const void* u, const void* delta, const float* A,
                     const void* B, const void* C, const float* D_skip, const void* z,
                     const float* delta_bias, int flags, void* y, int batch,
                     int dim, int dstate, int dtype, void* stream);

/*
 * ssm_conv_scan_fwd -- ssm_scan_fwd with the block's convolution prologue
 * fused in: the scan's u is computed in the kernel from x as
 *
 *   u[b,d,t] = silu(conv_b[d] + sum_{k<K} conv_w[d,k] * x[b,d,t-K+1+k])
 *
 * (depthwise, causal, tap K-1 on the current input), and u feeds both the
 * recurrence and the D_skip term; x is read from HBM once.  Source: "Mamba"
 * paper review, "Mamba" block description (before the SSM the input goes
 * through a convolution and then a nonlinear function) and the NN LAB "Mamba"
 * page, "Kernel Fusion in On-Chip SRAM" (the causal 1-D convolution fused
 * with discretisation and scan).  Width, tap order and silu as the
 * non-linearity are not fixed by the pages; they are this interface's
 * choice.
 *
 *   x              in   (batch, dim, seqlen), dtype           required
 *   conv_w         in   (dim, conv_width) float32              required
 *   conv_b         in   (dim) float32                          NULL -> 0
 *   conv_width     1..4 (SSM_ERR_SHAPE otherwise)
 *   conv_state_in  in   (batch, dim, conv_width-1) float32: the inputs before
 *                       t = 0, oldest first                    NULL -> zeros
 *   conv_state_out out  (batch, dim, conv_width-1) float32: the last
 *                       conv_width-1 inputs (from conv_state_in where
 *                       seqlen < conv_width-1)                 NULL -> not written;
 *                       must not be conv_state_in, y or last_state
 *   every other argument as for ssm_scan_fwd (y must not be x), with the
 *   same workspace (ssm_scan_fwd_workspace_bytes).
 */
int ssm_conv_scan_fwd(const void* x, const float* conv_w, const float* conv_b, int conv_width,
                      const float* conv_state_in, float* conv_state_out, const void* delta,
                      const float* A, const void* B, const void* C, const float* D_skip,
                      const void* z, const float* delta_bias, int flags, const float* h0, void* y,
                      float* last_state, int batch, int dim, int dstate, int64_t seqlen, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_conv_state_update -- ssm_state_update with the convolution prologue:
 * u = silu(conv_b[d] + sum_{k<K-1} conv_w[d,k] * conv_state[b,d,k]
 *          + conv_w[d,K-1] * x[b,d]),
 * then conv_state is shifted in place to end with x.  Source as for
 * ssm_conv_scan_fwd.
 *
 *   conv_state     in/out (batch, dim, conv_width-1) float32   required when
 *                         conv_width > 1; must not be state, x or y
 *   x              in   (batch, dim), dtype                     required
 *   conv_w, conv_b, conv_width as for ssm_conv_scan_fwd; every other argument
 *   as for ssm_state_update.
 */
int ssm_conv_state_update(float* conv_state, float* state, const void* x, const float* conv_w,
                          const float* conv_b, int conv_width, const void* delta, const float* A,
                          const void* B, const void* C, const float* D_skip, const void* z,
                          const float* delta_bias, int flags, void* y, int batch, int dim,
                          int dstate, int dtype, void* stream);

/*
 * ssm_scan_bwd_workspace_bytes -- bytes of device workspace ssm_scan_bwd
 * needs: the forward workspace, the state entering every 16-step tile
 * (batch * ceil(seqlen/16) * dstate * dim floats), partial sums of dB and dC
 * per 64-channel group (batch * ceil(dim/64) * 2 * dstate * seqlen floats),
 * and small per-segment terms.  Pure host function; 0 for an empty problem
 * and for arguments ssm_scan_bwd would reject.
 */
size_t ssm_scan_bwd_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen, int dtype);

/*
 * ssm_scan_bwd -- gradients of a loss L through ssm_scan_fwd, given
 * dy = dL/dy and optionally dlast_state = dL/dlast_state.  The states are
 * recomputed from the inputs, not read from a saved forward pass: the
 * "Mamba" paper review, "Optimization" (recomputation for backpropagation).
 * Per channel the adjoint lambda_t = dL/dh_t runs backwards,
 * lambda_t = ds_t C_t + Abar_{t+1} lambda_{t+1} with ds_t = dy_t silu(z_t),
 * and every gradient is the chain rule through the formula at the top.
 *
 *   u .. h0          in   as for ssm_scan_fwd (same layouts and dtype)
 *   flags            as for ssm_scan_fwd: SSM_DELTA_SOFTPLUS, SSM_BBAR_ZOH (the
 *                    zero-order-hold input term, dBbar/dDelta = Abar and
 *                    dBbar/dA = (x e^x - e^x + 1)/A^2, x = Delta A, with its
 *                    series Delta^2 (1/2 + x/3 + ...) where abs(x) < 1/4)
 *   dy               in   (batch, dim, seqlen), dtype          required
 *   dlast_state      in   (batch, dim, dstate) float32         NULL -> 0
 *   du, ddelta       out  (batch, dim, seqlen), dtype          required
 *                         (ddelta is dL/d(delta), before the bias and softplus)
 *   dA               out  (dim, dstate) float32                required
 *   dB, dC           out  (batch, dstate, seqlen), dtype       required
 *   dD               out  (dim) float32                        NULL -> not written
 *   dz               out  (batch, dim, seqlen), dtype          required when z is given
 *   ddelta_bias      out  (dim) float32                        NULL -> not written
 *   dh0              out  (batch, dim, dstate) float32         NULL -> not written
 *                         (dL/dh0, also when h0 is NULL)
 *   workspace        at least ssm_scan_bwd_workspace_bytes(...) bytes, 256-byte
 *                    aligned, owned by the caller.
 * Outputs must not alias the per-token inputs (SSM_ERR_ALIAS).  dA, dB, dC,
 * dD and ddelta_bias are sums formed in float32 in a fixed order: the same
 * inputs give the same bits.  seqlen == 0 writes zeros and dh0 = dlast_state.
 */
int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D_skip, const void* z, const float* delta_bias, int flags,
                 const float* h0, const void* dy, const float* dlast_state, void* du, void* ddelta,
                 float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                 float* dh0, int batch, int dim, int dstate, int64_t seqlen, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_ckpt_bytes -- bytes of the tile checkpoints of a scan: the state
 * entering every 16-step tile, (batch, ceil(seqlen/16), dstate, dim) float32
 * (tile j holds h_{16j-1}, the zero or h0 state for j = 0).  Pure host
 * function; 0 for an empty problem and for a dstate or size ssm_scan_fwd
 * would reject.
 */
size_t ssm_scan_ckpt_bytes(int batch, int dim, int dstate, int64_t seqlen);

/*
 * ssm_scan_fwd_ckpt -- ssm_scan_fwd for a training step: besides y and
 * last_state it writes the tile checkpoints, which ssm_scan_bwd_ckpt then
 * starts from instead of running the states forward again.  The backward
 * still recomputes every state inside a tile from that tile's checkpoint
 * ("Mamba" paper review, "Optimization": intermediate states recomputed for
 * backpropagation rather than stored); only one state in 16 is kept.
 *
 *   ckpt         out  at least ssm_scan_ckpt_bytes(...) bytes, 4-byte
 *                     aligned, owned by the caller            required when
 *                     the query is above 0 (SSM_ERR_NULL; too small:
 *                     SSM_ERR_WORKSPACE); must not overlap any other buffer
 *                     of the call (SSM_ERR_ALIAS)
 *   every other argument, result and error as for ssm_scan_fwd (the same
 *   workspace query); y and last_state carry the same bits as ssm_scan_fwd's.
 */
int ssm_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D_skip, const void* z,
                      const float* delta_bias, int flags, const float* h0, void* y,
                      float* last_state, float* ckpt, size_t ckpt_bytes, int batch, int dim,
                      int dstate, int64_t seqlen, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * ssm_scan_bwd_ckpt_workspace_bytes -- bytes of device workspace
 * ssm_scan_bwd_ckpt needs: ssm_scan_bwd's without the checkpoint region.
 * Pure host function; 0 for an empty problem and for arguments
 * ssm_scan_bwd_ckpt would reject.
 */
size_t ssm_scan_bwd_ckpt_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen,
                                         int dtype);

/*
 * ssm_scan_bwd_ckpt -- ssm_scan_bwd starting from the tile checkpoints that
 * ssm_scan_fwd_ckpt wrote for the same inputs, flags and h0, so the forward
 * checkpoint pass is skipped.  Given those checkpoints every gradient
 * carries the same bits as ssm_scan_bwd's.
 *
 *   ckpt         in   the checkpoints, ssm_scan_ckpt_bytes(...) bytes or more,
 *                     4-byte aligned                            required when
 *                     the query is above 0 (SSM_ERR_NULL; too small:
 *                     SSM_ERR_WORKSPACE); no output or the workspace may
 *                     overlap it (SSM_ERR_ALIAS)
 *   workspace    at least ssm_scan_bwd_ckpt_workspace_bytes(...) bytes,
 *                256-byte aligned, owned by the caller
 *   every other argument, result and error as for ssm_scan_bwd.
 */
int ssm_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D_skip, const void* z,
                      const float* delta_bias, int flags, const float* h0, const float* ckpt,
                      size_t ckpt_bytes, const void* dy, const float* dlast_state, void* du,
                      void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                      float* ddelta_bias, float* dh0, int batch, int dim, int dstate,
                      int64_t seqlen, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * ssm_ssd_scan_fwd -- the SSD (Mamba-2) form: the same recurrence with a
 * scalar A per head, computed by chunks on the matrix cores.  The dim =
 * nheads * headdim channels form heads of headdim consecutive channels;
 * every channel d of head h = d / headdim uses A[d, n] = A_head[h] for all
 * states n and the head's step Delta[b, h, t] = softplus(dt[b, h, t] +
 * dt_bias[h]); B and C are shared by all heads.  Source: "Mamba" paper
 * review, "Mamba 2" (scalar-identity A; M_ji = A_{j:i} (C_j . B_i); small
 * chunks in the quadratic form, the linear recurrence across chunks); NN LAB
 * "Mamba" page, "Bridging Tensor Cores and Recurrence" (A = alpha I;
 * intra-chunk matrix products, inter-chunk state propagation).
 *
 *   x, z, y        (batch, nheads*headdim, seqlen), dtype    x, y required; z NULL -> no gate
 *   dt             (batch, nheads, seqlen), dtype            required (raw: bias and softplus inside)
 *   A_head         (nheads) float32                          required
 *   B, C           (batch, dstate, seqlen), dtype            required
 *   D_skip         (nheads*headdim) float32                  NULL -> 0
 *   dt_bias        (nheads) float32                          NULL -> 0
 *   flags          SSM_DELTA_SOFTPLUS, SSM_BBAR_ZOH as for ssm_scan_fwd
 *   h0, last_state (batch, nheads*headdim, dstate) float32   NULL -> zero start / not written
 *   headdim must be 64; dstate in {16, 32, 64, 128} (128 for SSM_BF16 only);
 *   seqlen * max(64, dstate) * element bytes below 2^31 (SSM_ERR_SHAPE).
 *   workspace      at least ssm_ssd_scan_fwd_workspace_bytes(...) bytes, 256-byte
 *                  aligned, owned by the caller (C with the state index
 *                  contiguous and, per 64-step chunk, the causal tiles of
 *                  C^T B, which all heads share; rewritten by every call)
 * bf16 storage feeds the matrix cores bf16 operands: the chunk matrix, the
 * decayed x and the state are rounded to bf16 for the products, which are
 * accumulated in float32; the state itself is carried in float32.
 * Non-finite inputs: a NaN or Inf in x at (channel, step t) makes that
 * channel's outputs non-finite from t on, as in the recurrence, and can
 * also reach its outputs of the same 64-step chunk before t (the chunk's
 * masked product multiplies it by the zeros above the diagonal, and
 * 0 * Inf is NaN); a non-finite dt, B or C reaches the whole chunk of its
 * head (dt) or batch row (B, C).  Outputs before the chunk are unaffected.
 * Otherwise as ssm_scan_fwd.
 */
int ssm_ssd_scan_fwd(const void* x, const void* dt, const float* A_head, const void* B,
                     const void* C, const float* D_skip, const void* z, const float* dt_bias,
                     int flags, const float* h0, void* y, float* last_state, int batch, int nheads,
                     int headdim, int dstate, int64_t seqlen, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ssm_ssd_scan_fwd_workspace_bytes -- batch * seqlen * dstate elements of
 * dtype rounded up to 256 bytes, plus 40 KiB (10 tiles of 16 x 16 float32)
 * per batch row and 64-step chunk; 0 for an empty problem.  Pure host
 * function. */
size_t ssm_ssd_scan_fwd_workspace_bytes(int batch, int dstate, int64_t seqlen, int dtype);

/* ssm_status_string -- a static, human-readable name for a status code. */
const char* ssm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
