/*
 * mssm.h -- C ABI of the MI355X (gfx950) selective-scan library libmssm.so.
 *
 * The operation is the selective state-space scan of Mamba (selective SSM
 * layer, Mamba paper Section 3 / Algorithm 2, named in the description section
 * of the page "Mamba SSM 架构"): for every batch b and channel d, with state
 * h[n], n < N,
 *
 *     x_t     = delta[b,t,d] + dt_bias[d]
 *     Delta_t = softplus(x_t) if problem.delta_softplus else x_t
 *     h_t[n]  = exp(Delta_t * A[d,n]) * h_{t-1}[n] + Delta_t * Bm[b,t,n] * u[b,t,d]
 *     y[b,t,d]= (sum_n Cm[b,t,n] * h_t[n] + Dskip[d] * u[b,t,d]) * silu(z[b,t,d])
 *
 * with h_{-1} = h0 (zeros when h0 is NULL).  The state update and readout are
 * the sequential loop printed in the Hacker News comments of the page
 * "PyTorch 한 파일에서의 Mamba 구현" (deltaA = exp(Delta*A), deltaB_u =
 * Delta*B*u, y = contraction of the state with C); the pages name deltaA and
 * deltaB_u without a formula, and the zero-order-hold / Euler reading above is
 * the one this library implements.  The state lives only in registers: the
 * (B, L, D, N) expansion is never written to memory, which is the data
 * movement the page "mamba.py: 一个简单高效的Mamba实现" (performance section,
 * d_state paragraph, citing the paper's Appendix D) credits for the O(N)
 * reduction in memory reads and writes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts: row-major, contiguous, no strides.
 *     u, delta, z, y, dy, du, ddelta, dz : (B, L, D)   D fastest
 *     Bm, Cm, dB, dC                     : (B, L, N)   N fastest
 *     A, dA                              : (D, N)      float32
 *     Dskip, dt_bias, dD, ddt_bias       : (D)         float32
 *     h0, h_final, dh_final, dh0, state  : (B, D, N)   float32
 *   and for the conv1d + SiLU front end (mssm_conv_*):
 *     x, dx                              : (B, L, D)   as u
 *     x_prev, dx_prev, conv_state        : (B, d_conv - 1, D), in time order
 *     conv_w, dconv_w                    : (D, d_conv) float32 (torch.nn.Conv1d's (D, 1, d_conv))
 *     conv_b, dconv_b                    : (D)         float32
 * Element type: problem.dtype (MSSM_F32 or MSSM_BF16) for u, delta, z, Bm, Cm,
 *   y and their gradients; float32 for everything else.  Arithmetic is float32
 *   throughout; bfloat16 outputs are rounded to nearest even.
 * Memory: every pointer is a device pointer owned by the caller, 16-byte
 *   aligned.  The library allocates and frees nothing and keeps no state
 *   between calls; it is re-entrant.  (One exception, for callers that cannot
 *   allocate: mssm_scan_fwd_noalloc uses a fixed scratch array of the
 *   library's own, shared by its calls on a GPU.)  Scratch memory is the caller's
 *   `workspace`, of at least the size the matching *_workspace_bytes query
 *   returns for the same problem (NULL is accepted when that size is 0).
 * Streams: all work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 *   null stream); calls return once the work is enqueued.  Outputs are valid
 *   when the stream reaches that point.
 * Errors: argument errors are detected on the host before anything is
 *   enqueued, and return without touching any buffer.  A launch failure
 *   returns MSSM_ERR_HIP.  NaN and Inf in inputs are not trapped; they
 *   propagate.  No exception crosses the ABI.
 * Limits: 1 <= dstate <= MSSM_MAX_DSTATE (a dstate that is not a power of two
 *   runs the next power of two's kernels with the extra states inert --
 *   A, Bm, Cm and h0 zero for them, so they stay 0 and add nothing to y -- on
 *   zero-padded copies of Bm, Cm, A, h0 in the workspace, which the
 *   *_workspace_bytes queries include);
 *   batch, seqlen, dim >= 1; batch * dim and seqlen below 2^31; dim below
 *   2^24; all indexing of (B, L, D) tensors is 64-bit.
 */
#ifndef MSSM_H
#define MSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSSM_MAX_DSTATE 64
/* Widest causal conv1d the fused front end (mssm_conv_scan_fwd) takes. */
#define MSSM_MAX_DCONV 4

typedef enum { MSSM_F32 = 0, MSSM_BF16 = 1 } mssm_dtype;

typedef enum {
    MSSM_OK = 0,
    MSSM_ERR_NULL = -1,        /* a required pointer is NULL */
    MSSM_ERR_SHAPE = -2,       /* a dimension is out of range */
    MSSM_ERR_DTYPE = -3,       /* unknown problem.dtype */
    MSSM_ERR_UNSUPPORTED = -4, /* valid but not built: dstate > MSSM_MAX_DSTATE (SSD: other sizes) */
    MSSM_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    MSSM_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the query returns */
    MSSM_ERR_HIP = -7          /* a HIP launch failed */
} mssm_status;

typedef struct {
    int64_t batch;          /* B */
    int64_t seqlen;         /* L (ignored by mssm_step) */
    int64_t dim;            /* D: channels */
    int64_t dstate;         /* N: state size per channel */
    int32_t dtype;          /* mssm_dtype of u, delta, z, Bm, Cm, y and their gradients */
    int32_t delta_softplus; /* nonzero: Delta = softplus(delta + dt_bias) */
} mssm_problem;

/* Bytes of device scratch the forward needs (0 when the sequence is scanned
 * in one pass; otherwise the cross-chunk carries, O(B * D * N * chunks)).
 * Returns 0 for an invalid problem. */
size_t mssm_scan_fwd_workspace_bytes(const mssm_problem* p);

/* Bytes of device scratch the backward needs: the forward's own scratch, the
 * state before every 16-step tile, sbar = dy * silu(z) in float32, the partial
 * sums of dB, dC (per 64-channel block) and of dA, dD, ddt_bias (per batch row
 * and time chunk), and, when the reverse walk is cut into time chunks (few
 * channel blocks, long sequences), each chunk's adjoint carry.  0 for an
 * invalid problem. */
size_t mssm_scan_bwd_workspace_bytes(const mssm_problem* p);

/*
 * Forward scan.  Required: p, u, delta, A, Bm, Cm, y.  Optional (NULL):
 *   Dskip   -> 0             z       -> no gate (y = s)
 *   dt_bias -> 0             h0      -> zero initial state
 *   h_final -> not written
 * Writes y (B, L, D) and, if given, h_final = h_{L-1} (B, D, N).
 * y may not alias any input.  h_final may be the same buffer as h0: the state
 * is then advanced in place by L steps, a multi-token form of mssm_step (each
 * lane reads a channel's initial state before that channel's final state is
 * written, in every schedule the library uses).  No other partial overlap of
 * h0 and h_final is allowed.
 */
mssm_status mssm_scan_fwd(const mssm_problem* p,
                          const void* u, const void* delta, const float* A,
                          const void* Bm, const void* Cm,
                          const float* Dskip, const void* z, const float* dt_bias,
                          const float* h0,
                          void* y, float* h_final,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * The forward scan of mssm_scan_fwd for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc -- and so cannot provide a workspace: same arguments,
 * outputs and errors as mssm_scan_fwd minus workspace / workspace_bytes, same
 * kernels and results (bit for bit).  The scratch comes from a fixed device
 * array inside the library, MSSM_NOALLOC_SCRATCH_BYTES on every GPU the
 * library runs on, reserved when the library's code is loaded onto that GPU
 * and held until the process ends; its device address is looked up once per
 * GPU (hipGetSymbolAddress, on the first call with that GPU current).  The
 * call itself allocates and frees nothing.
 * A problem whose scratch exceeds MSSM_NOALLOC_SCRATCH_BYTES returns
 * MSSM_ERR_WORKSPACE before anything is enqueued; the scratch is what
 * mssm_scan_fwd_workspace_bytes returns, except for the short sequences
 * (at most 8 steps, or at most 64 steps over at most 32,768 (batch, channel)
 * rows) that run without any.  32 MiB covers every time-chunked plan up to
 * dstate 64 and the balanced schedule up to 8,192 channel blocks at dstate 16.  Everything in the array that
 * must start at zero is cleared by a kernel of the call itself, so the contents
 * left by an earlier call do not matter -- but all calls on one GPU share the
 * one array: calls that may run at the same time on one GPU (other streams,
 * other host threads, a replayed graph next to a live call) race and give wrong
 * results.  Serialise them, or use mssm_scan_fwd with a workspace each.
 */
#define MSSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
mssm_status mssm_scan_fwd_noalloc(const mssm_problem* p,
                                  const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm,
                                  const float* Dskip, const void* z, const float* dt_bias,
                                  const float* h0,
                                  void* y, float* h_final, void* hip_stream);

/*
 * Forward scan behind the Mamba block's causal conv1d + SiLU, fused: the scan
 * input is formed inside the kernels as
 *
 *   u[b,t,d] = silu(conv_b[d] + sum_{k<d_conv} conv_w[d,k] * x[b, t-d_conv+1+k, d])
 *
 * (a depthwise causal convolution of kernel size d_conv; the configurations on
 * the page "Mamba SSM 架构" use d_conv = 4, and the mamba-minimal page "PyTorch
 * 한 파일에서의 Mamba 구현" runs it as torch.nn.Conv1d, whose weight layout
 * (D, 1, d_conv) this matches) and never stored unless u_out is given.  Then
 * exactly mssm_scan_fwd with that u.
 *   x       (B, L, D) in p->dtype, the conv input (replaces u)
 *   conv_w  (D, d_conv) float32, row-major; 1 <= d_conv <= MSSM_MAX_DCONV
 *   conv_b  (D) float32, NULL -> 0
 *   x_prev  (B, d_conv - 1, D) in p->dtype, the d_conv - 1 inputs just before
 *           t = 0 in time order (streaming: the last d_conv - 1 rows of the
 *           previous call's x); NULL -> zeros (the convolution's left padding)
 *   u_out   (B, L, D) in p->dtype, NULL -> not written; else receives u (what
 *           mssm_scan_bwd needs as its u)
 * The other arguments, the workspace (mssm_scan_fwd_workspace_bytes) and the
 * errors are those of mssm_scan_fwd; d_conv out of range -> MSSM_ERR_SHAPE,
 * conv_w NULL -> MSSM_ERR_NULL.  y and u_out may not alias any input; h_final
 * may be h0 (the state advanced in place).
 */
mssm_status mssm_conv_scan_fwd(const mssm_problem* p, int32_t d_conv,
                               const void* x, const float* conv_w, const float* conv_b,
                               const void* x_prev,
                               const void* delta, const float* A,
                               const void* Bm, const void* Cm,
                               const float* Dskip, const void* z, const float* dt_bias,
                               const float* h0,
                               void* y, float* h_final, void* u_out,
                               void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of device scratch mssm_conv_bwd needs (per (batch row, time chunk)
 * partial sums of dconv_w and dconv_b); p->dstate is ignored.  0 for an
 * invalid problem or d_conv. */
size_t mssm_conv_bwd_workspace_bytes(const mssm_problem* p, int32_t d_conv);

/*
 * Backward of the conv1d + SiLU front end of mssm_conv_scan_fwd: given du =
 * dL/du for u = silu(conv_b + causal depthwise conv of x with conv_w) (the du
 * that mssm_scan_bwd returns for the u that mssm_conv_scan_fwd formed),
 * writes, with g = du * silu'(c) and c the convolution:
 *   dx       (B, L, D) p->dtype   dx[t] = sum_k conv_w[d,k] g[t + d_conv - 1 - k]
 *   dconv_w  (D, d_conv) float32  sum over (b, t) of g[t] x[t - d_conv + 1 + k]
 *   dconv_b  (D) float32, NULL -> not written; sum over (b, t) of g
 *   dx_prev  (B, d_conv - 1, D) p->dtype, NULL -> not written; the gradient of
 *            the history rows x_prev (zero history: the gradient of the padding)
 * x, conv_w, conv_b, x_prev and d_conv as in mssm_conv_scan_fwd; p->dstate
 * and p->delta_softplus are ignored.  Gradients are overwritten; dconv_w and
 * dconv_b are summed in a fixed order (bitwise reproducible).  Errors as for
 * mssm_conv_scan_fwd (required: x, conv_w, du, dx, dconv_w, workspace).
 */
mssm_status mssm_conv_bwd(const mssm_problem* p, int32_t d_conv,
                          const void* x, const float* conv_w, const float* conv_b, const void* x_prev,
                          const void* du, void* dx, float* dconv_w, float* dconv_b, void* dx_prev,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Backward scan: gradients of  sum(dy * y) + sum(dh_final * h_final)  with
 * respect to every input, by the reverse-time adjoint scan with the forward
 * states recomputed per chunk (nothing of the forward is stored between the
 * calls).  Inputs are those of the forward plus dy (B, L, D) and the optional
 * dh_final (B, D, N).
 * Required outputs: du, ddelta (gradient w.r.t. the raw delta input, before
 *   bias and softplus), dA, dB, dC.
 * Optional outputs (NULL -> not written): dD (needs nothing), dz (only with
 *   z; required when z is given), ddt_bias, dh0.
 * Every gradient is overwritten, not accumulated.  Reductions over channels
 * (dB, dC) and over batch and time (dA, dD, ddt_bias) use a fixed order:
 * repeated calls give bitwise identical results.
 */
mssm_status mssm_scan_bwd(const mssm_problem* p,
                          const void* u, const void* delta, const float* A,
                          const void* Bm, const void* Cm,
                          const float* Dskip, const void* z, const float* dt_bias,
                          const float* h0,
                          const void* dy, const float* dh_final,
                          void* du, void* ddelta, float* dA, void* dB, void* dC,
                          float* dD, void* dz, float* ddt_bias, float* dh0,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Training pair: a forward that saves what its backward needs, and that
 * backward.  mssm_scan_bwd recomputes the forward's states with a pre-pass
 * over the whole recurrence; mssm_scan_fwd_train instead writes them, once
 * per 16-step tile, into a caller-owned context buffer, and
 * mssm_scan_bwd_saved starts its reverse walk from them (the forward-state
 * recomputation of the page "mamba.py: 一个简单高效的Mamba实现", performance
 * section, then covers one tile at a time).  The gradients are those of
 * mssm_scan_bwd (same definitions, same fixed reduction order).
 *
 * Context (ctx): device memory of at least mssm_scan_ctx_bytes(p), 16-byte
 * aligned, owned by the caller; its contents are the library's (the state
 * before every 16-step tile, (B, ceil(L/16), N, D) float32, and the readout
 * before the gate, sum_n Cm h_t + Dskip u_t, (B, L, D) float32, written only
 * when z is given).  Valid for the inputs of the forward that wrote it.  A
 * dstate that is not a power of two runs as elsewhere at the next power of
 * two with inert extra states, and the context is that problem's (the size
 * query accounts for it).  ctx_bytes below the query returns
 * MSSM_ERR_WORKSPACE.
 */
size_t mssm_scan_ctx_bytes(const mssm_problem* p);

/* Forward of mssm_scan_fwd that also writes the context: same arguments (the
 * workspace is mssm_scan_fwd_workspace_bytes), outputs and aliasing rules,
 * plus ctx (required).  Always runs the tiled kernels, so its results are bit
 * for bit those of mssm_scan_fwd except for the short sequences (at most 64
 * steps) that mssm_scan_fwd runs on its short-sequence path. */
mssm_status mssm_scan_fwd_train(const mssm_problem* p,
                                const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm,
                                const float* Dskip, const void* z, const float* dt_bias,
                                const float* h0,
                                void* y, float* h_final,
                                void* ctx, size_t ctx_bytes,
                                void* workspace, size_t workspace_bytes, void* hip_stream);

/* The forward behind the fused conv1d + SiLU front end (mssm_conv_scan_fwd)
 * that also writes the context for mssm_scan_bwd_saved: same arguments,
 * outputs and errors as mssm_conv_scan_fwd, plus ctx (required, as for
 * mssm_scan_fwd_train).  The backward of a Mamba block's scan then runs as
 * mssm_scan_bwd_saved with u = the front end's output (u_out of this call),
 * followed by mssm_conv_bwd for dx, dconv_w, dconv_b. */
mssm_status mssm_conv_scan_fwd_train(const mssm_problem* p, int32_t d_conv,
                                     const void* x, const float* conv_w, const float* conv_b,
                                     const void* x_prev,
                                     const void* delta, const float* A,
                                     const void* Bm, const void* Cm,
                                     const float* Dskip, const void* z, const float* dt_bias,
                                     const float* h0,
                                     void* y, float* h_final, void* u_out,
                                     void* ctx, size_t ctx_bytes,
                                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of device scratch mssm_scan_bwd_saved needs (the partial sums of
 * dB, dC, dA, dD, ddt_bias and, with time chunks, the adjoint carries). */
size_t mssm_scan_bwd_saved_workspace_bytes(const mssm_problem* p);

/* Backward of mssm_scan_bwd from the context mssm_scan_fwd_train wrote for
 * the same u, delta, A, Bm, Cm, Dskip, z, dt_bias and h0 (h0 itself is not
 * needed: the context holds it as the state before the first tile).
 * Arguments, outputs and errors otherwise those of mssm_scan_bwd; workspace
 * from mssm_scan_bwd_saved_workspace_bytes (required). */
mssm_status mssm_scan_bwd_saved(const mssm_problem* p,
                                const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm,
                                const float* Dskip, const void* z, const float* dt_bias,
                                const void* ctx, size_t ctx_bytes,
                                const void* dy, const float* dh_final,
                                void* du, void* ddelta, float* dA, void* dB, void* dC,
                                float* dD, void* dz, float* ddt_bias, float* dh0,
                                void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * One token of the recurrent (RNN) form, for streaming decode: the step
 * function that the page "mamba.py: 一个简单高效的Mamba实现" lists in its
 * updates section.  p->seqlen is ignored.  Shapes: u_t, delta_t, z_t, y_t
 * (B, D) in p->dtype; Bm_t, Cm_t (B, N) in p->dtype; state (B, D, N) float32,
 * read and overwritten in place with h_t.  Optional: Dskip, z_t, dt_bias.
 * Calling it L times equals one mssm_scan_fwd over L steps with h0 = state.
 */
mssm_status mssm_step(const mssm_problem* p,
                      const void* u_t, const void* delta_t, const float* A,
                      const void* Bm_t, const void* Cm_t,
                      const float* Dskip, const void* z_t, const float* dt_bias,
                      float* state, void* y_t, void* hip_stream);

/*
 * One token through the conv1d + SiLU front end and the recurrent step, for
 * streaming decode of a Mamba block: u_t = silu(conv_b + sum_k conv_w[d,k] *
 * x_{t-d_conv+1+k}) with x_{t-d_conv+1} .. x_{t-1} read from conv_state, then
 * exactly mssm_step with that u_t.  conv_state (B, d_conv - 1, D) in
 * p->dtype, the previous inputs in time order (the x_prev of
 * mssm_conv_scan_fwd; after a prefill call, the last d_conv - 1 rows of its
 * history and x), is read and overwritten in place with x_{t-d_conv+2} .. x_t.
 * Shapes otherwise as mssm_step (x_t replaces u_t); conv_w, conv_b, d_conv as
 * in mssm_conv_scan_fwd (conv_state may be NULL only when d_conv = 1).
 * Calling it L times equals one mssm_conv_scan_fwd over L steps with
 * x_prev = conv_state and h0 = state.
 */
mssm_status mssm_conv_step(const mssm_problem* p, int32_t d_conv,
                           const void* x_t, const float* conv_w, const float* conv_b, void* conv_state,
                           const void* delta_t, const float* A,
                           const void* Bm_t, const void* Cm_t,
                           const float* Dskip, const void* z_t, const float* dt_bias,
                           float* state, void* y_t, void* hip_stream);

/*
 * Forward of the Mamba-2 layer, the state-space dual (SSD).  The pages name
 * Mamba-2 (the model list of "mamba.py: 一个简单高效的Mamba实现", the versions
 * paragraph of "Mamba SSM 架构") without its equations; the library reads it as
 * the selective scan above with, per head h, one scalar decay A[h] and one
 * step dt[b,t,h] shared by the head's headdim channels and all dstate states,
 * and Bm, Cm shared by all heads (one group):
 *
 *     Delta   = softplus(dt[b,t,h] + dt_bias[h])   (or without softplus)
 *     h_t[p,n] = exp(Delta A[h]) h_{t-1}[p,n] + Delta Bm[b,t,n] x[b,t,h,p]
 *     y[b,t,h,p] = sum_n Cm[b,t,n] h_t[p,n] + Dskip[h] x[b,t,h,p]
 *
 * i.e. mssm_scan_fwd over the H * P channels d = h * P + p with
 * A[d, n] = A[h], delta[b,t,d] = dt[b,t,h], Dskip[d] = Dskip[h].  Computed in
 * chunks of 64 steps as dense products on the matrix cores.
 *   x, y       (B, L, H, P)                dt        (B, L, H)
 *   Bm, Cm     (B, L, N)                   A, Dskip, dt_bias  (H) float32
 *   h0, h_final (B, H, P, N) float32
 * x, dt, Bm, Cm and y in p->dtype (MSSM_F32 or MSSM_BF16); arithmetic float32
 * throughout, bfloat16 outputs rounded to nearest even.
 * Required: p, x, dt, A, Bm, Cm, y.  Optional (NULL): Dskip, dt_bias (-> 0),
 * h0 (-> zeros), h_final (not written; may be the same buffer as h0, which
 * then advances in place).  y and the workspace may not alias any input.
 * Built for headdim P in {64, 128, 192, 256} and dstate N in {64, 128}: other
 * sizes -> MSSM_ERR_UNSUPPORTED (a head of P channels runs as P / 64 heads of
 * 64 channels that share its dt, A, Dskip and dt_bias).  Other errors as
 * mssm_scan_fwd; batch * nheads * headdim / 64 must be below 2^31 and
 * nheads * headdim below 2^23 (else MSSM_ERR_SHAPE).  workspace as
 * mssm_scan_fwd's, sized by mssm_ssd_fwd_workspace_bytes.
 */
typedef struct {
    int64_t batch;          /* B */
    int64_t seqlen;         /* L */
    int64_t nheads;         /* H */
    int64_t headdim;        /* P */
    int64_t dstate;         /* N */
    int32_t dtype;          /* mssm_dtype of x, dt, Bm, Cm, y */
    int32_t delta_softplus; /* nonzero: Delta = softplus(dt + dt_bias) */
} mssm_ssd_problem;

/* Bytes of device scratch mssm_ssd_fwd needs on the current device, which has
 * C compute units:
 *  - B * H >= C and not a multiple of C: one persistent workgroup per CU
 *    scans an equal share of all 64-step chunks, a (batch, head) pair split
 *    between two of them handing its state over; scratch: C + 1 flags (padded
 *    to 256 bytes) and C states of P * N floats;
 *  - otherwise 0 when there are at least 128 (batch, head) pairs or the
 *    sequence is shorter than 4 chunks;
 *  - otherwise the sequence is cut into time segments scanned in parallel, and
 *    the scratch holds each segment's state and log-decay,
 *    (B * H * segments * (P * N + 1)) floats, and with bfloat16 activations
 *    also float32 outputs (B * L * H * P floats) that the last pass completes
 *    and rounds once.
 * 0 for an invalid problem.  A workspace sized on one device may be too small
 * on another with more CUs (MSSM_ERR_WORKSPACE). */
size_t mssm_ssd_fwd_workspace_bytes(const mssm_ssd_problem* p);

mssm_status mssm_ssd_fwd(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                         const float* h0, void* y, float* h_final,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* Mamba-2 (state-space dual) backward: the adjoint of mssm_ssd_fwd (same
 * reading: one decay A[h] and one step size per head, shared by the head's P
 * channels and N states, and Bm, Cm shared by all heads).  Given dy (the
 * gradient of y) and optionally dh_final (of h_final), writes
 *   dx (B, L, H, P), ddt (B, L, H): gradient w.r.t. the raw step input dt
 *     (before dt_bias and softplus), dB, dC (B, L, N)  -- in p->dtype;
 *   dA (H), and optionally dD (H), ddt_bias (H), dh0 (B, H, P, N) -- float32.
 * Gradients are overwritten, not accumulated.  Computed in 64-step chunks on
 * the matrix cores: a pass storing the state entering every chunk, a reverse
 * pass storing the adjoint state leaving every chunk, a chunk-parallel pass
 * forming every gradient from them, and fixed-order reductions of the tied
 * parameters' gradients (bitwise reproducible; no atomics).
 * Required: p, x, dt, A, Bm, Cm, dy, dx, ddt, dA, dB, dC.  Optional (NULL):
 * Dskip, dt_bias (-> 0), h0 (-> zeros), dh_final (-> zeros), dD, ddt_bias,
 * dh0 (not written).  No output may alias an input or another output.
 * Sizes, errors and alignment as mssm_ssd_fwd; the workspace (sized by
 * mssm_ssd_bwd_workspace_bytes, never 0) holds the chunk states and adjoint
 * states, (B * H * (2 * ceil(L / 64) + 1) * P * N) floats, plus small
 * partials (with headdim above 64 also B * L * H * P / 64 floats of ddt per
 * 64-channel part of a head). */
size_t mssm_ssd_bwd_workspace_bytes(const mssm_ssd_problem* p);

mssm_status mssm_ssd_bwd(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                         const float* h0, const void* dy, const float* dh_final,
                         void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                         float* ddt_bias, float* dh0,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Training pair of the SSD layer, as mssm_scan_fwd_train / mssm_scan_bwd_saved
 * for the selective scan: the forward keeps the state entering every 64-step
 * chunk and the final state, (B, H, ceil(L / 64) + 1, P, N) float32 in the
 * caller-owned ctx (at least mssm_ssd_ctx_bytes), and the backward starts from
 * them instead of recomputing them with its first pass over the chunks.
 * mssm_ssd_fwd_train: arguments, outputs and errors of mssm_ssd_fwd plus ctx
 * (required); its workspace is mssm_ssd_fwd_train_workspace_bytes: that of
 * mssm_ssd_fwd, and where mssm_ssd_fwd cuts the sequence into time segments
 * (few (batch, head) pairs) also, from the next 256-byte boundary, one float
 * per (batch, sub-head, chunk): each chunk's decay from its segment's start,
 * with which a last pass turns the states a segment stored from its zero
 * start into the true ones.  y and h_final are those of mssm_ssd_fwd bit for
 * bit (the same kernels, which also store the states).
 * mssm_ssd_bwd_saved: arguments, outputs and errors of mssm_ssd_bwd with ctx
 * in place of h0 (the ctx holds it); workspace
 * mssm_ssd_bwd_saved_workspace_bytes (the states are not in it).
 */
size_t mssm_ssd_ctx_bytes(const mssm_ssd_problem* p);
size_t mssm_ssd_fwd_train_workspace_bytes(const mssm_ssd_problem* p);
mssm_status mssm_ssd_fwd_train(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                               const float* h0, void* y, float* h_final, void* ctx, size_t ctx_bytes,
                               void* workspace, size_t workspace_bytes, void* hip_stream);
size_t mssm_ssd_bwd_saved_workspace_bytes(const mssm_ssd_problem* p);
mssm_status mssm_ssd_bwd_saved(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                               const void* ctx, size_t ctx_bytes, const void* dy, const float* dh_final,
                               void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                               float* ddt_bias, float* dh0,
                               void* workspace, size_t workspace_bytes, void* hip_stream);

/* Static, human-readable name of a status code. */
const char* mssm_status_string(mssm_status s);

/* Build description: target architecture and library version. */
const char* mssm_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_H */
