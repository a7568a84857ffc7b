// launch.h -- host-side interface between the C ABI (mssm_api.cpp) and the
// kernel launchers (scan_fwd.hip, scan_bwd.hip, scan_step.hip).  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mssm {

// Every pointer and size of one call, already validated by the C ABI layer.
struct ScanArgs {
    // problem
    int64_t B, L, D, N;
    int dtype;      // 0 = f32, 1 = bf16 (storage of u, delta, z, Bm, Cm, y, grads)
    int softplus;   // Delta = softplus(delta + dt_bias) when nonzero
    // forward inputs
    const void* u;
    const void* delta;
    const void* z;       // nullable
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;    // nullable
    const float* dt_bias;  // nullable
    const float* h0;       // nullable
    // forward outputs
    void* y;
    float* h_final;        // nullable
    // fused causal conv1d + SiLU front end (forward only; u is then its input x)
    const float* conv_w;   // (D, d_conv); null: no front end, u is the scan input
    const float* conv_b;   // nullable
    const void* x_prev;    // (B, d_conv - 1, D), nullable
    void* u_out;           // (B, L, D), nullable
    int d_conv;
    // backward inputs / outputs
    const void* dy;
    const float* dh_final; // nullable
    void* du;
    void* ddelta;
    void* dz;              // nullable
    void* dB;
    void* dC;
    float* dA;
    float* dD;             // nullable
    float* ddt_bias;       // nullable
    float* dh0;            // nullable
    // training context (mssm_scan_fwd_train writes it, mssm_scan_bwd_saved reads it)
    float* ctx_ckpt;       // (B, tiles, N, D) state before every 16-step tile; null: no context
    float* ctx_s;          // (B, L, D) readout before the gate, sum_n Cm h + Dskip u (only with z)
    // scratch
    void* workspace;
    size_t workspace_bytes;
};

// Channels per workgroup: one wave64 lane per channel.
constexpr int kChannelsPerBlock = 64;

// Forward schedule: how the time axis is cut into chunks.
struct FwdPlan {
    int64_t chunks;      // K >= 1
    int64_t chunk_len;   // steps per chunk (multiple of the time tile)
    size_t ws_bytes;     // workspace bytes (0 when K == 1)
};
FwdPlan plan_fwd(int64_t B, int64_t L, int64_t D, int64_t N);
hipError_t launch_fwd(const ScanArgs& a, hipStream_t s);
// launch_fwd with the library's own fixed scratch array (mssm_scan_fwd_noalloc)
// as the workspace; the caller has checked that the plan fits it.
hipError_t launch_fwd_noalloc(ScanArgs a, hipStream_t s);
// The forward behind the fused front end: a.u is x, a.conv_w (a.conv_b,
// a.x_prev) its causal conv; u = silu(conv(x) + bias) is formed inside the
// kernels (and written to a.u_out if set).  Same schedule and workspace as
// launch_fwd.
hipError_t launch_conv_fwd(const ScanArgs& a, hipStream_t s);  // with a.ctx_ckpt set: the training forward
// Backward pre-pass: the forward recurrence with, instead of y, the state
// before every 16-step tile (ckpt, (B, tiles, N, D)), sbar = dy * silu(z)
// ((B, L, D) float32) and dz; fwd_scratch is plan_fwd(...).ws_bytes of scratch.
hipError_t launch_fwd_prepass(const ScanArgs& a, void* fwd_scratch, float* ckpt, float* sbar, hipStream_t s);

struct BwdPlan {
    int64_t tile;        // time steps per recompute tile
    int64_t tiles;       // ceil(L / tile)
    int64_t chunks;      // K >= 1: the reverse walk cut into K time chunks (carry of the adjoint between them)
    int64_t chunk_tiles; // tiles per chunk (the last may have fewer)
    int64_t head_chunks; // walk 0 covers chunks [0, head_chunks), each later walk one chunk
    int64_t units;       // reverse walks per channel block: chunks - head_chunks + 1
    size_t ws_bytes;
};
BwdPlan plan_bwd(int64_t B, int64_t L, int64_t D, int64_t N);
hipError_t launch_bwd(const ScanArgs& a, hipStream_t s);

// Training context saved by the forward for the backward (power-of-two N):
// the state before every 16-step tile and the readout before the gate.
struct CtxLayout {
    size_t ckpt, s, total;
};
CtxLayout ctx_layout(int64_t B, int64_t L, int64_t D, int64_t N);
// The forward that also writes the context at a.ctx_ckpt / a.ctx_s (always the
// tiled kernels: the short-sequence path keeps no checkpoints).
hipError_t launch_fwd_train(const ScanArgs& a, hipStream_t s);
// The backward from a saved context: no pre-pass; the reverse walk forms
// sbar = dy silu(z) and dz = dy s silu'(z) from dy, z and the saved s.
size_t bwd_saved_ws_bytes(int64_t B, int64_t L, int64_t D, int64_t N);
hipError_t launch_bwd_saved(const ScanArgs& a, hipStream_t s);

hipError_t launch_step(const ScanArgs& a, float* state, hipStream_t s);
// The forward for short sequences: the state in registers across the L steps,
// the step's lane mapping; no workspace.  Used where measured faster than the
// tiled forward: up to 8 steps, and up to 64 steps over at most 32,768 (b, d)
// rows (at D = 5,120: B = 256, 1 step 56 us against 178; 4 steps 91 against
// 190; 16 steps 229 against 213; B = 4, 64 steps 41 against 74).
constexpr int64_t kTokensMaxL = 64;
inline bool use_tokens(int64_t B, int64_t L, int64_t D) {
    return L <= 8 || (L <= kTokensMaxL && B * D <= 32768);
}
hipError_t launch_tokens(const ScanArgs& a, hipStream_t s);

// Any state size <= 64 (pad.hip): powers of two run as they are, other sizes
// at the next power of two with the extra states inert (zero-padded Bm, Cm,
// A, h0 in the workspace).  The *_ws_bytes give the workspace of either.
bool needs_padding(int64_t N);
size_t fwd_ws_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype);
size_t bwd_ws_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype);
hipError_t launch_fwd_any(const ScanArgs& a, hipStream_t s);
hipError_t launch_conv_fwd_any(const ScanArgs& a, hipStream_t s);
hipError_t launch_bwd_any(const ScanArgs& a, hipStream_t s);
// The training pair at any N <= 64: the context is that of the N'-state
// problem (N' = padded_dstate(N), the next power of two), the backward's
// workspace holds its padded copies.
int64_t padded_dstate(int64_t N);
size_t bwd_saved_ws_bytes_any(int64_t B, int64_t L, int64_t D, int64_t N, int dtype);
hipError_t launch_fwd_train_any(const ScanArgs& a, hipStream_t s);
hipError_t launch_bwd_saved_any(const ScanArgs& a, hipStream_t s);
// Below this many (b, d) rows the short-sequence path loads 8 tokens' inputs
// at a time, the next 8 in flight while the current ones are computed (a few
// waves run the whole call and would otherwise wait on every token's loads).
constexpr int64_t kTokensDeepMaxRows = 4096;

// Backward of the conv1d + SiLU front end (a.u = x, a.conv_w, a.conv_b,
// a.x_prev, a.d_conv as in launch_conv_fwd): time chunks of T steps, partial
// sums of dw and dbias per (batch row, chunk) in the workspace.
struct ConvBwdPlan {
    int64_t T;           // steps per chunk
    int64_t chunks;
    int64_t workgroups;  // of the main kernel (must fit a 1-D grid)
    size_t ws_bytes;
};
ConvBwdPlan plan_conv_bwd(int64_t B, int64_t L, int64_t D);
struct ConvBwdIO {
    const void* du;
    void* dx;
    void* dx_prev;       // nullable
    float* dconv_w;
    float* dconv_b;      // nullable
};
hipError_t launch_conv_bwd(const ScanArgs& a, const ConvBwdIO& io, hipStream_t s);

}  // namespace mssm
