// pad.hip -- state sizes that are not a power of two.
//
// The scan kernels are built for d_state N in {1, 2, 4, ..., 64} (state
// groups per wave, 16-byte rows).  Any other N <= 64 runs them at the next
// power of two N' with the extra states made inert: A = 0, Bm = 0, Cm = 0 and
// an initial state of 0 for them.  Such a state stays exactly 0 -- each step
// computes exp(Delta * 0) * 0 + Delta * 0 * u = 0 -- and adds Cm * h = 0 to
// every readout, so the N real states and y are those of the N-state scan.
// Bm, Cm, A and h0 are copied into zero-padded buffers in the caller's
// workspace (B*L*N' activations each for Bm and Cm: a small fraction of the
// B*L*D ones), and h_final and the gradients of Bm, Cm, A and h0 are copied
// back without the extra states.  The decode step has no workspace; it runs a
// kernel that loops over any N (scan_step.hip).
#include "launch.h"

#include <algorithm>

namespace mssm {
namespace {

size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t next_pow2(int64_t n) {
    int64_t p = 1;
    while (p < n) p <<= 1;
    return p;
}

// dst (rows, Np) <- src (rows, N), the extra columns zero; src null: all zero.
template <typename T>
__global__ __launch_bounds__(256) void pad_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows,
                                                  int N, int Np) {
    const int64_t total = rows * Np;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = i / Np;
        const int n = static_cast<int>(i - r * Np);
        dst[i] = (src && n < N) ? src[r * N + n] : T{};
    }
}

// dst (rows, N) <- the first N columns of src (rows, Np).
template <typename T>
__global__ __launch_bounds__(256) void unpad_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows,
                                                    int N, int Np) {
    const int64_t total = rows * N;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = i / N;
        const int n = static_cast<int>(i - r * N);
        dst[i] = src[r * Np + n];
    }
}

unsigned grid_for(int64_t n) { return static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 8192)); }

template <typename T>
hipError_t pad(const void* src, void* dst, int64_t rows, int64_t N, int64_t Np, hipStream_t st) {
    hipLaunchKernelGGL(pad_kernel<T>, dim3(grid_for(rows * Np)), dim3(256), 0, st, static_cast<const T*>(src),
                       static_cast<T*>(dst), rows, static_cast<int>(N), static_cast<int>(Np));
    return hipGetLastError();
}
template <typename T>
hipError_t unpad(const void* src, void* dst, int64_t rows, int64_t N, int64_t Np, hipStream_t st) {
    hipLaunchKernelGGL(unpad_kernel<T>, dim3(grid_for(rows * N)), dim3(256), 0, st, static_cast<const T*>(src),
                       static_cast<T*>(dst), rows, static_cast<int>(N), static_cast<int>(Np));
    return hipGetLastError();
}
hipError_t pad_act(int dtype, const void* src, void* dst, int64_t rows, int64_t N, int64_t Np, hipStream_t st) {
    return dtype == 1 ? pad<uint16_t>(src, dst, rows, N, Np, st) : pad<float>(src, dst, rows, N, Np, st);
}
hipError_t unpad_act(int dtype, const void* src, void* dst, int64_t rows, int64_t N, int64_t Np, hipStream_t st) {
    return dtype == 1 ? unpad<uint16_t>(src, dst, rows, N, Np, st) : unpad<float>(src, dst, rows, N, Np, st);
}

// Workspace of a padded call: the N'-state call's own, then the padded
// copies (each 256-byte aligned).  `saved`: the backward from a saved context.
struct PadLayout {
    size_t inner, bm, cm, A, h0, hf, dhf, dB, dC, dA, dh0, total;
};
PadLayout pad_layout(int64_t B, int64_t L, int64_t D, int64_t Np, int dtype, bool bwd, bool saved = false) {
    const size_t act = dtype == 1 ? 2 : 4;
    PadLayout p{};
    size_t off = 0;
    p.inner = off;
    off += al256(bwd ? (saved ? bwd_saved_ws_bytes(B, L, D, Np) : plan_bwd(B, L, D, Np).ws_bytes)
                     : plan_fwd(B, L, D, Np).ws_bytes);
    p.bm = off;    off += al256(static_cast<size_t>(B * L * Np) * act);
    p.cm = off;    off += al256(static_cast<size_t>(B * L * Np) * act);
    p.A = off;     off += al256(static_cast<size_t>(D * Np) * 4);
    p.h0 = off;    off += al256(static_cast<size_t>(B * D * Np) * 4);
    p.hf = off;    off += al256(static_cast<size_t>(B * D * Np) * 4);  // forward: h_final; backward: dh_final
    if (bwd) {
        p.dB = off;  off += al256(static_cast<size_t>(B * L * Np) * act);
        p.dC = off;  off += al256(static_cast<size_t>(B * L * Np) * act);
        p.dA = off;  off += al256(static_cast<size_t>(D * Np) * 4);
        p.dh0 = off; off += al256(static_cast<size_t>(B * D * Np) * 4);
    }
    p.dhf = p.hf;
    p.total = off;
    return p;
}

// Inputs common to the forward and the backward: Bm, Cm, A, h0 padded into
// the workspace and the arguments pointed at the copies.
hipError_t pad_inputs(ScanArgs& p, const ScanArgs& a, char* ws, const PadLayout& pl, hipStream_t st) {
    const int64_t Np = p.N, N = a.N;
    hipError_t e = pad_act(a.dtype, a.Bm, ws + pl.bm, a.B * a.L, N, Np, st);
    if (e == hipSuccess) e = pad_act(a.dtype, a.Cm, ws + pl.cm, a.B * a.L, N, Np, st);
    if (e == hipSuccess) e = pad<float>(a.A, ws + pl.A, a.D, N, Np, st);
    if (e == hipSuccess && a.h0) e = pad<float>(a.h0, ws + pl.h0, a.B * a.D, N, Np, st);
    p.Bm = ws + pl.bm;
    p.Cm = ws + pl.cm;
    p.A = reinterpret_cast<const float*>(ws + pl.A);
    p.h0 = a.h0 ? reinterpret_cast<const float*>(ws + pl.h0) : nullptr;
    p.workspace = ws + pl.inner;
    p.workspace_bytes = pl.bm - pl.inner;
    return e;
}

template <hipError_t (*LAUNCH)(const ScanArgs&, hipStream_t)>
hipError_t fwd_padded(const ScanArgs& a, hipStream_t st) {
    const int64_t Np = next_pow2(a.N);
    const PadLayout pl = pad_layout(a.B, a.L, a.D, Np, a.dtype, false);
    char* ws = static_cast<char*>(a.workspace);
    ScanArgs p = a;
    p.N = Np;
    hipError_t e = pad_inputs(p, a, ws, pl, st);
    p.h_final = a.h_final ? reinterpret_cast<float*>(ws + pl.hf) : nullptr;
    if (e == hipSuccess) e = LAUNCH(p, st);
    if (e == hipSuccess && a.h_final) e = unpad<float>(ws + pl.hf, a.h_final, a.B * a.D, a.N, Np, st);
    return e;
}

}  // namespace

bool needs_padding(int64_t N) { return N > 0 && (N & (N - 1)) != 0; }

size_t fwd_ws_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype) {
    if (!needs_padding(N)) return plan_fwd(B, L, D, N).ws_bytes;
    return pad_layout(B, L, D, next_pow2(N), dtype, false).total;
}

size_t bwd_ws_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype) {
    if (!needs_padding(N)) return plan_bwd(B, L, D, N).ws_bytes;
    return pad_layout(B, L, D, next_pow2(N), dtype, true).total;
}

hipError_t launch_fwd_any(const ScanArgs& a, hipStream_t st) {
    return needs_padding(a.N) ? fwd_padded<launch_fwd>(a, st) : launch_fwd(a, st);
}

hipError_t launch_conv_fwd_any(const ScanArgs& a, hipStream_t st) {
    return needs_padding(a.N) ? fwd_padded<launch_conv_fwd>(a, st) : launch_conv_fwd(a, st);
}

int64_t padded_dstate(int64_t N) { return needs_padding(N) ? next_pow2(N) : N; }

size_t bwd_saved_ws_bytes_any(int64_t B, int64_t L, int64_t D, int64_t N, int dtype) {
    if (!needs_padding(N)) return bwd_saved_ws_bytes(B, L, D, N);
    return pad_layout(B, L, D, next_pow2(N), dtype, true, true).total;
}

hipError_t launch_fwd_train_any(const ScanArgs& a, hipStream_t st) {
    return needs_padding(a.N) ? fwd_padded<launch_fwd_train>(a, st) : launch_fwd_train(a, st);
}

template <hipError_t (*LAUNCH)(const ScanArgs&, hipStream_t), bool SAVED>
hipError_t bwd_padded(const ScanArgs& a, hipStream_t st) {
    const int64_t Np = next_pow2(a.N), N = a.N;
    const PadLayout pl = pad_layout(a.B, a.L, a.D, Np, a.dtype, true, SAVED);
    char* ws = static_cast<char*>(a.workspace);
    ScanArgs p = a;
    p.N = Np;
    hipError_t e = pad_inputs(p, a, ws, pl, st);
    if (e == hipSuccess && a.dh_final) e = pad<float>(a.dh_final, ws + pl.dhf, a.B * a.D, N, Np, st);
    p.dh_final = a.dh_final ? reinterpret_cast<const float*>(ws + pl.dhf) : nullptr;
    p.dB = ws + pl.dB;
    p.dC = ws + pl.dC;
    p.dA = reinterpret_cast<float*>(ws + pl.dA);
    p.dh0 = a.dh0 ? reinterpret_cast<float*>(ws + pl.dh0) : nullptr;
    if (e == hipSuccess) e = LAUNCH(p, st);
    if (e == hipSuccess) e = unpad_act(a.dtype, ws + pl.dB, a.dB, a.B * a.L, N, Np, st);
    if (e == hipSuccess) e = unpad_act(a.dtype, ws + pl.dC, a.dC, a.B * a.L, N, Np, st);
    if (e == hipSuccess) e = unpad<float>(ws + pl.dA, a.dA, a.D, N, Np, st);
    if (e == hipSuccess && a.dh0) e = unpad<float>(ws + pl.dh0, a.dh0, a.B * a.D, N, Np, st);
    return e;
}

hipError_t launch_bwd_any(const ScanArgs& a, hipStream_t st) {
    return needs_padding(a.N) ? bwd_padded<launch_bwd, false>(a, st) : launch_bwd(a, st);
}

// The saved context holds N' states (its layout is that of the N'-state problem).
hipError_t launch_bwd_saved_any(const ScanArgs& a, hipStream_t st) {
    return needs_padding(a.N) ? bwd_padded<launch_bwd_saved, true>(a, st) : launch_bwd_saved(a, st);
}

}  // namespace mssm
