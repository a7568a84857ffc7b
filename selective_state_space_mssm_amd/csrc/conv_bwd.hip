// conv_bwd.hip -- backward of the causal conv1d + SiLU front end that
// mssm_conv_scan_fwd fuses into the forward scan.
//
// Forward (per batch row b and channel d, taps zero-padded to kConvTaps = 4,
// oldest input first): c_t = bias + sum_k w_k x_{t-3+k}, u_t = silu(c_t); the
// page "Mamba SSM 架构" configures the block with d_conv = 4, the mamba-minimal
// page ("PyTorch 한 파일에서의 Mamba 구현") runs the convolution as
// torch.nn.Conv1d.  Given du = dL/du:
//   g_t      = du_t * silu'(c_t),  silu'(c) = s (1 + c (1 - s)),  s = sigmoid(c)
//   dx_tau   = sum_k w_k g_{tau+3-k}          (tau from -3: the history x_prev)
//   dw_k     = sum_{b,t} g_t x_{t-3+k},  dbias = sum_{b,t} g_t
//
// HBM-bound (read x and du, write dx): one thread per channel and time chunk,
// walking the chunk in time with the last four inputs and the last four g in
// registers, so every access is one coalesced row of 256 channels per
// workgroup.  A chunk also recomputes g for the 3 steps after it (its last dx
// rows need them).  dw and dbias: per (batch row, chunk) partial sums, then a
// second kernel adds them in a fixed order (bitwise reproducible).
#include "device_common.h"
#include "launch.h"

namespace mssm {
namespace {

constexpr int kTaps = 4;          // widest conv; narrower ones run with leading taps zero
constexpr int kThreads = 256;     // channels per workgroup
constexpr int kPartRows = kTaps + 1;  // partial sums per channel: 4 taps and the bias

struct ConvBwdKArgs {
    const void* x;
    const float* w;        // (D, K)
    const float* bias;     // (D) nullable
    const void* x_prev;    // (B, K - 1, D) nullable
    const void* du;
    void* dx;
    void* dx_prev;         // (B, K - 1, D) nullable
    float* part;           // (B * chunks, kPartRows, D)
    float* dw;             // (D, K)
    float* dbias;          // (D) nullable
    int64_t B, L, D, T;    // T: steps per chunk
    int32_t K, chunks;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(ConvBwdKArgs a) {
    // workgroup -> (channel block, chunk, batch row), channel blocks fastest
    const int64_t dblocks = (a.D + kThreads - 1) / kThreads;
    const int64_t blk = blockIdx.x;
    const int64_t d = (blk % dblocks) * kThreads + threadIdx.x;
    const int64_t c = (blk / dblocks) % a.chunks;
    const int64_t b = blk / (dblocks * a.chunks);
    const int64_t D = a.D, L = a.L;
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - 1;
    const int K = a.K;
    float w[kTaps];
#pragma unroll
    for (int k = 0; k < kTaps; ++k) w[k] = k >= kTaps - K ? a.w[dc * K + k - (kTaps - K)] : 0.0f;
    const float bias = a.bias ? a.bias[dc] : 0.0f;
    const T* __restrict__ x = static_cast<const T*>(a.x) + b * L * D + dc;
    const T* __restrict__ du = static_cast<const T*>(a.du) + b * L * D + dc;
    T* __restrict__ dx = static_cast<T*>(a.dx) + b * L * D + dc;
    const T* xp = a.x_prev ? static_cast<const T*>(a.x_prev) + b * (K - 1) * D + dc : nullptr;

    const int64_t t0 = c * a.T;
    const int64_t t1 = t0 + a.T < L ? t0 + a.T : L;
    // inputs x_{t0-3}, x_{t0-2}, x_{t0-1}: the sequence, else the history, else zero
    float xw[kTaps];
#pragma unroll
    for (int k = 0; k < kTaps - 1; ++k) {
        const int64_t t = t0 - (kTaps - 1) + k;
        xw[k] = t >= 0 ? load_act(x, t * D) : ((xp && t >= 1 - K) ? load_act(xp, (K - 1 + t) * D) : 0.0f);
    }
    float g[kTaps] = {0.0f, 0.0f, 0.0f, 0.0f};  // g_{t-3} .. g_t (zero before the sequence)
    float pw[kTaps] = {0.0f, 0.0f, 0.0f, 0.0f}, pb = 0.0f;
    // one step t with inputs (x_t, du_t) (`data`: t < L; else g_t = 0 past the end):
    // g_t, the partial sums (t inside the chunk), and dx_{t-3} once its four g are known
    auto step = [&](int64_t t, float xt, float dut, bool data) {
        float gt = 0.0f;
        if (data) {
            xw[kTaps - 1] = xt;
            float cc = bias;
#pragma unroll
            for (int k = 0; k < kTaps; ++k) cc = __builtin_fmaf(w[k], xw[k], cc);
            const float s = sigmoid(cc);
            gt = dut * s * __builtin_fmaf(cc, 1.0f - s, 1.0f);
            if (t < t1) {
#pragma unroll
                for (int k = 0; k < kTaps; ++k) pw[k] = __builtin_fmaf(gt, xw[k], pw[k]);
                pb += gt;
            }
#pragma unroll
            for (int k = 0; k < kTaps - 1; ++k) xw[k] = xw[k + 1];
        }
#pragma unroll
        for (int k = 0; k < kTaps - 1; ++k) g[k] = g[k + 1];
        g[kTaps - 1] = gt;
        // dx_tau, tau = t - 3: sum_k w_k g_{tau+3-k} = w_0 g_t + w_1 g_{t-1} + w_2 g_{t-2} + w_3 g_{t-3}
        const int64_t tau = t - (kTaps - 1);
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < kTaps; ++k) v = __builtin_fmaf(w[k], g[kTaps - 1 - k], v);
        if (valid) {
            if (tau >= t0 && tau < t1)
                store_act(dx, tau * D, v);
            else if (tau < 0 && tau >= 1 - K && a.dx_prev)  // chunk 0 only: the history rows
                store_act(static_cast<T*>(a.dx_prev) + b * (K - 1) * D + dc, (K - 1 + tau) * D, v);
        }
    };
    // steps t0 .. t1 + 2; those with data in groups of 8 with all 16 loads issued first
    const int64_t tdata = t1 + kTaps - 1 < L ? t1 + kTaps - 1 : L;
    int64_t t = t0;
    constexpr int kGroup = 8;
    for (; t + kGroup <= tdata; t += kGroup) {
        float xv[kGroup], dv[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            xv[j] = load_act(x, (t + j) * D);
            dv[j] = load_act(du, (t + j) * D);
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) step(t + j, xv[j], dv[j], true);
    }
    for (; t < tdata; ++t) step(t, load_act(x, t * D), load_act(du, t * D), true);
    for (; t < t1 + kTaps - 1; ++t) step(t, 0.0f, 0.0f, false);
    if (valid) {
        float* p = a.part + ((b * a.chunks + c) * kPartRows) * D + d;
#pragma unroll
        for (int k = 0; k < kTaps; ++k) p[k * D] = pw[k];
        p[kTaps * D] = pb;
    }
}

// dw and dbias: the partial sums of every (batch row, chunk), added in order.
__global__ __launch_bounds__(256) void conv_bwd_reduce_kernel(ConvBwdKArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (row r, channel d)
    const int64_t D = a.D;
    if (i >= kPartRows * D) return;
    const int r = static_cast<int>(i / D);
    const int64_t d = i % D;
    const int K = a.K;
    if (r < kTaps - K || (r == kTaps && !a.dbias)) return;  // zero-padded taps; no bias gradient asked
    const int64_t parts = a.B * a.chunks;
    const float* p = a.part + r * D + d;
    float s = 0.0f;
#pragma unroll 8
    for (int64_t q = 0; q < parts; ++q) s += p[q * kPartRows * D];
    if (r == kTaps)
        a.dbias[d] = s;
    else
        a.dw[d * K + r - (kTaps - K)] = s;
}

}  // namespace

ConvBwdPlan plan_conv_bwd(int64_t B, int64_t L, int64_t D) {
    // chunks of at least 64 steps (the 3 recomputed steps per chunk stay < 5 %),
    // and at most about 1024 (batch row, chunk) partial sums per channel
    int64_t T = (B * L + 1023) / 1024;
    T = T < 64 ? 64 : T;
    ConvBwdPlan p{};
    p.T = T;
    p.chunks = (L + T - 1) / T;
    p.ws_bytes = static_cast<size_t>(B) * p.chunks * kPartRows * D * sizeof(float);
    p.workgroups = (D + kThreads - 1) / kThreads * p.chunks * B;
    return p;
}

hipError_t launch_conv_bwd(const ScanArgs& s, const ConvBwdIO& io, hipStream_t st) {
    const ConvBwdPlan pl = plan_conv_bwd(s.B, s.L, s.D);
    ConvBwdKArgs a{};
    a.x = s.u; a.w = s.conv_w; a.bias = s.conv_b; a.x_prev = s.x_prev; a.du = io.du;
    a.dx = io.dx; a.dx_prev = io.dx_prev; a.part = static_cast<float*>(s.workspace);
    a.dw = io.dconv_w; a.dbias = io.dconv_b;
    a.B = s.B; a.L = s.L; a.D = s.D; a.T = pl.T;
    a.K = s.d_conv; a.chunks = static_cast<int32_t>(pl.chunks);
    const dim3 grid(static_cast<unsigned>((s.D + kThreads - 1) / kThreads * pl.chunks * s.B));
    if (s.dtype == 1)
        hipLaunchKernelGGL(conv_bwd_kernel<uint16_t>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(conv_bwd_kernel<float>, grid, dim3(kThreads), 0, st, a);
    const int64_t n = kPartRows * s.D;
    hipLaunchKernelGGL(conv_bwd_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace mssm
