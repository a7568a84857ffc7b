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
// HBM-bound (read x and du, write dx): one thread per channel pair (one
// channel when D is odd) and time chunk, walking the chunk in time with the
// last four inputs and the last four g in registers, so every access is one
// coalesced row of 512 channels per workgroup.  A chunk also recomputes g for the 3 steps after it (its last dx
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

// V adjacent channels of one row: V = 2 moves 4-byte bf16 pairs / 8-byte fp32
// pairs (256 threads then cover 512 channels; wider rows per wave instruction).
template <int V>
__device__ __forceinline__ void load_vec(const float* p, int64_t i, float (&v)[V]) {
    if constexpr (V == 2) {
        const float2 q = *reinterpret_cast<const float2*>(p + i);
        v[0] = q.x;
        v[1] = q.y;
    } else {
        v[0] = p[i];
    }
}
template <int V>
__device__ __forceinline__ void load_vec(const uint16_t* p, int64_t i, float (&v)[V]) {
    if constexpr (V == 2) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(p + i);
        v[0] = bf16_lo(q);
        v[1] = bf16_hi(q);
    } else {
        v[0] = load_act(p, i);
    }
}
template <int V>
__device__ __forceinline__ void store_vec(float* p, int64_t i, const float (&v)[V]) {
    if constexpr (V == 2)
        *reinterpret_cast<float2*>(p + i) = make_float2(v[0], v[1]);
    else
        p[i] = v[0];
}
template <int V>
__device__ __forceinline__ void store_vec(uint16_t* p, int64_t i, const float (&v)[V]) {
    if constexpr (V == 2) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[0]));
        const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[1]));
        *reinterpret_cast<uint32_t*>(p + i) = lo | (hi << 16);
    } else {
        store_act(p, i, v[0]);
    }
}

// V channels per thread (V = 2 needs an even D: a pair never straddles the end).
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(ConvBwdKArgs a) {
    // workgroup -> (channel block, chunk, batch row), channel blocks fastest
    constexpr int kChan = kThreads * V;
    const int64_t dblocks = (a.D + kChan - 1) / kChan;
    const int64_t blk = blockIdx.x;
    const int64_t d = (blk % dblocks) * kChan + static_cast<int64_t>(threadIdx.x) * V;  // first of V channels
    const int64_t c = (blk / dblocks) % a.chunks;
    const int64_t b = blk / (dblocks * a.chunks);
    const int64_t D = a.D, L = a.L;
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - V;
    const int K = a.K;
    float w[V][kTaps], bias[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int k = 0; k < kTaps; ++k) w[v][k] = k >= kTaps - K ? a.w[(dc + v) * K + k - (kTaps - K)] : 0.0f;
        bias[v] = a.bias ? a.bias[dc + v] : 0.0f;
    }
    const T* __restrict__ x = static_cast<const T*>(a.x) + b * L * D + dc;
    const T* __restrict__ du = static_cast<const T*>(a.du) + b * L * D + dc;
    T* __restrict__ dx = static_cast<T*>(a.dx) + b * L * D + dc;
    const T* xp = a.x_prev ? static_cast<const T*>(a.x_prev) + b * (K - 1) * D + dc : nullptr;

    const int64_t t0 = c * a.T;
    const int64_t t1 = t0 + a.T < L ? t0 + a.T : L;
    // inputs x_{t0-3}, x_{t0-2}, x_{t0-1}: the sequence, else the history, else zero
    float xw[V][kTaps];
#pragma unroll
    for (int k = 0; k < kTaps - 1; ++k) {
        const int64_t t = t0 - (kTaps - 1) + k;
        float q[V];
        if (t >= 0)
            load_vec<V>(x, t * D, q);
        else if (xp && t >= 1 - K)
            load_vec<V>(xp, (K - 1 + t) * D, q);
        else
#pragma unroll
            for (int v = 0; v < V; ++v) q[v] = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) xw[v][k] = q[v];
    }
    float g[V][kTaps], pw[V][kTaps], pb[V];  // g_{t-3} .. g_t (zero before the sequence); partial sums
#pragma unroll
    for (int v = 0; v < V; ++v) {
        pb[v] = 0.0f;
#pragma unroll
        for (int k = 0; k < kTaps; ++k) g[v][k] = pw[v][k] = 0.0f;
    }
    // one step t with inputs (x_t, du_t) (`data`: t < L; else g_t = 0 past the end):
    // g_t, the partial sums (t inside the chunk), and dx_{t-3} once its four g are known
    auto step = [&](int64_t t, const float (&xt)[V], const float (&dut)[V], bool data) {
        float out[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float gt = 0.0f;
            if (data) {
                xw[v][kTaps - 1] = xt[v];
                float cc = bias[v];
#pragma unroll
                for (int k = 0; k < kTaps; ++k) cc = __builtin_fmaf(w[v][k], xw[v][k], cc);
                const float s = sigmoid(cc);
                gt = dut[v] * s * __builtin_fmaf(cc, 1.0f - s, 1.0f);
                if (t < t1) {
#pragma unroll
                    for (int k = 0; k < kTaps; ++k) pw[v][k] = __builtin_fmaf(gt, xw[v][k], pw[v][k]);
                    pb[v] += gt;
                }
#pragma unroll
                for (int k = 0; k < kTaps - 1; ++k) xw[v][k] = xw[v][k + 1];
            }
#pragma unroll
            for (int k = 0; k < kTaps - 1; ++k) g[v][k] = g[v][k + 1];
            g[v][kTaps - 1] = gt;
            // dx_tau, tau = t - 3: sum_k w_k g_{tau+3-k} = w_0 g_t + w_1 g_{t-1} + w_2 g_{t-2} + w_3 g_{t-3}
            float o = 0.0f;
#pragma unroll
            for (int k = 0; k < kTaps; ++k) o = __builtin_fmaf(w[v][k], g[v][kTaps - 1 - k], o);
            out[v] = o;
        }
        const int64_t tau = t - (kTaps - 1);
        if (valid) {
            if (tau >= t0 && tau < t1)
                store_vec<V>(dx, tau * D, out);
            else if (tau < 0 && tau >= 1 - K && a.dx_prev)  // chunk 0 only: the history rows
                store_vec<V>(static_cast<T*>(a.dx_prev) + b * (K - 1) * D + dc, (K - 1 + tau) * D, out);
        }
    };
    // steps t0 .. t1 + 2; those with data in groups of 8, the next group's
    // loads issued before the current group is computed (software pipeline)
    const int64_t tdata = t1 + kTaps - 1 < L ? t1 + kTaps - 1 : L;
    int64_t t = t0;
    constexpr int kGroup = 8;
    float xv[kGroup][V], dv[kGroup][V];
    auto fetch = [&](int64_t tt) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            load_vec<V>(x, (tt + j) * D, xv[j]);
            load_vec<V>(du, (tt + j) * D, dv[j]);
        }
    };
    if (t + kGroup <= tdata) fetch(t);
    for (; t + kGroup <= tdata; t += kGroup) {
        float xc[kGroup][V], dc_[kGroup][V];
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                xc[j][v] = xv[j][v];
                dc_[j][v] = dv[j][v];
            }
        if (t + 2 * kGroup <= tdata) fetch(t + kGroup);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) step(t + j, xc[j], dc_[j], true);
    }
    for (; t < tdata; ++t) {
        float xv[V], dv[V];
        load_vec<V>(x, t * D, xv);
        load_vec<V>(du, t * D, dv);
        step(t, xv, dv, true);
    }
    const float zero[V] = {};
    for (; t < t1 + kTaps - 1; ++t) step(t, zero, zero, false);
    if (valid) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float* p = a.part + ((b * a.chunks + c) * kPartRows) * D + d + v;
#pragma unroll
            for (int k = 0; k < kTaps; ++k) p[k * D] = pw[v][k];
            p[kTaps * D] = pb[v];
        }
    }
}

// dw and dbias: the partial sums of every (batch row, chunk), added in a fixed
// order.  A workgroup takes 64 of the (row, channel) sums; its 4 waves add one
// contiguous quarter of the partials each, then the quarters are added in order.
__global__ __launch_bounds__(256) void conv_bwd_reduce_kernel(ConvBwdKArgs a) {
    __shared__ float sq[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + lane;  // (row r, channel d)
    const int64_t D = a.D;
    const bool in = i < kPartRows * D;
    const int64_t ic = in ? i : 0;
    const int r = static_cast<int>(ic / D);
    const int64_t d = ic % D;
    const int64_t parts = a.B * a.chunks;
    const int64_t q0 = parts * wv / 4, q1 = parts * (wv + 1) / 4;
    const float* p = a.part + r * D + d;
    float s = 0.0f;
#pragma unroll 8
    for (int64_t q = q0; q < q1; ++q) s += p[q * kPartRows * D];
    sq[wv][lane] = s;
    __syncthreads();
    if (wv != 0 || !in) return;
    const int K = a.K;
    if (r < kTaps - K || (r == kTaps && !a.dbias)) return;  // zero-padded taps; no bias gradient asked
    const float t = ((sq[0][lane] + sq[1][lane]) + sq[2][lane]) + sq[3][lane];
    if (r == kTaps)
        a.dbias[d] = t;
    else
        a.dw[d * K + r - (kTaps - K)] = t;
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
    const int64_t chan = (D % 2 == 0 ? 2 : 1) * kThreads;  // channels per workgroup (pairs when D is even)
    p.workgroups = (D + chan - 1) / chan * p.chunks * B;
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
    const dim3 grid(static_cast<unsigned>(pl.workgroups));
    const bool pairs = s.D % 2 == 0;
    if (s.dtype == 1) {
        if (pairs)
            hipLaunchKernelGGL((conv_bwd_kernel<uint16_t, 2>), grid, dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((conv_bwd_kernel<uint16_t, 1>), grid, dim3(kThreads), 0, st, a);
    } else {
        if (pairs)
            hipLaunchKernelGGL((conv_bwd_kernel<float, 2>), grid, dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((conv_bwd_kernel<float, 1>), grid, dim3(kThreads), 0, st, a);
    }
    const int64_t n = kPartRows * s.D;
    hipLaunchKernelGGL(conv_bwd_reduce_kernel, dim3(static_cast<unsigned>((n + 63) / 64)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace mssm
