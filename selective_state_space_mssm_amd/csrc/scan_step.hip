// scan_step.hip -- one token of the recurrent form (streaming decode).
//
// The step function of the page "mamba.py: 一个简单高效的Mamba实现" (updates
// section: RNN form for inference): read the carried state h (B, D, N), apply
// one iteration of the selective-scan recurrence, write h back in place and
// emit y_t.  The cost is the state read + write (8 B per state element) plus
// the launch, so one thread per (b, d) streams its N contiguous states with
// 16-byte accesses; consecutive threads touch consecutive 4*N-byte rows.
#include "device_common.h"
#include "launch.h"

namespace mssm {
namespace {

struct StepKArgs {
    const void* u;
    const void* delta;
    const void* z;
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;
    const float* dt_bias;
    float* state;
    void* y;
    int64_t B, D;
    int32_t softplus;
};

template <typename T, int N>
__global__ __launch_bounds__(256) void scan_step_kernel(StepKArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (b, d)
    if (i >= a.B * a.D) return;
    const int64_t b = i / a.D, d = i % a.D;
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm) + b * N;
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm) + b * N;
    const float uu = load_act(static_cast<const T*>(a.u), i);
    const float x = load_act(static_cast<const T*>(a.delta), i) + (a.dt_bias ? a.dt_bias[d] : 0.0f);
    const float dt = a.softplus ? softplus(x) : x;
    const float du = dt * uu;
    const float dtl = dt * kLog2e;
    float* __restrict__ st = a.state + i * N;
    const float* __restrict__ Ad = a.A + d * N;
    float s = 0.0f;
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int n = 0; n < N; n += 4) {
            float4 h = *reinterpret_cast<const float4*>(st + n);
            const float4 av = *reinterpret_cast<const float4*>(Ad + n);
            h.x = __builtin_fmaf(fast_exp2(dtl * av.x), h.x, du * load_act(Bm, n + 0));
            h.y = __builtin_fmaf(fast_exp2(dtl * av.y), h.y, du * load_act(Bm, n + 1));
            h.z = __builtin_fmaf(fast_exp2(dtl * av.z), h.z, du * load_act(Bm, n + 2));
            h.w = __builtin_fmaf(fast_exp2(dtl * av.w), h.w, du * load_act(Bm, n + 3));
            s = __builtin_fmaf(load_act(Cm, n + 0), h.x, s);
            s = __builtin_fmaf(load_act(Cm, n + 1), h.y, s);
            s = __builtin_fmaf(load_act(Cm, n + 2), h.z, s);
            s = __builtin_fmaf(load_act(Cm, n + 3), h.w, s);
            *reinterpret_cast<float4*>(st + n) = h;
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float h = __builtin_fmaf(fast_exp2(dtl * Ad[n]), st[n], du * load_act(Bm, n));
            s = __builtin_fmaf(load_act(Cm, n), h, s);
            st[n] = h;
        }
    }
    s = __builtin_fmaf(a.Dskip ? a.Dskip[d] : 0.0f, uu, s);
    if (a.z) s *= silu(load_act(static_cast<const T*>(a.z), i));
    store_act(static_cast<T*>(a.y), i, s);
}

template <typename T>
hipError_t dispatch(const StepKArgs& k, int64_t N, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((k.B * k.D + 255) / 256));
    switch (N) {
        case 1: hipLaunchKernelGGL((scan_step_kernel<T, 1>), grid, dim3(256), 0, st, k); break;
        case 2: hipLaunchKernelGGL((scan_step_kernel<T, 2>), grid, dim3(256), 0, st, k); break;
        case 4: hipLaunchKernelGGL((scan_step_kernel<T, 4>), grid, dim3(256), 0, st, k); break;
        case 8: hipLaunchKernelGGL((scan_step_kernel<T, 8>), grid, dim3(256), 0, st, k); break;
        case 16: hipLaunchKernelGGL((scan_step_kernel<T, 16>), grid, dim3(256), 0, st, k); break;
        case 32: hipLaunchKernelGGL((scan_step_kernel<T, 32>), grid, dim3(256), 0, st, k); break;
        case 64: hipLaunchKernelGGL((scan_step_kernel<T, 64>), grid, dim3(256), 0, st, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const ScanArgs& s, float* state, hipStream_t st) {
    StepKArgs k{};
    k.u = s.u; k.delta = s.delta; k.z = s.z; k.Bm = s.Bm; k.Cm = s.Cm;
    k.A = s.A; k.Dskip = s.Dskip; k.dt_bias = s.dt_bias;
    k.state = state; k.y = s.y; k.B = s.B; k.D = s.D; k.softplus = s.softplus;
    return s.dtype == 1 ? dispatch<uint16_t>(k, s.N, st) : dispatch<float>(k, s.N, st);
}

}  // namespace mssm
