// scan_step.hip -- one token of the recurrent form (streaming decode).
//
// The step function of the page "mamba.py: 一个简单高效的Mamba实现" (updates
// section: RNN form for inference): read the carried state h (B, D, N), apply
// one iteration of the selective-scan recurrence, write h back in place and
// emit y_t.  The cost is the state read + write (8 B per state element) plus
// the launch.  A (b, d) row of N states is handled by N/4 lanes (one lane for
// N < 4), each owning 4 consecutive states as one 16-byte access, so a wave
// reads and writes one contiguous stretch of the state; the row's lanes add
// their partial readouts with lane shuffles and the first one stores y.
//
// With the fused conv front end (mssm_conv_step), the step's u is formed from
// x_t and the conv state, the d_conv - 1 previous inputs (B, d_conv - 1, D):
// u = silu(bias + sum_k w_k x_{t-d_conv+1+k}), and x_t is shifted into the
// conv state in place.  Every address of the conv state is read and written
// by one lane (lane q owns row q when a row has four lanes or more, else the
// row's first lane owns all rows), so its read precedes its write in program
// order.
//
// scan_tokens_kernel: mssm_scan_fwd's path for short sequences (a few tokens
// over many rows), the same mapping with the state held in registers across
// the L tokens.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

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
    // fused conv front end (u is then x_t)
    const float* conv_w;   // (D, K)
    const float* conv_b;   // (D) nullable
    void* conv_state;      // (B, K - 1, D), in/out
    int32_t K;
};

template <typename T, int N, bool CONV>
__global__ __launch_bounds__(256) void scan_step_kernel(StepKArgs a) {
    constexpr int V = N >= 4 ? 4 : N;  // states per lane
    constexpr int R = N / V;           // lanes per (b, d) row: a power of two dividing 64
    const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t i = g / R;  // (b, d); the R lanes of a row are all in range or all out
    const int q = static_cast<int>(g % R);
    if (i >= a.B * a.D) return;
    const int64_t b = i / a.D, d = i % a.D;
    const int n0 = q * V;
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm) + b * N + n0;
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm) + b * N + n0;
    float uu = load_act(static_cast<const T*>(a.u), i);
    if constexpr (CONV) {
        // the row's first lane alone reads and shifts the conv state (its loads
        // and stores of one address then come from one thread, in program
        // order); the row's other lanes take c from it
        constexpr int kTaps = 4;
        float c = 0.0f;
        if constexpr (R >= kTaps) {
            // four or more lanes per row: lane q < K takes tap q, whose input is
            // conv-state row q (x_t for q = K - 1); lane q < K - 1 then writes
            // row q from lane q + 1's input (each state address is read and
            // written by one lane); the products are summed over the row
            const int K = a.K;
            T* cs = static_cast<T*>(a.conv_state) + b * (K - 1) * a.D + d;  // (b, 0, d)
            const float in = q < K - 1 ? load_act(cs, q * a.D) : uu;
            float prod = q < K ? a.conv_w[d * K + q] * in : 0.0f;
            // lane q + 1's input (row_shl:1 within the 16-lane row; a row's last lane gets 0, and only lanes
            // q < K - 1 <= 2 use it, which never end a row)
            const float next = dpp_move<0x101>(in);
            if (q < K - 1) store_act(cs, q * a.D, next);
            prod = group_sum<R>(prod);
            c = (a.conv_b ? a.conv_b[d] : 0.0f) + prod;
        } else if (q == 0) {
            const int K = a.K;
            T* cs = static_cast<T*>(a.conv_state) + b * (K - 1) * a.D + d;  // (b, 0, d)
            float xs[kTaps - 1];  // x_{t-3} .. x_{t-1}; the state holds x_{t-K+1} .. x_{t-1} in its K - 1 rows
#pragma unroll
            for (int k = 0; k < kTaps - 1; ++k)
                xs[k] = k >= kTaps - K ? load_act(cs, (k - (kTaps - K)) * a.D) : 0.0f;
            c = a.conv_b ? a.conv_b[d] : 0.0f;
#pragma unroll
            for (int k = 0; k < kTaps - 1; ++k)
                if (k >= kTaps - K) c = __builtin_fmaf(a.conv_w[d * K + k - (kTaps - K)], xs[k], c);
            c = __builtin_fmaf(a.conv_w[d * K + K - 1], uu, c);
            // shift x_t in: row j <- row j + 1, the last row <- x_t
#pragma unroll
            for (int k = kTaps - 1 - (kTaps - 2); k < kTaps - 1; ++k)
                if (k - 1 >= kTaps - K) store_act(cs, (k - 1 - (kTaps - K)) * a.D, xs[k]);
            if (K > 1) store_act(cs, (K - 2) * a.D, uu);
        }
        if constexpr (R == 2) c = dpp_move<0xA0>(c);  // the pair's first lane's c: quad_perm [0, 0, 2, 2]
        static_assert(R == 1 || R == 2 || R >= kTaps, "rows of 1, 2 or at least kTaps lanes");
        uu = silu(c);
    }
    const float x = load_act(static_cast<const T*>(a.delta), i) + (a.dt_bias ? a.dt_bias[d] : 0.0f);
    const float dt = a.softplus ? softplus(x) : x;
    const float du = dt * uu;
    const float dtl = dt * kLog2e;
    float* __restrict__ st = a.state + i * N + n0;
    const float* __restrict__ Ad = a.A + d * N + n0;
    float s = 0.0f;
    if constexpr (V == 4) {
        float4 h = *reinterpret_cast<const float4*>(st);
        const float4 av = *reinterpret_cast<const float4*>(Ad);
        h.x = __builtin_fmaf(fast_exp2(dtl * av.x), h.x, du * load_act(Bm, 0));
        h.y = __builtin_fmaf(fast_exp2(dtl * av.y), h.y, du * load_act(Bm, 1));
        h.z = __builtin_fmaf(fast_exp2(dtl * av.z), h.z, du * load_act(Bm, 2));
        h.w = __builtin_fmaf(fast_exp2(dtl * av.w), h.w, du * load_act(Bm, 3));
        s = load_act(Cm, 0) * h.x;
        s = __builtin_fmaf(load_act(Cm, 1), h.y, s);
        s = __builtin_fmaf(load_act(Cm, 2), h.z, s);
        s = __builtin_fmaf(load_act(Cm, 3), h.w, s);
        *reinterpret_cast<float4*>(st) = h;
    } else {
#pragma unroll
        for (int n = 0; n < V; ++n) {
            const float h = __builtin_fmaf(fast_exp2(dtl * Ad[n]), st[n], du * load_act(Bm, n));
            s = __builtin_fmaf(load_act(Cm, n), h, s);
            st[n] = h;
        }
    }
    s = group_sum<R>(s);
    if (q == 0) {
        s = __builtin_fmaf(a.Dskip ? a.Dskip[d] : 0.0f, uu, s);
        if (a.z) s *= silu(load_act(static_cast<const T*>(a.z), i));
        store_act(static_cast<T*>(a.y), i, s);
    }
}

// The step for a state size that is not a power of two (any N <= 64): one
// lane per (b, d) row, looping over the N states of the row in memory.
template <typename T, bool CONV>
__global__ __launch_bounds__(256) void scan_step_any_kernel(StepKArgs a, int N) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= a.B * a.D) return;
    const int64_t b = i / a.D, d = i % a.D;
    float uu = load_act(static_cast<const T*>(a.u), i);
    if constexpr (CONV) {
        // as the single-lane rows of scan_step_kernel: x_{t-K+1} .. x_{t-1} from the conv state, x_t shifted in
        const int K = a.K;
        T* cs = static_cast<T*>(a.conv_state) + b * (K - 1) * a.D + d;  // (b, 0, d)
        float c = a.conv_b ? a.conv_b[d] : 0.0f;
        for (int k = 0; k < K - 1; ++k) {  // row k is read before row k is rewritten (as row (k + 1) - 1)
            const float xk = load_act(cs, k * a.D);
            c = __builtin_fmaf(a.conv_w[d * K + k], xk, c);
            if (k > 0) store_act(cs, (k - 1) * a.D, xk);
        }
        c = __builtin_fmaf(a.conv_w[d * K + K - 1], uu, c);
        if (K > 1) store_act(cs, (K - 2) * a.D, uu);
        uu = silu(c);
    }
    const float x = load_act(static_cast<const T*>(a.delta), i) + (a.dt_bias ? a.dt_bias[d] : 0.0f);
    const float dt = a.softplus ? softplus(x) : x;
    const float du = dt * uu;
    const float dtl = dt * kLog2e;
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm) + b * N;
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm) + b * N;
    float* __restrict__ st = a.state + i * N;
    const float* __restrict__ Ad = a.A + d * N;
    float s = 0.0f;
    for (int n = 0; n < N; ++n) {
        const float h = __builtin_fmaf(fast_exp2(dtl * Ad[n]), st[n], du * load_act(Bm, n));
        s = __builtin_fmaf(load_act(Cm, n), h, s);
        st[n] = h;
    }
    s = __builtin_fmaf(a.Dskip ? a.Dskip[d] : 0.0f, uu, s);
    if (a.z) s *= silu(load_act(static_cast<const T*>(a.z), i));
    store_act(static_cast<T*>(a.y), i, s);
}

// V consecutive values (V = 4: one 8-byte bf16 / 16-byte fp32 load; the
// lane's first state index is a multiple of 4, so the address is aligned).
template <int V>
__device__ __forceinline__ void load_states(const uint16_t* p, float (&v)[V]) {
    if constexpr (V == 4) {
        const uint2 q = *reinterpret_cast<const uint2*>(p);
        v[0] = bf16_lo(q.x);
        v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y);
        v[3] = bf16_hi(q.y);
    } else {
#pragma unroll
        for (int n = 0; n < V; ++n) v[n] = load_act(p, n);
    }
}
template <int V>
__device__ __forceinline__ void load_states(const float* p, float (&v)[V]) {
    if constexpr (V == 4) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    } else {
#pragma unroll
        for (int n = 0; n < V; ++n) v[n] = p[n];
    }
}

// Short sequences: the forward over L steps with the step's mapping (N/4
// lanes per (b, d) row, 4 states per lane, rows of the state contiguous),
// the state in registers from h0 to h_final, so it moves once per call
// rather than once per token; inputs at (b, t, d) and (b, t, n) as the
// forward takes them.  The forward kernel's tile pipeline needs whole 16-step
// tiles to pay for itself; for a few tokens over many (b, d) rows this is
// the faster form.
struct TokKArgs {
    const void* u;
    const void* delta;
    const void* z;
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;
    const float* dt_bias;
    const float* h0;      // nullable: zeros
    float* h_final;       // nullable; may be h0
    void* y;
    int64_t B, L, D;
    int32_t softplus;
};

template <typename T, int N>
__global__ __launch_bounds__(256) void scan_tokens_kernel(TokKArgs a) {
    constexpr int V = N >= 4 ? 4 : N;
    constexpr int R = N / V;
    const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t i = g / R;  // (b, d); a row's lanes are all in range or all out
    const int q = static_cast<int>(g % R);
    if (i >= a.B * a.D) return;
    const int64_t b = i / a.D, d = i % a.D;
    const int n0 = q * V;
    const int64_t D = a.D, L = a.L;
    float A2[V], h[V];
#pragma unroll
    for (int n = 0; n < V; ++n) {
        A2[n] = a.A[d * N + n0 + n] * kLog2e;
        h[n] = a.h0 ? a.h0[i * N + n0 + n] : 0.0f;
    }
    const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
    const float Dk = a.Dskip ? a.Dskip[d] : 0.0f;
    const T* __restrict__ u = static_cast<const T*>(a.u) + b * L * D + d;
    const T* __restrict__ dl = static_cast<const T*>(a.delta) + b * L * D + d;
    const T* __restrict__ z = a.z ? static_cast<const T*>(a.z) + b * L * D + d : nullptr;
    T* __restrict__ y = static_cast<T*>(a.y) + b * L * D + d;
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm) + b * L * N + n0;
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm) + b * L * N + n0;
    // token t's inputs are loaded during token t - 1 (one token of prefetch)
    float nu = load_act(u, 0), nx = load_act(dl, 0), nz = z ? load_act(z, 0) : 0.0f;
    float nb[V], nc[V];
    load_states<V>(Bm, nb);
    load_states<V>(Cm, nc);
    for (int64_t t = 0; t < L; ++t) {
        const float uu = nu, zz = nz;
        const float x = nx + bias;
        float bv[V], cv[V];  // this lane's V values of Bm_t, Cm_t: one vector load each
#pragma unroll
        for (int n = 0; n < V; ++n) {
            bv[n] = nb[n];
            cv[n] = nc[n];
        }
        if (t + 1 < L) {
            nu = load_act(u, (t + 1) * D);
            nx = load_act(dl, (t + 1) * D);
            if (z) nz = load_act(z, (t + 1) * D);
            load_states<V>(Bm + (t + 1) * N, nb);
            load_states<V>(Cm + (t + 1) * N, nc);
        }
        const float dt = a.softplus ? softplus(x) : x;
        const float du = dt * uu;
        float s = 0.0f;
#pragma unroll
        for (int n = 0; n < V; ++n) {
            h[n] = __builtin_fmaf(fast_exp2(dt * A2[n]), h[n], du * bv[n]);  // A2 = A log2(e)
            s = __builtin_fmaf(cv[n], h[n], s);
        }
        s = group_sum<R>(s);
        if (q == 0) {
            s = __builtin_fmaf(Dk, uu, s);
            if (z) s *= silu(zz);
            store_act(y, t * D, s);
        }
    }
    if (a.h_final) {
#pragma unroll
        for (int n = 0; n < V; ++n) a.h_final[i * N + n0 + n] = h[n];
    }
}

// The same for few (b, d) rows, where a handful of waves run the whole call
// and each token's loads would sit on the critical path: the inputs of P
// tokens are loaded together, and the next P tokens' loads are issued before
// the current P are computed (two register sets used in turn), so only the
// first group's load latency is exposed.
template <typename T, int N, int P>
__global__ __launch_bounds__(256) void scan_tokens_deep_kernel(TokKArgs a) {
    // one state per lane up to 16 states (more waves share the work than with
    // four, and the readout sum stays within a 16-lane DPP row): V states per
    // lane, R = N / V <= 16 lanes per (b, d) row
    constexpr int V = N > 16 ? N / 16 : 1;
    constexpr int R = N / V;
    const int g = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
    const int i = g / R;
    const int q = g % R;
    if (i >= a.B * a.D) return;
    // few rows of few tokens: every offset below fits 32 bits
    const int D = static_cast<int>(a.D), L = static_cast<int>(a.L);
    const int b = i / D, d = i % D;
    const int n0 = q * V;
    float A2[V], h[V];
#pragma unroll
    for (int n = 0; n < V; ++n) {
        A2[n] = a.A[d * N + n0 + n] * kLog2e;
        h[n] = a.h0 ? a.h0[static_cast<int64_t>(i) * N + n0 + n] : 0.0f;
    }
    const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
    const float Dk = a.Dskip ? a.Dskip[d] : 0.0f;
    const int row = b * L * D + d;  // element (b, 0, d)
    const T* __restrict__ u = static_cast<const T*>(a.u) + row;
    const T* __restrict__ dl = static_cast<const T*>(a.delta) + row;
    const T* __restrict__ z = a.z ? static_cast<const T*>(a.z) + row : nullptr;
    T* __restrict__ y = static_cast<T*>(a.y) + row;
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm) + b * L * N + n0;
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm) + b * L * N + n0;
    float ru[2][P], rx[2][P], rz[2][P], rb[2][P][V], rc[2][P][V];
    // inputs of tokens t0 .. t0 + P - 1 into set S (past the end: the last token again, never used)
    auto load = [&](auto set, int t0) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int t = min(t0 + j, L - 1);
            ru[S][j] = load_act(u, t * D);
            rx[S][j] = load_act(dl, t * D);
            rz[S][j] = z ? load_act(z, t * D) : 0.0f;
            load_states<V>(Bm + t * N, rb[S][j]);
            load_states<V>(Cm + t * N, rc[S][j]);
        }
    };
    auto compute = [&](auto set, int t0) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            if (t0 + j < L) {
                const float x = rx[S][j] + bias;
                const float dt = a.softplus ? softplus(x) : x;
                const float du = dt * ru[S][j];
                float s = 0.0f;
#pragma unroll
                for (int n = 0; n < V; ++n) {
                    h[n] = __builtin_fmaf(fast_exp2(dt * A2[n]), h[n], du * rb[S][j][n]);
                    s = __builtin_fmaf(rc[S][j][n], h[n], s);
                }
                s = group_sum<R>(s);
                if (q == 0) {
                    s = __builtin_fmaf(Dk, ru[S][j], s);
                    if (z) s *= silu(rz[S][j]);
                    store_act(y, (t0 + j) * D, s);
                }
            }
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    load(S0{}, 0);
    for (int t0 = 0; t0 < L; t0 += 2 * P) {
        load(S1{}, t0 + P);
        compute(S0{}, t0);
        if (t0 + P >= L) break;
        load(S0{}, t0 + 2 * P);
        compute(S1{}, t0 + P);
    }
    if (a.h_final) {
#pragma unroll
        for (int n = 0; n < V; ++n) a.h_final[static_cast<int64_t>(i) * N + n0 + n] = h[n];
    }
}

template <typename T, bool CONV>
hipError_t dispatch(const StepKArgs& k, int64_t N, hipStream_t st) {
    if ((N & (N - 1)) != 0) {  // not a power of two: one lane per row
        hipLaunchKernelGGL((scan_step_any_kernel<T, CONV>), dim3(static_cast<unsigned>((k.B * k.D + 255) / 256)),
                           dim3(256), 0, st, k, static_cast<int>(N));
        return hipGetLastError();
    }
    const int64_t lanes = k.B * k.D * (N >= 4 ? N / 4 : 1);  // N/4 lanes per (b, d) row
    const dim3 grid(static_cast<unsigned>((lanes + 255) / 256));
    switch (N) {
        case 1: hipLaunchKernelGGL((scan_step_kernel<T, 1, CONV>), grid, dim3(256), 0, st, k); break;
        case 2: hipLaunchKernelGGL((scan_step_kernel<T, 2, CONV>), grid, dim3(256), 0, st, k); break;
        case 4: hipLaunchKernelGGL((scan_step_kernel<T, 4, CONV>), grid, dim3(256), 0, st, k); break;
        case 8: hipLaunchKernelGGL((scan_step_kernel<T, 8, CONV>), grid, dim3(256), 0, st, k); break;
        case 16: hipLaunchKernelGGL((scan_step_kernel<T, 16, CONV>), grid, dim3(256), 0, st, k); break;
        case 32: hipLaunchKernelGGL((scan_step_kernel<T, 32, CONV>), grid, dim3(256), 0, st, k); break;
        case 64: hipLaunchKernelGGL((scan_step_kernel<T, 64, CONV>), grid, dim3(256), 0, st, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t dispatch_tokens(const TokKArgs& k, int64_t N, hipStream_t st) {
    const int64_t lanes = k.B * k.D * (N >= 4 ? N / 4 : 1);
    const dim3 grid(static_cast<unsigned>((lanes + 255) / 256));
    if (k.B * k.D <= kTokensDeepMaxRows && k.L > 8) {  // few rows: loads of 8 tokens at a time, 8 ahead
        constexpr int P = 8;
        const int64_t deep_lanes = k.B * k.D * (N > 16 ? 16 : N);  // one state per lane up to N = 16
        const dim3 grid(static_cast<unsigned>((deep_lanes + 255) / 256));
        switch (N) {
            case 1: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 1, P>), grid, dim3(256), 0, st, k); break;
            case 2: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 2, P>), grid, dim3(256), 0, st, k); break;
            case 4: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 4, P>), grid, dim3(256), 0, st, k); break;
            case 8: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 8, P>), grid, dim3(256), 0, st, k); break;
            case 16: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 16, P>), grid, dim3(256), 0, st, k); break;
            case 32: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 32, P>), grid, dim3(256), 0, st, k); break;
            case 64: hipLaunchKernelGGL((scan_tokens_deep_kernel<T, 64, P>), grid, dim3(256), 0, st, k); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (N) {
        case 1: hipLaunchKernelGGL((scan_tokens_kernel<T, 1>), grid, dim3(256), 0, st, k); break;
        case 2: hipLaunchKernelGGL((scan_tokens_kernel<T, 2>), grid, dim3(256), 0, st, k); break;
        case 4: hipLaunchKernelGGL((scan_tokens_kernel<T, 4>), grid, dim3(256), 0, st, k); break;
        case 8: hipLaunchKernelGGL((scan_tokens_kernel<T, 8>), grid, dim3(256), 0, st, k); break;
        case 16: hipLaunchKernelGGL((scan_tokens_kernel<T, 16>), grid, dim3(256), 0, st, k); break;
        case 32: hipLaunchKernelGGL((scan_tokens_kernel<T, 32>), grid, dim3(256), 0, st, k); break;
        case 64: hipLaunchKernelGGL((scan_tokens_kernel<T, 64>), grid, dim3(256), 0, st, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_tokens(const ScanArgs& s, hipStream_t st) {
    TokKArgs k{};
    k.u = s.u; k.delta = s.delta; k.z = s.z; k.Bm = s.Bm; k.Cm = s.Cm;
    k.A = s.A; k.Dskip = s.Dskip; k.dt_bias = s.dt_bias; k.h0 = s.h0; k.h_final = s.h_final; k.y = s.y;
    k.B = s.B; k.L = s.L; k.D = s.D; k.softplus = s.softplus;
    return s.dtype == 1 ? dispatch_tokens<uint16_t>(k, s.N, st) : dispatch_tokens<float>(k, s.N, st);
}

hipError_t launch_step(const ScanArgs& s, float* state, hipStream_t st) {
    StepKArgs k{};
    k.u = s.u; k.delta = s.delta; k.z = s.z; k.Bm = s.Bm; k.Cm = s.Cm;
    k.A = s.A; k.Dskip = s.Dskip; k.dt_bias = s.dt_bias;
    k.state = state; k.y = s.y; k.B = s.B; k.D = s.D; k.softplus = s.softplus;
    k.conv_w = s.conv_w; k.conv_b = s.conv_b; k.conv_state = const_cast<void*>(s.x_prev); k.K = s.d_conv;
    if (s.conv_w)
        return s.dtype == 1 ? dispatch<uint16_t, true>(k, s.N, st) : dispatch<float, true>(k, s.N, st);
    return s.dtype == 1 ? dispatch<uint16_t, false>(k, s.N, st) : dispatch<float, false>(k, s.N, st);
}

}  // namespace mssm
