// ssd_fwd.hip -- forward of the Mamba-2 layer (the state-space dual, SSD) on
// the gfx950 matrix cores.
//
// The pages name Mamba-2 (the model list of "mamba.py: 一个简单高效的Mamba实现",
// the versions paragraph of "Mamba SSM 架构") without defining it.  This is the
// reading the library implements: the selective scan of Mamba with one scalar
// decay A_h and one step size Delta per head h, shared by the head's P
// channels and all N states, and Bm, Cm shared by every head.  With channel
// d = (h, p) it is exactly the selective scan's recurrence.
//
// Computed in the chunked dual form.  Per chunk of Q = 64 steps, with the
// chunk-local cumulative log-decay cum_i = sum_{j <= i} Delta_j A_h and the
// state S (P x N) entering the chunk:
//     G   = C B^T                                        (Q x Q, over N)
//     M   = G o Lmask,  Lmask_ij = exp(cum_i - cum_j) Delta_j  for j <= i, else 0
//     Y   = diag(exp(cum)) C S^T + M X + D_h X           (Q x P)
//     S'  = exp(cum_last) S + (w o X)^T B,   w_j = exp(cum_last - cum_j) Delta_j
// All four products are dense fp32 contractions: they run as
// v_mfma_f32_32x32x2f32, one 32 x 32 output tile per wave per product, with
// the operands staged in LDS.  A workgroup owns one (batch, head) and walks its
// chunks in order, keeping S in the accumulators of its four waves.
//
// MFMA 32x32x2 f32 lane layout (wave64, lane l, half hl = l / 32):
//   A operand: lane holds A[l % 32][k + hl]; B operand: lane holds B[k + hl][l % 32];
//   accumulator item r: row (r / 4) * 8 + hl * 4 + r % 4, column l % 32.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ssd.h"

namespace mssm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQ = kSsdChunk;
constexpr int kP = kSsdHeadDim;
constexpr int kThreads = 256;

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Tile row of accumulator item r for a lane in half hl.
__device__ __forceinline__ int acc_row(int r, int hl) { return (r >> 2) * 8 + hl * 4 + (r & 3); }

__device__ __forceinline__ float fexp(float x) { return fast_exp2(x * kLog2e); }

// One chunk's operands.  Rows padded by one float so that reading a column
// (32 rows at one k, the A-operand pattern) hits 32 different banks.
template <int N>
struct SsdSmem {
    float x[kQ][kP + 1];   // X: the chunk's inputs of this head
    float b[kQ][N + 1];    // Bm rows
    float c[kQ][N + 1];    // Cm rows
    float m[kQ][kQ + 1];   // M = G o Lmask
    float st[N][kP + 1];   // S^T, the state entering the chunk
    float cum[kQ];         // chunk-local cumulative Delta * A_h
    float dlt[kQ];         // Delta (0 past the sequence end)
    float w[kQ];           // exp(cum_last - cum_j) Delta_j
};

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_fwd_kernel(SsdArgs a) {
    constexpr int NT = N / 64;  // state tiles per wave: the P x N state is 2 x (N / 32) tiles over 4 waves
    __shared__ SsdSmem<N> s;
    const int tid = threadIdx.x;
    const int wv = wave_id();
    const int lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int64_t H = a.H, L = a.L;
    const int64_t bi = blockIdx.x / H, h = blockIdx.x % H;

    const float Ah = a.A[h];
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Dh = a.Dskip ? a.Dskip[h] : 0.0f;

    // this wave's state tiles: rows p in [sp * 32, +32), columns n in [(wv & 1) * NT + k) * 32, +32)
    const int sp = wv >> 1;
    const int64_t state_base = (bi * H + h) * kP * N;
    f32x16 S[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            S[k][r] = a.h0 ? a.h0[state_base + (int64_t)(sp * 32 + acc_row(r, hl)) * N + n] : 0.0f;
    }

    // this wave's tile (ti, tj) of M (Q x Q) and of Y (Q x P)
    const int ti = wv >> 1, tj = wv & 1;

    for (int64_t t0 = 0; t0 < L; t0 += kQ) {
        const int nv = (int)imin64(kQ, L - t0);

        // ---- stage: S^T and the chunk's operands into LDS; cum, Delta, w ----
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) s.st[n][sp * 32 + acc_row(r, hl)] = S[k][r];
        }
        for (int e = tid; e < kQ * kP / 4; e += kThreads) {
            const int i = e / (kP / 4), p = (e % (kP / 4)) * 4;
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (i < nv) v = *reinterpret_cast<const float4*>(a.x + ((bi * L + t0 + i) * H + h) * kP + p);
            s.x[i][p] = v.x; s.x[i][p + 1] = v.y; s.x[i][p + 2] = v.z; s.x[i][p + 3] = v.w;
        }
        for (int e = tid; e < kQ * N / 4; e += kThreads) {
            const int i = e / (N / 4), n = (e % (N / 4)) * 4;
            float4 vb = make_float4(0.0f, 0.0f, 0.0f, 0.0f), vc = vb;
            if (i < nv) {
                const int64_t o = (bi * L + t0 + i) * N + n;
                vb = *reinterpret_cast<const float4*>(a.Bm + o);
                vc = *reinterpret_cast<const float4*>(a.Cm + o);
            }
            s.b[i][n] = vb.x; s.b[i][n + 1] = vb.y; s.b[i][n + 2] = vb.z; s.b[i][n + 3] = vb.w;
            s.c[i][n] = vc.x; s.c[i][n + 1] = vc.y; s.c[i][n + 2] = vc.z; s.c[i][n + 3] = vc.w;
        }
        if (wv == 0) {
            float d = 0.0f;
            if (lane < nv) {
                const float v = a.dt[(bi * L + t0 + lane) * H + h] + bias;
                d = a.softplus ? softplus(v) : v;
            }
            float c = d * Ah;  // inclusive prefix sum over the wave
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(c, off);
                if (lane >= off) c += o;
            }
            const float last = __shfl(c, 63);
            s.cum[lane] = c;
            s.dlt[lane] = d;
            s.w[lane] = fexp(last - c) * d;
        }
        __syncthreads();

        // ---- M = (C B^T) o Lmask, tile (ti, tj); the tile above the diagonal is zero ----
        {
            f32x16 g = {};
            if (ti >= tj) {
#pragma unroll 8
                for (int k = 0; k < N; k += 2)
                    g = mfma32(s.c[ti * 32 + l32][k + hl], s.b[tj * 32 + l32][k + hl], g);
            }
            const int j = tj * 32 + l32;
            const float cj = s.cum[j], dj = s.dlt[j];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ti * 32 + acc_row(r, hl);
                s.m[i][j] = j <= i ? g[r] * fexp(s.cum[i] - cj) * dj : 0.0f;
            }
        }
        __syncthreads();

        // ---- Y tile (ti, tj): exp(cum_i) (C S^T) + M X + D X ----
        {
            f32x16 y = {};
#pragma unroll 8
            for (int k = 0; k < N; k += 2) y = mfma32(s.c[ti * 32 + l32][k + hl], s.st[k + hl][tj * 32 + l32], y);
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] *= fexp(s.cum[ti * 32 + acc_row(r, hl)]);
            for (int kb = 0; kb <= ti; ++kb) {  // M is zero right of the diagonal tile
#pragma unroll
                for (int k = kb * 32; k < kb * 32 + 32; k += 2)
                    y = mfma32(s.m[ti * 32 + l32][k + hl], s.x[k + hl][tj * 32 + l32], y);
            }
            const int p = tj * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ti * 32 + acc_row(r, hl);
                if (i < nv) a.y[((bi * L + t0 + i) * H + h) * kP + p] = y[r] + Dh * s.x[i][p];
            }
        }

        // ---- S' = exp(cum_last) S + (w o X)^T B ----
        {
            const float decay = fexp(s.cum[kQ - 1]);
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const int n0 = ((wv & 1) * NT + k) * 32;
                f32x16 acc = S[k] * decay;
#pragma unroll 8
                for (int j = 0; j < kQ; j += 2)
                    acc = mfma32(s.w[j + hl] * s.x[j + hl][sp * 32 + l32], s.b[j + hl][n0 + l32], acc);
                S[k] = acc;
            }
        }
        __syncthreads();
    }

    if (a.h_final) {
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                a.h_final[state_base + (int64_t)(sp * 32 + acc_row(r, hl)) * N + n] = S[k][r];
        }
    }
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H)), block(kThreads);
    if (a.N == 64)
        hipLaunchKernelGGL(ssd_fwd_kernel<64>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(ssd_fwd_kernel<128>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace mssm
