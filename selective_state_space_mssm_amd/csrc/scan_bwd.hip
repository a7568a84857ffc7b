// scan_bwd.hip -- backward selective scan (reverse-time adjoint) for gfx950.
//
// Gradients of sum(dy * y) + sum(dh_final * h_final).  With Delta_t, a_t[n] =
// exp(Delta_t A[d,n]), h_t, s_t = sum_n Cm h_t + Dskip u_t, per (b, d):
//   sbar_t = dy_t silu(z_t),   dz_t = dy_t s_t silu'(z_t)
//   lam_t[n] = sbar_t Cm_t[n] + a_{t+1}[n] lam_{t+1}[n]   (reverse in time;
//              lam_{L-1} starts from dh_final)
//   du_t = sbar_t Dskip + Delta_t sum_n lam_t Bm_t
//   dDelta_t = sum_n lam_t (A a_t h_{t-1} + Bm_t u_t),  ddelta = dDelta sig(x)
//   dA += lam_t Delta_t a_t h_{t-1},  dB_t += lam_t Delta_t u_t (over d),
//   dC_t += sbar_t h_t (over d),  dD += sbar_t u_t,  ddt_bias += ddelta,
//   dh0 = a_0 lam_0.
// The forward states are recomputed instead of stored (the recomputation the
// page "mamba.py: 一个简单高效的Mamba实现" describes for the official backward,
// performance section), and the adjoint runs natively in reverse time, with
// no flipped copies (the reverse scan listed in that page's to-do section).
//
// Three kernels:
//  1. checkpoint: forward over the sequence, storing the state at the start
//     of every TB-step tile (B, tiles, D, N);
//  2. reverse: tiles in reverse order; per tile the states are recomputed
//     from the checkpoint into VGPRs, then the adjoint runs backwards over the
//     tile.  Same mapping as the forward (lane = channel, wave = state group,
//     Delta shared through LDS).  dB/dC are summed over the wave's 64 channels
//     with a cross-lane transpose-reduce and written as per-block partials;
//  3. reduce: fixed-order sums of the partials (dB, dC over channel blocks;
//     dA, dD, ddt_bias over the batch).  No atomics: results are bitwise
//     reproducible.
#include "device_common.h"
#include "launch.h"

namespace mssm {
namespace {

constexpr int kTB = 16;  // tile length (checkpoint spacing, VGPR history depth)

struct BwdKArgs {
    const void* u;
    const void* delta;
    const void* z;
    const void* Bm;
    const void* Cm;
    const void* dy;
    const float* A;
    const float* Dskip;
    const float* dt_bias;
    const float* h0;
    const float* dh_final;
    void* du;
    void* ddelta;
    void* dz;
    void* dB;
    void* dC;
    float* dA;
    float* dD;
    float* ddt_bias;
    float* dh0;
    float* ckpt;   // (B, tiles, D, N)
    float* pB;     // (B, L, dblocks, N)
    float* pC;     // (B, L, dblocks, N)
    float* pA;     // (B, D, N)
    float* pD;     // (B, D)
    float* pbias;  // (B, D)
    int64_t B, L, D, N;
    int64_t tiles;
    int32_t dblocks;
    int32_t softplus;
};

template <int NG>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&v)[NG]) {
#pragma unroll
    for (int k = 0; k < NG; ++k) v[k] = p[k];
}
template <int NG>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ p, float (&v)[NG]) {
    if constexpr (NG % 2 == 0) {
        const uint32_t* __restrict__ q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int k = 0; k < NG / 2; ++k) {
            const uint32_t w = q[k];
            v[2 * k] = bf16_lo(w);
            v[2 * k + 1] = bf16_hi(w);
        }
    } else {
#pragma unroll
        for (int k = 0; k < NG; ++k) v[k] = load_act(p, k);
    }
}

// ---- cross-lane sums -------------------------------------------------------
// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of every row; every lane of the row gets the sum.
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<kDppQuadSwap1>(v);
    v += dpp<kDppQuadSwap2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    return v;
}

// v_permlane32_swap: lanes 32..63 of `a` <-> lanes 0..31 of `b`.
__device__ __forceinline__ void swap32(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// v_permlane16_swap: odd rows of `a` <-> even rows of `b`.
__device__ __forceinline__ void swap16(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Full 64-lane sum of one value (every lane gets it).
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    float w = v;
    swap16(v, w);
    v += w;
    w = v;
    swap32(v, w);
    return v + w;
}

// Sum over the 64 lanes of four values at once (transpose-reduce).  On
// return, every lane of row r (= lane / 16) holds the sum of v[perm(r)] with
// perm = {0, 2, 1, 3}.
__device__ __forceinline__ float wave_sum4(float v0, float v1, float v2, float v3) {
    swap32(v0, v1);  // v0 = [v0 lo, v1 lo], v1 = [v0 hi, v1 hi]
    swap32(v2, v3);
    float s01 = v0 + v1;  // lanes 0-31: v0 halves summed; lanes 32-63: v1
    float s23 = v2 + v3;
    swap16(s01, s23);     // rows: s01 = [v0 r0, v2 r0, v1 r2, v3 r2], s23 = [v0 r1, v2 r1, v1 r3, v3 r3]
    return row_sum16(s01 + s23);
}

// ---- kernel 1: checkpoints ---------------------------------------------------
template <typename T, int NG, int G>
__global__ __launch_bounds__(64 * G) void bwd_ckpt_kernel(BwdKArgs a) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / G;
    __shared__ float sD[kTB][64];
    __shared__ float sDU[kTB][64];
    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ dl = static_cast<const T*>(a.delta);
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm);
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int64_t b = blockIdx.x / a.dblocks;
    const int64_t dblk = blockIdx.x % a.dblocks;
    const int64_t D = a.D, L = a.L;
    const int64_t d = dblk * 64 + lane;
    const bool dvalid = d < D;
    const int64_t dc = dvalid ? d : D - 1;
    const int n0 = w * NG;
    float A2[NG], h[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        A2[k] = a.A[dc * N + n0 + k] * kLog2e;
        h[k] = a.h0 ? a.h0[(b * D + dc) * N + n0 + k] : 0.0f;
    }
    const float bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    for (int64_t tile = 0; tile < a.tiles; ++tile) {
        const int64_t tb = tile * kTB;
        if (dvalid) {
            float* cp = a.ckpt + ((b * a.tiles + tile) * D + d) * N + n0;
#pragma unroll
            for (int k = 0; k < NG; ++k) cp[k] = h[k];
        }
        if (tile == a.tiles - 1) break;  // the last tile's end state is not needed
        const int nval = kTB;            // every tile but the last is full
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            const int64_t e = (b * L + tb + j) * D + dc;
            const float x = load_act(dl, e) + bias;
            const float dt = a.softplus ? softplus(x) : x;
            sD[j][lane] = dt;
            sDU[j][lane] = dt * load_act(u, e);
        }
        __syncthreads();
        const T* __restrict__ brow = Bm + (b * L + tb) * N + n0;
#pragma unroll
        for (int j = 0; j < nval; ++j) {
            float bv[NG];
            load_row<NG>(brow + j * N, bv);
            const float dt = sD[j][lane];
            const float du = sDU[j][lane];
#pragma unroll
            for (int k = 0; k < NG; ++k) h[k] = __builtin_fmaf(fast_exp2(dt * A2[k]), h[k], du * bv[k]);
        }
        __syncthreads();
    }
}

// ---- kernel 2: reverse adjoint -------------------------------------------------
template <typename T, int NG, int G>
__global__ __launch_bounds__(64 * G) void bwd_reverse_kernel(BwdKArgs a) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / G;
    __shared__ float sD[kTB][64];
    __shared__ float sDU[kTB][64];
    __shared__ float sS[kTB][64];       // sbar
    __shared__ float sP[G][kTB][64];    // partial readout, then partial sum lam*Bm
    __shared__ float sQ[G][kTB][64];    // partial sum A * lam * a * h_prev
    __shared__ float sRed[2][G][64];

    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ dl = static_cast<const T*>(a.delta);
    const T* __restrict__ z = static_cast<const T*>(a.z);
    const T* __restrict__ dy = static_cast<const T*>(a.dy);
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm);
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm);

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int64_t b = blockIdx.x / a.dblocks;
    const int64_t dblk = blockIdx.x % a.dblocks;
    const int64_t D = a.D, L = a.L;
    const int64_t d = dblk * 64 + lane;
    const bool dvalid = d < D;
    const int64_t dc = dvalid ? d : D - 1;
    const int n0 = w * NG;

    float A2[NG], Aval[NG], lam[NG], dAacc[NG], anext[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        Aval[k] = a.A[dc * N + n0 + k];
        A2[k] = Aval[k] * kLog2e;
        lam[k] = (a.dh_final && dvalid) ? a.dh_final[(b * D + d) * N + n0 + k] : 0.0f;
        dAacc[k] = 0.0f;
        anext[k] = 1.0f;  // no step after L-1
    }
    const float bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    const float Dk = a.Dskip ? a.Dskip[dc] : 0.0f;
    float accD = 0.0f, accBias = 0.0f;

    for (int64_t tile = a.tiles - 1; tile >= 0; --tile) {
        const int64_t tb = tile * kTB;
        const int nval = static_cast<int>(imin64(kTB, L - tb));
        // ---- rows of this wave: inputs and step sizes
        float ru[SPW], rx[SPW], rdy[SPW], rz[SPW], rdt[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            ru[i] = rx[i] = rdy[i] = rz[i] = rdt[i] = 0.0f;
            if (j < nval) {
                const int64_t e = (b * L + tb + j) * D + dc;
                ru[i] = load_act(u, e);
                rx[i] = load_act(dl, e) + bias;
                rdy[i] = dvalid ? load_act(dy, e) : 0.0f;
                if (z) rz[i] = load_act(z, e);
                rdt[i] = a.softplus ? softplus(rx[i]) : rx[i];
                sD[j][lane] = rdt[i];
                sDU[j][lane] = rdt[i] * ru[i];
            }
        }
        __syncthreads();
        // ---- recompute the tile's states from the checkpoint
        float hin[NG], hist[kTB][NG], ahist[kTB][NG];
        {
            const float* cp = a.ckpt + ((b * a.tiles + tile) * D + dc) * N + n0;
#pragma unroll
            for (int k = 0; k < NG; ++k) hin[k] = cp[k];
        }
        const T* __restrict__ brow = Bm + (b * L + tb) * N + n0;
        const T* __restrict__ crow = Cm + (b * L + tb) * N + n0;
        {
            float h[NG];
#pragma unroll
            for (int k = 0; k < NG; ++k) h[k] = hin[k];
#pragma unroll
            for (int j = 0; j < kTB; ++j) {
                if (j < nval) {
                    float bv[NG], cv[NG];
                    load_row<NG>(brow + j * N, bv);
                    load_row<NG>(crow + j * N, cv);
                    const float dt = sD[j][lane];
                    const float du = sDU[j][lane];
                    float yp = 0.0f;
#pragma unroll
                    for (int k = 0; k < NG; ++k) {
                        const float aa = fast_exp2(dt * A2[k]);
                        h[k] = __builtin_fmaf(aa, h[k], du * bv[k]);
                        ahist[j][k] = aa;
                        hist[j][k] = h[k];
                        yp = __builtin_fmaf(cv[k], h[k], yp);
                    }
                    sP[w][j][lane] = yp;
                } else {
#pragma unroll
                    for (int k = 0; k < NG; ++k) ahist[j][k] = hist[j][k] = 0.0f;
                }
            }
        }
        __syncthreads();
        // ---- gate: sbar and dz for this wave's rows
        float rsbar[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            rsbar[i] = 0.0f;
            if (j < nval) {
                float s = Dk * ru[i];
#pragma unroll
                for (int g = 0; g < G; ++g) s += sP[g][j][lane];
                float sbar = rdy[i];
                if (z) {
                    const float sg = sigmoid(rz[i]);
                    sbar = rdy[i] * rz[i] * sg;
                    if (dvalid) {
                        const float gz = rdy[i] * s * sg * (1.0f + rz[i] * (1.0f - sg));
                        store_act(static_cast<T*>(a.dz), (b * L + tb + j) * D + d, gz);
                    }
                }
                rsbar[i] = sbar;
                sS[j][lane] = sbar;
            }
        }
        __syncthreads();
        // ---- reverse over the tile
#pragma unroll
        for (int j = kTB - 1; j >= 0; --j) {
            if (j < nval) {
                float bv[NG], cv[NG];
                load_row<NG>(brow + j * N, bv);
                load_row<NG>(crow + j * N, cv);
                const float sbar = sS[j][lane];
                const float dt = sD[j][lane];
                const float du = sDU[j][lane];
                float lb = 0.0f, lq = 0.0f, gB[NG], gC[NG];
#pragma unroll
                for (int k = 0; k < NG; ++k) {
                    const int jn = j + 1 < kTB ? j + 1 : j;  // next row inside the tile
                    const float an = (j + 1 < kTB && j + 1 < nval) ? ahist[jn][k] : anext[k];
                    lam[k] = __builtin_fmaf(an, lam[k], sbar * cv[k]);
                    const int jp = j > 0 ? j - 1 : 0;
                    const float hp = j > 0 ? hist[jp][k] : hin[k];
                    const float q = lam[k] * ahist[j][k] * hp;
                    lb = __builtin_fmaf(lam[k], bv[k], lb);
                    lq = __builtin_fmaf(Aval[k], q, lq);
                    dAacc[k] = __builtin_fmaf(dt, q, dAacc[k]);
                    gB[k] = dvalid ? lam[k] * du : 0.0f;
                    gC[k] = dvalid ? sbar * hist[j][k] : 0.0f;
                }
                sP[w][j][lane] = lb;
                sQ[w][j][lane] = lq;
                // sum dB, dC over this wave's 64 channels
                const int64_t prow = ((b * L + tb + j) * a.dblocks + dblk) * N + n0;
                if constexpr (NG == 4) {
                    const float rb = wave_sum4(gB[0], gB[1], gB[2], gB[3]);
                    const float rc = wave_sum4(gC[0], gC[1], gC[2], gC[3]);
                    if ((lane & 15) == 0) {
                        const int r = lane >> 4;
                        const int k = ((r & 1) << 1) | (r >> 1);
                        a.pB[prow + k] = rb;
                        a.pC[prow + k] = rc;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < NG; ++k) {
                        const float rb = wave_sum(gB[k]);
                        const float rc = wave_sum(gC[k]);
                        if (lane == 0) {
                            a.pB[prow + k] = rb;
                            a.pC[prow + k] = rc;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NG; ++k) anext[k] = ahist[0][k];
        __syncthreads();
        // ---- per-element gradients for this wave's rows
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            if (j < nval && dvalid) {
                float lb = 0.0f, lq = 0.0f;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    lb += sP[g][j][lane];
                    lq += sQ[g][j][lane];
                }
                const int64_t e = (b * L + tb + j) * D + d;
                store_act(static_cast<T*>(a.du), e, __builtin_fmaf(rsbar[i], Dk, rdt[i] * lb));
                const float dDelta = __builtin_fmaf(ru[i], lb, lq);
                const float gx = a.softplus ? dDelta * sigmoid(rx[i]) : dDelta;
                store_act(static_cast<T*>(a.ddelta), e, gx);
                accD = __builtin_fmaf(rsbar[i], ru[i], accD);
                accBias += gx;
            }
        }
        __syncthreads();
    }
    // ---- per-(b, d) results
    if (dvalid) {
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            a.pA[(b * D + d) * N + n0 + k] = dAacc[k];
            if (a.dh0) a.dh0[(b * D + d) * N + n0 + k] = anext[k] * lam[k];
        }
    }
    sRed[0][w][lane] = accD;
    sRed[1][w][lane] = accBias;
    __syncthreads();
    if (w == 0 && dvalid) {
        float sd = 0.0f, sb = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            sd += sRed[0][g][lane];
            sb += sRed[1][g][lane];
        }
        a.pD[b * D + d] = sd;
        a.pbias[b * D + d] = sb;
    }
}

// ---- kernel 3: fixed-order reductions ---------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdKArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nBC = a.B * a.L * a.N;
    if (i < nBC) {  // dB, dC: sum over channel blocks
        const int64_t n = i % a.N, bt = i / a.N;
        const float* pb = a.pB + bt * a.dblocks * a.N + n;
        const float* pc = a.pC + bt * a.dblocks * a.N + n;
        float sb = 0.0f, sc = 0.0f;
        for (int32_t k = 0; k < a.dblocks; ++k) {
            sb += pb[k * a.N];
            sc += pc[k * a.N];
        }
        store_act(static_cast<T*>(a.dB), i, sb);
        store_act(static_cast<T*>(a.dC), i, sc);
        return;
    }
    const int64_t j = i - nBC;
    if (j < a.D * a.N) {  // dA: sum over the batch
        float s = 0.0f;
        for (int64_t b = 0; b < a.B; ++b) s += a.pA[b * a.D * a.N + j];
        a.dA[j] = s;
        if (j % a.N == 0) {
            const int64_t d = j / a.N;
            float sd = 0.0f, sb = 0.0f;
            for (int64_t b = 0; b < a.B; ++b) {
                sd += a.pD[b * a.D + d];
                sb += a.pbias[b * a.D + d];
            }
            if (a.dD) a.dD[d] = sd;
            if (a.ddt_bias) a.ddt_bias[d] = sb;
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
    size_t ckpt, pB, pC, pA, pD, pbias, total;
};
WsLayout ws_layout(int64_t B, int64_t L, int64_t D, int64_t N, int64_t tiles) {
    const int64_t dblocks = (D + 63) / 64;
    WsLayout w{};
    size_t off = 0;
    w.ckpt = off; off += align256(static_cast<size_t>(B) * tiles * D * N * 4);
    w.pB = off;   off += align256(static_cast<size_t>(B) * L * dblocks * N * 4);
    w.pC = off;   off += align256(static_cast<size_t>(B) * L * dblocks * N * 4);
    w.pA = off;   off += align256(static_cast<size_t>(B) * D * N * 4);
    w.pD = off;   off += align256(static_cast<size_t>(B) * D * 4);
    w.pbias = off; off += align256(static_cast<size_t>(B) * D * 4);
    w.total = off;
    return w;
}

template <typename T, int NG, int G>
hipError_t launch_bwd_t(const ScanArgs& s, hipStream_t st) {
    const BwdPlan pl = plan_bwd(s.B, s.L, s.D, s.N);
    const WsLayout wl = ws_layout(s.B, s.L, s.D, s.N, pl.tiles);
    char* ws = static_cast<char*>(s.workspace);
    BwdKArgs a{};
    a.u = s.u; a.delta = s.delta; a.z = s.z; a.Bm = s.Bm; a.Cm = s.Cm; a.dy = s.dy;
    a.A = s.A; a.Dskip = s.Dskip; a.dt_bias = s.dt_bias; a.h0 = s.h0; a.dh_final = s.dh_final;
    a.du = s.du; a.ddelta = s.ddelta; a.dz = s.dz; a.dB = s.dB; a.dC = s.dC;
    a.dA = s.dA; a.dD = s.dD; a.ddt_bias = s.ddt_bias; a.dh0 = s.dh0;
    a.ckpt = reinterpret_cast<float*>(ws + wl.ckpt);
    a.pB = reinterpret_cast<float*>(ws + wl.pB);
    a.pC = reinterpret_cast<float*>(ws + wl.pC);
    a.pA = reinterpret_cast<float*>(ws + wl.pA);
    a.pD = reinterpret_cast<float*>(ws + wl.pD);
    a.pbias = reinterpret_cast<float*>(ws + wl.pbias);
    a.B = s.B; a.L = s.L; a.D = s.D; a.N = s.N;
    a.tiles = pl.tiles;
    a.dblocks = static_cast<int32_t>((s.D + 63) / 64);
    a.softplus = s.softplus;
    const dim3 grid(static_cast<unsigned>(s.B * a.dblocks));
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, NG, G>), grid, dim3(64 * G), 0, st, a);
    hipLaunchKernelGGL((bwd_reverse_kernel<T, NG, G>), grid, dim3(64 * G), 0, st, a);
    const int64_t nred = s.B * s.L * s.N + s.D * s.N;
    hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3(static_cast<unsigned>((nred + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_n(const ScanArgs& s, hipStream_t st) {
    switch (s.N) {
        case 1: return launch_bwd_t<T, 1, 1>(s, st);
        case 2: return launch_bwd_t<T, 1, 2>(s, st);
        case 4: return launch_bwd_t<T, 1, 4>(s, st);
        case 8: return launch_bwd_t<T, 2, 4>(s, st);
        case 16: return launch_bwd_t<T, 4, 4>(s, st);
        case 32: return launch_bwd_t<T, 8, 4>(s, st);
        case 64: return launch_bwd_t<T, 16, 4>(s, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

BwdPlan plan_bwd(int64_t B, int64_t L, int64_t D, int64_t N) {
    BwdPlan p{};
    p.tile = kTB;
    p.tiles = (L + kTB - 1) / kTB;
    p.ws_bytes = ws_layout(B, L, D, N, p.tiles).total;
    return p;
}

hipError_t launch_bwd(const ScanArgs& s, hipStream_t st) {
    return s.dtype == 1 ? dispatch_n<uint16_t>(s, st) : dispatch_n<float>(s, st);
}

}  // namespace mssm
