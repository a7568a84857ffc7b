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
// Three launches:
//  1. pre-pass (scan_fwd.hip, the forward kernel in pre-pass mode): the
//     forward recurrence storing the state before every 16-step tile
//     (B, tiles, N, D), sbar (B, L, D) float32 and dz;
//  2. reverse (this file): one workgroup per 64-channel block walks the tiles
//     from last to first.  Lane = channel; each state wave owns a group of
//     states, as in the forward (N = 16: 8 state waves of 2 states), plus
//     helper waves.  Per tile each state wave recomputes the tile's states and
//     decays from the checkpoint into VGPRs, then runs the adjoint backwards
//     over the tile.  Bm/Cm reach the lanes by DPP row broadcast; (Delta,
//     Delta*u, sbar) is prepared by the helper waves and shared through LDS.
//     Each state wave leaves its partial sums over its states of lam*Bm and
//     A*lam*a*h_prev in LDS (two buffers, one barrier per tile), and in the
//     next interval the helpers finish the tile's rows (du, ddelta).  dB/dC are summed over the wave's 64 channels by a
//     transpose-reduce across lanes (16 values in 35 instructions) and
//     stored per channel block;
//  3. reduce: fixed-order sums of the per-block dB/dC partials and of the
//     per-batch-row dA/dD/ddt_bias partials.  No atomics: results are
//     bitwise reproducible.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace mssm {
namespace {

constexpr int kTB = 16;  // tile length (checkpoint spacing, VGPR history depth)

// Helper waves: besides the G state waves (recompute and adjoint of their
// states), a workgroup has G/2 (at least one) helper waves that run the
// per-element front end and the finishing of rows (du, ddelta).
constexpr int helper_waves(int G) { return G >= 2 ? G / 2 : 1; }

struct BwdKArgs {
    const void* u;
    const void* delta;
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;
    const float* dt_bias;
    const float* dh_final;
    const float* ckpt;   // (B, tiles, N, D) state before every tile (pre-pass, or the saved context)
    const float* sbar;   // (B, L, D) (pre-pass); null with a saved context
    // saved context: sbar and dz are formed from dy, z and the forward's readout s
    const void* dy;
    const void* z;        // nullable: no gate
    const float* s_saved; // (B, L, D) sum_n Cm h + Dskip u (with z)
    void* dz;             // (B, L, D) (with z)
    void* du;
    void* ddelta;
    void* dB;
    void* dC;
    float* dA;
    float* dD;
    float* ddt_bias;
    float* dh0;
    float* pBC;    // (B, L, dblocks, 2, N): per channel block, dB partial then dC partial
    float* pA;     // (B, units, D, N): per walk
    float* pD;     // (B, units, D)
    float* pbias;  // (B, units, D)
    float* qlam;   // (B, K - 1, D, N): chunks 1 .. K-1, a_{t0} lam_{t0} from a zero adjoint at the chunk's end
    float* slam;   // (B, K - 1, D): chunks 1 .. K-1, sum of Delta over the chunk
    float* pin;    // (B, K, D, N): a_{t1} lam_{t1} entering each chunk at its end (t1 = its end step)
    int64_t B, L, D, N;
    int64_t tiles;
    int32_t dblocks;
    int32_t softplus;
    int32_t chunks;       // K
    int32_t chunk_tiles;  // tiles per chunk
    int32_t head_chunks;  // walk 0 covers chunks [0, head_chunks), walk u >= 1 chunk head_chunks + u - 1
    int32_t units;        // walks per channel block: K - head_chunks + 1
};

// ---- cross-lane sums -------------------------------------------------------------
// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror (lane i <-> 7 - i within 8 lanes), row_ror:8 (i <-> i + 8
// within a 16-lane row).  All four are involutions.
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// v_permlane32_swap: lanes 32..63 of `a` <-> lanes 0..31 of `b`.
__device__ __forceinline__ void swap32(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// v_permlane16_swap: odd 16-lane rows of `a` <-> even rows of `b`.
__device__ __forceinline__ void swap16(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Sums over the 64 lanes of 16 values at once, in 35 instructions.  Each
// stage pairs the registers, exchanges half of the lanes of each pair with a
// lane permutation and adds, so the register count halves while every
// partial folds twice as many lanes: lanes 32 apart and 16 apart through the
// permlane swaps, then 8 and 4 apart inside a row through DPP with a lane
// select of which register is sent; two quad adds finish.  On return the
// four lanes 4g .. 4g + 3 hold the full sum of v[bitrev4(g)].
__device__ __forceinline__ float wave_sum16(float (&v)[16]) {
    const int lane = threadIdx.x & 63;
    float s[8], t[4], q[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float x = v[2 * i], y = v[2 * i + 1];
        swap32(x, y);
        s[i] = x + y;  // lanes 0-31: v[2i] folded over 32 lanes; 32-63: v[2i+1]
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = s[2 * i], y = s[2 * i + 1];
        swap16(x, y);
        t[i] = x + y;
    }
    const bool hi8 = (lane & 8) != 0, hi4 = (lane & 4) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float x = t[2 * i], y = t[2 * i + 1];
        const float send = hi8 ? x : y, keep = hi8 ? y : x;
        q[i] = keep + dpp<kDppRor8>(send);
    }
    const float send = hi4 ? q[0] : q[1], keep = hi4 ? q[1] : q[0];
    float r = keep + dpp<kDppHalfMirror>(send);
    r += dpp<kDppQuadSwap1>(r);
    r += dpp<kDppQuadSwap2>(r);
    return r;
}

__device__ __forceinline__ int bitrev4(int g) {
    return ((g & 1) << 3) | ((g & 2) << 1) | ((g & 4) >> 1) | ((g & 8) >> 3);
}

// This wave's Bm (or Cm) values of one tile: lane l loads step l % 16 (row
// clamped to the sequence's last row).
template <typename T, int NG>
__device__ __forceinline__ void fetch_tile_rows(const T* __restrict__ M, int64_t row0, int64_t last_row, int N,
                                                int n0, int lane, uint32_t (&q)[LaneRow<T, NG>::kWords]) {
    const int64_t r = imin64(row0 + (lane & (kTB - 1)), last_row);
    load_lane_row<T, NG>(M + r * N + n0, q);
}

// Raw u, delta, sbar of this wave's rows of tile `tile` (tile clamped to >= 0,
// row to the sequence's last row: every address is inside the tensors).
template <typename T, int SPW>
__device__ __forceinline__ void fetch_rows(const T* __restrict__ u_b, const T* __restrict__ d_b,
                                           const float* __restrict__ s_b, int tile, int L32, int D32,
                                           int first_row, int lo, float (&ru)[SPW], float (&rd)[SPW],
                                           float (&rs)[SPW]) {
    const int t0 = max(tile, 0) * kTB;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int t = min(t0 + first_row + i, L32 - 1);
        const int64_t off = static_cast<int64_t>(t) * D32 + lo;
        ru[i] = load_act(u_b, off);
        rd[i] = load_act(d_b, off);
        rs[i] = s_b[off];
    }
}

// Saved context: raw u, delta, dy, z and the forward's readout s of this
// wave's rows of tile `tile` (clamped as fetch_rows).
template <typename T, int SPW>
__device__ __forceinline__ void fetch_rows_saved(const T* __restrict__ u_b, const T* __restrict__ d_b,
                                                 const T* __restrict__ dy_b, const T* __restrict__ z_b,
                                                 const float* __restrict__ s_b, int tile, int L32, int D32,
                                                 int first_row, int lo, float (&ru)[SPW], float (&rd)[SPW],
                                                 float (&rdy)[SPW], float (&rz)[SPW], float (&rs)[SPW]) {
    const int t0 = max(tile, 0) * kTB;
    // without a gate, z is read from dy and s from the context's (unused) readout: the loads stay
    // unconditional, with no branch for the wait counters to merge over; gate_rows ignores both
    const T* zl = z_b ? z_b : dy_b;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int t = min(t0 + first_row + i, L32 - 1);
        const int64_t off = static_cast<int64_t>(t) * D32 + lo;
        ru[i] = load_act(u_b, off);
        rd[i] = load_act(d_b, off);
        rdy[i] = load_act(dy_b, off);
        rz[i] = load_act(zl, off);
        rs[i] = s_b[off];
    }
}

// What a wave keeps of one of its rows from preparing it until finishing it.
struct RowKeep {
    float u, sig, dt, sb;  // u, dDelta/dx (sigmoid(x) with softplus, else 1), Delta, sbar
};

// Per-element front end of this wave's rows of one tile: (Delta, Delta*u,
// sbar) to LDS for all waves.  Lanes past the last channel get u = sbar = 0,
// so they add nothing to the dB/dC sums over the 64 lanes.
template <int SPW>
__device__ __forceinline__ void prep_rows(const float (&ru)[SPW], const float (&rd)[SPW], const float (&rs)[SPW],
                                          float bias, int softplus_on, bool dvalid, int w, int lane,
                                          float4 (&dst)[kTB][64], RowKeep (&keep)[SPW]) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const float x = rd[i] + bias;
        const float dt = softplus_on ? softplus(x) : x;
        const float sg = softplus_on ? sigmoid(x) : 1.0f;
        const float uu = dvalid ? ru[i] : 0.0f;
        const float sb = dvalid ? rs[i] : 0.0f;
        dst[w * SPW + i][lane] = make_float4(dt, dt * uu, sb, 0.0f);
        keep[i] = RowKeep{uu, sg, dt, sb};
    }
}

// Saved context: the gate's two factors of each row from dy, z and the
// forward's readout s: rs[i] <- sbar = dy silu(z) (dy without a gate), and dz
// = dy s silu'(z) stored for rows [0, nstore) of the tile at dz_tile (none
// for a tile outside this walk: another walk stores it).
template <typename T, int SPW>
__device__ __forceinline__ void gate_rows(const float (&rdy)[SPW], const float (&rz)[SPW], float (&rs)[SPW],
                                          bool has_z, int w, int lane, bool dvalid, int nstore, T* dz_tile,
                                          int D32) {
    const __amdgpu_buffer_rsrc_t rdz =
        make_rsrc(has_z ? dz_tile : nullptr, static_cast<uint32_t>(kTB) * static_cast<uint32_t>(D32) * sizeof(T));
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        if (has_z) {
            const float zz = rz[i], sg = sigmoid(zz);
            const float dzf = rdy[i] * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
            const int j = w * SPW + i;
            const uint32_t off = (dvalid && j < nstore) ? (static_cast<uint32_t>(j) * static_cast<uint32_t>(D32) +
                                                           static_cast<uint32_t>(lane)) * sizeof(T)
                                                        : kNoStore;
            buffer_store_act(rs[i] * dzf, rdz, off, T{});
            rs[i] = rdy[i] * zz * sg;
        } else {
            rs[i] = rdy[i];
        }
    }
}

// Finish this wave's rows of a tile from the G partial sums in LDS: du and
// ddelta to memory (rows past `nvalid` dropped by the buffer range check),
// the dD and ddt_bias sums in registers.
template <typename T, int SPW, int G>
__device__ __forceinline__ void finish_rows(const float2 (&sLQ)[G][kTB][64], const RowKeep (&kp)[SPW], int w,
                                            int lane, bool dvalid, int nvalid, float Dk, T* du_tile,
                                            T* dd_tile, int D32, float& accD, float& accBias) {
    const uint32_t bytes = static_cast<uint32_t>(kTB) * static_cast<uint32_t>(D32) * sizeof(T);
    const __amdgpu_buffer_rsrc_t rdu = make_rsrc(du_tile, bytes);
    const __amdgpu_buffer_rsrc_t rdd = make_rsrc(dd_tile, bytes);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int j = w * SPW + i;
        float lb = 0.0f, lq = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float2 p = sLQ[g][j][lane];
            lb += p.x;
            lq += p.y;
        }
        const float gu = __builtin_fmaf(kp[i].sb, Dk, kp[i].dt * lb);
        const float gx = __builtin_fmaf(kp[i].u, lb, lq) * kp[i].sig;
        const bool ok = dvalid && j < nvalid;
        const uint32_t off =
            ok ? (static_cast<uint32_t>(j) * static_cast<uint32_t>(D32) + static_cast<uint32_t>(lane)) * sizeof(T)
               : kNoStore;
        buffer_store_act(gu, rdu, off, T{});
        buffer_store_act(gx, rdd, off, T{});
        if (ok) {
            accD = __builtin_fmaf(kp[i].sb, kp[i].u, accD);
            accBias += gx;
        }
    }
}

// Recompute of one tile from its checkpoint, in two passes over the steps:
// every step's decay and input first (independent of the state), then the
// dependent state updates.  Steps past the end of a ragged last tile hold
// state 0 and decay 1.
template <int NG, bool FULL, int J>
__device__ __forceinline__ void rec_pre(int nval, const float (&A2)[NG], const float (&Bt)[NG],
                                        const float4 (&xt)[kTB], float (&g)[kTB][NG], float (&ahist)[kTB][NG]) {
    if (FULL || J < nval) {
        const float4 x = xt[J];
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            ahist[J][k] = fast_exp2(x.x * A2[k]);
            g[J][k] = row_bcast<J>(Bt[k]) * x.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            ahist[J][k] = 1.0f;
            g[J][k] = 0.0f;
        }
    }
}

template <int NG, bool FULL, int J>
__device__ __forceinline__ void rec_step(int nval, float (&h)[NG], const float (&g)[kTB][NG],
                                         const float (&ahist)[kTB][NG], float (&hist)[kTB][NG]) {
    if (FULL || J < nval) {
#pragma unroll
        for (int k = 0; k < NG; ++k) hist[J][k] = h[k] = __builtin_fmaf(ahist[J][k], h[k], g[J][k]);
    } else {
#pragma unroll
        for (int k = 0; k < NG; ++k) hist[J][k] = 0.0f;
    }
}

template <int NG, bool FULL, int... J>
__device__ __forceinline__ void rec_steps(std::integer_sequence<int, J...>, int nval, const float (&A2)[NG],
                                          float (&h)[NG], const float (&Bt)[NG], const float4 (&xt)[kTB],
                                          float (&hist)[kTB][NG], float (&ahist)[kTB][NG]) {
    float g[kTB][NG];
    (rec_pre<NG, FULL, J>(nval, A2, Bt, xt, g, ahist), ...);
    (rec_step<NG, FULL, J>(nval, h, g, ahist, hist), ...);
}

// Four or more states per wave keep fewer registers per tile (the 168 of a
// 12-wave workgroup would not hold 2 * 16 * NG of states and decays beside
// the tile's (Delta, Delta*u, sbar)): the rows are read from LDS at each use,
// the recompute computes each step's decay and input in place and keeps only
// the states, and the reverse step recomputes the decay (one exp more per
// state-step).
template <int NG>
constexpr bool kLowReg = NG >= 4;

template <int NG, bool FULL, int XS, int J>
__device__ __forceinline__ void rec_step_fused(int nval, const float (&A2)[NG], float (&h)[NG],
                                               const float (&Bt)[NG], const float4* xt, float (&hist)[kTB][NG]) {
    if (FULL || J < nval) {
        const float4 x = xt[J * XS];
#pragma unroll
        for (int k = 0; k < NG; ++k)
            hist[J][k] = h[k] = __builtin_fmaf(fast_exp2(x.x * A2[k]), h[k], row_bcast<J>(Bt[k]) * x.y);
    } else {
#pragma unroll
        for (int k = 0; k < NG; ++k) hist[J][k] = 0.0f;
    }
}
template <int NG, bool FULL, int XS, int... J>
__device__ __forceinline__ void rec_steps_fused(std::integer_sequence<int, J...>, int nval, const float (&A2)[NG],
                                                float (&h)[NG], const float (&Bt)[NG], const float4* xt,
                                                float (&hist)[kTB][NG]) {
    (rec_step_fused<NG, FULL, XS, J>(nval, A2, h, Bt, xt, hist), ...);
}

// State that the reverse steps of one tile read and update.  xt[J * XS] is
// step J's (Delta, Delta*u, sbar): registers (XS = 1) or the LDS rows (XS = 64).
template <int NG, int G>
struct RevCtx {
    static constexpr int XS = kLowReg<NG> ? 64 : 1;
    const float* Aval;       // [NG]
    const float* A2;         // [NG] A * log2(e)
    const float* Bt;         // [NG]
    const float* Ct;         // [NG]
    const float4* xt;        // [kTB * XS]
    const float (*hist)[NG];
    const float (*ahist)[NG];  // unused with kLowReg (the decay is recomputed)
    const float* hin;        // [NG] state before the tile
    float2 (*sLQ)[kTB][64];  // [G]
    __amdgpu_buffer_rsrc_t rp;  // this block's dB/dC partial rows of the tile
    int nval, w, lane, dblocks, N, n0;
};

// Reverse step J for this wave's NG states: the adjoint, its partial sums
// for du/ddelta (to LDS), dA, and the step's dB/dC terms into the 16-value
// batch `vals`; when the batch is complete (its lowest step), its sums over
// the wave's channels are stored.  `pc` carries a_{t+1} lam_{t+1} from the
// step after (dh_final before the last step), so that
// lam_t = pc + sbar_t Cm_t is one DPP fmac and a_t lam_t serves both the
// dA / ddelta term and the next step.
template <int NG, int G, bool FULL, int J>
__device__ __forceinline__ void rev_step(const RevCtx<NG, G>& c, float (&pc)[NG], float (&dA)[NG],
                                         float (&vals)[16]) {
    constexpr int S = 16 / (2 * NG);  // steps per batch
    constexpr int slot = (J % S) * 2 * NG;
    if (FULL || J < c.nval) {
        const float4 x = c.xt[J * RevCtx<NG, G>::XS];  // (Delta, Delta*u, sbar, -)
        float lam[NG];
#pragma unroll
        for (int k = 0; k < NG; ++k) lam[k] = pc[k];
        if constexpr (NG % 2 == 0) {
#pragma unroll
            for (int k = 0; k < NG; k += 2)
                fmac_row_bcast2<J>(lam[k], c.Ct[k], x.z, lam[k + 1], c.Ct[k + 1], x.z);
        } else {
#pragma unroll
            for (int k = 0; k < NG; ++k) lam[k] = fmac_row_bcast<J>(lam[k], c.Ct[k], x.z);
        }
        float lb = 0.0f, lq = 0.0f;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            lb = k == 0 ? row_bcast<J>(c.Bt[0]) * lam[0] : fmac_row_bcast<J>(lb, c.Bt[k], lam[k]);
            float hp;
            if constexpr (J > 0) hp = c.hist[J - 1][k];
            else hp = c.hin[k];
            if constexpr (kLowReg<NG>)
                pc[k] = lam[k] * fast_exp2(x.x * c.A2[k]);
            else
                pc[k] = lam[k] * c.ahist[J][k];
            const float q = pc[k] * hp;
            lq = __builtin_fmaf(c.Aval[k], q, lq);
            dA[k] = __builtin_fmaf(x.x, q, dA[k]);
            vals[slot + k] = lam[k] * x.y;           // this channel's dB term
            vals[slot + NG + k] = x.z * c.hist[J][k];  // this channel's dC term
        }
        c.sLQ[c.w][J][c.lane] = make_float2(lb, lq);
    } else {
#pragma unroll
        for (int k = 0; k < NG; ++k) vals[slot + k] = vals[slot + NG + k] = 0.0f;
    }
    if constexpr (J % S == 0) {
        const float sum = wave_sum16(vals);
        const int v = bitrev4(c.lane >> 2);
        const int step = J + v / (2 * NG);
        const int which = (v / NG) & 1;  // 0: dB, 1: dC
        const int k = v % NG;
        const bool store = (c.lane & 3) == 0 && step < c.nval;
        const uint32_t off =
            ((static_cast<uint32_t>(step) * c.dblocks * 2u + which) * c.N + c.n0 + k) * 4u;
        buffer_store_act(sum, c.rp, store ? off : kNoStore, 0.0f);
    }
}

template <int NG, int G, bool FULL, int... I>
__device__ __forceinline__ void rev_steps(std::integer_sequence<int, I...>, const RevCtx<NG, G>& c,
                                          float (&pc)[NG], float (&dA)[NG]) {
    float vals[16];
    (rev_step<NG, G, FULL, kTB - 1 - I>(c, pc, dA, vals), ...);  // J = 15 .. 0: backwards in time
}

// Registers carried from one reverse interval to the next.
template <typename T, int NG, int G>
struct RevRegs {
    static constexpr int SPW = kTB / helper_waves(G);
    float ru[SPW], rd[SPW], rs[SPW];  // raw u, delta, sbar (saved context: s) of the next tile to prepare
    float rdy[SPW], rz[SPW];          // saved context: its raw dy, z
    uint32_t qb[LaneRow<T, NG>::kWords], qc[LaneRow<T, NG>::kWords];  // Bm/Cm of the next tile
    float hin_next[NG];               // checkpoint of the next tile
    RowKeep keep_c[SPW], keep_p[SPW];  // rows of the tile in flight / of the tile to finish
    float pc[NG], dA[NG];  // a_{t+1} lam_{t+1} into the next step back; the dA sums
    float accD, accBias;
};

// Uniform facts of one workgroup (and the lane's channel).
template <typename T>
struct RevBlock {
    int w, lane, lo, n0, D32, L32, dblk, dblocks, softplus_on;
    int tile_begin, tile_end;  // this workgroup's time chunk: tiles [tile_begin, tile_end)
    int hw;  // helper waves: index among the helpers
    bool dvalid;
    float bias, Dk;
    int64_t row_b, last_row, ck_stride;
    const T* u_b;
    const T* d_b;
    const float* s_b;   // sbar, or with a saved context the forward's readout s
    const T* dy_b;      // saved context: dy, z, dz of the block's first row (z, dz null without a gate)
    const T* z_b;
    T* dz_b;
    const T* Bm;
    const T* Cm;
    T* du_b;
    T* dd_b;
    const float* ck_b;
    float* pBC;
};

// Interval of tile k (tiles - 1 .. 0), one barrier after it:
//   A. read tile k's (Delta, Delta*u, sbar) from LDS; finish tile k + 1's
//      rows from the partial sums its reverse steps left; recompute tile k's
//      states from its checkpoint; prepare tile k - 1's rows into the other
//      LDS buffer; issue the loads of tile k - 1's Bm/Cm/checkpoint and of
//      tile k - 2's raw rows;
//   B. the reverse steps of tile k, whose partial sums go to the other of
//      the two partial-sum buffers (tile k + 1's are still being read).
// FULL: all 16 steps of the tile exist (every tile but a ragged last one).
// HELPER: a helper wave (rows' front end and finishing), else a state wave.
template <bool FULL, bool HELPER, bool SAVED, typename T, int NG, int G>
__device__ __forceinline__ void rev_interval(const RevBlock<T>& bk, int k, int nval, const float (&A2)[NG],
                                             const float (&Aval)[NG], RevRegs<T, NG, G>& r,
                                             float4 (&sX)[2][kTB][64], float2 (&sLQ)[2][G][kTB][64]) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / helper_waves(G);
    const int cur = k & 1, prv = cur ^ 1;
    const int w = bk.w, lane = bk.lane;
    if constexpr (HELPER) {
        if (k + 1 < bk.tile_end) {
            const int64_t off = static_cast<int64_t>(k + 1) * kTB * bk.D32;
            finish_rows<T, SPW, G>(sLQ[prv], r.keep_p, bk.hw, lane, bk.dvalid, min(kTB, bk.L32 - (k + 1) * kTB),
                                   bk.Dk, bk.du_b + off, bk.dd_b + off, bk.D32, r.accD, r.accBias);
        }
        RowKeep keep_n[SPW];
        if constexpr (SAVED) {  // tile k - 1's dz, unless that tile belongs to the walk before
            const int tp = max(k - 1, 0);
            gate_rows<T, SPW>(r.rdy, r.rz, r.rs, bk.z_b != nullptr, bk.hw, lane, bk.dvalid,
                              k - 1 >= bk.tile_begin ? min(kTB, bk.L32 - tp * kTB) : 0,
                              bk.dz_b + static_cast<int64_t>(tp) * kTB * bk.D32, bk.D32);
        }
        prep_rows<SPW>(r.ru, r.rd, r.rs, bk.bias, bk.softplus_on, bk.dvalid, bk.hw, lane, sX[prv],
                       keep_n);  // k == 0: unused
        if constexpr (SAVED)
            fetch_rows_saved<T, SPW>(bk.u_b, bk.d_b, bk.dy_b, bk.z_b, bk.s_b, k - 2, bk.L32, bk.D32, bk.hw * SPW,
                                     bk.lo, r.ru, r.rd, r.rdy, r.rz, r.rs);
        else
            fetch_rows<T, SPW>(bk.u_b, bk.d_b, bk.s_b, k - 2, bk.L32, bk.D32, bk.hw * SPW, bk.lo, r.ru, r.rd, r.rs);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            r.keep_p[i] = r.keep_c[i];
            r.keep_c[i] = keep_n[i];
        }
    } else {
        // ---- tile k's (Delta, Delta*u, sbar); its states recomputed from the checkpoint
        constexpr bool LOWREG = kLowReg<NG>;
        float4 xt[LOWREG ? 1 : kTB];
        if constexpr (!LOWREG) {
#pragma unroll
            for (int j = 0; j < kTB; ++j) xt[j] = sX[cur][j][lane];
        }
        const float4* xp = LOWREG ? &sX[cur][0][lane] : xt;
        float Bt[NG], Ct[NG], hin[NG];
        unpack_lane_row<T, NG>(r.qb, Bt);
        unpack_lane_row<T, NG>(r.qc, Ct);
#pragma unroll
        for (int q = 0; q < NG; ++q) hin[q] = r.hin_next[q];
        {
            const int tp = max(k - 1, 0);
            const int64_t rowp = bk.row_b + static_cast<int64_t>(tp) * kTB;
            fetch_tile_rows<T, NG>(bk.Bm, rowp, bk.last_row, N, bk.n0, lane, r.qb);
            fetch_tile_rows<T, NG>(bk.Cm, rowp, bk.last_row, N, bk.n0, lane, r.qc);
#pragma unroll
            for (int q = 0; q < NG; ++q) r.hin_next[q] = bk.ck_b[tp * bk.ck_stride + q * bk.D32];
        }
        float hist[kTB][NG], ahist[LOWREG ? 1 : kTB][NG];
        {
            float h[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) h[q] = hin[q];
            if constexpr (LOWREG)
                rec_steps_fused<NG, FULL, 64>(std::make_integer_sequence<int, kTB>{}, nval, A2, h, Bt, xp, hist);
            else
                rec_steps<NG, FULL>(std::make_integer_sequence<int, kTB>{}, nval, A2, h, Bt, xt, hist, ahist);
        }
        // ---- the reverse steps of tile k; partials to the other buffer than
        // those of tile k + 1 that the helpers are reading
        const int64_t row0 = bk.row_b + static_cast<int64_t>(k) * kTB;
        RevCtx<NG, G> c{Aval, A2, Bt, Ct, xp, hist, ahist, hin, sLQ[cur],
                        make_rsrc(bk.pBC + (row0 * bk.dblocks + bk.dblk) * 2 * N,
                                  static_cast<uint32_t>(kTB) * bk.dblocks * 2u * N * 4u),
                        nval, w, lane, bk.dblocks, N, bk.n0};
        rev_steps<NG, G, FULL>(std::make_integer_sequence<int, kTB>{}, c, r.pc, r.dA);
    }
}

// The reverse walk over the chunk's tiles.  Both roles execute the same barriers.
template <bool HELPER, bool SAVED, typename T, int NG, int G>
__device__ __forceinline__ void rev_run(const RevBlock<T>& bk, const float (&A2)[NG], const float (&Aval)[NG],
                                        RevRegs<T, NG, G>& r, float4 (&sX)[2][kTB][64],
                                        float2 (&sLQ)[2][G][kTB][64]) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / helper_waves(G);
    const int lane = bk.lane, n0 = bk.n0;
    // ---- prologue: last tile prepared; its Bm/Cm/checkpoint and the next raw rows in flight
    {
        const int tl = bk.tile_end - 1;
        const int64_t rowl = bk.row_b + static_cast<int64_t>(tl) * kTB;
        if constexpr (HELPER) {
            if constexpr (SAVED) {
                fetch_rows_saved<T, SPW>(bk.u_b, bk.d_b, bk.dy_b, bk.z_b, bk.s_b, tl, bk.L32, bk.D32, bk.hw * SPW,
                                         bk.lo, r.ru, r.rd, r.rdy, r.rz, r.rs);
                gate_rows<T, SPW>(r.rdy, r.rz, r.rs, bk.z_b != nullptr, bk.hw, lane, bk.dvalid,
                                  min(kTB, bk.L32 - tl * kTB), bk.dz_b + static_cast<int64_t>(tl) * kTB * bk.D32,
                                  bk.D32);
            } else {
                fetch_rows<T, SPW>(bk.u_b, bk.d_b, bk.s_b, tl, bk.L32, bk.D32, bk.hw * SPW, bk.lo, r.ru, r.rd, r.rs);
            }
            prep_rows<SPW>(r.ru, r.rd, r.rs, bk.bias, bk.softplus_on, bk.dvalid, bk.hw, lane, sX[tl & 1],
                           r.keep_c);
            if constexpr (SAVED)
                fetch_rows_saved<T, SPW>(bk.u_b, bk.d_b, bk.dy_b, bk.z_b, bk.s_b, tl - 1, bk.L32, bk.D32,
                                         bk.hw * SPW, bk.lo, r.ru, r.rd, r.rdy, r.rz, r.rs);
            else
                fetch_rows<T, SPW>(bk.u_b, bk.d_b, bk.s_b, tl - 1, bk.L32, bk.D32, bk.hw * SPW, bk.lo, r.ru, r.rd,
                                   r.rs);
        } else {
            fetch_tile_rows<T, NG>(bk.Bm, rowl, bk.last_row, N, n0, lane, r.qb);
            fetch_tile_rows<T, NG>(bk.Cm, rowl, bk.last_row, N, n0, lane, r.qc);
#pragma unroll
            for (int q = 0; q < NG; ++q) r.hin_next[q] = bk.ck_b[tl * bk.ck_stride + q * bk.D32];
        }
    }
    __syncthreads();

    for (int k = bk.tile_end - 1; k >= bk.tile_begin; --k) {
        const int nval = min(kTB, bk.L32 - k * kTB);
        if (nval == kTB)
            rev_interval<true, HELPER, SAVED>(bk, k, kTB, A2, Aval, r, sX, sLQ);
        else
            rev_interval<false, HELPER, SAVED>(bk, k, nval, A2, Aval, r, sX, sLQ);
        __syncthreads();
    }
    // ---- epilogue: finish the chunk's first tile
    if constexpr (HELPER) {
        const int kb = bk.tile_begin;
        const int64_t off = static_cast<int64_t>(kb) * kTB * bk.D32;
        finish_rows<T, SPW, G>(sLQ[kb & 1], r.keep_p, bk.hw, lane, bk.dvalid, min(kTB, bk.L32 - kb * kTB), bk.Dk,
                               bk.du_b + off, bk.dd_b + off, bk.D32, r.accD, r.accBias);
    }
}

// Reverse kernel.  Grid: (B * dblocks, units) workgroups of G state waves +
// the helper waves; workgroup (blk, u) walks the time chunks of walk u of
// channel block blk backwards, starting from the adjoint that enters its last
// chunk at that chunk's end.
template <typename T, int NG, int G, bool SAVED>
__global__ __launch_bounds__(64 * (G + helper_waves(G))) void bwd_reverse_kernel(BwdKArgs a) {
    constexpr int N = NG * G;
    constexpr int H = helper_waves(G);
    static_assert(kTB % H == 0 && 16 % (2 * NG) == 0, "tile and batch must split evenly");
    // (Delta, Delta*u, sbar, -) per row and channel; after the walk, the
    // helper waves' dD / ddt_bias sums
    __shared__ float4 sX[2][kTB][64];
    __shared__ float2 sLQ[2][G][kTB][64];  // per state group: (sum lam*Bm, sum A*lam*a*h_prev)
    float (&sRed)[2][H][64] = *reinterpret_cast<float (*)[2][H][64]>(&sX[0][0][0]);
    static_assert(sizeof(float) * 2 * H * 64 <= sizeof(sX), "reduction scratch must fit in sX");
    constexpr int SPW = kTB / H;

    RevBlock<T> bk;
    bk.lane = threadIdx.x & 63;
    bk.w = wave_id();
    const int64_t b = blockIdx.x / a.dblocks;
    bk.dblk = static_cast<int>(blockIdx.x % a.dblocks);
    bk.dblocks = a.dblocks;
    const int64_t chan0 = static_cast<int64_t>(bk.dblk) * 64;
    const int64_t D = a.D, L = a.L;
    bk.D32 = static_cast<int>(D);
    bk.L32 = static_cast<int>(L);
    bk.dvalid = chan0 + bk.lane < D;
    bk.lo = bk.dvalid ? bk.lane : static_cast<int>(D - 1 - chan0);
    const int64_t dc = chan0 + bk.lo;
    const bool state_wave = bk.w < G;
    bk.n0 = state_wave ? bk.w * NG : 0;
    bk.hw = state_wave ? 0 : bk.w - G;
    const int64_t unit = blockIdx.y;
    const int c_first = unit == 0 ? 0 : a.head_chunks + static_cast<int>(unit) - 1;
    const int c_last = unit == 0 ? a.head_chunks - 1 : c_first;
    bk.tile_begin = c_first * a.chunk_tiles;
    bk.tile_end = min((c_last + 1) * a.chunk_tiles, static_cast<int>(a.tiles));
    bk.softplus_on = a.softplus;
    bk.bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    bk.Dk = a.Dskip ? a.Dskip[dc] : 0.0f;
    bk.row_b = b * L;
    bk.last_row = bk.row_b + L - 1;
    bk.ck_stride = D * N;
    bk.u_b = static_cast<const T*>(a.u) + bk.row_b * D + chan0;
    bk.d_b = static_cast<const T*>(a.delta) + bk.row_b * D + chan0;
    bk.s_b = (SAVED ? a.s_saved : a.sbar) + bk.row_b * D + chan0;  // the context always holds the readout
    bk.dy_b = SAVED ? static_cast<const T*>(a.dy) + bk.row_b * D + chan0 : nullptr;
    bk.z_b = (SAVED && a.z) ? static_cast<const T*>(a.z) + bk.row_b * D + chan0 : nullptr;
    bk.dz_b = (SAVED && a.z) ? static_cast<T*>(a.dz) + bk.row_b * D + chan0 : nullptr;
    bk.Bm = static_cast<const T*>(a.Bm);
    bk.Cm = static_cast<const T*>(a.Cm);
    bk.du_b = static_cast<T*>(a.du) + bk.row_b * D + chan0;
    bk.dd_b = static_cast<T*>(a.ddelta) + bk.row_b * D + chan0;
    bk.ck_b = a.ckpt + (b * a.tiles * N + bk.n0) * D + dc;  // + tile * N * D + state * D
    bk.pBC = a.pBC;
    const int w = bk.w, lane = bk.lane, n0 = bk.n0;

    float A2[NG], Aval[NG];
    RevRegs<T, NG, G> r;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        Aval[k] = state_wave ? a.A[dc * N + n0 + k] : 0.0f;
        A2[k] = Aval[k] * kLog2e;
        const float dhf = (state_wave && a.dh_final && bk.dvalid) ? a.dh_final[(b * D + dc) * N + n0 + k] : 0.0f;
        if (a.head_chunks > 1 && unit == 0) {
            // one long walk and the last chunk's: the carry over that one chunk, Q + exp(A sum Delta) dh_final
            const int64_t q = (b * (a.chunks - 1) + (a.chunks - 2)) * D + dc;
            r.pc[k] = (state_wave && bk.dvalid) ? __builtin_fmaf(expf(Aval[k] * a.slam[q]), dhf, a.qlam[q * N + n0 + k])
                                                : 0.0f;
        } else if (a.chunks > 1 && c_last < a.chunks - 1) {
            r.pc[k] = (state_wave && bk.dvalid) ? a.pin[((b * a.chunks + c_last) * D + dc) * N + n0 + k] : 0.0f;
        } else {
            r.pc[k] = dhf;  // the walk over the last chunk starts from dh_final
        }
        r.dA[k] = 0.0f;
    }
    r.accD = r.accBias = 0.0f;
#pragma unroll
    for (int i = 0; i < SPW; ++i) r.keep_p[i] = RowKeep{0.0f, 0.0f, 0.0f, 0.0f};

    if (state_wave)
        rev_run<false, SAVED>(bk, A2, Aval, r, sX, sLQ);
    else
        rev_run<true, SAVED>(bk, A2, Aval, r, sX, sLQ);
    // ---- per-(b, d) results
    if (state_wave && bk.dvalid) {
        float* pa = a.pA + ((b * a.units + unit) * D + dc) * N + n0;
#pragma unroll
        for (int k = 0; k < NG; ++k) pa[k] = r.dA[k];
        if (a.dh0 && unit == 0) {
            float* g0 = a.dh0 + (b * D + dc) * N + n0;
#pragma unroll
            for (int k = 0; k < NG; ++k) g0[k] = r.pc[k];  // a_0 lam_0
        }
    }
    if (!state_wave) {
        sRed[0][bk.hw][lane] = r.accD;
        sRed[1][bk.hw][lane] = r.accBias;
    }
    __syncthreads();
    if (w == G && bk.dvalid) {
        float sd = 0.0f, sb = 0.0f;
#pragma unroll
        for (int g = 0; g < H; ++g) {
            sd += sRed[0][g][lane];
            sb += sRed[1][g][lane];
        }
        a.pD[(b * a.units + unit) * D + dc] = sd;
        a.pbias[(b * a.units + unit) * D + dc] = sb;
    }
}

// ---- reverse chunk carry -----------------------------------------------------------
// The adjoint is linear in what enters a time chunk at its end.  With
// p = a_{t1} lam_{t1} entering chunk c = steps [t0, t1) and p_out =
// a_{t0} lam_{t0} leaving it, p_out = Q_c + R_c p, where R_c = prod_{t in c}
// a_t = exp(A sum_{t in c} Delta_t) (the forward's chunk decay) and Q_c is
// p_out for p = 0.  bwd_chunk_lambda_kernel computes Q_c and the chunk's sum
// of Delta for the chunks after the first walk's (every chunk but the first
// when each walk is one chunk); bwd_lambda_carry_kernel chains them from the
// last chunk (p = dh_final) back to the first walk's last chunk; then every
// walk runs from its own entering p, all at once.

// Reverse step J of the zero-started adjoint: lam = p + sbar Cm, p = a lam.
template <int NG, bool FULL, int J>
__device__ __forceinline__ void lam_step(int nval, const float (&A2)[NG], const float (&Ct)[NG],
                                         const float2 (&xs)[kTB], float (&p)[NG]) {
    if (FULL || J < nval) {
        const float2 x = xs[J];  // (Delta, sbar)
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const float lam = __builtin_fmaf(row_bcast<J>(Ct[k]), x.y, p[k]);
            p[k] = lam * fast_exp2(x.x * A2[k]);
        }
    }
}
template <int NG, bool FULL, int... I>
__device__ __forceinline__ void lam_steps(std::integer_sequence<int, I...>, int nval, const float (&A2)[NG],
                                          const float (&Ct)[NG], const float2 (&xs)[kTB], float (&p)[NG]) {
    (lam_step<NG, FULL, kTB - 1 - I>(nval, A2, Ct, xs, p), ...);  // J = 15 .. 0
}

// Grid: (B * dblocks, K - head_chunks), G waves; workgroup (blk, c -
// head_chunks) walks chunk c backwards.  Per tile each wave prepares (Delta, sbar) of its rows of the
// tile before into the other LDS buffer while every wave runs the adjoint of
// its states over this tile: one barrier per tile.
template <int K>
using Slot = std::integral_constant<int, K>;
// f(Slot<0>), f(Slot<1>), ... in order
template <typename F, int... S>
__device__ __forceinline__ void for_slots(F&& f, std::integer_sequence<int, S...>) {
    (f(Slot<S>{}), ...);
}

template <typename T, int NG, int G, int PF, bool SAVED>
__global__ __launch_bounds__(64 * G) void bwd_chunk_lambda_kernel(BwdKArgs a) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / G;
    constexpr int W = LaneRow<T, NG>::kWords;
    static_assert(kTB % G == 0, "tile must split evenly over the waves");
    __shared__ float2 sDS[2][kTB][64];  // (Delta, sbar) per row and channel
    __shared__ float sSum[G][64];

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int64_t b = blockIdx.x / a.dblocks;
    const int64_t chan0 = static_cast<int64_t>(blockIdx.x % a.dblocks) * 64;
    const int64_t c = static_cast<int64_t>(blockIdx.y) + a.head_chunks;
    const int64_t D = a.D, L = a.L;
    const int L32 = static_cast<int>(L);
    const bool dvalid = chan0 + lane < D;
    const int lo = dvalid ? lane : static_cast<int>(D - 1 - chan0);
    const int64_t dc = chan0 + lo;
    const int n0 = w * NG;

    float A2[NG], p[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        A2[k] = a.A[dc * N + n0 + k] * kLog2e;
        p[k] = 0.0f;
    }
    const float bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    float psum = 0.0f;  // sum of Delta over this wave's rows

    const int tb = static_cast<int>(c) * a.chunk_tiles;
    const int te = min(tb + a.chunk_tiles, static_cast<int>(a.tiles));
    const int64_t row_b = b * L;
    const int64_t last_row = row_b + L - 1;
    const T* d_b = static_cast<const T*>(a.delta) + row_b * D + chan0;
    const float* s_b = SAVED ? nullptr : a.sbar + row_b * D + chan0;
    // saved context: sbar = dy silu(z) formed here from dy and z
    const T* dy_b = SAVED ? static_cast<const T*>(a.dy) + row_b * D + chan0 : nullptr;
    const T* z_b = (SAVED && a.z) ? static_cast<const T*>(a.z) + row_b * D + chan0 : nullptr;
    const T* zl = z_b ? z_b : dy_b;  // without a gate: an unconditional load from dy, its value unused
    const T* Cm = static_cast<const T*>(a.Cm);
    // loads of PF tiles in flight, in a ring of register slots: tile t's raw rows and Cm sit in slot
    // (te - 1 - t) % PF, issued PF tiles before its steps (one tile of steps does not cover a load's latency)
    float rd[PF][SPW], rs[PF][SPW], rz[PF][SPW];
    uint32_t qc[PF][W];

    // raw delta and sbar (saved context: dy, and z in zz) of this wave's rows of `tile` (clamped to the
    // last row), and the tile's Cm
    auto fetch = [&](int tile, float (&d)[SPW], float (&sb)[SPW], float (&zz)[SPW], uint32_t (&q)[W]) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = min(tile * kTB + w * SPW + i, L32 - 1);
            const int64_t off = static_cast<int64_t>(t) * D + lo;
            d[i] = load_act(d_b, off);
            if constexpr (SAVED) {
                sb[i] = load_act(dy_b, off);
                zz[i] = load_act(zl, off);
            } else {
                sb[i] = s_b[off];
            }
        }
        fetch_tile_rows<T, NG>(Cm, row_b + static_cast<int64_t>(tile) * kTB, last_row, N, n0, lane, q);
    };
    // (Delta, sbar) of this wave's rows of `tile` into buffer `buf`; a tile before the chunk (the one after
    // its first, in the unconditional main loop) is written to the unused buffer and left out of the sum
    auto prep = [&](int tile, int buf, const float (&d)[SPW], const float (&sb)[SPW], const float (&zz)[SPW]) {
        const int nval = min(kTB, L32 - tile * kTB);
        const bool in = tile >= tb;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            if (j < nval) {
                const float x = d[i] + bias;
                const float dt = a.softplus ? softplus(x) : x;
                const float sbar = (SAVED && z_b) ? sb[i] * zz[i] * sigmoid(zz[i]) : sb[i];  // as the pre-pass
                sDS[buf][j][lane] = make_float2(dt, sbar);
                psum += in ? dt : 0.0f;
            }
        }
    };
    // the steps of `tile` (slot S), after preparing the tile before it and issuing the loads of tile - PF.
    // MAIN: a tile of the loop over whole groups of PF tiles, whose loads and preparation are unconditional
    // (a load past the chunk's first tile reads that tile again): a branch around them would make the
    // compiler wait for every load in flight where the paths join
    auto walk = [&](auto slot, auto main, int tile) {
        constexpr int S = decltype(slot)::value;
        constexpr bool MAIN = decltype(main)::value;
        if (!MAIN && tile < tb) return;  // uniform over the workgroup
        const int cur = tile & 1;
        float Ct[NG];
        unpack_lane_row<T, NG>(qc[S], Ct);
        if (MAIN || tile - 1 >= tb) prep(tile - 1, cur ^ 1, rd[(S + 1) % PF], rs[(S + 1) % PF], rz[(S + 1) % PF]);
        if (MAIN) fetch(max(tile - PF, tb), rd[S], rs[S], rz[S], qc[S]);
        const int nval = min(kTB, L32 - tile * kTB);
        float2 xs[kTB];
#pragma unroll
        for (int j = 0; j < kTB; ++j) xs[j] = sDS[cur][j][lane];
        if (nval == kTB)
            lam_steps<NG, true>(std::make_integer_sequence<int, kTB>{}, kTB, A2, Ct, xs, p);
        else
            lam_steps<NG, false>(std::make_integer_sequence<int, kTB>{}, nval, A2, Ct, xs, p);
        __syncthreads();
    };
    using Main = std::true_type;
    using Rest = std::false_type;

#pragma unroll
    for (int i = 0; i < PF; ++i) fetch(max(te - 1 - i, tb), rd[i], rs[i], rz[i], qc[i]);
    prep(te - 1, (te - 1) & 1, rd[0], rs[0], rz[0]);
    __syncthreads();
    int base = te - 1;
    // groups of PF tiles, every slot index a constant; then the fewer than PF tiles left, their loads issued
    for (int g = (te - tb) / PF; g > 0; --g, base -= PF)
        for_slots([&](auto slot) { walk(slot, Main{}, base - decltype(slot)::value); },
                  std::make_integer_sequence<int, PF>{});
    for_slots([&](auto slot) { walk(slot, Rest{}, base - decltype(slot)::value); },
              std::make_integer_sequence<int, PF - 1>{});
    sSum[w][lane] = psum;
    __syncthreads();
    if (dvalid) {
        const int64_t q = (b * (a.chunks - 1) + (c - 1)) * D + dc;
        float* qo = a.qlam + q * N + n0;
#pragma unroll
        for (int k = 0; k < NG; ++k) qo[k] = p[k];
        if (w == 0) {
            float ssum = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g) ssum += sSum[g][lane];
            a.slam[q] = ssum;
        }
    }
}

// pin of the chunks from the last (dh_final, or 0) back to the first walk's
// last chunk: p_in(c - 1) = Q_c + exp(A sum Delta_c) p_in(c).  One thread per
// (b, d, n).
__global__ __launch_bounds__(256) void bwd_lambda_carry_kernel(BwdKArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= a.B * a.D * a.N) return;
    const int64_t n = i % a.N, bd = i / a.N;
    const int64_t d = bd % a.D, b = bd / a.D;
    const int64_t K = a.chunks;
    const float A = a.A[d * a.N + n];
    float p = a.dh_final ? a.dh_final[i] : 0.0f;
    a.pin[((b * K + (K - 1)) * a.D + d) * a.N + n] = p;
    for (int64_t c = K - 1; c >= a.head_chunks; --c) {
        const int64_t q = (b * (K - 1) + (c - 1)) * a.D + d;
        p = __builtin_fmaf(expf(A * a.slam[q]), p, a.qlam[q * a.N + n]);
        a.pin[((b * K + (c - 1)) * a.D + d) * a.N + n] = p;
    }
}

// ---- fixed-order reductions ----------------------------------------------------------
// Items [0, B*L*N): dB, dC of (b, t, n), summed over the channel blocks;
// items [B*L*N, + D*N): dA of (d, n), summed over the (batch row, time
// chunk) partials in order; items [B*L*N + D*N, + D): dD and ddt_bias of d,
// likewise.  Grid-stride.  The loops over partials are unrolled so their
// loads are issued together; the additions stay in order.
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdKArgs a) {
    const int64_t nBC = a.B * a.L * a.N;
    const int64_t nA = a.D * a.N;
    const int64_t total = nBC + nA + a.D;
    const int64_t parts = a.B * a.units;  // (b, walk) in order
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        if (i < nBC) {
            const int64_t n = i % a.N, bt = i / a.N;
            const float* p = a.pBC + bt * a.dblocks * 2 * a.N + n;
            float sb = 0.0f, sc = 0.0f;
#pragma unroll 8
            for (int32_t k = 0; k < a.dblocks; ++k) {
                sb += p[(2 * k) * a.N];
                sc += p[(2 * k + 1) * a.N];
            }
            store_act(static_cast<T*>(a.dB), i, sb);
            store_act(static_cast<T*>(a.dC), i, sc);
        } else if (i < nBC + nA) {
            const int64_t j = i - nBC;
            float s = 0.0f;
#pragma unroll 8
            for (int64_t q = 0; q < parts; ++q) s += a.pA[q * nA + j];
            a.dA[j] = s;
        } else {
            const int64_t d = i - nBC - nA;
            float sd = 0.0f, sb = 0.0f;
#pragma unroll 8
            for (int64_t q = 0; q < parts; ++q) {
                sd += a.pD[q * a.D + d];
                sb += a.pbias[q * a.D + d];
            }
            if (a.dD) a.dD[d] = sd;
            if (a.ddt_bias) a.ddt_bias[d] = sb;
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace: the forward schedule's own scratch, then the pre-pass outputs,
// then the partial sums.
struct WsLayout {
    size_t fwd, ckpt, sbar, pBC, pA, pD, pbias, qlam, slam, pin, total;
};
// `saved`: the backward from a saved context, with no pre-pass (no forward
// scratch, checkpoints or sbar).
WsLayout ws_layout(int64_t B, int64_t L, int64_t D, int64_t N, int64_t tiles, int64_t K, bool saved = false) {
    const int64_t dblocks = (D + 63) / 64;
    WsLayout w{};
    size_t off = 0;
    w.fwd = off;   off += saved ? 0 : align256(plan_fwd(B, L, D, N).ws_bytes);
    w.ckpt = off;  off += saved ? 0 : align256(static_cast<size_t>(B) * tiles * D * N * 4);
    w.sbar = off;  off += saved ? 0 : align256(static_cast<size_t>(B) * L * D * 4);
    w.pBC = off;   off += align256(static_cast<size_t>(B) * L * dblocks * 2 * N * 4);
    w.pA = off;    off += align256(static_cast<size_t>(B) * K * D * N * 4);
    w.pD = off;    off += align256(static_cast<size_t>(B) * K * D * 4);
    w.pbias = off; off += align256(static_cast<size_t>(B) * K * D * 4);
    w.qlam = off;  off += align256(static_cast<size_t>(B) * (K - 1) * D * N * 4);
    w.slam = off;  off += align256(static_cast<size_t>(B) * (K - 1) * D * 4);
    w.pin = off;   off += align256(K > 1 ? static_cast<size_t>(B) * K * D * N * 4 : 0);
    w.total = off;
    return w;
}

// SAVED: from the context a training forward saved (checkpoints and readout),
// with no pre-pass; else the pre-pass recomputes the checkpoints.
template <typename T, int NG, int G, bool SAVED>
hipError_t launch_bwd_t(const ScanArgs& s, hipStream_t st) {
    const BwdPlan pl = plan_bwd(s.B, s.L, s.D, s.N);
    const WsLayout wl = ws_layout(s.B, s.L, s.D, s.N, pl.tiles, pl.chunks, SAVED);
    char* ws = static_cast<char*>(s.workspace);
    float* ckpt = SAVED ? s.ctx_ckpt : reinterpret_cast<float*>(ws + wl.ckpt);
    float* sbar = SAVED ? nullptr : reinterpret_cast<float*>(ws + wl.sbar);
    if constexpr (!SAVED) {
        hipError_t e = launch_fwd_prepass(s, ws + wl.fwd, ckpt, sbar, st);
        if (e != hipSuccess) return e;
    }
    BwdKArgs a{};
    if constexpr (SAVED) {
        a.dy = s.dy;
        a.z = s.z;
        a.s_saved = s.ctx_s;
        a.dz = s.dz;
    }
    a.u = s.u; a.delta = s.delta; a.Bm = s.Bm; a.Cm = s.Cm;
    a.A = s.A; a.Dskip = s.Dskip; a.dt_bias = s.dt_bias; a.dh_final = s.dh_final;
    a.ckpt = ckpt; a.sbar = sbar;
    a.du = s.du; a.ddelta = s.ddelta; a.dB = s.dB; a.dC = s.dC;
    a.dA = s.dA; a.dD = s.dD; a.ddt_bias = s.ddt_bias; a.dh0 = s.dh0;
    a.pBC = reinterpret_cast<float*>(ws + wl.pBC);
    a.pA = reinterpret_cast<float*>(ws + wl.pA);
    a.pD = reinterpret_cast<float*>(ws + wl.pD);
    a.pbias = reinterpret_cast<float*>(ws + wl.pbias);
    a.qlam = reinterpret_cast<float*>(ws + wl.qlam);
    a.slam = reinterpret_cast<float*>(ws + wl.slam);
    a.pin = reinterpret_cast<float*>(ws + wl.pin);
    a.B = s.B; a.L = s.L; a.D = s.D; a.N = s.N;
    a.tiles = pl.tiles;
    a.dblocks = static_cast<int32_t>((s.D + 63) / 64);
    a.softplus = s.softplus;
    a.chunks = static_cast<int32_t>(pl.chunks);
    a.chunk_tiles = static_cast<int32_t>(pl.chunk_tiles);
    a.head_chunks = static_cast<int32_t>(pl.head_chunks);
    a.units = static_cast<int32_t>(pl.units);
    const unsigned nblk = static_cast<unsigned>(s.B * a.dblocks);
    if (pl.head_chunks > 1) {
        // one long walk per block and the last chunk's: Q of that chunk alone, one workgroup per block on a
        // GPU that is otherwise idle, so up to 16 waves of one state or more (four waves per SIMD); the
        // reverse kernel forms the long walk's entering adjoint itself (no carry pass)
        constexpr int Gq = NG * G < 16 ? NG * G : 16;
        constexpr int NGq = NG * G / Gq;
        hipLaunchKernelGGL((bwd_chunk_lambda_kernel<T, NGq, Gq, 4, SAVED>), dim3(nblk, 1u), dim3(64 * Gq), 0, st, a);
    } else if (pl.chunks > 1) {
        // its own layout: four states per wave where N allows (no LDS partial sums to keep small)
        constexpr int NGc = NG * G >= 16 ? (NG > 4 ? NG : 4) : NG;
        constexpr int Gc = NG * G / NGc;
        hipLaunchKernelGGL((bwd_chunk_lambda_kernel<T, NGc, Gc, 4, SAVED>),
                           dim3(nblk, static_cast<unsigned>(pl.chunks - pl.head_chunks)),
                           dim3(64 * Gc), 0, st, a);
        const int64_t threads = s.B * s.D * s.N;
        hipLaunchKernelGGL(bwd_lambda_carry_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                           st, a);
    }
    // walk 0 of every block first: with one long walk per block and the short ones after it, the hardware's
    // in-order dispatch gives each long walk a CU of its own and runs the short ones on the rest as they free up
    hipLaunchKernelGGL((bwd_reverse_kernel<T, NG, G, SAVED>), dim3(nblk, static_cast<unsigned>(pl.units)),
                       dim3(64 * (G + helper_waves(G))), 0, st, a);
    const int64_t items = s.B * s.L * s.N + s.D * s.N + s.D;
    const int64_t blocks = std::min<int64_t>((items + 255) / 256, 16384);
    hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, bool SAVED>
hipError_t dispatch_n(const ScanArgs& s, hipStream_t st) {
    switch (s.N) {  // NG states per wave x G waves; NG divides 8 (16-value batches)
        case 1: return launch_bwd_t<T, 1, 1, SAVED>(s, st);
        case 2: return launch_bwd_t<T, 1, 2, SAVED>(s, st);
        case 4: return launch_bwd_t<T, 1, 4, SAVED>(s, st);
        case 8: return launch_bwd_t<T, 2, 4, SAVED>(s, st);
        case 16: return launch_bwd_t<T, 2, 8, SAVED>(s, st);
        case 32: return launch_bwd_t<T, 4, 8, SAVED>(s, st);
        case 64: return launch_bwd_t<T, 8, 8, SAVED>(s, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Time chunks of the reverse walk, for a 256-CU MI355X (the workspace size
// query has no device, so the plan depends only on the problem).
// * Channel blocks fill at most half of the CUs: enough chunks for about three
//   workgroups per CU, each at least 4 tiles long, one walk per chunk.  (The
//   chunk carry's extra pass costs about a quarter of the reverse walk over
//   the chunks it covers.)
// * More blocks than half the CUs but fewer than all (the training shape: 192
//   blocks): with m = ceil(blocks / idle CUs), K = m + 1 chunks; each block's
//   first walk covers chunks 0 .. K - 2 on a CU of its own and its last chunk
//   is a walk of its own, m of them in turn on each otherwise idle CU.  The
//   carry then needs the last chunk's Q alone (one pass over 1/K of the
//   sequence), and every CU walks (K - 1)/K of it.  Only where a reverse
//   workgroup takes a CU by itself (N >= 4: 96 KB of LDS or more), so that no
//   short walk shares a long one's CU, with chunks of at least 4 tiles and at
//   most 8 short walks per idle CU.  Training shape, fp32: reverse 408 ->
//   303-337 us (all 256 CUs busy run at a lower clock than 192), plus 44 us for
//   the last chunk's Q.
BwdPlan plan_bwd(int64_t B, int64_t L, int64_t D, int64_t N) {
    constexpr int64_t kCUs = 256;
    BwdPlan p{};
    p.tile = kTB;
    p.tiles = (L + kTB - 1) / kTB;
    const int64_t nblk = B * ((D + 63) / 64);
    int64_t K = 1;
    bool tail = false;
    if (nblk <= kCUs / 2) {
        K = std::min<int64_t>((3 * kCUs + nblk - 1) / nblk, p.tiles / 4);
    } else if (nblk < kCUs && N >= 4) {
        const int64_t m = (nblk + (kCUs - nblk) - 1) / (kCUs - nblk);
        if (m <= 8 && p.tiles / (m + 1) >= 4) {
            K = m + 1;
            tail = true;
        }
    }
    K = std::max<int64_t>(K, 1);
    p.chunk_tiles = (p.tiles + K - 1) / K;
    p.chunks = (p.tiles + p.chunk_tiles - 1) / p.chunk_tiles;  // no empty chunk
    p.head_chunks = (tail && p.chunks > 1) ? p.chunks - 1 : 1;
    p.units = p.chunks - p.head_chunks + 1;
    p.ws_bytes = ws_layout(B, L, D, N, p.tiles, p.chunks).total;
    return p;
}

hipError_t launch_bwd(const ScanArgs& s, hipStream_t st) {
    return s.dtype == 1 ? dispatch_n<uint16_t, false>(s, st) : dispatch_n<float, false>(s, st);
}

CtxLayout ctx_layout(int64_t B, int64_t L, int64_t D, int64_t N) {
    CtxLayout c{};
    const int64_t tiles = (L + kTB - 1) / kTB;
    c.ckpt = 0;
    c.s = align256(static_cast<size_t>(B) * tiles * N * D * 4);
    c.total = c.s + align256(static_cast<size_t>(B) * L * D * 4);
    return c;
}

size_t bwd_saved_ws_bytes(int64_t B, int64_t L, int64_t D, int64_t N) {
    const BwdPlan p = plan_bwd(B, L, D, N);
    return ws_layout(B, L, D, N, p.tiles, p.chunks, true).total;
}

hipError_t launch_bwd_saved(const ScanArgs& s, hipStream_t st) {
    if (!s.ctx_ckpt || (s.z && !s.ctx_s)) return hipErrorInvalidValue;
    return s.dtype == 1 ? dispatch_n<uint16_t, true>(s, st) : dispatch_n<float, true>(s, st);
}

}  // namespace mssm
