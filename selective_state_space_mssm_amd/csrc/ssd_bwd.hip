// ssd_bwd.hip -- backward of the Mamba-2 layer (the state-space dual, SSD) on
// the gfx950 matrix cores.
//
// The reading is the forward's (ssd_fwd.hip): the selective scan with one
// scalar decay A_h and one step size Delta per head, shared by the head's P
// channels and N states, and Bm, Cm shared by all heads.  The backward is its
// adjoint in the chunked dual form, per chunk of Q = 64 steps with chunk-local
// cum_i = sum_{s <= i} Delta_s A_h, S_in the state entering the chunk, S_out
// the one leaving it and dS the adjoint of S_out:
//   G = C B^T,  Lmask_ij = exp(cum_i - cum_j) Delta_j (j <= i),
//   U_jk = exp(cum_k - cum_j) (k >= j),  e_j = exp(cum_last - cum_j),
//   dC   = diag(exp(cum)) dY S_in + ((dY X^T) o Lmask) B
//   V    = (G^T o U) dY + diag(e) B dS^T                 (V_j = lambda_j B_j)
//   dX   = diag(Delta) V + D dY
//   dB   = diag(Delta) [((X dY^T) o U) C + diag(e) X dS]
//   r_i  = x_i . V_i,  dcum_i = C_i . dC_i - Delta_i r_i (+ <dS, S_out> at the chunk's last row)
//   dDelta_t = A_h sum_{i >= t} dcum_i + r_t,  dA_h += sum_i dcum_i sum_{s <= i} Delta_s
//   dS_in = dY^T diag(exp(cum)) C + exp(cum_last) dS.
// dB and dC sum over heads; dA, dDskip and ddt_bias over batch and time.
//
// Four passes:
//   1. states (ssd_fwd.hip, launch_ssd_states): the forward recurrence alone,
//      storing the state entering every chunk (and the final state);
//   2. adjoint states (ssd_dstate_kernel): one workgroup per (batch, head)
//      walks the chunks backwards carrying dS in its accumulators, storing the
//      dS of every chunk; dh0 is the last dS_in;
//   3. chunk gradients (ssd_bwd_chunk_kernel): one workgroup per (batch,
//      chunk, head group), independent of every other: Bm, Cm and G = C B^T
//      are staged and formed once, then for each head of the group the
//      products above, dB and dC summed over the group's heads in the
//      accumulators, and <dS, S_out> from S_in and the X dS products;
//   4. reductions (ssd_bwd_reduce_*_kernel): dA, dDskip, ddt_bias over (batch,
//      chunk) and, with several head groups, dB and dC over the groups, in a
//      fixed order (no atomics: bitwise reproducible).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ssd.h"
#include "ssd_common.h"

namespace mssm {
namespace {
using namespace ssdk;

// Cross-lane partners without the LDS crossbar (ds_bpermute would queue behind
// the matrix operands' LDS reads): DPP within rows of 16 lanes and gfx950's
// v_permlane16_swap / v_permlane32_swap across them.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]: lane l ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]: lane l ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane l ^ 7 (reversal within 8 lanes)
constexpr int kDppMirror = 0x140;      // lane l ^ 15 (reversal within 16 lanes)
// value of lane l ^ 16: the swap moves rows 0 <-> 1 and 2 <-> 3 of 16 lanes
__device__ __forceinline__ float xor16(float v, int lane) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
// value of lane l ^ 32
__device__ __forceinline__ float xor32(float v, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
}

// Sum over the 64 lanes (every lane gets it).
__device__ __forceinline__ float wave_sum(float v, int lane) {
    v += dpp_mov<kDppXor1>(v);
    v += dpp_mov<kDppXor2>(v);
    v += dpp_mov<kDppHalfMirror>(v);
    v += dpp_mov<kDppMirror>(v);
    v += xor16(v, lane);
    return v + xor32(v, lane);
}

// Row sums of an accumulator tile: the 16 items of a lane (rows acc_row(r, hl))
// summed over the 32 lanes of its half.  Each butterfly step pairs lanes that
// differ in one bit b (partners l ^ 16, l ^ 15, l ^ 7, l ^ 2, l ^ 1, each
// flipping b and leaving the bits of earlier steps alone) and hands half of the
// remaining rows to the partner, so 16 exchanges do all 16 rows; afterwards
// lanes l and l ^ 1 (l = l32) hold the sum of item r = (l >> 1) & 15.  Returns
// that sum; the caller writes it from the even lanes.
__device__ __forceinline__ float tile_row_sums(f32x16 v, int lane) {
    // the items as opaque scalars: selecting between two elements of the vector would otherwise be folded
    // into an element read at a per-lane index, which lowers to a 16-way compare-and-select chain
    float w[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        w[r] = v[r];
        asm volatile("" : "+v"(w[r]));
    }
    float a8[8], a4[4], a2[2];
    const bool b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float send = b4 ? w[q] : w[q + 8], keep = b4 ? w[q + 8] : w[q];
        a8[q] = keep + xor16(send, lane);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float send = b3 ? a8[q] : a8[q + 4], keep = b3 ? a8[q + 4] : a8[q];
        a4[q] = keep + dpp_mov<kDppMirror>(send);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float send = b2 ? a4[q] : a4[q + 2], keep = b2 ? a4[q + 2] : a4[q];
        a2[q] = keep + dpp_mov<kDppHalfMirror>(send);
    }
    const float send = b1 ? a2[0] : a2[1], keep = b1 ? a2[1] : a2[0];
    const float a1 = keep + dpp_mov<kDppXor2>(send);
    return a1 + dpp_mov<kDppXor1>(a1);
}

// Offset of accumulator item r of the (P, N) state tile set a wave of the
// state passes keeps: rows sp * 32 + acc_row(r, hl), columns ((w & 1) * NT + k) * 32 + l32.
template <int N>
__device__ __forceinline__ int state_item(int wv, int k, int r, int hl, int l32) {
    constexpr int NT = N / 64;
    return ((wv >> 1) * 32 + acc_row(r, hl)) * N + ((wv & 1) * NT + k) * 32 + l32;
}

// ---------------------------------------------------------------------------
// Passes 1 and 2: the chains over chunks.  Both carry a P x N matrix through
// the chunks of one (batch, head) as the same update,
//   M <- exp(cum_last) M + sum_i q_i U_i^T V_i        (U: Q x P, V: Q x N rows),
// the states forward (M = S, U = X, V = Bm, q_i = exp(cum_last - cum_i) Delta_i:
// the forward's state update) and the adjoint states backward (M = dS, U = dY,
// V = Cm, q_i = exp(cum_i): dS_in from dS), and store M as it enters each
// chunk: the state entering chunk c (and the final state) for pass 3's dY S_in,
// the adjoint of the state leaving chunk c for its dB and V.  The matrix lives
// in the accumulators of the four waves as in the forward's state update.
template <int N>
struct alignas(16) ChainSmem {
    float u[kQ][kP + kPadRow];
    float v[kQ][N + kPadRow];
    float q[kQ];
    float decay;
};

template <class T, int N>
struct ChainRegs {
    static constexpr int kU = kQ * kP / 4 / kThreads;  // float4 of U per thread
    static constexpr int kV = kQ * N / 4 / kThreads;   // float4 of V per thread
    float4 u[kU], v[kV];
    float dt;
};

// Chunk [t0, t0 + 64)'s U rows (this head), V rows and step sizes into
// registers; rows at or past L lie outside the resources and read as zeros.
template <class T, int N>
__device__ __forceinline__ void load_chain_chunk(const SsdBwdArgs& a, const void* U, const void* V, int64_t bi,
                                                 int64_t h, int64_t t0, int tid, ChainRegs<T, N>& g) {
    const int64_t H = a.H;
    const int64_t nv = a.L - t0 < 0 ? 0 : imin64(kQ, a.L - t0);
    const int64_t row0 = bi * a.L + t0;
    const T* tag = nullptr;
    const auto ru = make_rsrc(static_cast<const T*>(U) + row0 * H * kP, (uint32_t)(nv * H * kP * sizeof(T)));
    const auto rv = make_rsrc(static_cast<const T*>(V) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
    const int64_t Hd = H / a.hsub;  // dt has a row of heads; sub-head h reads its head's
    const auto rd = make_rsrc(static_cast<const T*>(a.dt) + row0 * Hd, (uint32_t)(nv * Hd * sizeof(T)));
#pragma unroll
    for (int e = 0; e < ChainRegs<T, N>::kU; ++e) {
        int i, p;
        stage_pos(e * kThreads + tid, kP / 4, i, p);
        g.u[e] = load4(tag, ru, (int)((i * H + h) * kP + 4 * p));
    }
#pragma unroll
    for (int e = 0; e < ChainRegs<T, N>::kV; ++e) {
        int i, n;
        stage_pos(e * kThreads + tid, N / 4, i, n);
        g.v[e] = load4(tag, rv, i * N + 4 * n);
    }
    g.dt = load1(tag, rd, (int)((tid & 63) * Hd + h / a.hsub));
}

// One workgroup per (batch, sub-head) and time segment, kept small (about
// 50 KB of LDS, under 170 registers) so that three run on a CU and all
// chains of a training batch run at once.  REV: the adjoint states (pass 2),
// else the states (pass 1).  With time segments (a.nseg > 1) each segment
// starts from zero -- the first from h0, the last adjoint from dh_final --
// and leaves its end state (start adjoint) in seg_state; ssd_chain_carry_kernel
// and ssd_chain_fix_kernel then add what the true boundary matrix contributes
// to every stored one.
template <class T, int N, bool REV>
__global__ __launch_bounds__(kThreads) void ssd_chain_kernel(SsdBwdArgs a) {
    constexpr int NT = N / 64;
    __shared__ ChainSmem<N> s;
    const int tid = threadIdx.x;
    const int wv = wave_id();
    const int lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int sp = wv >> 1;
    const int64_t H = a.H, L = a.L, PN = kP * N;
    const int64_t nch = (L + kQ - 1) / kQ;
    const int64_t job = xcd_order(blockIdx.x, gridDim.x);
    const int64_t bh = job / a.nseg, seg = job % a.nseg;
    const int64_t bi = bh / H, h = bh % H;
    const int64_t c_begin = seg * a.seg_chunks, c_end = imin64(nch, c_begin + a.seg_chunks);
    const int64_t steps = c_end - c_begin;
    const bool first_seg = REV ? c_end == nch : seg == 0;  // the segment whose walk starts at the true boundary
    const float Ah = a.A[h / a.hsub];
    const float bias = a.dt_bias ? a.dt_bias[h / a.hsub] : 0.0f;
    const void* U = REV ? a.dy : a.x;
    const void* V = REV ? a.Cm : a.Bm;
    // where chunk c's entering matrix goes: the states (nch + 1 per job: the final state last), the adjoints
    float* const store_base = REV ? a.dstates + bh * nch * PN : a.states + bh * (nch + 1) * PN;

    const float* init = first_seg ? (REV ? a.dh_final : a.h0) : nullptr;
    f32x16 M[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
#pragma unroll
        for (int r = 0; r < 16; ++r) M[k][r] = init ? init[bh * PN + state_item<N>(wv, k, r, hl, l32)] : 0.0f;
    }

    ChainRegs<T, N> g;
    load_chain_chunk<T, N>(a, U, V, bi, h, (REV ? c_end - 1 : c_begin) * kQ, tid, g);
    float run = 0.0f;  // wave 0, lane 63: log-decay of the chunks walked so far in this segment
    for (int64_t step = 0; step < steps; ++step) {
        const int64_t c = REV ? c_end - 1 - step : c_begin + step;
        const int64_t t0 = c * kQ;
        const int nv = (int)imin64(kQ, L - t0);
        // ---- stage U, V; the weights q and the chunk's decay ----
#pragma unroll
        for (int e = 0; e < ChainRegs<T, N>::kU; ++e) {
            int i, p;
            stage_pos(e * kThreads + tid, kP / 4, i, p);
            p *= 4;
            s.u[i][p] = g.u[e].x; s.u[i][p + 1] = g.u[e].y; s.u[i][p + 2] = g.u[e].z; s.u[i][p + 3] = g.u[e].w;
        }
#pragma unroll
        for (int e = 0; e < ChainRegs<T, N>::kV; ++e) {
            int i, n;
            stage_pos(e * kThreads + tid, N / 4, i, n);
            n *= 4;
            s.v[i][n] = g.v[e].x; s.v[i][n + 1] = g.v[e].y; s.v[i][n + 2] = g.v[e].z; s.v[i][n + 3] = g.v[e].w;
        }
        if (wv == 0) {
            const ChunkScan cs = chunk_scan(g.dt, nv, bias, Ah, a.softplus, lane);
            s.q[lane] = REV ? fexp(cs.cum + cs.lo) : cs.w;
            if (lane == kQ - 1) {
                s.decay = fexp(cs.cum + cs.lo);
                if (a.nseg > 1) {  // for the correction: the decay from the segment's boundary to this chunk
                    a.chunk_dec[bh * nch + c] = fexp(run);
                    run += cs.cum + cs.lo;
                }
            }
        }
        // ---- the matrix entering this chunk, stored ----
        {
            const auto rout = make_rsrc(store_base + c * PN, (uint32_t)(PN * sizeof(float)));
            const int lo = opaque(state_item<N>(wv, 0, 0, hl, l32));
#pragma unroll
            for (int k = 0; k < NT; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    store1<float>(M[k][r], rout, lo + state_item<N>(wv, k, r, 0, 0) - state_item<N>(wv, 0, 0, 0, 0));
        }
        __syncthreads();
        // the next chunk's inputs travel during this chunk's products (none after the last)
        if (step + 1 < steps) load_chain_chunk<T, N>(a, U, V, bi, h, (REV ? c - 1 : c + 1) * kQ, tid, g);

        // ---- M = exp(cum_last) M + (q o U)^T V ----
        const float decay = s.decay;
        constexpr int SU = kP + kPadRow, SV = N + kPadRow;
        const float* uf = &s.u[0][0];
        const float* vf = &s.v[0][0];
        const int ou = opaque(hl * SU + sp * 32 + l32);
        const int ov = opaque(hl * SV + (wv & 1) * NT * 32 + l32);
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            M[k] = mfma_chain_scaled<kQ / 2>(
                M[k] * decay,
                [&](int j, float& av, float& a2, float& bv) {
                    av = s.q[2 * j + hl];
                    a2 = uf[ou + 2 * j * SU];
                    bv = vf[ov + k * 32 + 2 * j * SV];
                },
                [](int) {});
        }
        __syncthreads();  // every wave is done with u, v, q before the next chunk stages over them
    }
    if (a.nseg > 1 && tid == kQ - 1) a.seg_lam[bh * a.nseg + seg] = run;
    // the final state (pass 1) or dh0 (pass 2) from the segment that reaches it, else the segment's own end
    const bool at_end = REV ? seg == 0 : c_end == nch;
    float* const last = at_end ? (REV ? (a.dh0 ? a.dh0 + bh * PN : nullptr) : store_base + nch * PN)
                               : a.seg_state + (bh * a.nseg + seg) * PN;
    if (last) {
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) last[state_item<N>(wv, k, r, hl, l32)] = M[k][r];
    }
}

// The chains' time segments joined: walking the segments outwards from the
// one whose walk was exact, the true matrix T at a segment's outer boundary
// (the state entering it, the adjoint leaving it) is the neighbour's own end
// value plus the neighbour's decay (exp of its chunks' log-decays, summed)
// times the neighbour's T.  One thread per (batch, sub-head, item of the
// P x N matrix) carries T and leaves each segment's T in place of the
// segment's own end value (read a segment ahead); pass 1 also completes the
// final state, pass 2 dh0.
template <int N, bool REV>
__global__ __launch_bounds__(256) void ssd_chain_carry_kernel(SsdBwdArgs a) {
    const int64_t PN = kP * N, nch = (a.L + kQ - 1) / kQ;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.B * a.H * PN) return;
    const int64_t bh = i / PN, e = i % PN;
    const float* __restrict__ lam = a.seg_lam + bh * a.nseg;
    float* __restrict__ seg_t = a.seg_state + bh * a.nseg * PN + e;
    float T = 0.0f;  // the first segment walked is exact
    auto seg_of = [&](int64_t q) { return REV ? a.nseg - 1 - q : q; };
    float own_next = seg_t[seg_of(0) * PN];
    for (int64_t q = 0; q < a.nseg; ++q) {
        const int64_t seg = seg_of(q);
        const float own = own_next;
        if (q + 1 < a.nseg) own_next = seg_t[seg_of(q + 1) * PN];
        const float decay = fexp(lam[seg]);
        seg_t[seg * PN] = T;
        if (q < a.nseg - 1) {
            T = own + decay * T;
        } else {  // the last segment walked: its end value is the final state (pass 1) or dh0 (pass 2)
            float* const end = REV ? (a.dh0 ? a.dh0 + bh * PN + e : nullptr)
                                   : a.states + (bh * (nch + 1) + nch) * PN + e;
            if (end) *end += decay * T;
        }
    }
}

// Every matrix stored inside a segment other than the exact one gains its
// segment's boundary matrix T times the decay between them: one workgroup
// per (batch, sub-head, chunk), its threads over the P x N items.
template <int N, bool REV>
__global__ __launch_bounds__(256) void ssd_chain_fix_kernel(SsdBwdArgs a) {
    constexpr int64_t PN = kP * N;
    const int64_t nch = (a.L + kQ - 1) / kQ;
    const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
    const int64_t seg = c / a.seg_chunks;
    if (seg == (REV ? a.nseg - 1 : 0)) return;  // the exact segment
    const float d = a.chunk_dec[bh * nch + c];
    const float* __restrict__ t = a.seg_state + (bh * a.nseg + seg) * PN;
    float* __restrict__ m = (REV ? a.dstates + (bh * nch + c) * PN : a.states + (bh * (nch + 1) + c) * PN);
#pragma unroll 4
    for (int64_t e = threadIdx.x; e < PN; e += 256) m[e] += d * t[e];
}

// ---------------------------------------------------------------------------
// Pass 3: chunk gradients.
//
// mm holds two Q x Q triangular operands in one array: M2 = G^T o U on and
// above the diagonal (mm[j][k], k >= j) and M3^T = (dY X^T) o U^T strictly
// below it (mm[k][j] = M3[j][k], k > j), M3's diagonal in d3.  Read as
//   M2[j][k] = k >= j ? mm[j][k] : 0
//   M3[j][k] = k > j ? mm[k][j] : k == j ? d3[j] : 0
//   M1[i][k] = (dY X^T o Lmask)[i][k] = M3[k][i] Delta_k.
template <int N>
struct alignas(16) BwdSmem {
    static constexpr int kSB = N + kPadCol, kSX = kP + kPadRow, kSM = kQ + kPadCol;
    float b[kQ][kSB];
    float c[kQ][kSB];
    float x[kQ][kSX];
    float dy[kQ][kSX];
    float dst[N][kSX];   // dS^T: dst[n][p] = dS[p][n]
    float mm[kQ][kSM];
    float d3[kQ];
    float cum[kQ];       // chunk-local cumulative Delta * A_h, as cum + cum_lo (ssdk::chunk_scan)
    float cum_lo[kQ];
    float dlt[kQ];
    float ecum[kQ];      // exp(cum_i)
    float elast[kQ];     // exp(cum_last - cum_j)
    float red_c[N / 32][kQ];  // per n-block row sums of C o dC
    float red_r[2][kQ];       // per p-block row sums of X o V
    float red_d[2][4];        // per wave sums of dY o X (double-buffered by head parity)
    float red_o[2][4];        // per wave parts of <dS, S_out> (double-buffered by head parity)
    float dcd[kQ];            // sum over the group's heads of Delta_i (dY_i . x_i): dC's same-step terms / Bm_i
    float junk[kThreads];     // target of the masked operands' writes that belong to no operand
};

// Per-thread registers of one head's inputs, loaded a head ahead.
template <int N>
struct HeadRegs {
    static constexpr int kX = kQ * kP / 4 / kThreads;  // float4 of X, of dY
    static constexpr int kS = kP * N / kThreads;       // floats of dS
    float4 x[kX], y[kX];
    float ds[kS];
    float dt;
};

// One head's loads, numbered so that a caller can spread their issue over
// matrix products (piece k < kPieces, a compile-time constant after
// unrolling): the X and dY float4s, the dS floats, the step sizes.
template <class T, int N>
struct HeadLoader {
    static constexpr int kX = HeadRegs<N>::kX, kS = HeadRegs<N>::kS;
    static constexpr int kPieces = kX + kS + 1;
    __amdgpu_buffer_rsrc_t rx, ry, rds, rd;
    int64_t H, h, Hd, hd;  // sub-heads and this sub-head (x, dy); heads and this sub-head's head (dt)
    int tid;

    __device__ __forceinline__ HeadLoader(const SsdBwdArgs& a, int64_t bi, int64_t c, int64_t h_, int tid_)
        : H(a.H), h(h_), Hd(a.H / a.hsub), hd(h_ / a.hsub), tid(tid_) {
        const int64_t L = a.L, PN = kP * N;
        const int64_t nch = (L + kQ - 1) / kQ;
        const int64_t t0 = c * kQ;
        const int64_t nv = imin64(kQ, L - t0);
        const int64_t row0 = bi * L + t0;
        const int64_t bh = bi * H + h;
        rx = make_rsrc(static_cast<const T*>(a.x) + row0 * H * kP, (uint32_t)(nv * H * kP * sizeof(T)));
        ry = make_rsrc(static_cast<const T*>(a.dy) + row0 * H * kP, (uint32_t)(nv * H * kP * sizeof(T)));
        // dS through a buffer resource: a lane offset plus per-load constants kept in scalar offsets, not
        // 64-bit addresses per load
        rds = make_rsrc(a.dstates + (bh * nch + c) * PN, (uint32_t)(PN * sizeof(float)));
        rd = make_rsrc(static_cast<const T*>(a.dt) + row0 * Hd, (uint32_t)(nv * Hd * sizeof(T)));
    }

    __device__ __forceinline__ void piece(int k, HeadRegs<N>& g) const {
        const T* tag = nullptr;
        if (k < kX) {
            int i, p;
            stage_pos(k * kThreads + tid, kP / 4, i, p);
            const int off = (int)((i * H + h) * kP + 4 * p);
            g.x[k] = load4(tag, rx, off);
            g.y[k] = load4(tag, ry, off);
        } else if (k < kX + kS) {
            const float* ftag = nullptr;
            g.ds[k - kX] = load1(ftag, rds, (k - kX) * kThreads + tid);
        } else {
            g.dt = load1(tag, rd, (int)((tid & 63) * Hd + hd));
        }
    }

    __device__ __forceinline__ void all(HeadRegs<N>& g) const {
#pragma unroll
        for (int k = 0; k < kPieces; ++k) piece(k, g);
    }
};

// S_in[2 k + hl][nb * 32 + l32], k < 32: the B operand of dY S_in for n-block nb (loaded when the head
// starts, so that it is not held across the previous head's products).
template <int N>
__device__ __forceinline__ void load_sin(const SsdBwdArgs& a, int64_t bh, int64_t c, int nb, int lane, float (&sin)[32]) {
    const int64_t PN = kP * N, nch = (a.L + kQ - 1) / kQ;
    const float* ftag = nullptr;
    const auto rsi = make_rsrc(a.states + (bh * (nch + 1) + c) * PN, (uint32_t)(PN * sizeof(float)));
    const int lo = (lane >> 5) * N + nb * 32 + (lane & 31);
#pragma unroll
    for (int k = 0; k < 32; ++k) sin[k] = load1(ftag, rsi, lo + 2 * k * N);
}

template <class T, int N>
__global__ __launch_bounds__(kThreads) void ssd_bwd_chunk_kernel(SsdBwdArgs a) {
    constexpr int NB = N / 32;           // n-blocks
    constexpr int NTC = NB / 2;          // dC (and dB) tiles per wave: N = 128: (0, w), (1, w); N = 64: (w / 2, w % 2)
    constexpr int SB = BwdSmem<N>::kSB, SX = BwdSmem<N>::kSX, SM = BwdSmem<N>::kSM;
    __shared__ BwdSmem<N> s;
    const int tid = threadIdx.x;
    const int wv = wave_id();
    const int lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int64_t H = a.H, L = a.L;
    const int64_t nch = (L + kQ - 1) / kQ;
    const int64_t g_idx = blockIdx.x % a.groups, rest = blockIdx.x / a.groups;
    const int64_t c = rest % nch, bi = rest / nch;
    const int64_t t0 = c * kQ;
    const int nv = (int)imin64(kQ, L - t0);
    const int64_t h_begin = g_idx * a.heads_per_group, h_end = imin64(H, h_begin + a.heads_per_group);
    const float* bf = &s.b[0][0];
    const float* cf = &s.c[0][0];
    const float* xf = &s.x[0][0];
    const float* yf = &s.dy[0][0];
    const float* sf = &s.dst[0][0];
    const float* mf = &s.mm[0][0];

    // this wave's tiles: dC and dB tiles (row block, n-block) for t < NTC; the V tile (jb, pb)
    auto tile_rb = [&](int t) { return NB == 4 ? t : (wv >> 1); };
    const int nb = NB == 4 ? wv : (wv & 1);
    const int vjb = wv >> 1, vpb = wv & 1;

    // ---- Bm, Cm rows of the chunk, once for all heads ----
    {
        const int64_t row0 = bi * L + t0;
        const T* tag = nullptr;
        const auto rb = make_rsrc(static_cast<const T*>(a.Bm) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
        const auto rc = make_rsrc(static_cast<const T*>(a.Cm) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
#pragma unroll
        for (int e = 0; e < kQ * N / 4 / kThreads; ++e) {
            int i, n;
            stage_pos(e * kThreads + tid, N / 4, i, n);
            const float4 vb = load4(tag, rb, i * N + 4 * n), vc = load4(tag, rc, i * N + 4 * n);
            n *= 4;
            s.b[i][n] = vb.x; s.b[i][n + 1] = vb.y; s.b[i][n + 2] = vb.z; s.b[i][n + 3] = vb.w;
            s.c[i][n] = vc.x; s.c[i][n + 1] = vc.y; s.c[i][n + 2] = vc.z; s.c[i][n + 3] = vc.w;
        }
    }
    HeadRegs<N> g;
    if (h_begin < h_end) HeadLoader<T, N>(a, bi, c, h_begin, tid).all(g);
    __syncthreads();

    // ---- G = C B^T, tiles (0, 0), (1, 0), (1, 1) on waves 0, 1, 2, kept for all heads ----
    const int gti = wv == 0 ? 0 : 1, gtj = wv == 2 ? 1 : 0;
    f32x16 Gt = {};
    if (wv < 3) {
        const int oc = opaque((gti * 32 + l32) * SB + hl), ob = opaque((gtj * 32 + l32) * SB + hl);
        Gt = mfma_chain<N / 2>(Gt, [&](int k, float& av, float& bv) {
            av = cf[oc + 2 * k];
            bv = bf[ob + 2 * k];
        });
    }

    f32x16 dCacc[NTC], dBacc[NTC];
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        dCacc[t] = f32x16{};
        dBacc[t] = f32x16{};
    }

    float sig = 1.0f, dlt_l = 0.0f, cumd = 0.0f;  // wave 3: this head's sigmoid factor, Delta, sum_{s<=t} Delta_s
    float dcd = 0.0f;  // wave 3: sum over the heads so far of Delta_t (dY_t . x_t)
    int par = 0;
    for (int64_t h = h_begin; h < h_end; ++h, par ^= 1) {
        const int64_t hd = h / a.hsub;  // the head this sub-head belongs to
        const float Ah = a.A[hd];
        const float Dh = a.Dskip ? a.Dskip[hd] : 0.0f;
        // ---- (a) stage X, dY, dS^T; step quantities (wave 3) ----
        float pd = 0.0f;
#pragma unroll
        for (int e = 0; e < HeadRegs<N>::kX; ++e) {
            int i, p;
            stage_pos(e * kThreads + tid, kP / 4, i, p);
            p *= 4;
            s.x[i][p] = g.x[e].x; s.x[i][p + 1] = g.x[e].y; s.x[i][p + 2] = g.x[e].z; s.x[i][p + 3] = g.x[e].w;
            s.dy[i][p] = g.y[e].x; s.dy[i][p + 1] = g.y[e].y; s.dy[i][p + 2] = g.y[e].z; s.dy[i][p + 3] = g.y[e].w;
            pd += g.x[e].x * g.y[e].x + g.x[e].y * g.y[e].y + g.x[e].z * g.y[e].z + g.x[e].w * g.y[e].w;
        }
#pragma unroll
        for (int e = 0; e < HeadRegs<N>::kS; ++e) {
            const int f = e * kThreads + tid;  // element (p, n) = (f / N, f % N) of dS
            s.dst[f % N][f / N] = g.ds[e];
        }
        pd = wave_sum(pd, lane);
        if (lane == 0) s.red_d[par][wv] = pd;
        if (wv == 3) {
            const float bias = a.dt_bias ? a.dt_bias[hd] : 0.0f;
            const float v = g.dt + bias;
            const ChunkScan cs = chunk_scan(g.dt, nv, bias, Ah, a.softplus, lane);
            sig = a.softplus ? sigmoid(v) : 1.0f;
            dlt_l = cs.d;
            cumd = wave_prefix_sum(cs.d, lane);
            s.cum[lane] = cs.cum;
            s.cum_lo[lane] = cs.lo;
            s.dlt[lane] = cs.d;
            s.ecum[lane] = fexp(cs.cum + cs.lo);
            const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs.cum), 63));
            const float last_lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs.lo), 63));
            s.elast[lane] = fexp((last - cs.cum) + (last_lo - cs.lo));
        }
        __syncthreads();

        float sin[32];
        load_sin<N>(a, bi * H + h, c, nb, lane, sin);

        // ---- (b) dY X^T tiles and the masked operands (waves 0, 1, 2) ----
        if (wv < 3) {
            const int oy = opaque((gti * 32 + l32) * SX + hl), ox = opaque((gtj * 32 + l32) * SX + hl);
            const f32x16 dyx = mfma_chain<kP / 2>(f32x16{}, [&](int k, float& av, float& bv) {
                av = yf[oy + 2 * k];
                bv = xf[ox + 2 * k];
            });
            // (opaque: the item addresses below are formed per head, not kept in registers across the loop)
            const int j = opaque(gtj * 32 + l32);
            const float cj = s.cum[j], cjl = s.cum_lo[j];
            float ci[16], cil[16];
            acc_row_cum(s.cum, gti, hl, ci);
            acc_row_cum(s.cum_lo, gti, hl, cil);
            // M2[j][i] = G[i][j] f for i >= j, M3[j][i] = dYX[i][j] f for i > j (stored transposed) and on
            // the diagonal (d3), f = exp(cum_i - cum_j) (1 on the diagonal); the items with i < j belong to
            // neither and go to a junk word, so that every lane writes twice per item without a branch
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = gti * 32 + acc_row(r, hl);
                const float f = fexp((ci[r] - cj) + (cil[r] - cjl));
                float* p2 = i >= j ? &s.mm[j][i] : &s.junk[tid];
                float* p3 = i > j ? &s.mm[i][j] : i == j ? &s.d3[j] : &s.junk[tid];
                *p2 = Gt[r] * f;
                *p3 = dyx[r] * f;
            }
        }
        __syncthreads();

        // ---- (c) products ----
        // the next head's inputs travel during this head's products
        const bool more = h + 1 < h_end;
        // <dS, S_out>, the adjoint's pairing with the state leaving the chunk, from the products at hand:
        // S_out = exp(cum_last) S_in + sum_j Delta_j e_j X_j^T B_j, so it is exp(cum_last) <dS, S_in> plus
        // sum_j Delta_j e_j X_j . (B dS^T)_j, whose (B dS^T) tiles the V products below form anyway
        float odot = 0.0f;
        // dC tiles (rb, nb): diag(exp(cum)) dY S_in + M1 B
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const int rb = tile_rb(t);
            const int oy = opaque((rb * 32 + l32) * SX + hl);
            f32x16 acc = mfma_chain<kP / 2>(f32x16{}, [&](int k, float& av, float& bv) {
                av = yf[oy + 2 * k];
                bv = sin[k];
            });
            float ci[16];
            acc_row_cum(s.ecum, rb, hl, ci);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] *= ci[r];
            // M1[i][k] B[k][n] over k <= i: k-blocks 0 .. rb, the last one the diagonal block
            const int i = rb * 32 + l32;
            const int om = opaque(i * SM + hl);
            const int ob = opaque(hl * SB + nb * 32 + l32);
            // (the diagonal k = i is left out here and added below: see the row sums)
            auto ld_m1 = [&](int kb) {
                return [&, kb](int k, float& av, float& a2, float& bv) {
                    const int kk = kb * 32 + 2 * k + hl;
                    const float m = mf[om + kb * 32 + 2 * k];
                    av = kb < rb ? m : (kk < i ? m : 0.0f);
                    a2 = s.dlt[kk];
                    bv = bf[ob + (kb * 32 + 2 * k) * SB];
                };
            };
            if (rb == 1) acc = mfma_chain_scaled<16>(acc, ld_m1(0), [](int) {});
            acc = mfma_chain_scaled<16>(acc, ld_m1(rb), [](int) {});
            // row sums of C o dC over this n-block, without dC's same-step term Delta_i (dY_i . x_i) B_i: in
            // dcum_i = C_i . dC_i - Delta_i x_i . V_i that term cancels exactly against Delta_i (x_i . dY_i)
            // G_ii of the second sum, and with a large step and a fast decay it would dominate both, leaving
            // dcum to the rounding of their difference
            f32x16 cdc;
#pragma unroll
            for (int r = 0; r < 16; ++r) cdc[r] = acc[r] * s.c[rb * 32 + acc_row(r, hl)][nb * 32 + l32];
            const float rs = tile_row_sums(cdc, lane);
            if ((l32 & 1) == 0) s.red_c[nb][rb * 32 + acc_row((l32 >> 1) & 15, hl)] = rs;
            dCacc[t] += acc;  // the same-step terms, summed over the group's heads, are added at the end
        }
        // <dS, S_in> over this wave's n-block (N = 64: waves 2 and 3 hold the blocks of waves 0 and 1)
        if (wv < NB) {
            float sdot = 0.0f;
            const int os = opaque((nb * 32 + l32) * SX + hl);
#pragma unroll
            for (int k = 0; k < 32; ++k) sdot += sin[k] * sf[os + 2 * k];
            odot = s.ecum[kQ - 1] * sdot;
        }
        // the next head's loads go out one per product of the X dS chains (all together, they would hold
        // the wave); past the group's last head, a loader of the last head again (never used)
        const HeadLoader<T, N> next(a, bi, c, more ? h + 1 : h, tid);
        static_assert(HeadLoader<T, N>::kPieces <= NTC * kP / 2, "the X dS chains have a slot for every load");

        // dB tiles (rb, nb): diag(Delta) [diag(e) X dS + M3 C]
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const int rb = tile_rb(t);
            const int ox = opaque((rb * 32 + l32) * SX + hl);
            const int os = opaque((nb * 32 + l32) * SX + hl);
            f32x16 acc = mfma_chain<kP / 2>(
                f32x16{},
                [&](int k, float& av, float& bv) {
                    av = xf[ox + 2 * k];
                    bv = sf[os + 2 * k];
                },
                [&](int k) {
                    const int piece = t * (kP / 2) + k;
                    if (piece < HeadLoader<T, N>::kPieces) next.piece(piece, g);
                });
            float el[16], dl[16];
            acc_row_cum(s.elast, rb, hl, el);
            acc_row_cum(s.dlt, rb, hl, dl);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[r] *= el[r];
            }
            // M3[j][k] C[k][n] over k >= j: k-blocks rb .. 1, the first one the diagonal block
            const int j = rb * 32 + l32;
            const int om = opaque(hl * SM + j);
            const int oc = opaque(hl * SB + nb * 32 + l32);
            auto ld_m3 = [&](int kb) {
                return [&, kb](int k, float& av, float& bv) {
                    const int kk = kb * 32 + 2 * k + hl;
                    const float m = mf[om + (kb * 32 + 2 * k) * SM];
                    av = kb > rb ? m : (kk > j ? m : (kk == j ? s.d3[j] : 0.0f));
                    bv = cf[oc + (kb * 32 + 2 * k) * SB];
                };
            };
            acc = mfma_chain<16>(acc, ld_m3(rb));
            if (rb == 0) acc = mfma_chain<16>(acc, ld_m3(1));
#pragma unroll
            for (int r = 0; r < 16; ++r) dBacc[t][r] += dl[r] * acc[r];
        }

        // V tile (vjb, vpb): diag(e) B dS^T + M2 dY; dX = diag(Delta) V + D dY; row sums of X o V
        {
            const int ob = opaque((vjb * 32 + l32) * SB + hl);
            const int os = opaque(hl * SX + vpb * 32 + l32);
            f32x16 acc = mfma_chain<N / 2>(f32x16{}, [&](int k, float& av, float& bv) {
                av = bf[ob + 2 * k];
                bv = sf[os + 2 * k * SX];
            });
            float el[16], dl[16];
            acc_row_cum(s.elast, vjb, hl, el);
            acc_row_cum(s.dlt, vjb, hl, dl);
            const int px = vpb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[r] *= el[r];
                odot += dl[r] * acc[r] * s.x[vjb * 32 + acc_row(r, hl)][px];
            }
            // M2[j][k] dY[k][p] over k > j: k-blocks vjb .. 1, the first one the diagonal block (whose own
            // diagonal, G_jj dY_j, is added after the row sums: see dC's)
            const int j = vjb * 32 + l32;
            const int om = opaque(j * SM + hl);
            const int oy = opaque(hl * SX + vpb * 32 + l32);
            auto ld_m2 = [&](int kb) {
                return [&, kb](int k, float& av, float& bv) {
                    const int kk = kb * 32 + 2 * k + hl;
                    const float m = mf[om + kb * 32 + 2 * k];
                    av = kb > vjb ? m : (kk > j ? m : 0.0f);
                    bv = yf[oy + (kb * 32 + 2 * k) * SX];
                };
            };
            acc = mfma_chain<16>(acc, ld_m2(vjb));
            if (vjb == 0) acc = mfma_chain<16>(acc, ld_m2(1));
            // dX = Delta_j (V without its same-step term) + (Delta_j G_jj + Dskip) dY_j (rows past the end
            // dropped by the resource); row sums of X o V without the same-step term
            const int p = vpb * 32 + l32;
            const auto rx = make_rsrc(static_cast<T*>(a.dx) + (bi * L + t0) * H * kP,
                                      (uint32_t)(nv * H * kP * sizeof(T)));
            f32x16 xv;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jr = vjb * 32 + acc_row(r, hl);
                const float dyj = s.dy[jr][p];
                store1<T>(dl[r] * (acc[r] + s.mm[jr][jr] * dyj) + Dh * dyj, rx, (int)((jr * H + h) * kP + p));
                xv[r] = s.x[jr][p] * acc[r];
            }
            const float rs = tile_row_sums(xv, lane);
            if ((l32 & 1) == 0) s.red_r[vpb][vjb * 32 + acc_row((l32 >> 1) & 15, hl)] = rs;
        }
        odot = wave_sum(odot, lane);
        if (lane == 0) s.red_o[par][wv] = odot;
        __syncthreads();

        // ---- (d) per-step scalars (wave 3): dcum, dDelta, ddt; this head's dA, dDskip, ddt_bias parts ----
        if (wv == 3) {
            float cdc = 0.0f;
#pragma unroll
            for (int q = 0; q < NB; ++q) cdc += s.red_c[q][lane];
            // both row sums leave out the same-step terms (equal, they cancel in dcum); r_t, the direct
            // derivative by Delta_t, has it: G_tt (x_t . dY_t), M2's and d3's diagonals
            const float r = s.red_r[0][lane] + s.red_r[1][lane];
            const float d3t = s.d3[lane];
            const float r_full = r + s.mm[lane][lane] * d3t;
            dcd += dlt_l * d3t;
            const float dot = s.red_o[par][0] + s.red_o[par][1] + s.red_o[par][2] + s.red_o[par][3];
            const float dcum = cdc - dlt_l * r + (lane == kQ - 1 ? dot : 0.0f);
            const float incl = wave_prefix_sum(dcum, lane);
            const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
            const float dDelta = Ah * (total - incl + dcum) + r_full;
            const float ddt = dDelta * sig;
            if (a.ddt_ws) {  // sub-heads of one head: summed per head in pass 4
                const auto rt = make_rsrc(a.ddt_ws + (bi * L + t0) * H, (uint32_t)(nv * H * sizeof(float)));
                store1<float>(ddt, rt, (int)(lane * H + h));
            } else {
                const auto rt = make_rsrc(static_cast<T*>(a.ddt) + (bi * L + t0) * H, (uint32_t)(nv * H * sizeof(T)));
                store1<T>(ddt, rt, (int)(lane * H + h));
            }
            const float pa = wave_sum(dcum * cumd, lane);
            const float pb = wave_sum(lane < nv ? ddt : 0.0f, lane);
            if (lane == 0) {
                float* part = a.parts + ((bi * nch + c) * H + h) * 3;
                part[0] = pa;
                part[1] = s.red_d[par][0] + s.red_d[par][1] + s.red_d[par][2] + s.red_d[par][3];
                part[2] = pb;
            }
        }
        // no barrier: the next head's staging writes x, dy, dst (read above only before the last barrier), and
        // red_d of the other parity; wave 3 rewrites the step quantities after its own reads
    }

    // ---- dB, dC of the chunk summed over this group's heads; dC's same-step terms Bm_i dcd_i first ----
    __syncthreads();  // every wave is past its last reads of the head's operands (wave 3 past its dcd)
    if (wv == 3) s.dcd[lane] = dcd;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        const int rb = tile_rb(t);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = rb * 32 + acc_row(r, hl);
            dCacc[t][r] += s.dcd[i] * s.b[i][nb * 32 + l32];
        }
    }
    const int64_t row0 = bi * L + t0;
    if (a.groups == 1) {
        const auto rb_ = make_rsrc(static_cast<T*>(a.dB) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
        const auto rc_ = make_rsrc(static_cast<T*>(a.dC) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const int rb = tile_rb(t);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int e = (rb * 32 + acc_row(r, hl)) * N + nb * 32 + l32;
                store1<T>(dBacc[t][r], rb_, e);
                store1<T>(dCacc[t][r], rc_, e);
            }
        }
    } else {
        float* db = a.dbc + (g_idx * a.B * L + row0) * N;
        float* dc = a.dbc + ((a.groups + g_idx) * a.B * L + row0) * N;
        const auto rb_ = make_rsrc(db, (uint32_t)(nv * N * sizeof(float)));
        const auto rc_ = make_rsrc(dc, (uint32_t)(nv * N * sizeof(float)));
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const int rb = tile_rb(t);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int e = (rb * 32 + acc_row(r, hl)) * N + nb * 32 + l32;
                store1<float>(dBacc[t][r], rb_, e);
                store1<float>(dCacc[t][r], rc_, e);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 4: reductions in a fixed order (bitwise reproducible).  One workgroup per
// head h: dA, dDskip, ddt_bias over the (batch, chunk) partials of its
// sub-heads, each thread a strided share, then a tree over the workgroup.
__global__ __launch_bounds__(256) void ssd_bwd_reduce_heads_kernel(SsdBwdArgs a) {
    __shared__ float red[3][256];
    const int64_t h = blockIdx.x, H = a.H, G = a.hsub;
    const int64_t nbc = a.B * ((a.L + kQ - 1) / kQ);
    const int tid = threadIdx.x;
    float sa = 0.0f, sd = 0.0f, sb = 0.0f;
    for (int64_t bc = tid; bc < nbc; bc += 256) {
        for (int64_t q = 0; q < G; ++q) {
            const float* p = a.parts + (bc * H + h * G + q) * 3;
            sa += p[0];
            sd += p[1];
            sb += p[2];
        }
    }
    red[0][tid] = sa;
    red[1][tid] = sd;
    red[2][tid] = sb;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            red[0][tid] += red[0][tid + w];
            red[1][tid] += red[1][tid + w];
            red[2][tid] += red[2][tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.dA[h] = red[0][0];
        if (a.dD) a.dD[h] = red[1][0];
        if (a.ddt_bias) a.ddt_bias[h] = red[2][0];
    }
}

// With sub-heads: ddt of one (batch, step, head) summed over the head's sub-heads.
template <class T>
__global__ __launch_bounds__(256) void ssd_bwd_ddt_kernel(SsdBwdArgs a) {
    const int64_t G = a.hsub, Hd = a.H / G;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= a.B * a.L * Hd) return;
    float v = 0.0f;
    for (int64_t q = 0; q < G; ++q) v += a.ddt_ws[e * G + q];
    store_act(static_cast<T*>(a.ddt), e, v);
}

// With several head groups: dB and dC of one element summed over the groups.
template <class T>
__global__ __launch_bounds__(256) void ssd_bwd_reduce_groups_kernel(SsdBwdArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x, BLN = a.B * a.L * a.N;
    if (e >= BLN) return;
    float sb = 0.0f, sc = 0.0f;
    for (int64_t g = 0; g < a.groups; ++g) {
        sb += a.dbc[g * BLN + e];
        sc += a.dbc[(a.groups + g) * BLN + e];
    }
    store_act(static_cast<T*>(a.dB), e, sb);
    store_act(static_cast<T*>(a.dC), e, sc);
}

// SAVED: a.states holds what the first chain computes (a training forward
// stored it), so only the adjoint chain runs.
template <class T, int N, bool SAVED>
hipError_t launch_bwd_typed(const SsdBwdArgs& a, hipStream_t st) {
    const dim3 chains((unsigned)(a.B * a.H * a.nseg));
    const dim3 carry((unsigned)((a.B * a.H * kP * N + 255) / 256));
    const dim3 fix((unsigned)(a.B * a.H * ((a.L + kQ - 1) / kQ)));
    if constexpr (!SAVED) {
        hipLaunchKernelGGL((ssd_chain_kernel<T, N, false>), chains, dim3(kThreads), 0, st, a);
        if (a.nseg > 1) {
            hipLaunchKernelGGL((ssd_chain_carry_kernel<N, false>), carry, dim3(256), 0, st, a);
            hipLaunchKernelGGL((ssd_chain_fix_kernel<N, false>), fix, dim3(256), 0, st, a);
        }
    }
    hipLaunchKernelGGL((ssd_chain_kernel<T, N, true>), chains, dim3(kThreads), 0, st, a);
    if (a.nseg > 1) {
        hipLaunchKernelGGL((ssd_chain_carry_kernel<N, true>), carry, dim3(256), 0, st, a);
        hipLaunchKernelGGL((ssd_chain_fix_kernel<N, true>), fix, dim3(256), 0, st, a);
    }
    const int64_t nch = (a.L + kQ - 1) / kQ;
    hipLaunchKernelGGL((ssd_bwd_chunk_kernel<T, N>), dim3((unsigned)(a.B * nch * a.groups)), dim3(kThreads), 0, st,
                       a);
    hipLaunchKernelGGL(ssd_bwd_reduce_heads_kernel, dim3((unsigned)(a.H / a.hsub)), dim3(256), 0, st, a);
    if (a.ddt_ws) {
        const int64_t n = a.B * a.L * (a.H / a.hsub);
        hipLaunchKernelGGL((ssd_bwd_ddt_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    }
    if (a.groups > 1) {
        const int64_t n = a.B * a.L * a.N;
        hipLaunchKernelGGL((ssd_bwd_reduce_groups_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_bwd(const SsdBwdArgs& a, hipStream_t st) {
    if (a.dtype == 1)
        return a.N == 64 ? launch_bwd_typed<uint16_t, 64, false>(a, st) : launch_bwd_typed<uint16_t, 128, false>(a, st);
    return a.N == 64 ? launch_bwd_typed<float, 64, false>(a, st) : launch_bwd_typed<float, 128, false>(a, st);
}

hipError_t launch_ssd_bwd_saved(const SsdBwdArgs& a, hipStream_t st) {
    if (a.dtype == 1)
        return a.N == 64 ? launch_bwd_typed<uint16_t, 64, true>(a, st) : launch_bwd_typed<uint16_t, 128, true>(a, st);
    return a.N == 64 ? launch_bwd_typed<float, 64, true>(a, st) : launch_bwd_typed<float, 128, true>(a, st);
}

}  // namespace mssm
