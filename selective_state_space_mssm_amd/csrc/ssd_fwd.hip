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
//     Y   = diag(exp(cum)) C S^T + (M + D_h I) X         (Q x P)
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

#include "balanced_plan.h"
#include "device_common.h"
#include "ssd.h"
#include "ssd_common.h"

namespace mssm {
namespace {
using namespace ssdk;

// One chunk's operands.  16-byte aligned: cum is read four floats at a time.
template <int N>
struct alignas(16) SsdSmem {
    static constexpr int kSB = N + kPadCol;    // row stride of b, c
    static constexpr int kSX = kP + kPadRow;   // row stride of x, st
    static constexpr int kSM = kQ + kPadCol;   // row stride of m
    float x[kQ][kSX];      // X: the chunk's inputs of this head
    float b[kQ][kSB];      // Bm rows
    float c[kQ][kSB];      // Cm rows
    float m[kQ][kSM];      // M = G o Lmask
    float st[N][kSX];      // S^T, the state entering the chunk
    float cum[kQ];         // chunk-local cumulative Delta * A_h, as cum + cum_lo (ssdk::chunk_scan)
    float cum_lo[kQ];
    float dlt[kQ];         // Delta (0 past the sequence end)
    float w[kQ];           // exp(cum_last - cum_j) Delta_j
};

// One chunk's global inputs, held in registers from the previous chunk's
// compute until they are staged into LDS.
template <int N>
struct ChunkRegs {
    static constexpr int kX = kQ * kP / 4 / kThreads;  // float4 per thread of X
    static constexpr int kB = kQ * N / 4 / kThreads;   // float4 per thread of Bm, of Cm
    float4 x[kX], b[kB], c[kB];
    float dt;
};

// Loads chunk [t0, t0 + 64) into registers through buffer resources that
// cover only the chunk's valid rows (those before t_end): a row past the
// sequence end lies outside its resource and reads as zeros, with no branch and
// no address select (a chunk wholly past the end has an empty resource and
// touches no memory).  The loads are numbered (piece k < kPieces: the X float4s,
// then Bm's, Cm's, then the step sizes) so that a caller can spread their
// issue over other work; k must be a compile-time constant after unrolling.
template <class T, int N>
struct ChunkLoader {
    static constexpr int kX = ChunkRegs<N>::kX, kB = ChunkRegs<N>::kB;
    static constexpr int kPieces = kX + 2 * kB + 1;
    __amdgpu_buffer_rsrc_t rx, rb, rc, rd;
    int64_t H, h, Hd, hd;  // sub-heads and this sub-head (x); heads and this sub-head's head (dt)
    int tid;

    __device__ __forceinline__ ChunkLoader(const SsdArgs& a, int64_t bi, int64_t h_, int64_t t0, int64_t t_end,
                                           int tid_)
        : H(a.H), h(h_), Hd(a.H / a.hsub), hd(h_ / a.hsub), tid(tid_) {
        const int64_t nv = t_end - t0 < 0 ? 0 : imin64(kQ, t_end - t0);
        const int64_t row0 = bi * a.L + t0;
        rx = make_rsrc(static_cast<const T*>(a.x) + row0 * H * kP, (uint32_t)(nv * H * kP * sizeof(T)));
        rb = make_rsrc(static_cast<const T*>(a.Bm) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
        rc = make_rsrc(static_cast<const T*>(a.Cm) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
        rd = make_rsrc(static_cast<const T*>(a.dt) + row0 * Hd, (uint32_t)(nv * Hd * sizeof(T)));
    }

    __device__ __forceinline__ void piece(int k, ChunkRegs<N>& g) const {
        const T* tag = nullptr;  // selects the load4 / load1 overload of the activation type
        if (k < kX) {
            int i, p;
            stage_pos(k * kThreads + tid, kP / 4, i, p);
            g.x[k] = load4(tag, rx, (int)((i * H + h) * kP + 4 * p));
        } else if (k < kPieces - 1) {
            const int e = (k - kX) % kB;
            int i, n;
            stage_pos(e * kThreads + tid, N / 4, i, n);
            if (k < kX + kB)
                g.b[e] = load4(tag, rb, i * N + 4 * n);
            else
                g.c[e] = load4(tag, rc, i * N + 4 * n);
        } else {
            g.dt = load1(tag, rd, (int)((tid & 63) * Hd + hd));  // lane = step; used by wave 1
        }
    }

    __device__ __forceinline__ void all(ChunkRegs<N>& g) const {
#pragma unroll
        for (int k = 0; k < kPieces; ++k) piece(k, g);
    }
};

// SAVE: the training forward, which also stores the state entering every
// chunk and the final state (a.states); with time segments, those of the
// segment's zero start and each chunk's decay from the segment's start, for
// ssd_states_fix_kernel.
template <class T, int N, bool SAVE>
__global__ __launch_bounds__(kThreads) void ssd_fwd_kernel(SsdArgs a) {
    constexpr int NT = N / 64;  // state tiles per wave: the P x N state is 2 x (N / 32) tiles over 4 waves
    __shared__ SsdSmem<N> s;
    const int tid = threadIdx.x;
    const int wv = wave_id();
    const int lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int64_t H = a.H, L = a.L;
    // this wave's state tiles: rows p in [sp * 32, +32), columns n in [((wv & 1) * NT + k) * 32, +32)
    const int sp = wv >> 1;
    // this wave's tile (ti, tj) of M (Q x Q) and of Y (Q x P)
    const int ti = wv >> 1, tj = wv & 1;
    // offset of state item (tile k, accumulator item r) of this lane in a (P, N) state
    auto state_off = [&](int k, int r) { return (sp * 32 + acc_row(r, hl)) * N + ((wv & 1) * NT + k) * 32 + l32; };

    // What this workgroup scans, as segments: a (batch, head) job and its steps [t_begin, t_end).
    //  * workers == 0: one segment, (batch, head, time segment) number xcd_order(blockIdx.x);
    //  * workers > 0: worker xcd_order(blockIdx.x) of the balanced persistent schedule
    //    (balanced_plan.h) over B * H jobs of nch chunks each: every CU scans the same number of
    //    chunks, and a job split between two workers hands its state over through the workspace.
    //    Consecutive workers run on one XCD, so a handed-over state and the Bm, Cm rows of a batch
    //    mostly stay in one L2.
    const int64_t nch = (L + kQ - 1) / kQ;
    const int64_t worker = xcd_order(blockIdx.x, gridDim.x);
    BalancedRange rg{};
    int nsegs = 1;
    if (a.workers > 0) {
        rg = balanced_range(a.B * H, nch, a.workers, worker);
        nsegs = rg.nseg;
    }
    for (int sg = 0; sg < nsegs; ++sg) {
        int64_t bh, seg = 0, t_begin, t_end;
        int from = kFromH0, to = kFinal;
        if (a.workers == 0) {
            bh = worker / a.nseg;
            seg = worker % a.nseg;
            t_begin = seg * a.seg_len;
            t_end = imin64(L, t_begin + a.seg_len);
        } else {
            const BalancedSegment bs = balanced_segment(rg, nch, sg);
            bh = bs.blk;
            t_begin = bs.tile_begin * kQ;
            t_end = imin64(L, bs.tile_end * kQ);
            from = bs.from;
            to = bs.to;
        }
        const int64_t bi = bh / H, h = bh % H;

        const int64_t hd = h / a.hsub;  // the head this sub-head belongs to
        const float Ah = a.A[hd];
        const float bias = a.dt_bias ? a.dt_bias[hd] : 0.0f;
        const float Dh = a.Dskip ? a.Dskip[hd] : 0.0f;

        const int64_t state_base = bh * kP * N;
        f32x16 S[NT];
#pragma unroll
        for (int k = 0; k < NT; ++k) S[k] = f32x16{};
        if (from == kFromPublished) {
            // the previous worker scanned this job up to t_begin first of all its segments and published
            // the state; bounded wait: past the limit (minutes; a legitimate wait lasts at most one
            // worker's range) the worker records the failure in the word after the flags and goes on
            // instead of hanging the GPU
            if (tid == 0) {
                uint32_t spins = 0;
                while (__hip_atomic_load(a.flags + worker - 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
                    if (++spins == kSsdMaxWaitSpins) {
                        __hip_atomic_store(a.flags + a.workers, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            float* src = a.carry + (worker - 1) * kP * N;
#pragma unroll
            for (int k = 0; k < NT; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    S[k][r] = __hip_atomic_load(src + state_off(k, r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (a.h0 && seg == 0) {  // later time segments start from zero; the carry pass supplies their state
#pragma unroll
            for (int k = 0; k < NT; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[k][r] = a.h0[state_base + state_off(k, r)];
        }

        ChunkRegs<N> g;
        ChunkLoader<T, N>(a, bi, h, t_begin, t_end, tid).all(g);
        float lam = 0.0f;  // the segment's total log-decay, sum of Delta A_h
        // wave 1, the one with the least matrix work (its M tile lies above the
        // diagonal), forms each chunk's step quantities one chunk ahead, off the
        // path to the first barrier
        ChunkScan cs{};
        if (wv == 1) cs = chunk_scan(g.dt, (int)imin64(kQ, t_end - t_begin), bias, Ah, a.softplus, lane);

        for (int64_t t0 = t_begin; t0 < t_end; t0 += kQ) {
            const int nv = (int)imin64(kQ, t_end - t0);
            if constexpr (SAVE) {  // the state entering this chunk, in the (P, N) layout of the backward's chains
                if (a.nseg > 1 && tid == 0) a.chunk_dec[bh * nch + t0 / kQ] = fexp(lam);
                float* st_out = a.states + (bh * (nch + 1) + t0 / kQ) * kP * N;
#pragma unroll
                for (int k = 0; k < NT; ++k)
#pragma unroll
                    for (int r = 0; r < 16; ++r) st_out[state_off(k, r)] = S[k][r];
            }

            // ---- stage: the chunk's operands and S^T into LDS; cum, Delta, w ----
#pragma unroll
            for (int e = 0; e < ChunkRegs<N>::kX; ++e) {
                int i, p;
                stage_pos(e * kThreads + tid, kP / 4, i, p);
                p *= 4;
                s.x[i][p] = g.x[e].x; s.x[i][p + 1] = g.x[e].y; s.x[i][p + 2] = g.x[e].z; s.x[i][p + 3] = g.x[e].w;
            }
#pragma unroll
            for (int e = 0; e < ChunkRegs<N>::kB; ++e) {
                int i, n;
                stage_pos(e * kThreads + tid, N / 4, i, n);
                n *= 4;
                s.b[i][n] = g.b[e].x; s.b[i][n + 1] = g.b[e].y; s.b[i][n + 2] = g.b[e].z; s.b[i][n + 3] = g.b[e].w;
                s.c[i][n] = g.c[e].x; s.c[i][n + 1] = g.c[e].y; s.c[i][n + 2] = g.c[e].z; s.c[i][n + 3] = g.c[e].w;
            }
            // S^T is the B operand of C S^T
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) s.st[n][sp * 32 + acc_row(r, hl)] = S[k][r];
            }
            if (wv == 1) {
                s.cum[lane] = cs.cum;
                s.cum_lo[lane] = cs.lo;
                s.dlt[lane] = cs.d;
                s.w[lane] = cs.w;
            }
            __syncthreads();

            // the next chunk's inputs travel while this chunk computes (past the end: no access)
            const ChunkLoader<T, N> next(a, bi, h, t0 + kQ, t_end, tid);
            lam += s.cum[kQ - 1] + s.cum_lo[kQ - 1];

            // per-lane LDS base offsets (floats) of the MFMA operands; step k adds a constant
            constexpr int SB = SsdSmem<N>::kSB, SX = SsdSmem<N>::kSX, SM = SsdSmem<N>::kSM;
            const float* cf = &s.c[0][0];
            const float* bf = &s.b[0][0];
            const float* xf = &s.x[0][0];
            const float* mf = &s.m[0][0];
            const float* stf = &s.st[0][0];
            const int oc = opaque((ti * 32 + l32) * SB + hl);   // C[i][k + hl]
            const int ob = opaque((tj * 32 + l32) * SB + hl);   // B^T[k + hl][j]
            const int ost = opaque(hl * SX + tj * 32 + l32);     // S^T[k + hl][p]
            const int om = opaque((ti * 32 + l32) * SM + hl);   // M[i][k + hl]
            const int ox = opaque(hl * SX + tj * 32 + l32);     // X[k + hl][p]
            const int oxs = opaque(hl * SX + sp * 32 + l32);     // X[j + hl][p] of the state rows
            const int ob_s = opaque(hl * SB + (wv & 1) * NT * 32 + l32);   // B[j + hl][n]

            // ---- M = (C B^T) o Lmask, tile (ti, tj); the tile above the diagonal is zero ----
            {
                f32x16 gm = {};
                if (ti >= tj) {
                    // the next chunk's loads go out one every other product, while the matrix core runs:
                    // issued back to back they hold the wave for thousands of cycles
                    gm = mfma_chain<N / 2>(
                        gm,
                        [&](int k, float& av, float& bv) {
                            av = cf[oc + 2 * k];
                            bv = bf[ob + 2 * k];
                        },
                        [&](int k) {
                            if (k % 2 == 0 && k / 2 < next.kPieces) next.piece(k / 2, g);
                        });
                    static_assert(ChunkLoader<T, N>::kPieces <= N / 4, "the G chain has a slot for every load");
                } else {
                    next.all(g);
                }
                const int j = tj * 32 + l32;
                const float cj = s.cum[j], cjl = s.cum_lo[j], dj = s.dlt[j];
                float ci[16], cil[16];
                acc_row_cum(s.cum, ti, hl, ci);
                acc_row_cum(s.cum_lo, ti, hl, cil);
                // above the diagonal: exponent -inf and a selected 0 (a non-finite future Bm row must not
                // reach an earlier output), both as selects rather than a branch around the exponential; on the
                // diagonal the skip weight D_h joins M (Y = (M + D_h I) X: the skip term rides the M X product)
                const float dsk = ti == tj ? Dh : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = ti * 32 + acc_row(r, hl);
                    const bool keep = j <= i;
                    const float v = gm[r] * fexp(keep ? (ci[r] - cj) + (cil[r] - cjl) : -__builtin_inff()) * dj;
                    s.m[i][j] = keep ? (i == j ? v + dsk : v) : 0.0f;
                }
            }
            __syncthreads();  // M is read by other waves below

            // ---- Y tile (ti, tj): exp(cum_i) (C S^T) + (M + D_h I) X ----
            f32x16 y = {};
            {
                y = mfma_chain<N / 2>(f32x16{}, [&](int k, float& av, float& bv) {
                    av = cf[oc + 2 * k];
                    bv = stf[ost + 2 * k * SX];
                });
                float ci[16], cil[16];
                acc_row_cum(s.cum, ti, hl, ci);
                acc_row_cum(s.cum_lo, ti, hl, cil);
#pragma unroll
                for (int r = 0; r < 16; ++r) y[r] *= fexp(ci[r] + cil[r]);
                auto ld_mx = [&](int k, float& av, float& bv) {
                    av = mf[om + 2 * k];
                    bv = xf[ox + 2 * k * SX];
                };
                // M is zero right of the diagonal tile: row block ti contracts over k < (ti + 1) * 32
                if (ti == 0)
                    y = mfma_chain<16>(y, ld_mx);
                else
                    y = mfma_chain<32>(y, ld_mx);
            }
            // rows past the sequence end fall outside the resource and are dropped; a bf16 output of a
            // time segment the correction completes stays float32 until then
            const bool to_ws = a.ws_y && seg > 0;
            const auto ry = to_ws ? make_rsrc(a.ws_y + (bi * L + t0) * H * kP, (uint32_t)(nv * H * kP * 4))
                                  : make_rsrc(static_cast<T*>(a.y) + (bi * L + t0) * H * kP,
                                              (uint32_t)(nv * H * kP * sizeof(T)));
            auto store_y = [&](int r) {
                const int e = (int)(((ti * 32 + acc_row(r, hl)) * H + h) * kP + tj * 32 + l32);
                if (to_ws)
                    store1<float>(y[r], ry, e);
                else
                    store1<T>(y[r], ry, e);
            };

            if (wv == 1) cs = chunk_scan(g.dt, (int)imin64(kQ, t_end - t0 - kQ), bias, Ah, a.softplus, lane);

            // ---- S' = exp(cum_last) S + (w o X)^T B ----
            {
                const float decay = fexp(s.cum[kQ - 1] + s.cum_lo[kQ - 1]);
#pragma unroll
                for (int k = 0; k < NT; ++k) {
                    const int obs = ob_s + k * 32;
                    // the Y tile goes out one item every other product of the first update
                    S[k] = mfma_chain_scaled<kQ / 2>(
                        S[k] * decay,
                        [&](int j, float& av, float& a2, float& bv) {
                            av = s.w[2 * j + hl];
                            a2 = xf[oxs + 2 * j * SX];
                            bv = bf[obs + 2 * j * SB];
                        },
                        [&](int j) {
                            if (k == 0 && j % 2 == 0) store_y(j / 2);
                        });
                }
            }
            __syncthreads();
        }

        // The segment's end state: h_final; with time segments, this segment's state from zero and its
        // log-decay, for the carry pass; a split job's first part, the state the next worker continues from.
        float* out = to == kPublish ? a.carry + worker * kP * N
                     : a.nseg > 1   ? a.ws + (bh * a.nseg + seg) * kP * N
                     : a.h_final    ? a.h_final + state_base
                                    : nullptr;
        if (out) {
#pragma unroll
            for (int k = 0; k < NT; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r) out[state_off(k, r)] = S[k][r];
        }
        if (SAVE && to == kFinal && t_end == L) {  // the final state, after the states entering the chunks
            float* st_out = a.states + (bh * (nch + 1) + nch) * kP * N;
#pragma unroll
            for (int k = 0; k < NT; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r) st_out[state_off(k, r)] = S[k][r];
        }
        if (a.nseg > 1 && tid == 0) a.ws[a.B * H * a.nseg * kP * N + bh * a.nseg + seg] = lam;
        if (to == kPublish) {
            __threadfence();
            __syncthreads();
            if (tid == 0) __hip_atomic_store(a.flags + worker, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Carry pass over the segments, one thread per (batch, head, p, n): the state
// entering segment k is exp(lam_{k-1}) times the state entering k - 1 plus
// segment k - 1's own final state.  Segment 0 was scanned from h0, so its
// final state is already exact and the carry starts from zero.  Each entering
// state replaces the segment's slot in the workspace; the last carry is h_final.
__global__ __launch_bounds__(256) void ssd_carry_kernel(SsdArgs a) {
    const int64_t PN = a.P * a.N, e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= a.B * a.H * PN) return;
    const int64_t bh = e / PN, pn = e % PN;
    const float* lam = a.ws + a.B * a.H * a.nseg * PN + bh * a.nseg;
    float cur = 0.0f;
    for (int64_t k = 0; k < a.nseg; ++k) {
        float* slot = a.ws + (bh * a.nseg + k) * PN + pn;
        const float loc = *slot;
        *slot = cur;
        cur = fexp(lam[k]) * cur + loc;
    }
    if (a.h_final) a.h_final[e] = cur;
}

// The training forward's stored states of time segments k >= 1, which started
// from zero: adds the segment's true entering state (the carry pass's) times
// the decay from the segment's start to each chunk, and to the final state the
// last segment's total decay times its entering state.  One workgroup per
// (batch, head, chunk or the final slot).
__global__ __launch_bounds__(256) void ssd_states_fix_kernel(SsdArgs a) {
    const int64_t PN = a.P * a.N, nch = (a.L + kQ - 1) / kQ;
    const int64_t bh = blockIdx.x / (nch + 1), c = blockIdx.x % (nch + 1);
    const float* lam = a.ws + a.B * a.H * a.nseg * PN + bh * a.nseg;
    int64_t seg;
    float d;
    if (c == nch) {
        seg = a.nseg - 1;
        d = fexp(lam[seg]);
    } else {
        seg = c / (a.seg_len / kQ);
        if (seg == 0) return;  // segment 0 started from h0: its states are exact
        d = a.chunk_dec[bh * nch + c];
    }
    const float* sin = a.ws + (bh * a.nseg + seg) * PN;
    float* out = a.states + (bh * (nch + 1) + c) * PN;
    for (int64_t e = threadIdx.x; e < PN; e += 256) out[e] = __builtin_fmaf(d, sin[e], out[e]);
}

// Correction pass, one workgroup per (batch, head, segment k >= 1): adds the
// entering state's contribution exp(cum_t) C_t S_in^T to every output row of
// the segment, cum_t being the log-decay from the segment's start through t.
template <int N>
struct SsdCorrSmem {
    float c[kQ][N + kPadCol];
    float st[N][kP + kPadRow];
    float cum[kQ];
};

template <class T, int N>
__global__ __launch_bounds__(kThreads) void ssd_correct_kernel(SsdArgs a) {
    __shared__ SsdCorrSmem<N> s;
    constexpr int SB = N + kPadCol, SX = kP + kPadRow;
    const int tid = threadIdx.x;
    const int wv = wave_id();
    const int lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int64_t H = a.H, L = a.L, S1 = a.nseg - 1;
    const int64_t job = xcd_order(blockIdx.x, gridDim.x);
    const int64_t seg = job % S1 + 1, bi = job / S1 / H, h = job / S1 % H;
    const int64_t t_begin = seg * a.seg_len, t_end = imin64(L, t_begin + a.seg_len);
    const int64_t Hd = H / a.hsub, hd = h / a.hsub;  // heads; the head this sub-head belongs to
    const float Ah = a.A[hd];
    const float bias = a.dt_bias ? a.dt_bias[hd] : 0.0f;
    const int ti = wv >> 1, tj = wv & 1;

    // S_in^T into LDS, once: the state is the same for the whole segment
    const float* sin = a.ws + ((bi * H + h) * a.nseg + seg) * kP * N;
    for (int e = tid; e < kP * N; e += kThreads) s.st[e % N][e / N] = sin[e];

    // one chunk's Cm rows and step sizes, loaded a chunk ahead; rows past the segment's end read zeros
    constexpr int kC = kQ * N / 4 / kThreads;
    float4 cr[kC];
    float dtv;
    auto load = [&](int64_t t0) {
        const int64_t nv = t_end - t0 < 0 ? 0 : imin64(kQ, t_end - t0), row0 = bi * L + t0;
        const T* cm = static_cast<const T*>(a.Cm);
        const auto rc = make_rsrc(cm + row0 * N, (uint32_t)(nv * N * sizeof(T)));
#pragma unroll
        for (int e = 0; e < kC; ++e) {
            const int q = e * kThreads + tid, i = q / (N / 4), n = (q % (N / 4)) * 4;
            cr[e] = load4(cm, rc, i * N + n);
        }
        const auto rd = make_rsrc(static_cast<const T*>(a.dt) + row0 * Hd, (uint32_t)(nv * Hd * sizeof(T)));
        dtv = load1(cm, rd, (int)(lane * Hd + hd));
    };
    load(t_begin);

    float carry = 0.0f;  // log-decay from the segment's start to the current chunk's start
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kQ) {
        const int nv = (int)imin64(kQ, t_end - t0);
        const int64_t row0 = bi * L + t0;
#pragma unroll
        for (int e = 0; e < kC; ++e) {
            const int q = e * kThreads + tid, i = q / (N / 4), n = (q % (N / 4)) * 4;
            s.c[i][n] = cr[e].x; s.c[i][n + 1] = cr[e].y; s.c[i][n + 2] = cr[e].z; s.c[i][n + 3] = cr[e].w;
        }
        if (wv == 0) {
            const float v = dtv + bias;
            float c = lane < nv ? (a.softplus ? softplus(v) : v) * Ah : 0.0f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(c, off);
                if (lane >= off) c += o;
            }
            s.cum[lane] = carry + c;
        }
        __syncthreads();
        load(t0 + kQ);  // the next chunk's inputs travel during this chunk (past the end: no access)

        // the outputs this lane adds to, read before the products; rows past the end fall outside the resource
        T* yp = static_cast<T*>(a.y);
        const auto ry = make_rsrc(yp + row0 * H * kP, (uint32_t)(nv * H * kP * sizeof(T)));
        const int p = tj * 32 + l32;
        float old[16];
        if (a.ws_y) {  // the segment pass's float32 outputs (bf16 problems)
            const float* wy = a.ws_y;
            const auto rw = make_rsrc(wy + row0 * H * kP, (uint32_t)(nv * H * kP * 4));
#pragma unroll
            for (int r = 0; r < 16; ++r)
                old[r] = load1(wy, rw, (int)(((ti * 32 + acc_row(r, hl)) * H + h) * kP + p));
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                old[r] = load1(yp, ry, (int)(((ti * 32 + acc_row(r, hl)) * H + h) * kP + p));
        }
        const int oc = opaque((ti * 32 + l32) * SB + hl);
        const int ost = opaque(hl * SX + tj * 32 + l32);
        const float* cf = &s.c[0][0];
        const float* stf = &s.st[0][0];
        f32x16 y = mfma_chain<N / 2>(f32x16{}, [&](int k, float& av, float& bv) {
            av = cf[oc + 2 * k];
            bv = stf[ost + 2 * k * SX];
        });
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = ti * 32 + acc_row(r, hl);
            store1<T>(old[r] + y[r] * fexp(s.cum[i]), ry, (int)((i * H + h) * kP + p));
        }
        carry = s.cum[kQ - 1];
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void ssd_zero_flags_kernel(uint32_t* flags, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) flags[i] = 0u;
}

template <class T, int N>
hipError_t launch_typed(const SsdArgs& a, hipStream_t st) {
    const dim3 block(kThreads);
    if (a.workers > 0) {  // a fill kernel rather than a memset: the launch may be captured in a graph
        hipLaunchKernelGGL(ssd_zero_flags_kernel, dim3((unsigned)((a.workers + 1 + 255) / 256)), dim3(256), 0, st,
                           a.flags, a.workers + 1);
        if (a.states)
            hipLaunchKernelGGL((ssd_fwd_kernel<T, N, true>), dim3((unsigned)a.workers), block, 0, st, a);
        else
            hipLaunchKernelGGL((ssd_fwd_kernel<T, N, false>), dim3((unsigned)a.workers), block, 0, st, a);
        return hipGetLastError();
    }
    if (a.states && a.nseg > 1 && !a.chunk_dec) return hipErrorInvalidValue;
    if (a.states)
        hipLaunchKernelGGL((ssd_fwd_kernel<T, N, true>), dim3((unsigned)(a.B * a.H * a.nseg)), block, 0, st, a);
    else
        hipLaunchKernelGGL((ssd_fwd_kernel<T, N, false>), dim3((unsigned)(a.B * a.H * a.nseg)), block, 0, st, a);
    if (a.nseg > 1) {
        const int64_t n = a.B * a.H * a.P * a.N;
        hipLaunchKernelGGL(ssd_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
        hipLaunchKernelGGL((ssd_correct_kernel<T, N>), dim3((unsigned)(a.B * a.H * (a.nseg - 1))), block, 0, st, a);
        if (a.states) {
            const int64_t slots = a.B * a.H * ((a.L + kQ - 1) / kQ + 1);
            hipLaunchKernelGGL(ssd_states_fix_kernel, dim3((unsigned)slots), dim3(256), 0, st, a);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st) {
    if (a.dtype == 1) return a.N == 64 ? launch_typed<uint16_t, 64>(a, st) : launch_typed<uint16_t, 128>(a, st);
    return a.N == 64 ? launch_typed<float, 64>(a, st) : launch_typed<float, 128>(a, st);
}

}  // namespace mssm
