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

// Activation access through a buffer resource, by element offset: T = float,
// or uint16_t holding bfloat16 bits (widened exactly to float32).
__device__ __forceinline__ float4 load4(const float*, __amdgpu_buffer_rsrc_t r, int e) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, 0));
}
__device__ __forceinline__ float4 load4(const uint16_t*, __amdgpu_buffer_rsrc_t r, int e) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, e * 2, 0, 0);
    return make_float4(bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]));
}
__device__ __forceinline__ float load1(const float*, __amdgpu_buffer_rsrc_t r, int e) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, e * 4, 0, 0));
}
__device__ __forceinline__ float load1(const uint16_t*, __amdgpu_buffer_rsrc_t r, int e) {
    return bf16_lo(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, e * 2, 0, 0)));
}
template <class T>
__device__ __forceinline__ void store1(float v, __amdgpu_buffer_rsrc_t r, int e) {
    buffer_store_act(v, r, static_cast<uint32_t>(e) * sizeof(T), T{});
}

// An integer the compiler must treat as unknown at this point (an empty asm
// statement, no instruction).  Recomputing a lane's LDS base offsets through
// it once per chunk keeps them out of loop-invariant hoisting: each step's
// address stays base + constant, with the constant folded into the ds_read
// offset field, instead of one precomputed address register per step.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Row padding (floats) of the LDS operands: kPadCol for arrays read down a
// column (32 rows at one k, the A-operand pattern), kPadRow for arrays read
// along rows by both lane halves (two rows, 32 consecutive columns each).
constexpr int kPadCol = 1;
constexpr int kPadRow = 1;

// One chunk's operands.
template <int N>
struct SsdSmem {
    static constexpr int kSB = N + kPadCol;    // row stride of b, c
    static constexpr int kSX = kP + kPadRow;   // row stride of x, st
    static constexpr int kSM = kQ + kPadCol;   // row stride of m
    float x[kQ][kSX];      // X: the chunk's inputs of this head
    float b[kQ][kSB];      // Bm rows
    float c[kQ][kSB];      // Cm rows
    float m[kQ][kSM];      // M = G o Lmask
    float st[N][kSX];      // S^T, the state entering the chunk
    float cum[kQ];         // chunk-local cumulative Delta * A_h
    float dlt[kQ];         // Delta (0 past the sequence end)
    float w[kQ];           // exp(cum_last - cum_j) Delta_j
};

// acc += sum over STEPS k-steps of A_s B_s, the operands of step s read by
// ld(s, a, b).  The reads run DIST steps ahead of the MFMAs, so the LDS
// latency hides behind the matrix core (one wave per SIMD has no other wave
// to cover it).  DIST times the reads per step stays within the 15 LDS
// operations the wave's lgkm counter can track.
template <int STEPS, int DIST = 6, class F>
__device__ __forceinline__ f32x16 mfma_chain(f32x16 acc, F&& ld) {
    float av[STEPS], bv[STEPS];
#pragma unroll
    for (int s = 0; s < DIST && s < STEPS; ++s) ld(s, av[s], bv[s]);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (s + DIST < STEPS) ld(s + DIST, av[s + DIST], bv[s + DIST]);
        // keep the reads issued ahead: the scheduler would otherwise sink each
        // one next to its MFMA and wait out its latency there
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(av[s], bv[s], acc);
    }
    return acc;
}

// As mfma_chain, with the A operand of step s the product of two values
// ld(s, a, a2, b) reads: the product is formed when the step issues, so its
// reads stay DIST steps ahead too.
template <int STEPS, int DIST = 4, class F>
__device__ __forceinline__ f32x16 mfma_chain_scaled(f32x16 acc, F&& ld) {
    float av[STEPS], a2[STEPS], bv[STEPS];
#pragma unroll
    for (int s = 0; s < DIST && s < STEPS; ++s) ld(s, av[s], a2[s], bv[s]);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (s + DIST < STEPS) ld(s + DIST, av[s + DIST], a2[s + DIST], bv[s + DIST]);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(av[s] * a2[s], bv[s], acc);
    }
    return acc;
}

// The (batch, head) a workgroup takes.  Workgroups are dealt to the eight
// XCDs round robin (workgroup i to XCD i % 8), each XCD with its own L2; this
// order gives XCD x a contiguous run of (batch, head) pairs, so the heads of a
// batch, which all read the same Bm and Cm rows, share one L2 instead of each
// XCD fetching those rows again.  A bijection of [0, n) for any n.
__device__ __forceinline__ int64_t xcd_order(int64_t i, int64_t n) {
    constexpr int64_t kXcds = 8;
    const int64_t per = n / kXcds, rem = n % kXcds;
    const int64_t x = i % kXcds, slot = i / kXcds;
    return x * per + (x < rem ? x : rem) + slot;
}

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
// cover only the chunk's valid rows (those before t_end): a row past the sequence end lies outside
// its resource and reads as zeros, with no branch and no address select (a
// chunk wholly past the end has an empty resource and touches no memory).
template <class T, int N>
__device__ __forceinline__ void load_chunk(const SsdArgs& a, int64_t bi, int64_t h, int64_t t0, int64_t t_end,
                                           int tid, ChunkRegs<N>& g) {
    const int64_t H = a.H, L = a.L;
    const int64_t nv = t_end - t0 < 0 ? 0 : imin64(kQ, t_end - t0);
    const int64_t row0 = bi * L + t0;
    const T* x = static_cast<const T*>(a.x);
    const auto rx = make_rsrc(x + row0 * H * kP, (uint32_t)(nv * H * kP * sizeof(T)));
    const auto rb = make_rsrc(static_cast<const T*>(a.Bm) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
    const auto rc = make_rsrc(static_cast<const T*>(a.Cm) + row0 * N, (uint32_t)(nv * N * sizeof(T)));
    const auto rd = make_rsrc(static_cast<const T*>(a.dt) + row0 * H, (uint32_t)(nv * H * sizeof(T)));
#pragma unroll
    for (int e = 0; e < ChunkRegs<N>::kX; ++e) {
        const int q = e * kThreads + tid, i = q / (kP / 4), p = (q % (kP / 4)) * 4;
        g.x[e] = load4(x, rx, (int)((i * H + h) * kP + p));
    }
#pragma unroll
    for (int e = 0; e < ChunkRegs<N>::kB; ++e) {
        const int q = e * kThreads + tid, i = q / (N / 4), n = (q % (N / 4)) * 4;
        g.b[e] = load4(x, rb, i * N + n);
        g.c[e] = load4(x, rc, i * N + n);
    }
    // step sizes, used by wave 0 only
    g.dt = load1(x, rd, (int)((tid & 63) * H + h));
}

template <class T, int N>
__global__ __launch_bounds__(kThreads) void ssd_fwd_kernel(SsdArgs a) {
    constexpr int NT = N / 64;  // state tiles per wave: the P x N state is 2 x (N / 32) tiles over 4 waves
    __shared__ SsdSmem<N> s;
    const int tid = threadIdx.x;
    const int wv = wave_id();
    const int lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int64_t H = a.H, L = a.L;
    // job = (batch, head, time segment); the segment's steps are [t_begin, t_end)
    const int64_t job = xcd_order(blockIdx.x, gridDim.x);
    const int64_t seg = job % a.nseg, bi = job / a.nseg / H, h = job / a.nseg % H;
    const int64_t t_begin = seg * a.seg_len, t_end = imin64(L, t_begin + a.seg_len);

    const float Ah = a.A[h];
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Dh = a.Dskip ? a.Dskip[h] : 0.0f;

    // this wave's state tiles: rows p in [sp * 32, +32), columns n in [((wv & 1) * NT + k) * 32, +32)
    const int sp = wv >> 1;
    const int64_t state_base = (bi * H + h) * kP * N;
    f32x16 S[NT];
    if (a.h0 && seg == 0) {  // later segments start from zero; the carry pass supplies their state
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) S[k][r] = a.h0[state_base + (int64_t)(sp * 32 + acc_row(r, hl)) * N + n];
        }
    } else {
#pragma unroll
        for (int k = 0; k < NT; ++k) S[k] = f32x16{};
    }

    // this wave's tile (ti, tj) of M (Q x Q) and of Y (Q x P)
    const int ti = wv >> 1, tj = wv & 1;

    ChunkRegs<N> g;
    load_chunk<T, N>(a, bi, h, t_begin, t_end, tid, g);
    float lam = 0.0f;  // the segment's total log-decay, sum of Delta A_h

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kQ) {
        const int nv = (int)imin64(kQ, t_end - t0);

        // ---- stage: the chunk's operands and S^T into LDS; cum, Delta, w ----
#pragma unroll
        for (int e = 0; e < ChunkRegs<N>::kX; ++e) {
            const int q = e * kThreads + tid, i = q / (kP / 4), p = (q % (kP / 4)) * 4;
            s.x[i][p] = g.x[e].x; s.x[i][p + 1] = g.x[e].y; s.x[i][p + 2] = g.x[e].z; s.x[i][p + 3] = g.x[e].w;
        }
#pragma unroll
        for (int e = 0; e < ChunkRegs<N>::kB; ++e) {
            const int q = e * kThreads + tid, i = q / (N / 4), n = (q % (N / 4)) * 4;
            s.b[i][n] = g.b[e].x; s.b[i][n + 1] = g.b[e].y; s.b[i][n + 2] = g.b[e].z; s.b[i][n + 3] = g.b[e].w;
            s.c[i][n] = g.c[e].x; s.c[i][n + 1] = g.c[e].y; s.c[i][n + 2] = g.c[e].z; s.c[i][n + 3] = g.c[e].w;
        }
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) s.st[n][sp * 32 + acc_row(r, hl)] = S[k][r];
        }
        if (wv == 0) {
            float d = 0.0f;
            if (lane < nv) {
                const float v = g.dt + bias;
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

        // the next chunk's inputs travel while this chunk computes (past the end: no access)
        load_chunk<T, N>(a, bi, h, t0 + kQ, t_end, tid, g);
        lam += s.cum[kQ - 1];

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
            if (ti >= tj)
                gm = mfma_chain<N / 2>(gm, [&](int k, float& av, float& bv) {
                    av = cf[oc + 2 * k];
                    bv = bf[ob + 2 * k];
                });
            const int j = tj * 32 + l32;
            const float cj = s.cum[j], dj = s.dlt[j];
            // above the diagonal: exponent -inf and a selected 0 (a non-finite future Bm row must not
            // reach an earlier output), both as selects rather than a branch around the exponential
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ti * 32 + acc_row(r, hl);
                const bool keep = j <= i;
                const float v = gm[r] * fexp(keep ? s.cum[i] - cj : -__builtin_inff()) * dj;
                s.m[i][j] = keep ? v : 0.0f;
            }
        }
        __syncthreads();

        // ---- Y tile (ti, tj): exp(cum_i) (C S^T) + M X + D X ----
        {
            f32x16 y = mfma_chain<N / 2>(f32x16{}, [&](int k, float& av, float& bv) {
                av = cf[oc + 2 * k];
                bv = stf[ost + 2 * k * SX];
            });
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] *= fexp(s.cum[ti * 32 + acc_row(r, hl)]);
            auto ld_mx = [&](int k, float& av, float& bv) {
                av = mf[om + 2 * k];
                bv = xf[ox + 2 * k * SX];
            };
            // M is zero right of the diagonal tile: row block ti contracts over k < (ti + 1) * 32
            if (ti == 0)
                y = mfma_chain<16>(y, ld_mx);
            else
                y = mfma_chain<32>(y, ld_mx);
            // rows past the sequence end fall outside the resource and are dropped
            const int p = tj * 32 + l32;
            if (a.ws_y && seg > 0) {  // a bf16 segment output the correction completes: kept in float32 until then
                const auto rw = make_rsrc(a.ws_y + (bi * L + t0) * H * kP, (uint32_t)(nv * H * kP * 4));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = ti * 32 + acc_row(r, hl);
                    store1<float>(y[r] + Dh * s.x[i][p], rw, (int)((i * H + h) * kP + p));
                }
            } else {
                const auto ry = make_rsrc(static_cast<T*>(a.y) + (bi * L + t0) * H * kP,
                                          (uint32_t)(nv * H * kP * sizeof(T)));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = ti * 32 + acc_row(r, hl);
                    store1<T>(y[r] + Dh * s.x[i][p], ry, (int)((i * H + h) * kP + p));
                }
            }
        }

        // ---- S' = exp(cum_last) S + (w o X)^T B ----
        {
            const float decay = fexp(s.cum[kQ - 1]);
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const int obs = ob_s + k * 32;
                S[k] = mfma_chain_scaled<kQ / 2>(S[k] * decay, [&](int j, float& av, float& a2, float& bv) {
                    av = s.w[2 * j + hl];
                    a2 = xf[oxs + 2 * j * SX];
                    bv = bf[obs + 2 * j * SB];
                });
            }
        }
        __syncthreads();
    }

    // one segment: the final state; several: this segment's state from zero and its log-decay, for the carry pass
    float* out = a.nseg > 1 ? a.ws + ((bi * H + h) * a.nseg + seg) * kP * N : a.h_final ? a.h_final + state_base : nullptr;
    if (out) {
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int n = ((wv & 1) * NT + k) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) out[(int64_t)(sp * 32 + acc_row(r, hl)) * N + n] = S[k][r];
        }
    }
    if (a.nseg > 1 && tid == 0) a.ws[a.B * H * a.nseg * kP * N + (bi * H + h) * a.nseg + seg] = lam;
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
    const float Ah = a.A[h];
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
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
        const auto rd = make_rsrc(static_cast<const T*>(a.dt) + row0 * H, (uint32_t)(nv * H * sizeof(T)));
        dtv = load1(cm, rd, (int)(lane * H + h));
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

template <class T, int N>
hipError_t launch_typed(const SsdArgs& a, hipStream_t st) {
    const dim3 block(kThreads);
    hipLaunchKernelGGL((ssd_fwd_kernel<T, N>), dim3((unsigned)(a.B * a.H * a.nseg)), block, 0, st, a);
    if (a.nseg > 1) {
        const int64_t n = a.B * a.H * a.P * a.N;
        hipLaunchKernelGGL(ssd_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
        hipLaunchKernelGGL((ssd_correct_kernel<T, N>), dim3((unsigned)(a.B * a.H * (a.nseg - 1))), block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st) {
    if (a.dtype == 1) return a.N == 64 ? launch_typed<uint16_t, 64>(a, st) : launch_typed<uint16_t, 128>(a, st);
    return a.N == 64 ? launch_typed<float, 64>(a, st) : launch_typed<float, 128>(a, st);
}

}  // namespace mssm
