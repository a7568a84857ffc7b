// ssd_common.h -- device helpers shared by the SSD (Mamba-2) forward and
// backward kernels: the fp32 matrix-core product chains, activation access
// through buffer resources, the LDS staging map, the XCD-aware order and the
// per-chunk step quantities.
//
// MFMA 32x32x2 f32 lane layout (wave64, lane l, half hl = l / 32):
//   A operand: lane holds A[l % 32][k + hl]; B operand: lane holds B[k + hl][l % 32];
//   accumulator item r: row (r / 4) * 8 + hl * 4 + r % 4, column l % 32.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ssd.h"

namespace mssm {
namespace ssdk {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQ = kSsdChunk;
// spins of a bounded wait for a handed-over state (each with a short sleep)
constexpr uint32_t kSsdMaxWaitSpins = 1u << 27;
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

// acc += sum over STEPS k-steps of A_s B_s, the operands of step s read by
// ld(s, a, b).  The reads run DIST steps ahead of the MFMAs, so the LDS
// latency hides behind the matrix core (one wave per SIMD has no other wave
// to cover it).  DIST times the reads per step stays within the 15 LDS
// operations the wave's lgkm counter can track.
template <int STEPS, int DIST = 6, class F, class S>
__device__ __forceinline__ f32x16 mfma_chain(f32x16 acc, F&& ld, S&& side) {
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
        // other work of step s (side(s)) issues behind the product
        side(s);
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

template <int STEPS, int DIST = 6, class F>
__device__ __forceinline__ f32x16 mfma_chain(f32x16 acc, F&& ld) {
    return mfma_chain<STEPS, DIST>(acc, ld, [](int) {});
}

// As mfma_chain, with the A operand of step s the product of two values
// ld(s, a, a2, b) reads: the product is formed when the step issues, so its
// reads stay DIST steps ahead too.
template <int STEPS, int DIST = 4, class F, class S>
__device__ __forceinline__ f32x16 mfma_chain_scaled(f32x16 acc, F&& ld, S&& side) {
    float av[STEPS], a2[STEPS], bv[STEPS];
#pragma unroll
    for (int s = 0; s < DIST && s < STEPS; ++s) ld(s, av[s], a2[s], bv[s]);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (s + DIST < STEPS) ld(s + DIST, av[s + DIST], a2[s + DIST], bv[s + DIST]);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(av[s] * a2[s], bv[s], acc);
        side(s);
        __builtin_amdgcn_sched_barrier(0);
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

// Where float4 number f of a staged row-major array (cpr float4 per row, an
// odd row stride in LDS) goes: each 32 lanes take 4 rows x 8 float4, lane l at
// row l % 4 and float4 column l / 4.  A staging write of component j then puts
// lane l at bank (row + 4 * column + j) % 32 = (l + const) % 32, 32 distinct
// banks, where 32 lanes along one row would meet 8 banks four times each.  In
// global memory a 32-lane group still reads 4 runs of 128 contiguous bytes.
__device__ __forceinline__ void stage_pos(int f, int cpr, int& row, int& c4) {
    const int u = f >> 5, l = f & 31, upr = cpr / 8;
    row = (u / upr) * 4 + (l & 3);
    c4 = (u % upr) * 8 + (l >> 2);
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele shifts inside each
// row of 16 lanes (DPP row_shr, lanes before the shift add 0), then the
// totals of the earlier rows, read from lanes 15, 31 and 47.
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
    const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const int row = lane >> 4;
    return v + (row >= 1 ? t0 : 0.0f) + (row >= 2 ? t1 : 0.0f) + (row >= 3 ? t2 : 0.0f);
}

// Inclusive prefix sum over the 64 lanes of a value held as an unevaluated
// sum hi + lo, each addition exact: Knuth's TwoSum gives the rounding error
// of hi + hi' exactly, and it joins the lo parts.  cum_i - cum_j for two
// steps of a chunk is then (hi_i - hi_j) + (lo_i - lo_j): when the chunk's
// log-decay is large (|cum| in the thousands) and the steps between i and j
// are tiny, hi_i - hi_j is exact (Sterbenz) and the difference keeps its
// digits, where a plain float32 prefix sum would leave an error of
// ulp(cum) -- a relative error of ulp(cum) in exp(cum_i - cum_j).
// (No contraction anywhere here: an addend fused with the multiply that made
// it into one fma would no longer be the value the error terms refer to.)
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
#pragma clang fp contract(off)
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ void add_df(float& hi, float& lo, float h2, float l2) {
#pragma clang fp contract(off)
    float s, e;
    two_sum(hi, h2, s, e);
    hi = s;
    lo = lo + l2 + e;
}
template <int CTRL>
__device__ __forceinline__ float dpp_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ void wave_prefix_sum_df(float& hi, float& lo, int lane) {
    add_df(hi, lo, dpp_shr<0x111>(hi), dpp_shr<0x111>(lo));
    add_df(hi, lo, dpp_shr<0x112>(hi), dpp_shr<0x112>(lo));
    add_df(hi, lo, dpp_shr<0x114>(hi), dpp_shr<0x114>(lo));
    add_df(hi, lo, dpp_shr<0x118>(hi), dpp_shr<0x118>(lo));
    const int row = lane >> 4;
    float th = 0.0f, tl = 0.0f;  // the totals of the earlier rows, added in row order
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const float h2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hi), 16 * q + 15));
        const float l2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lo), 16 * q + 15));
        if (row > q) add_df(th, tl, h2, l2);
    }
    add_df(hi, lo, th, tl);
}

// One chunk's step quantities, lane t = step t of the chunk: Delta_t (0 for
// steps past the segment end, nv valid steps), the chunk-local cumulative
// log-decay cum_t = sum_{s <= t} Delta_s A_h as hi + lo (wave_prefix_sum_df;
// each product Delta_s A_h split exactly by an fma), and the state weight
// w_t = exp(cum_last - cum_t) Delta_t.
struct ChunkScan {
    float d, cum, lo, w;
};
__device__ __forceinline__ ChunkScan chunk_scan(float dtv, int nv, float bias, float Ah, int softplus_on, int lane) {
#pragma clang fp contract(off)
    float d = 0.0f;
    if (lane < nv) {
        const float v = dtv + bias;
        d = softplus_on ? softplus(v) : v;
    }
    float hi = d * Ah;
    float lo = __builtin_fmaf(d, Ah, -hi);
    wave_prefix_sum_df(hi, lo, lane);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hi), 63));
    const float last_lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lo), 63));
    return {d, hi, lo, fexp((last - hi) + (last_lo - lo)) * d};
}

// cum of the 16 accumulator rows a lane of half hl holds in row block ti
// (rows ti * 32 + g * 8 + hl * 4 + q for item r = 4 g + q): four 16-byte reads.
__device__ __forceinline__ void acc_row_cum(const float* cum, int ti, int hl, float (&ci)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(cum + ti * 32 + g * 8 + hl * 4);
        ci[4 * g] = v.x;
        ci[4 * g + 1] = v.y;
        ci[4 * g + 2] = v.z;
        ci[4 * g + 3] = v.w;
    }
}

}  // namespace ssdk
}  // namespace mssm
