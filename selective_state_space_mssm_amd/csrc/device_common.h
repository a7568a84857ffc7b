// device_common.h -- gfx950 device helpers shared by the scan kernels.
//
// Activation storage types: `float` for fp32 problems, `uint16_t` holding
// bfloat16 bit patterns for bf16 problems.  All arithmetic is float32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element load / store ------------------------------------------------

__device__ __forceinline__ float load_act(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_act(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);  // bf16 -> f32 is exact
}
__device__ __forceinline__ void store_act(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_act(uint16_t* p, int64_t i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // v_cvt_pk_bf16_f32: nearest even
}

// bf16 pair packed in one dword -> two floats (low half first in memory order)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- wave-uniform (scalar) loads ---------------------------------------------
// Reading through the constant address space tells the compiler the data is
// read-only for the kernel's lifetime, so a wave-uniform address becomes a
// scalar load into SGPRs (s_load) instead of a 64-lane vector load, and the
// value feeds VALU instructions as a scalar operand.
typedef const __attribute__((address_space(4))) float* cfloat_p;
typedef const __attribute__((address_space(4))) uint32_t* cu32_p;
typedef const __attribute__((address_space(4))) uint16_t* cu16_p;

// A pointer every lane holds the same value of, moved to scalar registers
// (free when the compiler already knows it is uniform).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// NG consecutive values of a wave-uniform row of a float / bf16 tensor.
template <int NG>
__device__ __forceinline__ void load_uniform_row(const float* p, float (&v)[NG]) {
    cfloat_p q = (cfloat_p)(p);
#pragma unroll
    for (int k = 0; k < NG; ++k) v[k] = q[k];
}
template <int NG>
__device__ __forceinline__ void load_uniform_row(const uint16_t* p, float (&v)[NG]) {
    if constexpr (NG % 2 == 0) {  // 4-byte aligned pairs: unpack on the scalar unit
        cu32_p q = (cu32_p)(p);
#pragma unroll
        for (int k = 0; k < NG / 2; ++k) {
            const uint32_t w = q[k];
            v[2 * k] = __uint_as_float(w << 16);
            v[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        }
    } else {
        cu16_p q = (cu16_p)(p);
#pragma unroll
        for (int k = 0; k < NG; ++k) v[k] = __uint_as_float(static_cast<uint32_t>(q[k]) << 16);
    }
}

// Raw 32-bit words of NG consecutive values of a wave-uniform row: NG words
// for float, NG / 2 for bf16 (NG even).  Kept raw in SGPRs while prefetched;
// unpacked to float on the scalar unit at use.
template <typename T, int NG>
struct RawRow {
    static constexpr bool kOk = sizeof(T) == 4 || NG % 2 == 0;
    static constexpr int kWords = sizeof(T) == 4 ? NG : (kOk ? NG / 2 : 1);  // 1: unused placeholder
};

template <typename T, int NG>
__device__ __forceinline__ void load_raw_row(const T* p, uint32_t (&q)[RawRow<T, NG>::kWords]) {
    cu32_p r = (cu32_p)(p);
#pragma unroll
    for (int k = 0; k < RawRow<T, NG>::kWords; ++k) q[k] = r[k];
}

template <typename T, int NG>
__device__ __forceinline__ void unpack_raw_row(const uint32_t (&q)[RawRow<T, NG>::kWords], float (&v)[NG]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < NG; ++k) v[k] = __uint_as_float(q[k]);
    } else {
#pragma unroll
        for (int k = 0; k < NG / 2; ++k) {
            v[2 * k] = __uint_as_float(q[k] << 16);
            v[2 * k + 1] = __uint_as_float(q[k] & 0xffff0000u);
        }
    }
}

// ---- per-lane row loads ------------------------------------------------------
// NG consecutive values starting at p (one lane's own address), with the
// widest aligned vector loads: NG * sizeof(T) bytes are 16-byte aligned for
// NG * sizeof(T) >= 16, 8-byte for 8, 4-byte for 4 (rows of N values at a
// multiple of NG; the C ABI requires 16-byte aligned tensors).
template <typename T, int NG>
struct LaneRow {
    static constexpr int kBytes = NG * static_cast<int>(sizeof(T));
    static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
};

template <typename T, int NG>
__device__ __forceinline__ void load_lane_row(const T* p, uint32_t (&q)[LaneRow<T, NG>::kWords]) {
    constexpr int bytes = LaneRow<T, NG>::kBytes;
    if constexpr (bytes >= 16) {
#pragma unroll
        for (int i = 0; i < bytes / 16; ++i) {
            const uint4 v = reinterpret_cast<const uint4*>(p)[i];
            q[4 * i] = v.x; q[4 * i + 1] = v.y; q[4 * i + 2] = v.z; q[4 * i + 3] = v.w;
        }
    } else if constexpr (bytes == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        q[0] = v.x; q[1] = v.y;
    } else if constexpr (bytes == 4) {
        q[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
        q[0] = *reinterpret_cast<const uint16_t*>(p);  // a single bf16
    }
}

template <typename T, int NG>
__device__ __forceinline__ void unpack_lane_row(const uint32_t (&q)[LaneRow<T, NG>::kWords], float (&v)[NG]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < NG; ++k) v[k] = __uint_as_float(q[k]);
    } else if constexpr (NG == 1) {
        v[0] = __uint_as_float(q[0] << 16);
    } else {
#pragma unroll
        for (int k = 0; k < NG / 2; ++k) {
            v[2 * k] = __uint_as_float(q[k] << 16);
            v[2 * k + 1] = __uint_as_float(q[k] & 0xffff0000u);
        }
    }
}

// ---- buffer stores with hardware range checking ---------------------------------
// A raw buffer resource over [base, base + bytes): a store whose byte offset
// is outside the range is dropped by the hardware, so a lane that must not
// write gets an out-of-range offset instead of a branch (branches split the
// instruction stream the scheduler interleaves).  Word 3 is the gfx9
// descriptor format for raw (untyped) buffer access.
constexpr uint32_t kBufferWord3 = 0x00020000u;
constexpr uint32_t kNoStore = 0xFFFFFFF0u;  // an offset beyond any range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufferWord3);
}
__device__ __forceinline__ void buffer_store_act(float v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off, float) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(byte_off), 0, 0);
}
__device__ __forceinline__ void buffer_store_act(float v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint16_t) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r,
                                          static_cast<int>(byte_off), 0, 0);
}

// ---- DPP row broadcast -----------------------------------------------------------
// row_newbcast:J -- every lane of a 16-lane row reads lane J of that row.  With
// a value replicated over the four rows (lane l holding element l % 16), this
// is a broadcast of element J to the whole wave at no instruction cost: the
// compiler folds it into the consuming v_mul_f32 as a DPP source modifier.
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + J, 0xF, 0xF, true));
}

// acc + row_bcast<J>(c) * h as one v_fmac_f32 with a DPP source (the
// compiler does not fold DPP into the tied-accumulator form by itself).
// Arithmetic only.  A DPP source must not have been written by either of the
// two preceding VALU instructions; the compiler does not check that for
// inline assembly, so the statement starts with two wait states of its own
// (s_nop 1) -- the register holding `c` may have just been written, e.g. by
// the bf16 unpacking of a Bm/Cm tile.
template <int J>
__device__ __forceinline__ float fmac_row_bcast(float acc, float c, float h) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+v"(acc)
        : "v"(c), "v"(h), "i"(J));
    return acc;
}
// Two independent fmac_row_bcast behind one pair of wait states.
template <int J>
__device__ __forceinline__ void fmac_row_bcast2(float& acc0, float c0, float h0, float& acc1, float c1, float h1) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %2, %3 row_newbcast:%6 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %4, %5 row_newbcast:%6 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+&v"(acc0), "+&v"(acc1)
        : "v"(c0), "v"(h0), "v"(c1), "v"(h1), "i"(J));
}
// Two steps J0, J0 + 1 of one state at once (as fmac_row_bcast_x4 below).
template <int J0>
__device__ __forceinline__ void fmac_row_bcast_x2(float (&acc)[2], float c, const float (&h)[2]) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %2, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %4 row_newbcast:%6 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+&v"(acc[0]), "+&v"(acc[1])
        : "v"(c), "v"(h[0]), "v"(h[1]), "i"(J0), "i"(J0 + 1));
}
// Four steps J0 .. J0 + 3 of one state at once: acc[j] += row_bcast<J0 + j>(c)
// * h[j], behind one pair of wait states.  Inside the statement the four
// accumulators are independent, so the next statement's update of acc[j]
// (the next state) comes at least three wait states after this one's.  The
// accumulators are early-clobber: no input shares a register with them.
template <int J0>
__device__ __forceinline__ void fmac_row_bcast_x4(float (&acc)[4], float c, const float (&h)[4]) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %4, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %2, %4, %7 row_newbcast:%11 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %3, %4, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+&v"(acc[0]), "+&v"(acc[1]), "+&v"(acc[2]), "+&v"(acc[3])
        : "v"(c), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "i"(J0), "i"(J0 + 1), "i"(J0 + 2), "i"(J0 + 3));
}

// Sum over aligned groups of R consecutive lanes (R = 1, 2, 4, 8 or 16),
// every lane of a group receiving the group's sum.  Within-row DPP moves (no
// LDS round trip, unlike a lane shuffle): swap neighbours, swap pairs of a
// quad, then mirror the half-rows and the row; each step adds a lane's value
// to the one at lane ^ m of the same partial sums, so the pairing, and the
// result, are those of the butterfly s += shfl_xor(s, m), m = 1, 2, 4, 8.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int R>
__device__ __forceinline__ float group_sum(float s) {
    static_assert(R == 1 || R == 2 || R == 4 || R == 8 || R == 16, "groups of 1, 2, 4, 8 or 16 lanes");
    if constexpr (R >= 2) s += dpp_move<0xB1>(s);   // quad_perm [1, 0, 3, 2]
    if constexpr (R >= 4) s += dpp_move<0x4E>(s);   // quad_perm [2, 3, 0, 1]
    if constexpr (R >= 8) s += dpp_move<0x141>(s);  // row_half_mirror: lane 7 - l of the half-row
    if constexpr (R >= 16) s += dpp_move<0x140>(s); // row_mirror: lane 15 - l of the row
    return s;
}

// ---- transcendental building blocks (hardware v_exp/v_log/v_rcp) --------

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = max(x, 0) + log1p(exp(-|x|)).
// log1p(e) for e in (0, 1] is formed as log(w) + c, where w = fl(1 + e) and
// c = e - (w - 1) is the exact rounding error of that sum (Fast2Sum, since
// 1 >= e).  log(1 + e) = log(w + c) = log(w) + c / w + O(c^2), and replacing
// c / w by c costs at most |c| (1 - 1/w) <= 2^-24 e, i.e. full relative
// accuracy also for the tiny e of strongly negative x, where log(w) alone
// would keep only the bits of e that survive the rounding of 1 + e.
__device__ __forceinline__ float softplus(float x) {
    const float e = fast_exp2(-__builtin_fabsf(x) * kLog2e);
    const float w = 1.0f + e;
    const float c = e - (w - 1.0f);
    const float l1p = __builtin_fmaf(fast_log2(w), kLn2, c);
    return __builtin_fmaxf(x, 0.0f) + l1p;
}

// logistic sigmoid 1 / (1 + e^-x)
__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

// silu(z) = z * sigmoid(z)
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }

__host__ __device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// ---- wave helpers ----------------------------------------------------------

// Wave index inside the workgroup, provably uniform (lets the compiler keep
// everything derived from it in scalar registers).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace mssm
