// scan_fwd.hip -- forward selective scan for gfx950 (MI355X).
//
// Operation: for each (b, d), h_t[n] = exp(Delta_t A[d,n]) h_{t-1}[n] +
// Delta_t Bm[b,t,n] u[b,t,d] and y[b,t,d] = (sum_n Cm[b,t,n] h_t[n] +
// Dskip[d] u[b,t,d]) silu(z[b,t,d]), Delta_t = softplus(delta + dt_bias) --
// the sequential loop of the mamba-minimal page ("PyTorch 한 파일에서의 Mamba
// 구현", Hacker News comments) with the selective-SSM discretisation (Mamba
// paper Section 3 / Algorithm 2, named on the page "Mamba SSM 架构").
//
// Mapping (one workgroup = one batch row b x 64 channels x one time chunk):
//  * lane = channel d: u, delta, z, y are read/written one row (b, t, 64 d)
//    at a time, consecutive lanes on consecutive addresses;
//  * wave w of the G waves = state group n in [w*NG, (w+1)*NG); the NG
//    states of each channel live in VGPRs and are never written to memory
//    (the (B,L,D,N) expansion does not exist);
//  * Bm[b,t,n], Cm[b,t,n] are the same for all 64 channels: a tile of them
//    sits in VGPRs with lane l holding step l % 16 (replicated over the four
//    16-lane rows), and step j reads it through a DPP row_newbcast:j source
//    modifier on the v_mul / v_fmac that consumes it -- a broadcast with no
//    extra instruction, no LDS traffic and no scalar-load waits;
//  * per time tile of TB steps: every wave turns TB/G rows of (u, delta)
//    into (Delta, Delta*u) in LDS (softplus once per element, shared by the
//    G waves); every wave runs the recurrence for its states over the tile
//    and leaves its partial readout in LDS; every wave then finishes TB/G
//    rows: sum of the G partials + Dskip*u, times silu(z), store.
//  * long sequences: the time axis is cut into K chunks.  A first kernel
//    computes per chunk the end state from zero and the step-size sum
//    (the chunk aggregate of the associative operator
//    (a1, g1) o (a2, g2) = (a1 a2, a2 g1 + g2)); a small kernel chains the
//    aggregates over chunks (the parallel-scan combination the page
//    "mamba.py: 一个简单高效的Mamba实现" credits for parallelising the time
//    dimension); the main kernel then scans every chunk from its true
//    initial state.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <utility>

namespace mssm {
namespace {

constexpr int kTB = 16;  // time steps per tile (= lanes per DPP row)

struct FwdKArgs {
    const void* u;
    const void* delta;
    const void* z;
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;
    const float* dt_bias;
    const float* h0;       // used by chunk 0 when h_in is null
    const float* h_in;     // (B, K, D, N) initial state of every chunk, or null
    void* y;
    float* h_final;
    float* agg_h;          // (B, K, D, N) chunk end state from zero (chunk 0: from h0)
    float* agg_s;          // (B, K, D) chunk sum of Delta
    uint32_t* flags;       // (nblk) balanced schedule: 1 once a block's split state is published
    float* carry;          // (nblk, 64, N) balanced schedule: the published states
    int64_t L, D;
    int64_t chunk_len;
    int32_t dblocks;       // ceil(D / 64)
    int32_t chunks;        // K
    int32_t softplus;
    int32_t workers;       // 0: one workgroup per (block, chunk); > 0: balanced persistent schedule
    int32_t nblk;          // B * dblocks
    // backward pre-pass only
    const void* dy;
    void* dz;              // nullable (no gate)
    float* sbar;           // (B, L, D) dy * silu(z), or dy without a gate
    float* ckpt;           // (B, tiles, D, N) state before every kTB-step tile
    int64_t tiles;         // ceil(L / kTB)
};

// Raw inputs of this wave's rows of one tile (u, delta, z at (b, t, chan0 +
// lane)), loaded with 32-bit offsets from a uniform row base.
template <typename T, int SPW>
__device__ __forceinline__ void fetch_rows(const T* __restrict__ u, const T* __restrict__ dl,
                                           const T* __restrict__ z, int64_t base, int first_row, int rows_left,
                                           int D32, int lo, float (&ru)[SPW], float (&rd)[SPW], float (&rz)[SPW]) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int j = first_row + i;
        if (j < rows_left) {
            const uint32_t off = static_cast<uint32_t>(j * D32 + lo);
            ru[i] = load_act(u + base, off);
            rd[i] = load_act(dl + base, off);
            if (z) rz[i] = load_act(z + base, off);
        }
    }
}

// This wave's Bm (and Cm) values of one tile: lane l loads step l % 16 (row
// clamped to the chunk's last row, so nothing outside the tensor is read).
template <typename T, int NG>
__device__ __forceinline__ void fetch_tile_rows(const T* __restrict__ M, int64_t row0, int64_t last_row, int N,
                                                int n0, int lane, uint32_t (&q)[LaneRow<T, NG>::kWords]) {
    const int64_t r = imin64(row0 + (lane & (kTB - 1)), last_row);
    load_lane_row<T, NG>(M + r * N + n0, q);
}

// One step J of the recurrence for this wave's NG states; leaves the partial
// readout in sP[w][J].
template <int NG, int G, bool FULL, int J>
__device__ __forceinline__ void fwd_step(int nval, int w, int lane, const float (&A2)[NG], float (&h)[NG],
                                         const float (&Bt)[NG], const float (&Ct)[NG], const float2 (&ddt)[kTB],
                                         float (&sP)[G][kTB][64]) {
    if (FULL || J < nval) {
        const float2 dd = ddt[J];
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const float dA = fast_exp2(dd.x * A2[k]);
            h[k] = __builtin_fmaf(dA, h[k], row_bcast<J>(Bt[k]) * dd.y);
        }
        float yp = row_bcast<J>(Ct[0]) * h[0];
#pragma unroll
        for (int k = 1; k < NG; ++k) yp = fmac_row_bcast<J>(yp, Ct[k], h[k]);
        sP[w][J][lane] = yp;
    }
}

template <int NG, int G, bool FULL, int... J>
__device__ __forceinline__ void fwd_steps(std::integer_sequence<int, J...>, int nval, int w, int lane,
                                          const float (&A2)[NG], float (&h)[NG], const float (&Bt)[NG],
                                          const float (&Ct)[NG], const float2 (&ddt)[kTB],
                                          float (&sP)[G][kTB][64]) {
    (fwd_step<NG, G, FULL, J>(nval, w, lane, A2, h, Bt, Ct, ddt, sP), ...);
}

template <int NG, bool FULL, int J>
__device__ __forceinline__ void state_step(int nval, const float (&A2)[NG], float (&h)[NG],
                                           const float (&Bt)[NG], const float2 (&ddt)[kTB], float& ssum) {
    if (FULL || J < nval) {
        const float2 dd = ddt[J];
        ssum += dd.x;
#pragma unroll
        for (int k = 0; k < NG; ++k)
            h[k] = __builtin_fmaf(fast_exp2(dd.x * A2[k]), h[k], row_bcast<J>(Bt[k]) * dd.y);
    }
}

template <int NG, bool FULL, int... J>
__device__ __forceinline__ void state_steps(std::integer_sequence<int, J...>, int nval, int lane,
                                            const float (&A2)[NG], float (&h)[NG], const float (&Bt)[NG],
                                            const float2 (&sDD)[kTB][64], float& ssum) {
    float2 ddt[kTB];
    ((ddt[J] = (FULL || J < nval) ? sDD[J][lane] : make_float2(0.0f, 0.0f)), ...);
    (state_step<NG, FULL, J>(nval, A2, h, Bt, ddt, ssum), ...);
}

// Raw inputs of this wave's rows of tile `tile` of the chunk, branch-free:
// the tile index is clamped to the chunk's last tile and the row to that
// tile's last valid row, so every address is inside the chunk (rows that do
// not exist are loaded from a valid row and never used).
template <typename T, int SPW, bool HAS_Z, bool PRE>
__device__ __forceinline__ void fetch_rows_clamped(const T* __restrict__ u_chunk, const T* __restrict__ d_chunk,
                                                   const T* __restrict__ z_chunk, const T* __restrict__ dy_chunk,
                                                   int tile, int ntiles, int t_len, int64_t D, int first_row,
                                                   int lo, float (&ru)[SPW], float (&rd)[SPW], float (&rz)[SPW],
                                                   float (&rdy)[SPW]) {
    const int te = min(tile, ntiles - 1);
    const int rows_left = t_len - te * kTB;  // >= 1
    const int64_t base = static_cast<int64_t>(te) * kTB * D;
    const int D32 = static_cast<int>(D);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int j = min(first_row + i, rows_left - 1);
        const uint32_t off = static_cast<uint32_t>(j * D32 + lo);
        ru[i] = load_act(u_chunk + base, off);
        rd[i] = load_act(d_chunk + base, off);
        if constexpr (HAS_Z) rz[i] = load_act(z_chunk + base, off);
        if constexpr (PRE) rdy[i] = load_act(dy_chunk + base, off);
    }
}

// Per-element front end of one row: Delta = softplus(delta + dt_bias) (or
// delta + dt_bias), Delta * u, the skip term Dskip * u and the gate silu(z).
template <bool HAS_Z>
__device__ __forceinline__ void prep_element(float uu, float dd, float zz, float bias, float Dk, int softplus_on,
                                             float2& dDU, float& skip, float& gate) {
    const float x = dd + bias;
    const float sp = softplus(x);
    const float dt = softplus_on ? sp : x;
    dDU = make_float2(dt, dt * uu);
    skip = Dk * uu;
    gate = HAS_Z ? silu(zz) : 1.0f;
}

// Backward pre-pass front end of one row: the forward's (Delta, Delta*u) and
// skip term, plus sbar = dy * silu(z) (dy without a gate) and the factor
// dzf = dy * silu'(z) that turns the row's readout s into dz = s * dzf.
template <bool HAS_Z>
__device__ __forceinline__ void prep_element_pre(float uu, float dd, float zz, float gy, float bias, float Dk,
                                                 int softplus_on, float2& dDU, float& skip, float& dzf,
                                                 float& sb) {
    const float x = dd + bias;
    const float sp = softplus(x);
    const float dt = softplus_on ? sp : x;
    dDU = make_float2(dt, dt * uu);
    skip = Dk * uu;
    if constexpr (HAS_Z) {
        const float sg = sigmoid(zz);
        sb = gy * zz * sg;
        dzf = gy * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
    } else {
        sb = gy;
        dzf = 0.0f;
    }
}

// Registers carried from one tile interval to the next.
template <typename T, int NG, int G>
struct FwdRegs {
    static constexpr int SPW = kTB / G;
    float ru[SPW], rd[SPW], rz[SPW], rdy[SPW];             // raw inputs of the next tile to prepare
    uint32_t qb[LaneRow<T, NG>::kWords], qc[LaneRow<T, NG>::kWords];  // Bm/Cm of the next recurrence tile
    float skip_c[SPW], gate_c[SPW];                        // rows of the tile in recurrence
    float skip_p[SPW], gate_p[SPW];                        // rows of the tile being finished
    // (backward pre-pass: "gate" holds dzf, the factor with s * dzf = dz)
};

// Uniform facts about one tile interval.
template <typename T, int NG, int G, bool HAS_Z, bool PRE>
struct FwdInterval {
    int k, ntiles, t_len, w, lane, lo;
    bool dvalid;
    int row_bytes, softplus_on;
    float bias, Dk;
    int64_t D;
    int N, n0;
    int64_t row0, last_row;
    const T* u_chunk;
    const T* d_chunk;
    const T* z_chunk;
    const T* Bm;
    const T* Cm;
    T* y_prev;  // first element (row0 - kTB, chan0) of the tile finished in this interval (k > 0)
    // backward pre-pass
    const T* dy_chunk;
    float* sbar_next;  // first element (row0 + kTB, chan0) of sbar for the tile prepared here
    float* ckpt_tile;  // ckpt row of this tile for channel chan0: ((b * tiles + tile) * D + chan0) * N
};

// One interval: read this interval's LDS first (tile k's (Delta, Delta*u), the
// partial readouts of tile k - 1), then -- in one straight-line block when
// FULL -- prepare tile k + 1, issue the loads of tiles k + 1 / k + 2, run the
// recurrence of tile k and store tile k - 1.  Work that does not exist
// (tile k + 1 past the end, tile -1) runs on clamped inputs and stores to an
// out-of-range offset, instead of branching.
template <bool FULL, typename T, int NG, int G, bool HAS_Z, bool PRE>
__device__ __forceinline__ void fwd_interval(const FwdInterval<T, NG, G, HAS_Z, PRE>& it, int nval,
                                             const float (&A2)[NG], float (&h)[NG], FwdRegs<T, NG, G>& r,
                                             float2 (&sDD)[2][kTB][64], float (&sP)[2][G][kTB][64]) {
    constexpr int SPW = kTB / G;
    const int cur = it.k & 1, prv = cur ^ 1;
    const int lane = it.lane, w = it.w;
    float2 ddt[kTB];
#pragma unroll
    for (int j = 0; j < kTB; ++j) ddt[j] = sDD[cur][j][lane];
    float part[SPW][G];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) part[i][g] = sP[prv][g][w * SPW + i][lane];
    float Bt[NG], Ct[NG];
    unpack_lane_row<T, NG>(r.qb, Bt);
    unpack_lane_row<T, NG>(r.qc, Ct);
    fetch_tile_rows<T, NG>(it.Bm, it.row0 + kTB, it.last_row, it.N, it.n0, lane, r.qb);
    fetch_tile_rows<T, NG>(it.Cm, it.row0 + kTB, it.last_row, it.N, it.n0, lane, r.qc);
    float skip_n[SPW], gate_n[SPW];
    const int D32 = static_cast<int>(it.D);
    if constexpr (PRE) {
        // rows of tile k + 1; sbar goes straight to memory (rows past the end: out of range)
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(it.sbar_next, static_cast<uint32_t>(kTB * D32 * 4));
        const int rows_next = it.t_len - (it.k + 1) * kTB;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            float2 v;
            float sb;
            prep_element_pre<HAS_Z>(r.ru[i], r.rd[i], r.rz[i], r.rdy[i], it.bias, it.Dk, it.softplus_on, v,
                                    skip_n[i], gate_n[i], sb);
            sDD[prv][w * SPW + i][lane] = v;
            const int j = w * SPW + i;
            const uint32_t off = (it.dvalid && j < rows_next) ? static_cast<uint32_t>((j * D32 + lane) * 4) : kNoStore;
            buffer_store_act(sb, rs, off, 0.0f);
        }
        // the state before tile k
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(it.ckpt_tile, static_cast<uint32_t>(64 * it.N * 4));
#pragma unroll
        for (int q = 0; q < NG; ++q)
            buffer_store_act(h[q], rc, it.dvalid ? static_cast<uint32_t>((lane * it.N + it.n0 + q) * 4) : kNoStore,
                             0.0f);
    } else {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            float2 v;
            prep_element<HAS_Z>(r.ru[i], r.rd[i], r.rz[i], it.bias, it.Dk, it.softplus_on, v, skip_n[i],
                                gate_n[i]);
            sDD[prv][w * SPW + i][lane] = v;
        }
    }
    fetch_rows_clamped<T, SPW, HAS_Z, PRE>(it.u_chunk, it.d_chunk, it.z_chunk, it.dy_chunk, it.k + 2, it.ntiles,
                                           it.t_len, it.D, w * SPW, it.lo, r.ru, r.rd, r.rz, r.rdy);
    fwd_steps<NG, G, FULL>(std::make_integer_sequence<int, kTB>{}, nval, w, lane, A2, h, Bt, Ct, ddt, sP[cur]);
    {
        // tile k - 1 (none when k == 0: every lane stores out of range)
        // (pre-pass: y_prev points into dz, and s * dzf is the gate gradient)
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(it.y_prev, static_cast<uint32_t>(kTB * it.row_bytes));
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g) s += part[i][g];
            const int j = w * SPW + i;
            const bool store = it.dvalid && it.k > 0 && (!PRE || HAS_Z);
            const uint32_t off = store ? static_cast<uint32_t>((j * D32 + lane) * static_cast<int>(sizeof(T)))
                                       : kNoStore;
            buffer_store_act((s + r.skip_p[i]) * r.gate_p[i], ry, off, T{});
        }
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        r.skip_p[i] = r.skip_c[i];
        r.gate_p[i] = r.gate_c[i];
        r.skip_c[i] = skip_n[i];
        r.gate_c[i] = gate_n[i];
    }
}

// Runs steps [t_begin, t_end) of channel block `blk` (batch row b = blk /
// dblocks, channels chan0 .. chan0 + 63) from the state in h, leaving the
// final state in h.  Software-pipelined over tiles of kTB steps with one
// barrier per tile: in the interval of tile k every wave prepares its rows of
// tile k + 1, runs the recurrence of tile k and finishes its rows of tile
// k - 1 (LDS double buffered), so the per-element work fills the latency gaps
// of the recurrence's dependency chains.
template <typename T, int NG, int G, bool HAS_Z, bool PRE>
__device__ __forceinline__ void fwd_segment(const FwdKArgs& a, int blk, int64_t t_begin, int64_t t_end,
                                            float (&h)[NG], float2 (&sDD)[2][kTB][64],
                                            float (&sP)[2][G][kTB][64]) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / G;  // rows prepared and finished per wave per tile

    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ dl = static_cast<const T*>(a.delta);
    const T* __restrict__ z = static_cast<const T*>(a.z);
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm);
    const T* __restrict__ Cm = static_cast<const T*>(a.Cm);
    T* __restrict__ y = static_cast<T*>(a.y);

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int64_t b = blk / a.dblocks;
    const int64_t chan0 = static_cast<int64_t>(blk % a.dblocks) * 64;
    const int64_t D = a.D, L = a.L;
    const int D32 = static_cast<int>(D);
    const bool dvalid = chan0 + lane < D;
    const int lo = dvalid ? lane : static_cast<int>(D - 1 - chan0);  // clamped lane offset for loads
    const int64_t dc = chan0 + lo;
    const int n0 = w * NG;

    float A2[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) A2[k] = a.A[dc * N + n0 + k] * kLog2e;
    const float bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    const float Dk = a.Dskip ? a.Dskip[dc] : 0.0f;
    const int softplus_on = a.softplus;

    const int t_len = static_cast<int>(t_end - t_begin);
    const int ntiles = (t_len + kTB - 1) / kTB;
    const int64_t row_begin = b * L + t_begin;  // row index of (b, t_begin)
    const int64_t last_row = row_begin + t_len - 1;
    const int64_t chunk_off = row_begin * D + chan0;  // element (b, t_begin, chan0)
    const T* u_chunk = u + chunk_off;
    const T* d_chunk = dl + chunk_off;
    const T* z_chunk = HAS_Z ? z + chunk_off : nullptr;
    const T* dy_chunk = PRE ? static_cast<const T*>(a.dy) + chunk_off : nullptr;
    const int row_bytes = D32 * static_cast<int>(sizeof(T));
    const int64_t gtile0 = t_begin / kTB;  // segments start on tile boundaries

    __syncthreads();  // LDS is reused from a previous segment
    // ---- prologue: tile 0 prepared, tile 1 raw inputs and tile 0 Bm/Cm in flight
    FwdRegs<T, NG, G> r;
    fetch_rows_clamped<T, SPW, HAS_Z, PRE>(u_chunk, d_chunk, z_chunk, dy_chunk, 0, ntiles, t_len, D, w * SPW, lo,
                                           r.ru, r.rd, r.rz, r.rdy);
    fetch_tile_rows<T, NG>(Bm, row_begin, last_row, N, n0, lane, r.qb);
    fetch_tile_rows<T, NG>(Cm, row_begin, last_row, N, n0, lane, r.qc);
    if constexpr (PRE) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.sbar + chunk_off, static_cast<uint32_t>(kTB * D32 * 4));
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            float2 v;
            float sb;
            prep_element_pre<HAS_Z>(r.ru[i], r.rd[i], r.rz[i], r.rdy[i], bias, Dk, softplus_on, v, r.skip_c[i],
                                    r.gate_c[i], sb);
            sDD[0][w * SPW + i][lane] = v;
            const int j = w * SPW + i;
            buffer_store_act(sb, rs, (dvalid && j < t_len) ? static_cast<uint32_t>((j * D32 + lane) * 4) : kNoStore,
                             0.0f);
        }
    } else {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            float2 v;
            prep_element<HAS_Z>(r.ru[i], r.rd[i], r.rz[i], bias, Dk, softplus_on, v, r.skip_c[i], r.gate_c[i]);
            sDD[0][w * SPW + i][lane] = v;  // rows past the segment end hold finite junk, never used
        }
    }
    fetch_rows_clamped<T, SPW, HAS_Z, PRE>(u_chunk, d_chunk, z_chunk, dy_chunk, 1, ntiles, t_len, D, w * SPW, lo,
                                           r.ru, r.rd, r.rz, r.rdy);
    __syncthreads();

    for (int k = 0; k < ntiles; ++k) {
        const int nval = min(kTB, t_len - k * kTB);
        const int64_t row0 = row_begin + static_cast<int64_t>(k) * kTB;
        FwdInterval<T, NG, G, HAS_Z, PRE> it{
            k, ntiles, t_len, w, lane, lo, dvalid, row_bytes, softplus_on, bias, Dk, D, N, n0, row0, last_row,
            u_chunk, d_chunk, z_chunk, Bm, Cm, y + (k > 0 ? row0 - kTB : row0) * D + chan0, dy_chunk,
            PRE ? a.sbar + (k + 1 < ntiles ? row0 + kTB : row0) * D + chan0 : nullptr,
            PRE ? a.ckpt + ((b * a.tiles + gtile0 + k) * D + chan0) * N : nullptr};
        if (nval == kTB)
            fwd_interval<true>(it, kTB, A2, h, r, sDD, sP);
        else
            fwd_interval<false>(it, nval, A2, h, r, sDD, sP);
        __syncthreads();
    }
    // ---- epilogue: finish the last tile
    {
        const int klast = ntiles - 1;
        const int nval = t_len - klast * kTB;
        const int64_t row0 = row_begin + static_cast<int64_t>(klast) * kTB;
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + row0 * D + chan0, kTB * row_bytes);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            float s = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g) s += sP[klast & 1][g][j][lane];
            const uint32_t off = (dvalid && j < nval && (!PRE || HAS_Z))
                                     ? static_cast<uint32_t>((j * D32 + lane) * static_cast<int>(sizeof(T)))
                                     : kNoStore;
            buffer_store_act((s + r.skip_p[i]) * r.gate_p[i], ry, off, T{});
        }
    }
}

// Main forward kernel.  Block: 64 * G threads.
//  * workers == 0 -- grid (B * dblocks, K): one workgroup per channel block
//    and time chunk (initial state from h_in when K > 1);
//  * workers > 0 -- balanced persistent schedule, one workgroup per worker:
//    the (block, tile) sequence is cut into `workers` equal contiguous ranges
//    of at least one block each.  A block is split between at most two
//    workers.  Each worker first runs its range's last piece if that piece
//    ends inside a block (it starts at t = 0, so it depends on nobody) and
//    publishes the end state; then its whole blocks; then its first piece if
//    that starts inside a block, from the state the previous worker
//    published.  Equal work per workgroup, no extra arithmetic.  A worker only
//    waits on a lower-numbered worker, which never waits before publishing
//    (workgroups are dispatched in increasing order), so every wait ends.
template <typename T, int NG, int G, bool HAS_Z, bool PRE>
__global__ __launch_bounds__(64 * G) void scan_fwd_kernel(FwdKArgs a) {
    constexpr int N = NG * G;
    static_assert(kTB % G == 0, "tile must split evenly over the waves");
    __shared__ float2 sDD[2][kTB][64];   // (Delta, Delta * u) per row and channel
    __shared__ float sP[2][G][kTB][64];  // partial readout of each state group
    float h[NG];
    const int lane = threadIdx.x & 63;
    const int n0 = wave_id() * NG;

    // Segments of this workgroup, in processing order.  Each is (block,
    // steps [t_begin, t_end), where its initial state comes from, what
    // happens to its final state).
    enum { kFromH0 = 0, kFromChunkCarry = 1, kFromPublished = 2 };
    enum { kKeep = 0, kFinal = 1, kPublish = 2 };
    int nseg = 1, tail_piece = 0, full_first = 0, b0 = 0, b1 = 0;
    int64_t t0 = 0, t1 = 0, T_ = 0;
    if (a.workers > 0) {
        T_ = (a.L + kTB - 1) / kTB;  // tiles per sequence
        const int64_t U = static_cast<int64_t>(a.nblk) * T_;
        const int64_t u0 = U * blockIdx.x / a.workers;
        const int64_t u1 = U * (blockIdx.x + 1) / a.workers;
        b0 = static_cast<int>(u0 / T_);
        t0 = u0 - b0 * T_;                               // first tile of the range, in block b0
        b1 = static_cast<int>((u1 - 1) / T_);
        t1 = u1 - static_cast<int64_t>(b1) * T_;        // end tile of the range, in block b1 (1..T)
        tail_piece = (b1 > b0 && t1 < T_) ? 1 : 0;       // ends inside b1: run it first and publish
        full_first = t0 == 0 ? b0 : b0 + 1;
        const int full_last = t1 == T_ ? b1 : b1 - 1;
        nseg = tail_piece + (full_last - full_first + 1) + (t0 > 0 ? 1 : 0);
    }
    for (int sg = 0; sg < nseg; ++sg) {
        int blk, from, to;
        int64_t t_begin, t_end;
        if (a.workers == 0) {  // grid: block blockIdx.x, chunk blockIdx.y
            blk = blockIdx.x;
            t_begin = static_cast<int64_t>(blockIdx.y) * a.chunk_len;
            t_end = imin64(a.L, t_begin + a.chunk_len);
            from = a.h_in ? kFromChunkCarry : kFromH0;
            to = static_cast<int>(blockIdx.y) == a.chunks - 1 ? kFinal : kKeep;
        } else if (sg < tail_piece) {  // last piece of the range, ends inside block b1
            blk = b1; t_begin = 0; t_end = t1 * kTB; from = kFromH0; to = kPublish;
        } else if (sg < nseg - (t0 > 0 ? 1 : 0)) {  // a whole block
            blk = full_first + (sg - tail_piece); t_begin = 0; t_end = a.L; from = kFromH0; to = kFinal;
        } else {  // first piece of the range, starts inside block b0
            blk = b0; t_begin = t0 * kTB; t_end = a.L; from = kFromPublished; to = kFinal;
        }
        const int64_t b = blk / a.dblocks;
        const int64_t chan0 = static_cast<int64_t>(blk % a.dblocks) * 64;
        const int64_t dcl = imin64(chan0 + lane, a.D - 1);
        float* carry_lane = a.carry ? a.carry + (static_cast<int64_t>(blk) * 64 + lane) * N + n0 : nullptr;
        if (from == kFromH0) {
#pragma unroll
            for (int k = 0; k < NG; ++k) h[k] = a.h0 ? a.h0[(b * a.D + dcl) * N + n0 + k] : 0.0f;
        } else if (from == kFromChunkCarry) {
            const float* hi = a.h_in + ((b * a.chunks + blockIdx.y) * a.D + dcl) * N + n0;
#pragma unroll
            for (int k = 0; k < NG; ++k) h[k] = hi[k];
        } else {
            if (threadIdx.x == 0) {
                while (__hip_atomic_load(a.flags + blk, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u)
                    __builtin_amdgcn_s_sleep(2);
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NG; ++k)
                h[k] = __hip_atomic_load(carry_lane + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        fwd_segment<T, NG, G, HAS_Z, PRE>(a, blk, t_begin, t_end, h, sDD, sP);
        if (to == kFinal) {
            if (a.h_final && chan0 + lane < a.D) {
                float* hf = a.h_final + (b * a.D + chan0 + lane) * N + n0;
#pragma unroll
                for (int k = 0; k < NG; ++k) hf[k] = h[k];
            }
        } else if (to == kPublish) {
#pragma unroll
            for (int k = 0; k < NG; ++k) carry_lane[k] = h[k];
            __threadfence();
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_store(a.flags + blk, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ __launch_bounds__(256) void zero_flags_kernel(uint32_t* flags, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) flags[i] = 0u;
}

// Chunk aggregates: end state of chunk c started from zero (chunk 0 from h0)
// and the chunk's sum of Delta.  Grid: (B * dblocks, K - 1).
template <typename T, int NG, int G>
__global__ __launch_bounds__(64 * G) void scan_chunk_state_kernel(FwdKArgs a) {
    constexpr int N = NG * G;
    constexpr int SPW = kTB / G;
    constexpr int W = LaneRow<T, NG>::kWords;
    __shared__ float2 sDD[kTB][64];

    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ dl = static_cast<const T*>(a.delta);
    const T* __restrict__ Bm = static_cast<const T*>(a.Bm);

    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int64_t b = blockIdx.x / a.dblocks;
    const int64_t chan0 = static_cast<int64_t>(blockIdx.x % a.dblocks) * 64;
    const int64_t c = blockIdx.y;
    const int64_t D = a.D, L = a.L;
    const int D32 = static_cast<int>(D);
    const bool dvalid = chan0 + lane < D;
    const int lo = dvalid ? lane : static_cast<int>(D - 1 - chan0);
    const int64_t dc = chan0 + lo;
    const int n0 = w * NG;

    float A2[NG], h[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) A2[k] = a.A[dc * N + n0 + k] * kLog2e;
    if (c == 0 && a.h0) {
        const float* hi = a.h0 + (b * D + dc) * N + n0;
#pragma unroll
        for (int k = 0; k < NG; ++k) h[k] = hi[k];
    } else {
#pragma unroll
        for (int k = 0; k < NG; ++k) h[k] = 0.0f;
    }
    const float bias = a.dt_bias ? a.dt_bias[dc] : 0.0f;
    float ssum = 0.0f;

    const int64_t t_begin = c * a.chunk_len;
    const int t_len = static_cast<int>(imin64(L, t_begin + a.chunk_len) - t_begin);
    const int ntiles = (t_len + kTB - 1) / kTB;
    const int64_t row_begin = b * L + t_begin;
    const int64_t last_row = row_begin + t_len - 1;
    float ru[SPW], rd[SPW], rz[SPW];
    uint32_t qb[W];
    fetch_rows<T, SPW>(u, dl, static_cast<const T*>(nullptr), row_begin * D + chan0, w * SPW, t_len, D32, lo,
                       ru, rd, rz);
    fetch_tile_rows<T, NG>(Bm, row_begin, last_row, N, n0, lane, qb);
    for (int tile = 0; tile < ntiles; ++tile) {
        const int nval = min(kTB, t_len - tile * kTB);
        const int64_t row0 = row_begin + static_cast<int64_t>(tile) * kTB;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int j = w * SPW + i;
            if (j < nval) {
                const float x = rd[i] + bias;
                const float dt = a.softplus ? softplus(x) : x;
                sDD[j][lane] = make_float2(dt, dt * ru[i]);
            }
        }
        float Bt[NG];
        unpack_lane_row<T, NG>(qb, Bt);
        if (tile + 1 < ntiles) {
            fetch_rows<T, SPW>(u, dl, static_cast<const T*>(nullptr), (row0 + kTB) * D + chan0, w * SPW,
                               t_len - (tile + 1) * kTB, D32, lo, ru, rd, rz);
            fetch_tile_rows<T, NG>(Bm, row0 + kTB, last_row, N, n0, lane, qb);
        }
        __syncthreads();
        if (nval == kTB)
            state_steps<NG, true>(std::make_integer_sequence<int, kTB>{}, kTB, lane, A2, h, Bt, sDD, ssum);
        else
            state_steps<NG, false>(std::make_integer_sequence<int, kTB>{}, nval, lane, A2, h, Bt, sDD, ssum);
        __syncthreads();
    }
    if (dvalid) {
        float* ho = a.agg_h + ((b * a.chunks + c) * D + chan0 + lane) * N + n0;
#pragma unroll
        for (int k = 0; k < NG; ++k) ho[k] = h[k];
        if (w == 0) a.agg_s[(b * a.chunks + c) * D + chan0 + lane] = ssum;
    }
}

// Chain the chunk aggregates: h_in[c] = P_{c-1} h_in[c-1] + H_{c-1}, with
// P = exp(A * sum Delta).  One thread per (b, d, n); sequential over chunks.
__global__ __launch_bounds__(256) void scan_carry_kernel(FwdKArgs a, int64_t B, int64_t N) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t D = a.D;
    if (i >= B * D * N) return;
    const int64_t n = i % N;
    const int64_t d = (i / N) % D;
    const int64_t b = i / (N * D);
    const float A2 = a.A[d * N + n] * kLog2e;
    float* hin = const_cast<float*>(a.h_in);
    const int64_t K = a.chunks;
    hin[((b * K + 0) * D + d) * N + n] = a.h0 ? a.h0[(b * D + d) * N + n] : 0.0f;
    float h = a.agg_h[((b * K + 0) * D + d) * N + n];   // chunk 0 aggregate includes h0
    for (int64_t c = 1; c < K; ++c) {
        hin[((b * K + c) * D + d) * N + n] = h;
        if (c + 1 < K) {
            const float P = fast_exp2(A2 * a.agg_s[(b * K + c) * D + d]);
            h = __builtin_fmaf(P, h, a.agg_h[((b * K + c) * D + d) * N + n]);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Smallest block count for which the balanced schedule may be chosen (a
// device partition has at least this many CUs).
constexpr int64_t kBalancedMinBlocks = 64;

// Extra outputs of the backward pre-pass (all null for the forward).
struct PreOut {
    const void* dy;
    void* dz;
    float* sbar;
    float* ckpt;
};

template <typename T, int NG, int G, bool PRE>
hipError_t launch_fwd_t(const ScanArgs& s, const FwdPlan& pl, void* scratch, const PreOut& pre, hipStream_t st) {
    FwdKArgs a{};
    a.u = s.u; a.delta = s.delta; a.z = s.z; a.Bm = s.Bm; a.Cm = s.Cm;
    a.A = s.A; a.Dskip = s.Dskip; a.dt_bias = s.dt_bias; a.h0 = s.h0;
    a.y = s.y; a.h_final = s.h_final;
    a.L = s.L; a.D = s.D;
    a.chunk_len = pl.chunk_len;
    a.chunks = static_cast<int32_t>(pl.chunks);
    a.dblocks = static_cast<int32_t>((s.D + 63) / 64);
    a.softplus = s.softplus;
    a.tiles = (s.L + kTB - 1) / kTB;
    if constexpr (PRE) {
        a.dy = pre.dy;
        a.dz = pre.dz;
        a.sbar = pre.sbar;
        a.ckpt = pre.ckpt;
        a.y = pre.dz ? pre.dz : static_cast<void*>(pre.sbar);  // dz goes where y would; never stored without z
        a.h_final = nullptr;
    }
    const dim3 block(64 * G);
    char* ws = static_cast<char*>(scratch);
    if (pl.chunks > 1) {
        const size_t nh = static_cast<size_t>(s.B) * pl.chunks * s.D * s.N * sizeof(float);
        const size_t ns = static_cast<size_t>(s.B) * pl.chunks * s.D * sizeof(float);
        a.agg_h = reinterpret_cast<float*>(ws);
        a.agg_s = reinterpret_cast<float*>(ws + align256(nh));
        a.h_in = nullptr;
        hipLaunchKernelGGL((scan_chunk_state_kernel<T, NG, G>),
                           dim3(static_cast<unsigned>(s.B * a.dblocks), static_cast<unsigned>(pl.chunks - 1)),
                           block, 0, st, a);
        a.h_in = reinterpret_cast<const float*>(ws + align256(nh) + align256(ns));
        const int64_t threads = s.B * s.D * s.N;
        hipLaunchKernelGGL(scan_carry_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st,
                           a, s.B, s.N);
    }
    dim3 grid(static_cast<unsigned>(s.B * a.dblocks), static_cast<unsigned>(pl.chunks));
    a.nblk = static_cast<int32_t>(s.B * a.dblocks);
    if (pl.chunks == 1 && pl.ws_bytes > 0) {
        // balanced persistent schedule when the blocks do not split evenly over the CUs
        int dev = 0, ncu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (ncu > 0 && a.nblk >= ncu && a.nblk % ncu != 0) {
            a.workers = ncu;
            a.flags = reinterpret_cast<uint32_t*>(ws);
            a.carry = reinterpret_cast<float*>(ws + align256(static_cast<size_t>(a.nblk) * sizeof(uint32_t)));
            hipLaunchKernelGGL(zero_flags_kernel, dim3(static_cast<unsigned>((a.nblk + 255) / 256)), dim3(256), 0,
                               st, a.flags, a.nblk);
            grid = dim3(static_cast<unsigned>(ncu));
        }
    }
    if (s.z)
        hipLaunchKernelGGL((scan_fwd_kernel<T, NG, G, true, PRE>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((scan_fwd_kernel<T, NG, G, false, PRE>), grid, block, 0, st, a);
    return hipGetLastError();
}

// Waves per workgroup (state groups) for N = 16, the state size of every
// pretrained Mamba model.
#ifndef MSSM_FWD_WAVES_N16
#define MSSM_FWD_WAVES_N16 8
#endif

template <typename T, bool PRE>
hipError_t dispatch_n(const ScanArgs& s, const FwdPlan& pl, void* scratch, const PreOut& pre, hipStream_t st) {
    switch (s.N) {
        case 1: return launch_fwd_t<T, 1, 1, PRE>(s, pl, scratch, pre, st);
        case 2: return launch_fwd_t<T, 1, 2, PRE>(s, pl, scratch, pre, st);
        case 4: return launch_fwd_t<T, 1, 4, PRE>(s, pl, scratch, pre, st);
        case 8: return launch_fwd_t<T, 2, 4, PRE>(s, pl, scratch, pre, st);
        case 16: return launch_fwd_t<T, 16 / MSSM_FWD_WAVES_N16, MSSM_FWD_WAVES_N16, PRE>(s, pl, scratch, pre, st);
        case 32: return launch_fwd_t<T, 8, 4, PRE>(s, pl, scratch, pre, st);
        case 64: return launch_fwd_t<T, 16, 4, PRE>(s, pl, scratch, pre, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

FwdPlan plan_fwd(int64_t B, int64_t L, int64_t D, int64_t N) {
    FwdPlan p{1, L, 0};
    const int64_t blocks = B * ((D + 63) / 64);
    if (blocks >= kBalancedMinBlocks) {
        // room for the balanced schedule (used when the blocks do not split
        // evenly over the CUs): a flag and a published 64 x N state per block
        p.ws_bytes = align256(static_cast<size_t>(blocks) * sizeof(uint32_t)) +
                     align256(static_cast<size_t>(blocks) * 64 * N * sizeof(float));
    }
    // Cut time only when the channel blocks alone cannot occupy the chip.
    constexpr int64_t kTargetBlocks = 1024;
    constexpr int64_t kMinChunk = 1024;
    if (blocks >= 128 || L < 2 * kMinChunk) return p;
    int64_t K = std::min<int64_t>((kTargetBlocks + blocks - 1) / blocks, L / kMinChunk);
    K = std::max<int64_t>(K, 1);
    int64_t len = (L + K - 1) / K;
    len = (len + kTB - 1) / kTB * kTB;
    K = (L + len - 1) / len;
    if (K <= 1) return p;
    p.chunks = K;
    p.chunk_len = len;
    const size_t nh = static_cast<size_t>(B) * K * D * N * sizeof(float);
    const size_t ns = static_cast<size_t>(B) * K * D * sizeof(float);
    p.ws_bytes = align256(nh) + align256(ns) + align256(nh);
    return p;
}

hipError_t launch_fwd(const ScanArgs& s, hipStream_t st) {
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut none{};
    return s.dtype == 1 ? dispatch_n<uint16_t, false>(s, pl, s.workspace, none, st)
                        : dispatch_n<float, false>(s, pl, s.workspace, none, st);
}

hipError_t launch_fwd_prepass(const ScanArgs& s, void* fwd_scratch, float* ckpt, float* sbar, hipStream_t st) {
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut pre{s.dy, s.dz, sbar, ckpt};
    return s.dtype == 1 ? dispatch_n<uint16_t, true>(s, pl, fwd_scratch, pre, st)
                        : dispatch_n<float, true>(s, pl, fwd_scratch, pre, st);
}

}  // namespace mssm
