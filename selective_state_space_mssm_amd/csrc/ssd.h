// ssd.h -- launcher interface of the state-space dual (Mamba-2) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

// Validated arguments of one SSD forward: x, y (B, L, H, P); dt (B, L, H);
// Bm, Cm (B, L, N) in the activation type (float32 or bfloat16 bits, `dtype`);
// A, Dskip, dt_bias (H); h0, h_final (B, H, P, N) float32.
//
// Heads as the kernels see them: sub-heads of P = 64 channels.  A head of
// hsub * 64 channels is hsub consecutive sub-heads (x, y and the state keep
// their layout: (B, L, H, hsub * 64) is (B, L, H * hsub, 64)) that share the
// head's step size, decay, skip weight and bias; here H counts sub-heads and
// dt, A, Dskip, dt_bias are indexed by sub-head / hsub (dt's row has H / hsub
// entries).
struct SsdArgs {
    int64_t B, L, H, P, N;  // H: sub-heads; P = 64
    int64_t hsub;           // sub-heads per head (the head dim / 64)
    int softplus;
    int dtype;             // 0: float32 activations, 1: bfloat16
    const void* x;
    const void* dt;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;    // may be null
    const float* dt_bias;  // may be null
    const float* h0;       // may be null
    void* y;
    float* h_final;        // may be null
    // time segments scanned in parallel (1: the whole sequence in one pass)
    int64_t nseg;
    int64_t seg_len;       // steps per segment, a multiple of the chunk length (L when nseg == 1)
    float* ws;             // nseg > 1: segment states (B, H, nseg, P, N), then log-decays (B, H, nseg)
    float* ws_y;           // nseg > 1 with bf16 outputs: float32 outputs (B, L, H, P) of segments 1.. before the
                           // correction (a bf16 partial would be rounded twice); else null
    // balanced persistent schedule (workers > 0, nseg == 1): one workgroup per worker
    int32_t workers;
    uint32_t* flags;       // (workers + 1): 1 once worker w has published; word `workers`: 1 if a wait gave up
    float* carry;          // (workers, P, N): the state worker w hands to worker w + 1
    // training forward: (B, H, nch + 1, P, N) float32, the state entering every 64-step chunk, then the final
    // state -- what the backward's first chain would recompute; null otherwise.  With time segments the main
    // kernel stores the states of a segment's zero start and, per chunk, the decay from the segment's start
    // (chunk_dec, (B, H, nch)); a fix pass adds the segment's true entering state times that decay
    float* states;
    float* chunk_dec;
};



constexpr int kSsdHeadDim = 64;   // P the kernel is built for
constexpr int kSsdChunk = 64;     // chunk length of the dual form

// Workspace of the training forward: the forward's, and with time segments
// the per-chunk decays of the stored states' fix pass.
inline size_t ssd_train_ws_bytes(size_t fwd_ws, int64_t nseg, int64_t B, int64_t L, int64_t H) {
    return nseg > 1 ? ((fwd_ws + 255) & ~static_cast<size_t>(255)) +
                          static_cast<size_t>(B * H * ((L + kSsdChunk - 1) / kSsdChunk)) * sizeof(float)
                    : fwd_ws;
}

constexpr int kSsdMaxSubHeads = 4;  // head dims 64, 128, 192, 256

// True when the kernels are built for this head dimension and state size.
inline bool ssd_supported(int64_t P, int64_t N) {
    return P % kSsdHeadDim == 0 && P / kSsdHeadDim <= kSsdMaxSubHeads && (N == 64 || N == 128);
}

// How the work is cut, for a device of ncu compute units (one workgroup fits
// a CU).  With fewer (batch, head) pairs than half the 256 CUs of an MI355X,
// the sequence splits into segments of at least two chunks, as many as fit
// one workgroup per CU in a single round (a second, partial round would
// double the time); each segment is scanned from a zero state, a carry pass
// forms the state entering every segment, and a correction pass adds that
// state's contribution to the segment's outputs.  Scratch: the segment states
// and log-decays, and for bfloat16 outputs a float32 copy of the outputs the
// correction completes.  With at least ncu pairs that do not divide evenly
// over the CUs (the last round of a grid would run partly empty), a
// persistent workgroup per CU scans an equal share of all chunks instead;
// scratch: a flag per worker and the one state each worker hands over.
struct SsdPlan {
    int64_t nseg;
    int64_t seg_len;
    int64_t workers;
    size_t ws_bytes;
};

inline SsdPlan plan_ssd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, bool bf16, int64_t ncu) {
    SsdPlan pl{1, L, 0, 0};
    const int64_t jobs = B * H, chunks = (L + kSsdChunk - 1) / kSsdChunk;
    if (ncu > 0 && jobs >= ncu && jobs % ncu != 0) {
        pl.workers = ncu;
        pl.ws_bytes = ((static_cast<size_t>(ncu + 1) * sizeof(uint32_t) + 255) & ~static_cast<size_t>(255)) +
                      static_cast<size_t>(ncu * P * N) * sizeof(float);
        return pl;
    }
    if (jobs >= 128 || chunks < 4) return pl;
    const int64_t want = 256 / jobs, most = chunks / 2;
    const int64_t segs = want < most ? want : most;
    const int64_t per = (chunks + segs - 1) / segs;  // chunks per segment
    pl.seg_len = per * kSsdChunk;
    pl.nseg = (L + pl.seg_len - 1) / pl.seg_len;
    if (pl.nseg == 1) {
        pl.seg_len = L;
        return pl;
    }
    pl.ws_bytes = static_cast<size_t>(jobs * pl.nseg * (P * N + 1) + (bf16 ? B * L * H * P : 0)) * sizeof(float);
    return pl;
}

// Validated arguments of one SSD backward (shapes as SsdArgs; dy, dx (B, L, H, P);
// ddt (B, L, H); dB, dC (B, L, N) in the activation type; dA, dD, ddt_bias (H),
// dh0, dh_final (B, H, P, N) float32).
struct SsdBwdArgs {
    int64_t B, L, H, P, N;  // H: sub-heads; P = 64 (as SsdArgs)
    int64_t hsub;
    int softplus;
    int dtype;
    const void* x;
    const void* dt;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;     // may be null
    const float* dt_bias;   // may be null
    const float* h0;        // may be null
    const void* dy;
    const float* dh_final;  // may be null
    void* dx;
    void* ddt;
    float* dA;
    void* dB;
    void* dC;
    float* dD;              // may be null
    float* ddt_bias;        // may be null
    float* dh0;             // may be null
    // workspace
    float* states;          // (B, H, nch + 1, P, N): state entering each 64-step chunk, then the final state
    float* dstates;         // (B, H, nch, P, N): adjoint of the state leaving each chunk
    float* parts;           // (B, nch, H, 3): per chunk and sub-head, the dA, dDskip, ddt_bias contributions
    float* ddt_ws;          // hsub > 1: (B, L, H) float32 ddt per sub-head, summed per head at the end; else null
    float* dbc;             // groups > 1: (2, groups, B, L, N) float32 dB, dC per head group; else null
    int64_t groups;         // head groups per (batch, chunk)
    int64_t heads_per_group;
    // the chains (passes 1 and 2) in time segments of seg_chunks chunks, scanned in parallel from zero and
    // then corrected (nseg == 1: one walk per (batch, sub-head))
    int64_t nseg, seg_chunks;
    float* seg_state;       // nseg > 1: (B, H, nseg, P, N) each segment's end state (pass 1) / start adjoint (pass 2)
    float* seg_lam;         // nseg > 1: (B, H, nseg) each segment's log-decay, sum of Delta A_h over it
    float* chunk_dec;       // nseg > 1: (B, H, nch) decay from the chunk's segment boundary to its stored matrix
};

// Workspace of the backward: states, adjoint states, partials, the
// head-group partials of dB, dC, with sub-heads their ddt, with time
// segments the chains' segment states, segment log-decays and per-chunk
// decays (each 256-byte aligned).  H counts sub-heads, P = 64.
struct SsdBwdPlan {
    int64_t groups, heads_per_group, nseg, seg_chunks;
    size_t states, dstates, parts, dbc, ddt, seg_state, seg_lam, chunk_dec, total;  // byte offsets (total: size)
};

// `saved`: the backward from a training forward's context, whose chunk states
// are not in the workspace.
inline SsdBwdPlan plan_ssd_bwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t hsub, int64_t ncu,
                               bool saved = false) {
    auto al = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
    SsdBwdPlan p{};
    const int64_t nch = (L + kSsdChunk - 1) / kSsdChunk;
    // one workgroup per (batch, chunk, head group): groups so that there are about 2 workgroups per CU
    const int64_t want = ncu > 0 ? 2 * ncu : 512;
    p.groups = (B * nch >= want) ? 1 : (want + B * nch - 1) / (B * nch);
    if (p.groups > H) p.groups = H;
    p.heads_per_group = (H + p.groups - 1) / p.groups;
    p.groups = (H + p.heads_per_group - 1) / p.heads_per_group;
    size_t off = 0;
    p.states = off;  off += saved ? 0 : al(static_cast<size_t>(B * H * (nch + 1) * P * N) * sizeof(float));
    p.dstates = off; off += al(static_cast<size_t>(B * H * nch * P * N) * sizeof(float));
    p.parts = off;   off += al(static_cast<size_t>(B * nch * H * 3) * sizeof(float));
    p.dbc = off;     off += p.groups > 1 ? al(static_cast<size_t>(2 * p.groups * B * L * N) * sizeof(float)) : 0;
    p.ddt = off;     off += hsub > 1 ? al(static_cast<size_t>(B * L * H) * sizeof(float)) : 0;
    // The chains walk their chunks one after another, three workgroups to a CU: with fewer (batch, sub-head)
    // pairs than fill the CUs that way, time segments of at least two chunks, about 768 workgroups in all
    p.nseg = 1;
    p.seg_chunks = nch;
    const int64_t jobs = B * H, slots = 3 * (ncu > 0 ? ncu : 256);
    if (jobs < slots / 3 && nch >= 4) {
        const int64_t want = slots / jobs, most = nch / 2;
        const int64_t segs = want < most ? want : most;
        p.seg_chunks = (nch + segs - 1) / segs;
        p.nseg = (nch + p.seg_chunks - 1) / p.seg_chunks;
    }
    p.seg_state = off; off += p.nseg > 1 ? al(static_cast<size_t>(jobs * p.nseg * P * N) * sizeof(float)) : 0;
    p.seg_lam = off;   off += p.nseg > 1 ? al(static_cast<size_t>(jobs * p.nseg) * sizeof(float)) : 0;
    p.chunk_dec = off; off += p.nseg > 1 ? al(static_cast<size_t>(jobs * nch) * sizeof(float)) : 0;
    p.total = off;
    return p;
}

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st);
hipError_t launch_ssd_bwd(const SsdBwdArgs& a, hipStream_t st);
// Bytes of an SSD training forward's context: the chunk states (B, H, nch + 1, P, N) float32.
inline size_t ssd_ctx_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N) {
    return static_cast<size_t>(B * H * ((L + kSsdChunk - 1) / kSsdChunk + 1) * P * N) * sizeof(float);
}
// The backward with a.states the context a training forward wrote: no first chain.
hipError_t launch_ssd_bwd_saved(const SsdBwdArgs& a, hipStream_t st);

}  // namespace mssm
