// ssd.h -- launcher interface of the state-space dual (Mamba-2) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

// Validated arguments of one SSD forward: x, y (B, L, H, P); dt (B, L, H);
// Bm, Cm (B, L, N) in the activation type (float32 or bfloat16 bits, `dtype`);
// A, Dskip, dt_bias (H); h0, h_final (B, H, P, N) float32.
struct SsdArgs {
    int64_t B, L, H, P, N;
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
};

constexpr int kSsdHeadDim = 64;   // P the kernel is built for
constexpr int kSsdChunk = 64;     // chunk length of the dual form

// True when the kernel is built for this head dimension and state size.
inline bool ssd_supported(int64_t P, int64_t N) { return P == kSsdHeadDim && (N == 64 || N == 128); }

// How the sequence is cut: with fewer (batch, head) pairs than half the 256
// CUs, the sequence splits into segments of at least two chunks, as many as
// fit one workgroup per CU in a single round (a second, partial round would
// double the time); each segment is scanned from a zero state, a
// carry pass forms the state entering every segment, and a correction pass
// adds that state's contribution to the segment's outputs.  Scratch: the
// segment states and log-decays, and for bfloat16 outputs a float32 copy of
// the outputs the correction completes.
struct SsdPlan {
    int64_t nseg;
    int64_t seg_len;
    size_t ws_bytes;
};

inline SsdPlan plan_ssd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, bool bf16) {
    SsdPlan pl{1, L, 0};
    const int64_t jobs = B * H, chunks = (L + kSsdChunk - 1) / kSsdChunk;
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

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st);

}  // namespace mssm
