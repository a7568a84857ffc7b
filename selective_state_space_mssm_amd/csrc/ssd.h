// ssd.h -- launcher interface of the state-space dual (Mamba-2) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

// Validated arguments of one SSD forward: x, y (B, L, H, P); dt (B, L, H);
// Bm, Cm (B, L, N); A, Dskip, dt_bias (H); h0, h_final (B, H, P, N).  Float32.
struct SsdArgs {
    int64_t B, L, H, P, N;
    int softplus;
    const float* x;
    const float* dt;
    const float* A;
    const float* Bm;
    const float* Cm;
    const float* Dskip;    // may be null
    const float* dt_bias;  // may be null
    const float* h0;       // may be null
    float* y;
    float* h_final;        // may be null
};

constexpr int kSsdHeadDim = 64;   // P the kernel is built for
constexpr int kSsdChunk = 64;     // chunk length of the dual form

// True when the kernel is built for this head dimension and state size.
inline bool ssd_supported(int64_t P, int64_t N) { return P == kSsdHeadDim && (N == 64 || N == 128); }

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st);

}  // namespace mssm
