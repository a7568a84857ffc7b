// scan_fwd.hip -- the forward selective scan and the backward pre-pass: the
// schedule (plan_fwd) and the launchers over the kernels of scan_fwd_kernels.h,
// whose header describes the mapping onto gfx950.
#include "scan_fwd_kernels.h"

namespace mssm {

FwdPlan plan_fwd(int64_t B, int64_t L, int64_t D, int64_t N) {
    FwdPlan p{1, L, 0};
    const int64_t blocks = B * ((D + 63) / 64);
    if (blocks >= kBalancedMinBlocks) {
        // room for the balanced schedule (used when the blocks do not split
        // evenly over the CUs): a flag and a published 64 x N state per block
        p.ws_bytes = align256(static_cast<size_t>(blocks) * sizeof(uint32_t)) +
                     align256(static_cast<size_t>(blocks) * 64 * N * sizeof(float));
    }
    // Cut time only when the channel blocks alone cannot occupy the chip:
    // at most 1024 (block, chunk) workgroups, a whole number of rounds on 256
    // CUs with one or two workgroups per CU (1032 would add a round of 8).
    constexpr int64_t kTargetBlocks = 1024;
    constexpr int64_t kMinChunk = 1024;
    if (blocks >= 128 || L < 2 * kMinChunk) return p;
    int64_t K = std::min<int64_t>(kTargetBlocks / blocks, L / kMinChunk);
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
    if (use_tokens(s.B, s.L, s.D)) return launch_tokens(s, st);  // a few tokens: the state moves once (scan_step.hip)
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut none{};
    return s.dtype == 1 ? dispatch_n<uint16_t, false, false>(s, pl, s.workspace, none, st)
                        : dispatch_n<float, false, false>(s, pl, s.workspace, none, st);
}

hipError_t launch_fwd_prepass(const ScanArgs& s, void* fwd_scratch, float* ckpt, float* sbar, hipStream_t st) {
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut pre{s.dy, s.dz, sbar, ckpt};
    return s.dtype == 1 ? dispatch_n<uint16_t, true, false>(s, pl, fwd_scratch, pre, st)
                        : dispatch_n<float, true, false>(s, pl, fwd_scratch, pre, st);
}

}  // namespace mssm

