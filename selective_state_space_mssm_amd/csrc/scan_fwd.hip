// scan_fwd.hip -- the forward selective scan and the backward pre-pass: the
// schedule (plan_fwd) and the launchers over the kernels of scan_fwd_kernels.h,
// whose header describes the mapping onto gfx950.
#include "scan_fwd_kernels.h"

#include <mutex>

#include "mssm.h"

namespace mssm {

// Scratch of mssm_scan_fwd_noalloc: a fixed array in device memory, one copy
// per GPU (reserved when the code object is loaded onto that GPU), shared by
// every such call on it.  In host code `scratch` is only a handle for the
// symbol lookup below: its device address differs per GPU and is what kernels
// are given.
static __device__ __align__(256) unsigned char scratch[MSSM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};  // device address of `scratch` per GPU, looked up on first use

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_fwd_noalloc(ScanArgs a, hipStream_t st) {
    void* p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return e;
    a.workspace = p;
    a.workspace_bytes = MSSM_NOALLOC_SCRATCH_BYTES;
    return launch_fwd_any(a, st);
}

FwdPlan plan_fwd(int64_t B, int64_t L, int64_t D, int64_t N) {
    FwdPlan p{1, L, 0};
    const int64_t blocks = B * ((D + 63) / 64);
    if (blocks >= kBalancedMinBlocks) {
        // room for the balanced schedule (used when the blocks do not split
        // evenly over the CUs): a flag and a published 64 x N state per
        // block, and the word that records a wait that gave up
        p.ws_bytes = align256(static_cast<size_t>(blocks + 1) * sizeof(uint32_t)) +
                     align256(static_cast<size_t>(blocks) * 64 * N * sizeof(float));
    }
    // Cut time only when the channel blocks alone cannot occupy the chip:
    // at most 1024 (block, chunk) workgroups, a whole number of rounds on 256
    // CUs with one or two workgroups per CU (1032 would add a round of 8),
    // chunks of at least 128 steps, and sequences of at least 512 steps.
    // Measured (bf16, D = 1536, B = 1): L = 1024 72 -> 34 us, 2048 162 -> 50,
    // 4096 174 -> 71; at L = 256 the three passes cost what the split gains.
    constexpr int64_t kTargetBlocks = 1024;
    constexpr int64_t kMinChunk = 128;
    if (blocks >= 128 || L < 4 * kMinChunk) return p;
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
    // a few tokens: the state moves once (scan_step.hip); a training forward keeps the tiled path's checkpoints
    if (!s.ctx_ckpt && use_tokens(s.B, s.L, s.D)) return launch_tokens(s, st);
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut none{};
    return s.dtype == 1 ? dispatch_n<uint16_t, false, false>(s, pl, s.workspace, none, st)
                        : dispatch_n<float, false, false>(s, pl, s.workspace, none, st);
}

hipError_t launch_fwd_train(const ScanArgs& s, hipStream_t st) { return s.ctx_ckpt ? launch_fwd(s, st) : hipErrorInvalidValue; }

hipError_t launch_fwd_prepass(const ScanArgs& s, void* fwd_scratch, float* ckpt, float* sbar, hipStream_t st) {
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut pre{s.dy, s.dz, sbar, ckpt};
    return s.dtype == 1 ? dispatch_n<uint16_t, true, false>(s, pl, fwd_scratch, pre, st)
                        : dispatch_n<float, true, false>(s, pl, fwd_scratch, pre, st);
}

}  // namespace mssm

