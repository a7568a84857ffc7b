// scan_conv_fwd.hip -- the forward selective scan behind a fused causal
// conv1d + SiLU front end, over the kernels of scan_fwd_kernels.h.
//
// The Mamba block feeds the scan u = silu(conv1d(x)), a depthwise causal
// convolution of kernel size d_conv (4 in every configuration the page "Mamba
// SSM 架构" shows; the mamba-minimal page, "PyTorch 한 파일에서의 Mamba
// 구현", runs it as torch.nn.Conv1d).  Here u is formed in the scan's helper
// waves from a window of x and never stored (unless u_out is asked for), which
// saves writing u and reading it back: 2 x B x L x D activations of HBM
// traffic per call.
#include "scan_fwd_kernels.h"

namespace mssm {

hipError_t launch_conv_fwd(const ScanArgs& s, hipStream_t st) {
    if (!s.conv_w || s.d_conv < 1 || s.d_conv > kConvTaps) return hipErrorInvalidValue;
    const FwdPlan pl = plan_fwd(s.B, s.L, s.D, s.N);
    const PreOut none{};
    return s.dtype == 1 ? dispatch_n<uint16_t, false, true>(s, pl, s.workspace, none, st)
                        : dispatch_n<float, false, true>(s, pl, s.workspace, none, st);
}

}  // namespace mssm
