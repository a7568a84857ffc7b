// mssm_api.cpp -- the C ABI declared in include/mssm.h.
//
// Host-only layer: validates every argument before anything is enqueued
// (so argument errors never touch a device buffer and need no GPU), sizes the
// workspace, and hands a validated ScanArgs to the kernel launchers.
#include "mssm.h"

#include <hip/hip_runtime.h>
#include <hip/hip_version.h>

#include <cstdint>
#include <initializer_list>

#include "launch.h"
#include "ssd.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Problem checks shared by every entry point.  `need_seq`: seqlen matters.
mssm_status check_problem(const mssm_problem* p, bool need_seq) {
    if (!p) return MSSM_ERR_NULL;
    if (p->dtype != MSSM_F32 && p->dtype != MSSM_BF16) return MSSM_ERR_DTYPE;
    if (p->batch < 1 || p->dim < 1 || p->dstate < 1) return MSSM_ERR_SHAPE;
    if (need_seq && p->seqlen < 1) return MSSM_ERR_SHAPE;
    if (p->batch * p->dim >= (int64_t{1} << 31)) return MSSM_ERR_SHAPE;
    if (p->dim >= (int64_t{1} << 24)) return MSSM_ERR_SHAPE;  // per-tile byte offsets are 31-bit
    if (need_seq && p->seqlen >= (int64_t{1} << 31)) return MSSM_ERR_SHAPE;
    if (p->dstate > MSSM_MAX_DSTATE) return MSSM_ERR_UNSUPPORTED;
    return MSSM_OK;
}

// All non-null pointers must be 16-byte aligned.
mssm_status check_align(std::initializer_list<const void*> ptrs) {
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return MSSM_ERR_ALIGN;
    return MSSM_OK;
}

mssm::ScanArgs base_args(const mssm_problem* p) {
    mssm::ScanArgs a{};
    a.B = p->batch;
    a.L = p->seqlen;
    a.D = p->dim;
    a.N = p->dstate;
    a.dtype = p->dtype;
    a.softplus = p->delta_softplus ? 1 : 0;
    return a;
}

mssm_status from_hip(hipError_t e) { return e == hipSuccess ? MSSM_OK : MSSM_ERR_HIP; }

// The conv front end's backward: the problem without its state size.
mssm_status check_conv_problem(const mssm_problem* p, int32_t d_conv) {
    if (!p) return MSSM_ERR_NULL;
    if (p->dtype != MSSM_F32 && p->dtype != MSSM_BF16) return MSSM_ERR_DTYPE;
    if (p->batch < 1 || p->dim < 1 || p->seqlen < 1) return MSSM_ERR_SHAPE;
    if (p->batch * p->dim >= (int64_t{1} << 31) || p->seqlen >= (int64_t{1} << 31)) return MSSM_ERR_SHAPE;
    if (d_conv < 1 || d_conv > MSSM_MAX_DCONV) return MSSM_ERR_SHAPE;
    if (mssm::plan_conv_bwd(p->batch, p->seqlen, p->dim).workgroups >= (int64_t{1} << 31)) return MSSM_ERR_SHAPE;
    return MSSM_OK;
}

}  // namespace

extern "C" {

size_t mssm_scan_fwd_workspace_bytes(const mssm_problem* p) {
    if (check_problem(p, true) != MSSM_OK) return 0;
    return mssm::fwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
}

size_t mssm_scan_bwd_workspace_bytes(const mssm_problem* p) {
    if (check_problem(p, true) != MSSM_OK) return 0;
    return mssm::bwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
}

mssm_status mssm_scan_fwd(const mssm_problem* p, const void* u, const void* delta, const float* A,
                          const void* Bm, const void* Cm, const float* Dskip, const void* z,
                          const float* dt_bias, const float* h0, void* y, float* h_final,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (!u || !delta || !A || !Bm || !Cm || !y) return MSSM_ERR_NULL;
    st = check_align({u, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, y, h_final, workspace});
    if (st != MSSM_OK) return st;
    const size_t need = mssm::fwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = u; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.y = y; a.h_final = h_final;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return from_hip(mssm::launch_fwd_any(a, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_scan_fwd_noalloc(const mssm_problem* p, const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm, const float* Dskip, const void* z,
                                  const float* dt_bias, const float* h0, void* y, float* h_final,
                                  void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (!u || !delta || !A || !Bm || !Cm || !y) return MSSM_ERR_NULL;
    st = check_align({u, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, y, h_final});
    if (st != MSSM_OK) return st;
    const size_t need = mssm::use_tokens(p->batch, p->seqlen, p->dim) && !mssm::needs_padding(p->dstate)
                            ? 0 : mssm::fwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (need > MSSM_NOALLOC_SCRATCH_BYTES) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = u; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.y = y; a.h_final = h_final;
    return from_hip(mssm::launch_fwd_noalloc(a, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_conv_scan_fwd(const mssm_problem* p, int32_t d_conv, const void* x, const float* conv_w,
                               const float* conv_b, const void* x_prev, const void* delta, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip, const void* z,
                               const float* dt_bias, const float* h0, void* y, float* h_final, void* u_out,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (d_conv < 1 || d_conv > MSSM_MAX_DCONV) return MSSM_ERR_SHAPE;
    if (!x || !conv_w || !delta || !A || !Bm || !Cm || !y) return MSSM_ERR_NULL;
    st = check_align({x, conv_w, conv_b, x_prev, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, y, h_final, u_out,
                      workspace});
    if (st != MSSM_OK) return st;
    const size_t need = mssm::fwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = x; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.y = y; a.h_final = h_final;
    a.conv_w = conv_w; a.conv_b = conv_b; a.x_prev = d_conv > 1 ? x_prev : nullptr; a.u_out = u_out;
    a.d_conv = d_conv;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return from_hip(mssm::launch_conv_fwd_any(a, static_cast<hipStream_t>(hip_stream)));
}

size_t mssm_conv_bwd_workspace_bytes(const mssm_problem* p, int32_t d_conv) {
    if (check_conv_problem(p, d_conv) != MSSM_OK) return 0;
    return mssm::plan_conv_bwd(p->batch, p->seqlen, p->dim).ws_bytes;
}

mssm_status mssm_conv_bwd(const mssm_problem* p, int32_t d_conv, const void* x, const float* conv_w,
                          const float* conv_b, const void* x_prev, const void* du, void* dx, float* dconv_w,
                          float* dconv_b, void* dx_prev, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
    mssm_status st = check_conv_problem(p, d_conv);
    if (st != MSSM_OK) return st;
    if (!x || !conv_w || !du || !dx || !dconv_w) return MSSM_ERR_NULL;
    st = check_align({x, conv_w, conv_b, x_prev, du, dx, dconv_w, dconv_b, dx_prev, workspace});
    if (st != MSSM_OK) return st;
    const size_t need = mssm::plan_conv_bwd(p->batch, p->seqlen, p->dim).ws_bytes;
    if (!workspace || workspace_bytes < need) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = x; a.conv_w = conv_w; a.conv_b = conv_b; a.x_prev = d_conv > 1 ? x_prev : nullptr; a.d_conv = d_conv;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    const mssm::ConvBwdIO io{du, dx, d_conv > 1 ? dx_prev : nullptr, dconv_w, dconv_b};
    return from_hip(mssm::launch_conv_bwd(a, io, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_scan_bwd(const mssm_problem* p, const void* u, const void* delta, const float* A,
                          const void* Bm, const void* Cm, const float* Dskip, const void* z,
                          const float* dt_bias, const float* h0, const void* dy,
                          const float* dh_final, void* du, void* ddelta, float* dA, void* dB,
                          void* dC, float* dD, void* dz, float* ddt_bias, float* dh0,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (!u || !delta || !A || !Bm || !Cm || !dy) return MSSM_ERR_NULL;
    if (!du || !ddelta || !dA || !dB || !dC) return MSSM_ERR_NULL;
    if (z && !dz) return MSSM_ERR_NULL;
    st = check_align({u, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, dy, dh_final, du, ddelta, dA, dB,
                      dC, dD, dz, ddt_bias, dh0, workspace});
    if (st != MSSM_OK) return st;
    const size_t need = mssm::bwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = u; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.dy = dy; a.dh_final = dh_final;
    a.du = du; a.ddelta = ddelta; a.dz = z ? dz : nullptr; a.dB = dB; a.dC = dC;
    a.dA = dA; a.dD = dD; a.ddt_bias = ddt_bias; a.dh0 = dh0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return from_hip(mssm::launch_bwd_any(a, static_cast<hipStream_t>(hip_stream)));
}

namespace {
// The context of a problem: that of its N'-state form (N' the next power of two).
mssm::CtxLayout ctx_of(const mssm_problem* p) {
    return mssm::ctx_layout(p->batch, p->seqlen, p->dim, mssm::padded_dstate(p->dstate));
}
}  // namespace

size_t mssm_scan_ctx_bytes(const mssm_problem* p) {
    if (check_problem(p, true) != MSSM_OK) return 0;
    return ctx_of(p).total;
}

size_t mssm_scan_bwd_saved_workspace_bytes(const mssm_problem* p) {
    if (check_problem(p, true) != MSSM_OK) return 0;
    return mssm::bwd_saved_ws_bytes_any(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
}

mssm_status mssm_scan_fwd_train(const mssm_problem* p, const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip, const void* z,
                                const float* dt_bias, const float* h0, void* y, float* h_final, void* ctx,
                                size_t ctx_bytes, void* workspace, size_t workspace_bytes, void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (!u || !delta || !A || !Bm || !Cm || !y || !ctx) return MSSM_ERR_NULL;
    st = check_align({u, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, y, h_final, ctx, workspace});
    if (st != MSSM_OK) return st;
    const mssm::CtxLayout cl = ctx_of(p);
    if (ctx_bytes < cl.total) return MSSM_ERR_WORKSPACE;
    const size_t need = mssm::fwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = u; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.y = y; a.h_final = h_final;
    a.ctx_ckpt = reinterpret_cast<float*>(static_cast<char*>(ctx) + cl.ckpt);
    a.ctx_s = reinterpret_cast<float*>(static_cast<char*>(ctx) + cl.s);
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return from_hip(mssm::launch_fwd_train_any(a, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_conv_scan_fwd_train(const mssm_problem* p, int32_t d_conv, const void* x, const float* conv_w,
                                     const float* conv_b, const void* x_prev, const void* delta, const float* A,
                                     const void* Bm, const void* Cm, const float* Dskip, const void* z,
                                     const float* dt_bias, const float* h0, void* y, float* h_final, void* u_out,
                                     void* ctx, size_t ctx_bytes, void* workspace, size_t workspace_bytes,
                                     void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (d_conv < 1 || d_conv > MSSM_MAX_DCONV) return MSSM_ERR_SHAPE;
    if (!x || !conv_w || !delta || !A || !Bm || !Cm || !y || !ctx) return MSSM_ERR_NULL;
    st = check_align({x, conv_w, conv_b, x_prev, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, y, h_final, u_out, ctx,
                      workspace});
    if (st != MSSM_OK) return st;
    const mssm::CtxLayout cl = ctx_of(p);
    if (ctx_bytes < cl.total) return MSSM_ERR_WORKSPACE;
    const size_t need = mssm::fwd_ws_bytes(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = x; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.y = y; a.h_final = h_final;
    a.conv_w = conv_w; a.conv_b = conv_b; a.x_prev = d_conv > 1 ? x_prev : nullptr; a.u_out = u_out;
    a.d_conv = d_conv;
    a.ctx_ckpt = reinterpret_cast<float*>(static_cast<char*>(ctx) + cl.ckpt);
    a.ctx_s = reinterpret_cast<float*>(static_cast<char*>(ctx) + cl.s);
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return from_hip(mssm::launch_conv_fwd_any(a, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_scan_bwd_saved(const mssm_problem* p, const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip, const void* z,
                                const float* dt_bias, const void* ctx, size_t ctx_bytes, const void* dy,
                                const float* dh_final, void* du, void* ddelta, float* dA, void* dB, void* dC,
                                float* dD, void* dz, float* ddt_bias, float* dh0, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
    mssm_status st = check_problem(p, true);
    if (st != MSSM_OK) return st;
    if (!u || !delta || !A || !Bm || !Cm || !dy || !ctx) return MSSM_ERR_NULL;
    if (!du || !ddelta || !dA || !dB || !dC) return MSSM_ERR_NULL;
    if (z && !dz) return MSSM_ERR_NULL;
    st = check_align({u, delta, A, Bm, Cm, Dskip, z, dt_bias, ctx, dy, dh_final, du, ddelta, dA, dB, dC, dD, dz,
                      ddt_bias, dh0, workspace});
    if (st != MSSM_OK) return st;
    const mssm::CtxLayout cl = ctx_of(p);
    if (ctx_bytes < cl.total) return MSSM_ERR_WORKSPACE;
    const size_t need = mssm::bwd_saved_ws_bytes_any(p->batch, p->seqlen, p->dim, p->dstate, p->dtype);
    if (!workspace || workspace_bytes < need) return MSSM_ERR_WORKSPACE;

    mssm::ScanArgs a = base_args(p);
    a.u = u; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias;
    a.dy = dy; a.dh_final = dh_final;
    a.du = du; a.ddelta = ddelta; a.dz = z ? dz : nullptr; a.dB = dB; a.dC = dC;
    a.dA = dA; a.dD = dD; a.ddt_bias = ddt_bias; a.dh0 = dh0;
    a.ctx_ckpt = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(ctx)) + cl.ckpt);
    a.ctx_s = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(ctx)) + cl.s);
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return from_hip(mssm::launch_bwd_saved_any(a, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_step(const mssm_problem* p, const void* u_t, const void* delta_t, const float* A,
                      const void* Bm_t, const void* Cm_t, const float* Dskip, const void* z_t,
                      const float* dt_bias, float* state, void* y_t, void* hip_stream) {
    mssm_status st = check_problem(p, false);
    if (st != MSSM_OK) return st;
    if (!u_t || !delta_t || !A || !Bm_t || !Cm_t || !state || !y_t) return MSSM_ERR_NULL;
    st = check_align({u_t, delta_t, A, Bm_t, Cm_t, Dskip, z_t, dt_bias, state, y_t});
    if (st != MSSM_OK) return st;
    mssm::ScanArgs a = base_args(p);
    a.L = 1;
    a.u = u_t; a.delta = delta_t; a.z = z_t; a.Bm = Bm_t; a.Cm = Cm_t;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.y = y_t;
    return from_hip(mssm::launch_step(a, state, static_cast<hipStream_t>(hip_stream)));
}

mssm_status mssm_conv_step(const mssm_problem* p, int32_t d_conv, const void* x_t, const float* conv_w,
                           const float* conv_b, void* conv_state, const void* delta_t, const float* A,
                           const void* Bm_t, const void* Cm_t, const float* Dskip, const void* z_t,
                           const float* dt_bias, float* state, void* y_t, void* hip_stream) {
    mssm_status st = check_problem(p, false);
    if (st != MSSM_OK) return st;
    if (d_conv < 1 || d_conv > MSSM_MAX_DCONV) return MSSM_ERR_SHAPE;
    if (!x_t || !conv_w || (d_conv > 1 && !conv_state) || !delta_t || !A || !Bm_t || !Cm_t || !state || !y_t)
        return MSSM_ERR_NULL;
    st = check_align({x_t, conv_w, conv_b, conv_state, delta_t, A, Bm_t, Cm_t, Dskip, z_t, dt_bias, state, y_t});
    if (st != MSSM_OK) return st;
    mssm::ScanArgs a = base_args(p);
    a.L = 1;
    a.u = x_t; a.delta = delta_t; a.z = z_t; a.Bm = Bm_t; a.Cm = Cm_t;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.y = y_t;
    a.conv_w = conv_w; a.conv_b = conv_b; a.x_prev = d_conv > 1 ? conv_state : nullptr; a.d_conv = d_conv;
    return from_hip(mssm::launch_step(a, state, static_cast<hipStream_t>(hip_stream)));
}

namespace {
// Compute units of the current device (0 if the query fails: no balanced schedule then).
int64_t device_cus() {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return ncu;
}

mssm_status check_ssd_problem(const mssm_ssd_problem* p) {
    if (!p) return MSSM_ERR_NULL;
    if (p->dtype != MSSM_F32 && p->dtype != MSSM_BF16) return MSSM_ERR_DTYPE;
    if (p->batch < 1 || p->seqlen < 1 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1) return MSSM_ERR_SHAPE;
    // the kernels' (batch, sub-head) pairs, a sub-head being 64 channels of a head
    if (p->batch * p->nheads * ((p->headdim + 63) / 64) >= (int64_t{1} << 31) || p->seqlen >= (int64_t{1} << 31))
        return MSSM_ERR_SHAPE;
    if (p->nheads * p->headdim >= (int64_t{1} << 23)) return MSSM_ERR_SHAPE;  // a 64-step chunk stays below 2^31 bytes
    if (!mssm::ssd_supported(p->headdim, p->dstate)) return MSSM_ERR_UNSUPPORTED;
    return MSSM_OK;
}

// The kernels' heads: sub-heads of 64 channels (a head of headdim channels is
// headdim / 64 of them, sharing its step size, decay, skip weight and bias).
int64_t ssd_subheads(const mssm_ssd_problem* p) { return p->headdim / mssm::kSsdHeadDim; }
}  // namespace

size_t mssm_ssd_fwd_workspace_bytes(const mssm_ssd_problem* p) {
    if (check_ssd_problem(p) != MSSM_OK) return 0;
    return mssm::plan_ssd(p->batch, p->seqlen, p->nheads * ssd_subheads(p), mssm::kSsdHeadDim, p->dstate,
                          p->dtype == MSSM_BF16, device_cus())
        .ws_bytes;
}

namespace {
// The SSD forward; with ctx, the training forward (no time segments; the chunk states into ctx).
mssm_status ssd_fwd_common(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                           const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                           const float* h0, void* y, float* h_final, void* ctx, size_t ctx_bytes,
                           void* workspace, size_t workspace_bytes, void* hip_stream, bool train) {
    const mssm_status chk = check_ssd_problem(p);
    if (chk != MSSM_OK) return chk;
    if (!x || !dt || !A || !Bm || !Cm || !y || (train && !ctx)) return MSSM_ERR_NULL;
    const mssm_status st = check_align({x, dt, A, Bm, Cm, Dskip, dt_bias, h0, y, h_final, ctx, workspace});
    if (st != MSSM_OK) return st;
    const int64_t hsub = ssd_subheads(p), Hs = p->nheads * hsub;
    const mssm::SsdPlan plan = mssm::plan_ssd(p->batch, p->seqlen, Hs, mssm::kSsdHeadDim, p->dstate,
                                              p->dtype == MSSM_BF16, device_cus());
    if (train && ctx_bytes < mssm::ssd_ctx_bytes(p->batch, p->seqlen, Hs, mssm::kSsdHeadDim, p->dstate))
        return MSSM_ERR_WORKSPACE;
    const size_t need = train ? mssm::ssd_train_ws_bytes(plan.ws_bytes, plan.nseg, p->batch, p->seqlen, Hs)
                              : plan.ws_bytes;
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSSM_ERR_WORKSPACE;

    mssm::SsdArgs a{};
    a.B = p->batch; a.L = p->seqlen; a.H = Hs; a.P = mssm::kSsdHeadDim; a.N = p->dstate; a.hsub = hsub;
    a.softplus = p->delta_softplus ? 1 : 0;
    a.dtype = p->dtype == MSSM_BF16 ? 1 : 0;
    a.x = x; a.dt = dt; a.A = A; a.Bm = Bm; a.Cm = Cm;
    a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0; a.y = y; a.h_final = h_final;
    a.nseg = plan.nseg; a.seg_len = plan.seg_len; a.ws = static_cast<float*>(workspace);
    a.ws_y = plan.nseg > 1 && p->dtype == MSSM_BF16
                 ? a.ws + p->batch * Hs * plan.nseg * (mssm::kSsdHeadDim * p->dstate + 1) : nullptr;
    if (plan.workers > 0) {
        a.workers = static_cast<int32_t>(plan.workers);
        a.flags = static_cast<uint32_t*>(workspace);
        a.carry = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           ((static_cast<size_t>(plan.workers + 1) * sizeof(uint32_t) + 255) &
                                            ~static_cast<size_t>(255)));
    }
    a.states = train ? static_cast<float*>(ctx) : nullptr;
    a.chunk_dec = train && plan.nseg > 1
                      ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                 ((plan.ws_bytes + 255) & ~static_cast<size_t>(255)))
                      : nullptr;
    return from_hip(mssm::launch_ssd_fwd(a, static_cast<hipStream_t>(hip_stream)));
}
}  // namespace

mssm_status mssm_ssd_fwd(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                         const float* h0, void* y, float* h_final,
                         void* workspace, size_t workspace_bytes, void* hip_stream) {
    return ssd_fwd_common(p, x, dt, A, Bm, Cm, Dskip, dt_bias, h0, y, h_final, nullptr, 0, workspace,
                          workspace_bytes, hip_stream, false);
}

size_t mssm_ssd_ctx_bytes(const mssm_ssd_problem* p) {
    if (check_ssd_problem(p) != MSSM_OK) return 0;
    return mssm::ssd_ctx_bytes(p->batch, p->seqlen, p->nheads * ssd_subheads(p), mssm::kSsdHeadDim, p->dstate);
}

size_t mssm_ssd_fwd_train_workspace_bytes(const mssm_ssd_problem* p) {
    if (check_ssd_problem(p) != MSSM_OK) return 0;
    const int64_t Hs = p->nheads * ssd_subheads(p);
    const mssm::SsdPlan plan = mssm::plan_ssd(p->batch, p->seqlen, Hs, mssm::kSsdHeadDim, p->dstate,
                                              p->dtype == MSSM_BF16, device_cus());
    return mssm::ssd_train_ws_bytes(plan.ws_bytes, plan.nseg, p->batch, p->seqlen, Hs);
}

mssm_status mssm_ssd_fwd_train(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                               const float* h0, void* y, float* h_final, void* ctx, size_t ctx_bytes,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
    return ssd_fwd_common(p, x, dt, A, Bm, Cm, Dskip, dt_bias, h0, y, h_final, ctx, ctx_bytes, workspace,
                          workspace_bytes, hip_stream, true);
}

size_t mssm_ssd_bwd_workspace_bytes(const mssm_ssd_problem* p) {
    if (check_ssd_problem(p) != MSSM_OK) return 0;
    return mssm::plan_ssd_bwd(p->batch, p->seqlen, p->nheads * ssd_subheads(p), mssm::kSsdHeadDim, p->dstate,
                              ssd_subheads(p), device_cus())
        .total;
}

namespace {
// The SSD backward; with ctx, from the chunk states a training forward saved (no first chain).
mssm_status ssd_bwd_common(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                           const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                           const float* h0, const void* ctx, size_t ctx_bytes, const void* dy,
                           const float* dh_final, void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                           float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes, void* hip_stream,
                           bool saved) {
    const mssm_status chk = check_ssd_problem(p);
    if (chk != MSSM_OK) return chk;
    if (!x || !dt || !A || !Bm || !Cm || !dy || !dx || !ddt || !dA || !dB || !dC) return MSSM_ERR_NULL;
    if (saved && !ctx) return MSSM_ERR_NULL;
    const mssm_status al = check_align({x, dt, A, Bm, Cm, Dskip, dt_bias, h0, ctx, dy, dh_final, dx, ddt, dA, dB,
                                        dC, dD, ddt_bias, dh0, workspace});
    if (al != MSSM_OK) return al;
    const bool bf16 = p->dtype == MSSM_BF16;
    const int64_t hsub = ssd_subheads(p), Hs = p->nheads * hsub;
    if (saved && ctx_bytes < mssm::ssd_ctx_bytes(p->batch, p->seqlen, Hs, mssm::kSsdHeadDim, p->dstate))
        return MSSM_ERR_WORKSPACE;
    const mssm::SsdBwdPlan plan =
        mssm::plan_ssd_bwd(p->batch, p->seqlen, Hs, mssm::kSsdHeadDim, p->dstate, hsub, device_cus(), saved);
    if (!workspace || workspace_bytes < plan.total) return MSSM_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);

    mssm::SsdBwdArgs a{};
    a.B = p->batch; a.L = p->seqlen; a.H = Hs; a.P = mssm::kSsdHeadDim; a.N = p->dstate; a.hsub = hsub;
    a.softplus = p->delta_softplus ? 1 : 0;
    a.dtype = bf16 ? 1 : 0;
    a.x = x; a.dt = dt; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.dy = dy; a.dh_final = dh_final;
    a.dx = dx; a.ddt = ddt; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.ddt_bias = ddt_bias; a.dh0 = dh0;
    a.states = saved ? static_cast<float*>(const_cast<void*>(ctx)) : reinterpret_cast<float*>(ws + plan.states);
    a.dstates = reinterpret_cast<float*>(ws + plan.dstates);
    a.parts = reinterpret_cast<float*>(ws + plan.parts);
    a.dbc = plan.groups > 1 ? reinterpret_cast<float*>(ws + plan.dbc) : nullptr;
    a.ddt_ws = hsub > 1 ? reinterpret_cast<float*>(ws + plan.ddt) : nullptr;
    a.nseg = plan.nseg;
    a.seg_chunks = plan.seg_chunks;
    a.seg_state = plan.nseg > 1 ? reinterpret_cast<float*>(ws + plan.seg_state) : nullptr;
    a.seg_lam = plan.nseg > 1 ? reinterpret_cast<float*>(ws + plan.seg_lam) : nullptr;
    a.chunk_dec = plan.nseg > 1 ? reinterpret_cast<float*>(ws + plan.chunk_dec) : nullptr;
    a.groups = plan.groups;
    a.heads_per_group = plan.heads_per_group;
    return from_hip(saved ? mssm::launch_ssd_bwd_saved(a, static_cast<hipStream_t>(hip_stream))
                          : mssm::launch_ssd_bwd(a, static_cast<hipStream_t>(hip_stream)));
}
}  // namespace

mssm_status mssm_ssd_bwd(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                         const float* h0, const void* dy, const float* dh_final,
                         void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                         float* ddt_bias, float* dh0,
                         void* workspace, size_t workspace_bytes, void* hip_stream) {
    return ssd_bwd_common(p, x, dt, A, Bm, Cm, Dskip, dt_bias, h0, nullptr, 0, dy, dh_final, dx, ddt, dA, dB, dC,
                          dD, ddt_bias, dh0, workspace, workspace_bytes, hip_stream, false);
}

size_t mssm_ssd_bwd_saved_workspace_bytes(const mssm_ssd_problem* p) {
    if (check_ssd_problem(p) != MSSM_OK) return 0;
    return mssm::plan_ssd_bwd(p->batch, p->seqlen, p->nheads * ssd_subheads(p), mssm::kSsdHeadDim, p->dstate,
                              ssd_subheads(p), device_cus(), true)
        .total;
}

mssm_status mssm_ssd_bwd_saved(const mssm_ssd_problem* p, const void* x, const void* dt, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip, const float* dt_bias,
                               const void* ctx, size_t ctx_bytes, const void* dy, const float* dh_final,
                               void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                               float* ddt_bias, float* dh0,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
    return ssd_bwd_common(p, x, dt, A, Bm, Cm, Dskip, dt_bias, nullptr, ctx, ctx_bytes, dy, dh_final, dx, ddt, dA,
                          dB, dC, dD, ddt_bias, dh0, workspace, workspace_bytes, hip_stream, true);
}

const char* mssm_status_string(mssm_status s) {
    switch (s) {
        case MSSM_OK: return "MSSM_OK: success";
        case MSSM_ERR_NULL: return "MSSM_ERR_NULL: a required pointer is NULL";
        case MSSM_ERR_SHAPE: return "MSSM_ERR_SHAPE: a dimension is out of range";
        case MSSM_ERR_DTYPE: return "MSSM_ERR_DTYPE: unknown element type";
        case MSSM_ERR_UNSUPPORTED: return "MSSM_ERR_UNSUPPORTED: dstate > 64 (or an SSD size not built)";
        case MSSM_ERR_ALIGN: return "MSSM_ERR_ALIGN: a pointer is not 16-byte aligned";
        case MSSM_ERR_WORKSPACE: return "MSSM_ERR_WORKSPACE: workspace missing or too small";
        case MSSM_ERR_HIP: return "MSSM_ERR_HIP: a HIP launch failed";
    }
    return "unknown mssm_status";
}

const char* mssm_build_info(void) { return "libmssm 0.1 (gfx950)"; }

}  // extern "C"
