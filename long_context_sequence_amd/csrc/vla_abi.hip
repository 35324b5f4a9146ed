// vla_abi.hip -- the library's extern "C" entry points (declared in include/vla.h):
// argument checks, then kernel selection by (d_h, input type).  Nothing is
// launched when a check fails.
#include <math.h>
#include <stdint.h>

#include "../../include/vla.h"
#include "vla_bwd.h"
#include "vla_common.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool ok_ptr(const void *p, bool required) { return p ? aligned16(p) : !required; }
bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 96 || d == 128; }
bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

vla_status check_common(int in_dtype, int B, int H, int d_h, float eps)
{
    if (B < 1 || H < 1) return VLA_ERR_INVALID_ARG;
    if ((long long)B * H > 0x7fffffffLL) return VLA_ERR_INVALID_ARG;
    if (!finite_pos(eps)) return VLA_ERR_INVALID_ARG;
    if (in_dtype != VLA_F32 && in_dtype != VLA_BF16) return VLA_ERR_UNSUPPORTED;
    if (!supported_d(d_h)) return VLA_ERR_UNSUPPORTED;
    return VLA_OK;
}

// d_h in {64, 96, 128}: sequences (T >= 1) run on the two-pass matrix-core
// kernels and a single decode token on the decode kernel (which reads and
// writes every state element from the same lane, so the state is updated in
// place); d_h in {16, 32} uses the LDS kernel for both.  T = 0 writes the
// initial state to the outputs.
vla_status launch(const vla::FwdArgs &a, bool step)
{
    hipError_t e;
    if (step)
        e = vla::chunk_supported(a.d) ? vla::launch_step(a) : vla::launch_forward_ref(a);
    else if (a.T == 0)
        e = vla::launch_state_init(a);
    else if (vla::chunk_supported(a.d))
        e = vla::launch_forward_twopass(a, 3);
    else
        e = vla::launch_forward_ref(a);
    return e == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

size_t workspace_bytes(int B, int H, int T, int d_h)
{
    if (!vla::chunk_supported(d_h) || T <= 0) return 0;
    return vla::twopass_workspace_bytes(B * H, T, d_h);
}

}  // namespace

// Every check of vla_forward except the workspace's (shared with
// vla_forward_noalloc, whose workspace is the library's own).
vla_status vla::check_forward(const void *q, const void *k, const void *v, const void *u,
                              int in_dtype, int B, int H, int T, int d_h, float lambda0, float eps,
                              const float *o, const float *S_out, const float *A_out,
                              const float *zkey_out, const float *S0, const float *A0,
                              const float *zkey0)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (T < 0 || !finite_pos(lambda0)) return VLA_ERR_INVALID_ARG;
    if (!vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    const bool need_tok = T > 0;
    if (!ok_ptr(q, need_tok) || !ok_ptr(k, need_tok) || !ok_ptr(v, need_tok) ||
        !ok_ptr(u, need_tok) || !ok_ptr(o, need_tok))
        return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(S_out, false) || !ok_ptr(A_out, false) || !ok_ptr(zkey_out, false) ||
        !ok_ptr(S0, false) || !ok_ptr(A0, false) || !ok_ptr(zkey0, false))
        return VLA_ERR_INVALID_ARG;
    return VLA_OK;
}

extern "C" vla_status vla_forward(const void *q, const void *k, const void *v, const void *u,
                                  vla_dtype in_dtype, int B, int H, int T, int d_h,
                                  float lambda0, float eps,
                                  float *o, float *S_out, float *A_out, float *zkey_out,
                                  const float *S0, const float *A0, const float *zkey0,
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    vla_status st = vla::check_forward(q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps, o, S_out,
                                       A_out, zkey_out, S0, A0, zkey0);
    if (st != VLA_OK) return st;
    const size_t need = ::workspace_bytes(B, H, T, d_h);
    if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need))
        return VLA_ERR_INVALID_ARG;
    if (T == 0 && !S_out && !A_out && !zkey_out) return VLA_OK;   // nothing to do

    vla::FwdArgs a{q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps,
                   o, S_out, A_out, zkey_out, S0, A0, zkey0, (hipStream_t)stream,
                   workspace, workspace_bytes};
    return launch(a, false);
}

// The two phases of the two-pass forward (d_h in {64, 96, 128}, T >= 1).
static vla_status check_phase(int in_dtype, int B, int H, int T, int d_h, float eps, void *workspace,
                       size_t workspace_bytes)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (!vla::chunk_supported(d_h)) return VLA_ERR_UNSUPPORTED;
    if (T < 1) return VLA_ERR_INVALID_ARG;
    if (!vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    const size_t need = ::workspace_bytes(B, H, T, d_h);
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return VLA_ERR_INVALID_ARG;
    return VLA_OK;
}

extern "C" vla_status vla_forward_penalty(const void *q, const void *k, const void *u, vla_dtype in_dtype,
                                          int B, int H, int T, int d_h, float lambda0, float eps,
                                          float *A_out, float *zkey_out, const float *A0,
                                          const float *zkey0, void *workspace,
                                          size_t workspace_bytes, void *stream)
{
    vla_status st = check_phase(in_dtype, B, H, T, d_h, eps, workspace, workspace_bytes);
    if (st != VLA_OK) return st;
    if (!finite_pos(lambda0)) return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(q, true) || !ok_ptr(k, true) || !ok_ptr(u, true) || !ok_ptr(A_out, false) ||
        !ok_ptr(zkey_out, false) || !ok_ptr(A0, false) || !ok_ptr(zkey0, false))
        return VLA_ERR_INVALID_ARG;
    vla::FwdArgs a{q, k, nullptr, u, in_dtype, B, H, T, d_h, lambda0, eps,
                   nullptr, nullptr, A_out, zkey_out, nullptr, A0, zkey0, (hipStream_t)stream,
                   workspace, workspace_bytes};
    return vla::launch_forward_twopass(a, 1) == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

extern "C" vla_status vla_forward_memory(const void *v, vla_dtype in_dtype, int B, int H, int T,
                                         int d_h, float *o, float *S_out, const float *S0,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    vla_status st = check_phase(in_dtype, B, H, T, d_h, 1.0f, workspace, workspace_bytes);
    if (st != VLA_OK) return st;
    if (!ok_ptr(v, true) || !ok_ptr(o, true) || !ok_ptr(S_out, false) || !ok_ptr(S0, false))
        return VLA_ERR_INVALID_ARG;
    vla::FwdArgs a{nullptr, nullptr, v, nullptr, in_dtype, B, H, T, d_h, 1.0f, 1.0f,
                   o, S_out, nullptr, nullptr, S0, nullptr, nullptr, (hipStream_t)stream,
                   workspace, workspace_bytes};
    return vla::launch_forward_twopass(a, 2) == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

extern "C" vla_status vla_forward_workspace_size(int B, int H, int T, int d_h, size_t *bytes)
{
    if (!bytes || B < 1 || H < 1 || T < 0 || (long long)B * H > 0x7fffffffLL) return VLA_ERR_INVALID_ARG;
    if (!supported_d(d_h) || !vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    *bytes = ::workspace_bytes(B, H, T, d_h);
    return VLA_OK;
}

extern "C" vla_status vla_step(const void *q, const void *k, const void *v, const void *u,
                               vla_dtype in_dtype, int B, int H, int d_h, float eps,
                               float *S, float *A, float *zkey, float *o, void *stream)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (!ok_ptr(q, true) || !ok_ptr(k, true) || !ok_ptr(v, true) || !ok_ptr(u, true) ||
        !ok_ptr(o, true) || !ok_ptr(S, true) || !ok_ptr(A, true) || !ok_ptr(zkey, true))
        return VLA_ERR_INVALID_ARG;
    // lambda0 only shapes the default A_0, which a step never uses (A is given).
    vla::FwdArgs a{q, k, v, u, in_dtype, B, H, 1, d_h, 1.0f, eps,
                   o, S, A, zkey, S, A, zkey, (hipStream_t)stream, nullptr, 0};
    return launch(a, true);
}

extern "C" vla_status vla_forward_scan_workspace_size(int B, int H, int T, int d_h, size_t *bytes)
{
    if (!bytes || B < 1 || H < 1 || T < 0 || (long long)B * H > 0x7fffffffLL) return VLA_ERR_INVALID_ARG;
    if (!vla::scan_supported(d_h) || !vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    *bytes = vla::scan_workspace_bytes(B * H, T, d_h);
    return VLA_OK;
}

extern "C" vla_status vla_forward_scan(const void *q, const void *k, const void *v, const void *u,
                                       vla_dtype in_dtype, int B, int H, int T, int d_h,
                                       float lambda0, float eps,
                                       float *o, float *S_out, float *A_out, float *zkey_out,
                                       const float *S0, const float *A0, const float *zkey0,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (!vla::scan_supported(d_h)) return VLA_ERR_UNSUPPORTED;
    if (T < 1 || !finite_pos(lambda0)) return VLA_ERR_INVALID_ARG;
    if (!vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    const size_t need = vla::scan_workspace_bytes(B * H, T, d_h);
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(q, true) || !ok_ptr(k, true) || !ok_ptr(v, true) || !ok_ptr(u, true) ||
        !ok_ptr(o, true))
        return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(S_out, false) || !ok_ptr(A_out, false) || !ok_ptr(zkey_out, false) ||
        !ok_ptr(S0, false) || !ok_ptr(A0, false) || !ok_ptr(zkey0, false))
        return VLA_ERR_INVALID_ARG;
    vla::FwdArgs a{q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps,
                   o, S_out, A_out, zkey_out, S0, A0, zkey0, (hipStream_t)stream,
                   workspace, workspace_bytes};
    return vla::launch_forward_scan(a) == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

extern "C" vla_status vla_backward_workspace_size(int B, int H, int T, int d_h, size_t *bytes)
{
    if (!bytes || B < 1 || H < 1 || T < 0 || (long long)B * H > 0x7fffffffLL) return VLA_ERR_INVALID_ARG;
    if (!supported_d(d_h) || !vla::twopass_size_ok(T, d_h, true)) return VLA_ERR_UNSUPPORTED;
    *bytes = vla::backward_workspace_bytes(B * H, T, d_h);
    return VLA_OK;
}

extern "C" vla_status vla_backward(const void *q, const void *k, const void *v, const void *u,
                                   vla_dtype in_dtype, int B, int H, int T, int d_h,
                                   float lambda0, float eps,
                                   const float *S0, const float *A0, const float *zkey0,
                                   const float *dO, const float *dS_T, const float *dA_T,
                                   const float *dzkey_T,
                                   float *dq, float *dk, float *dv, float *du,
                                   float *dS0, float *dA0, float *dzkey0,
                                   void *workspace, size_t workspace_bytes, void *stream)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (T < 0 || !finite_pos(lambda0)) return VLA_ERR_INVALID_ARG;
    if (!vla::twopass_size_ok(T, d_h, true)) return VLA_ERR_UNSUPPORTED;
    const size_t need = vla::backward_workspace_bytes(B * H, T, d_h);
    if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need))
        return VLA_ERR_INVALID_ARG;
    const bool need_tok = T > 0;
    if (!ok_ptr(q, need_tok) || !ok_ptr(k, need_tok) || !ok_ptr(v, need_tok) ||
        !ok_ptr(u, need_tok) || !ok_ptr(dO, need_tok) || !ok_ptr(dq, need_tok) ||
        !ok_ptr(dk, need_tok) || !ok_ptr(dv, need_tok) || !ok_ptr(du, need_tok))
        return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(S0, false) || !ok_ptr(A0, false) || !ok_ptr(zkey0, false) ||
        !ok_ptr(dS_T, false) || !ok_ptr(dA_T, false) || !ok_ptr(dzkey_T, false) ||
        !ok_ptr(dS0, false) || !ok_ptr(dA0, false) || !ok_ptr(dzkey0, false))
        return VLA_ERR_INVALID_ARG;
    if (T == 0 && !dS0 && !dA0 && !dzkey0) return VLA_OK;   // nothing to do

    vla::BwdArgs a{q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps, S0, A0, zkey0,
                   dO, dS_T, dA_T, dzkey_T, dq, dk, dv, du, dS0, dA0, dzkey0,
                   workspace, (hipStream_t)stream};
    return vla::launch_backward(a) == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

extern "C" vla_status vla_baseline_workspace_size(int B, int H, int T, int d_h, size_t *bytes)
{
    if (!bytes || B < 1 || H < 1 || T < 0 || (long long)B * H > 0x7fffffffLL) return VLA_ERR_INVALID_ARG;
    if (!vla::chunk_supported(d_h) || !vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    *bytes = vla::baseline_workspace_bytes(B * H, T, d_h);
    return VLA_OK;
}

extern "C" vla_status vla_baseline_forward(vla_baseline kind, const void *q, const void *k,
                                           const void *v, vla_dtype in_dtype, int B, int H, int T,
                                           int d_h, float beta, float eps, float *o, float *S_out,
                                           float *zkey_out, const float *S0, const float *zkey0,
                                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (kind != VLA_BASELINE_LINEAR && kind != VLA_BASELINE_DELTA) return VLA_ERR_UNSUPPORTED;
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (!vla::chunk_supported(d_h)) return VLA_ERR_UNSUPPORTED;
    if (T < 0 || !isfinite(beta)) return VLA_ERR_INVALID_ARG;
    if (!vla::twopass_size_ok(T, d_h, false)) return VLA_ERR_UNSUPPORTED;
    const size_t need = vla::baseline_workspace_bytes(B * H, T, d_h);
    if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need))
        return VLA_ERR_INVALID_ARG;
    const bool need_tok = T > 0;
    if (!ok_ptr(q, need_tok) || !ok_ptr(k, need_tok) || !ok_ptr(v, need_tok) || !ok_ptr(o, need_tok))
        return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(S_out, false) || !ok_ptr(zkey_out, false) || !ok_ptr(S0, false) ||
        !ok_ptr(zkey0, false))
        return VLA_ERR_INVALID_ARG;
    if (T == 0 && !S_out && !zkey_out) return VLA_OK;
    vla::FwdArgs a{q, k, v, nullptr, in_dtype, B, H, T, d_h, 1.0f, eps,
                   o, S_out, nullptr, zkey_out, S0, nullptr, zkey0, (hipStream_t)stream,
                   workspace, workspace_bytes};
    hipError_t e = T == 0 ? vla::launch_state_init(a)
                          : vla::launch_baseline(a, kind == VLA_BASELINE_DELTA, beta);
    return e == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

extern "C" const char *vla_status_string(vla_status status)
{
    switch (status) {
    case VLA_OK: return "VLA_OK: success";
    case VLA_ERR_INVALID_ARG: return "VLA_ERR_INVALID_ARG: null or misaligned pointer, bad size or constant";
    case VLA_ERR_UNSUPPORTED: return "VLA_ERR_UNSUPPORTED: no kernel for this head dimension or input type";
    case VLA_ERR_HIP: return "VLA_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown vla_status";
    }
}
