// vla_abi.hip -- the library's extern "C" entry points (declared in include/vla.h):
// argument checks, then kernel selection by (d_h, input type).  Nothing is
// launched when a check fails.
#include <math.h>
#include <stdint.h>

#include "../../include/vla.h"
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

// d_h in {64, 96, 128} runs on the chunked matrix-core kernel (also for a single
// decode token: every state element is read and written by the same lane, so the
// state may be updated in place); d_h in {16, 32} uses the LDS kernel.
vla_status launch(const vla::FwdArgs &a)
{
    hipError_t e = vla::chunk_supported(a.d) ? vla::launch_forward_chunk(a) : vla::launch_forward_ref(a);
    return e == hipSuccess ? VLA_OK : VLA_ERR_HIP;
}

}  // namespace

extern "C" vla_status vla_forward(const void *q, const void *k, const void *v, const void *u,
                                  int in_dtype, int B, int H, int T, int d_h,
                                  float lambda0, float eps,
                                  float *o, float *S_out, float *A_out, float *zkey_out,
                                  const float *S0, const float *A0, const float *zkey0,
                                  void *stream)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (T < 0 || !finite_pos(lambda0)) return VLA_ERR_INVALID_ARG;
    const bool need_tok = T > 0;
    if (!ok_ptr(q, need_tok) || !ok_ptr(k, need_tok) || !ok_ptr(v, need_tok) ||
        !ok_ptr(u, need_tok) || !ok_ptr(o, need_tok))
        return VLA_ERR_INVALID_ARG;
    if (!ok_ptr(S_out, false) || !ok_ptr(A_out, false) || !ok_ptr(zkey_out, false) ||
        !ok_ptr(S0, false) || !ok_ptr(A0, false) || !ok_ptr(zkey0, false))
        return VLA_ERR_INVALID_ARG;
    if (T == 0 && !S_out && !A_out && !zkey_out) return VLA_OK;   // nothing to do

    vla::FwdArgs a{q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps,
                   o, S_out, A_out, zkey_out, S0, A0, zkey0, (hipStream_t)stream};
    return launch(a);
}

extern "C" vla_status vla_step(const void *q, const void *k, const void *v, const void *u,
                               int in_dtype, int B, int H, int d_h, float eps,
                               float *S, float *A, float *zkey, float *o, void *stream)
{
    vla_status st = check_common(in_dtype, B, H, d_h, eps);
    if (st != VLA_OK) return st;
    if (!ok_ptr(q, true) || !ok_ptr(k, true) || !ok_ptr(v, true) || !ok_ptr(u, true) ||
        !ok_ptr(o, true) || !ok_ptr(S, true) || !ok_ptr(A, true) || !ok_ptr(zkey, true))
        return VLA_ERR_INVALID_ARG;
    // lambda0 only shapes the default A_0, which a step never uses (A is given).
    vla::FwdArgs a{q, k, v, u, in_dtype, B, H, 1, d_h, 1.0f, eps,
                   o, S, A, zkey, S, A, zkey, (hipStream_t)stream};
    return launch(a);
}

extern "C" const char *vla_status_string(int status)
{
    switch (status) {
    case VLA_OK: return "VLA_OK: success";
    case VLA_ERR_INVALID_ARG: return "VLA_ERR_INVALID_ARG: null or misaligned pointer, bad size or constant";
    case VLA_ERR_UNSUPPORTED: return "VLA_ERR_UNSUPPORTED: no kernel for this head dimension or input type";
    case VLA_ERR_HIP: return "VLA_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown vla_status";
    }
}
