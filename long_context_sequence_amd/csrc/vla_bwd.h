// vla_bwd.h -- internal declarations of the reverse-mode (gradient) kernel.
#pragma once
#include "vla_common.h"

namespace vla {

// Launch arguments of vla_backward after the C-ABI checks (include/vla.h).
struct BwdArgs {
    const void *q, *k, *v, *u;
    int dtype;            // 0 = fp32, 1 = bf16
    int B, H, T, d;
    float lambda0, eps;
    const float *S0, *A0, *zk0;
    const float *dO, *dS_T, *dA_T, *dzk_T;
    float *dq, *dk, *dv, *du, *dS0, *dA0, *dzk0;
    void *ws;
    hipStream_t stream;
};

// floats kept per token of a head (rec::Keep in vla_record.h): z, alpha^, e,
// the key sum zkey_t (d each) and 8 scalars
constexpr size_t backward_record_floats(int d) { return 4 * (size_t)d + 8; }
size_t backward_workspace_bytes(int BH, int T, int d);
hipError_t launch_backward(const BwdArgs &a);

}  // namespace vla
