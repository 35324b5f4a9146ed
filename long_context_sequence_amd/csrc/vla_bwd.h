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

// The reverse sweep as two chains running side by side (vla_bwd_split.hip), for
// d in {64, 96, 128}: per head a workgroup for the memory chain's adjoint (dS),
// which writes dv and the gate adjoint dL/dalpha^ per token (galpha,
// [B][H][T][d]), and one for the penalty chain's adjoint in the conjugated
// frame Q = A Sigma A, with S' and A, which follows it token by token and
// writes dq, dk and du.  rec holds the forward's per-token records, S_T and A_T
// its final state; sync is B H + 1 ints of workspace (role tickets and per-head
// progress), reset by the launch itself; qb is B H d^2 floats of workspace
// (Q_T when dL/dA_T is given, Q_0 when A_0 is).
// frec: the forward's per-chunk records (vla_record.h); at d = 64 both chains
// then go sixteen tokens at a time on the matrix cores; null, or another d,
// takes the token-by-token chains.
hipError_t launch_backward_split(const BwdArgs &a, const float *rec, const float *frec, const float *S_T,
                                 const float *A_T, float *galpha, int *sync, float *qb);

// x y + z w with both products rounded before the sum (no fused multiply-add):
// the same bits for (x, y, z, w) and (z, w, x, y), so that the two mirror
// entries of a symmetric rank-2 update receive identical terms.  (Rounded
// differently, Sigma gains an antisymmetric part that the reverse chain does
// not shrink, and it swamps the small gradients Sigma carries.)
__device__ __forceinline__ float sym_sum(float x, float y, float z, float w)
{
#pragma clang fp contract(off)
    return x * y + z * w;
}

// derivative of phi = ELU + 1
__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __expf(x); }

}  // namespace vla
