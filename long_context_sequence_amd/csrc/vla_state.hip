// vla_state.hip -- a forward over no tokens: the initial state of the recurrence
// written to the requested outputs.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.2: the
// default initial state is S_0 = 0, A_0 = I / lambda0 and an empty key sum
// (zkey_0 = 0); a caller-given state is copied as it is.
//
// Plain element-wise copy/fill, 16 bytes per thread and grid-stride loops.
// Every element is read and written by the same thread, so an output may alias
// its initial state (then that part is skipped altogether).
#include "vla_common.h"

namespace vla {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// n4 granules of 4 floats of a [BH][D][D] matrix: the copy of src, or the
// default (diag on the diagonal, 0 elsewhere) when src is NULL.
__device__ __forceinline__ void mat_part(size_t i4, int D, const float *src, float diag, float *dst)
{
    f4 x;
    if (src) {
        x = reinterpret_cast<const f4 *>(src)[i4];
    } else {
        const size_t e0 = 4 * i4, DD = (size_t)D * D;
        const int r = (int)((e0 % DD) / D), c0 = (int)(e0 % D);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = r == c0 + j ? diag : 0.f;
    }
    reinterpret_cast<f4 *>(dst)[i4] = x;
}

__global__ void __launch_bounds__(256)
vla_state_init(int BH, int D, float lambda0, const float *S0, const float *A0, const float *zk0,
               float *S_out, float *A_out, float *zk_out)
{
    const size_t nm = (size_t)BH * D * D / 4, nz = (size_t)BH * D / 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool doS = S_out && S_out != S0, doA = A_out && A_out != A0;
    const bool doZ = zk_out && zk_out != zk0;
    for (size_t i = i0; i < nm; i += stride) {
        if (doS) mat_part(i, D, S0, 0.f, S_out);
        if (doA) mat_part(i, D, A0, 1.f / lambda0, A_out);
    }
    if (doZ) {
        for (size_t i = i0; i < nz; i += stride) {
            f4 x = {0.f, 0.f, 0.f, 0.f};
            if (zk0) x = reinterpret_cast<const f4 *>(zk0)[i];
            reinterpret_cast<f4 *>(zk_out)[i] = x;
        }
    }
}

}  // namespace

hipError_t launch_state_init(const FwdArgs &a)
{
    const int BH = a.B * a.H;
    const size_t n4 = (size_t)BH * a.d * a.d / 4;
    const size_t want = (n4 + 255) / 256;
    const unsigned blocks = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
    hipLaunchKernelGGL(vla_state_init, dim3(blocks), dim3(256), 0, a.stream, BH, a.d, a.lambda0,
                       a.S0, a.A0, a.zk0, a.S_out, a.A_out, a.zk_out);
    return hipGetLastError();
}

}  // namespace vla
