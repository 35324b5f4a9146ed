// vla_ref_kernel.hip -- the VLA recurrence for the small head dimensions
// d_h in {16, 32}, forward and decode step.
//
// One workgroup of 256 threads owns one (batch, head) for the whole sequence
// and keeps A and S in LDS (row stride d+1).  Every step of a token is a
// separate block-synchronised phase: at these sizes a head is a few kilobytes
// of state and the sequence is latency-bound whatever the kernel.  The state
// is read into LDS before anything is written, so a decode step may update it
// in place.  Source: "Variational Linear Attention" (arXiv 2605.11196),
// section 3.3, Eqs. (9)-(11); initial A_0 = I / lambda0 from section 3.2.
#include "vla_common.h"

namespace vla {

template <int NW>
__device__ inline float block_sum(float x, float *red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();                 // previous use of red[] is finished
    if (l == 0) red[w] = x;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s += red[i];
    return s;
}

template <int D, typename Tin>
__global__ void __launch_bounds__(256)
vla_fwd_ref(const Tin *__restrict__ q, const Tin *__restrict__ k,
            const Tin *__restrict__ v, const Tin *__restrict__ u,
            int T, float lambda0, float eps,
            float *__restrict__ o, float *S_out, float *A_out, float *zk_out,
            const float *S0, const float *A0, const float *zk0)
{
    constexpr int NT = 256, NW = NT / 64, P = D + 1, DD = D * D;
    __shared__ float sA[D * P];
    __shared__ float sS[D * P];
    __shared__ float kh[D], uh[D], z[D], al[D], pq[D], zk[D], ev[D];
    __shared__ float red[NW];

    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x;

    for (int idx = tid; idx < DD; idx += NT) {
        const int i = idx / D, j = idx % D;
        sS[i * P + j] = S0 ? S0[bh * DD + idx] : 0.f;
        sA[i * P + j] = A0 ? A0[bh * DD + idx] : (i == j ? 1.f / lambda0 : 0.f);
    }
    if (tid < D) zk[tid] = zk0 ? zk0[bh * D + tid] : 0.f;
    __syncthreads();

    for (int t = 0; t < T; ++t) {
        const size_t base = (bh * (size_t)T + t) * D;
        float kv = 0.f, uv = 0.f, qv = 0.f, vv = 0.f;
        if (tid < D) {
            kv = load_in(k, base + tid);
            uv = load_in(u, base + tid);
            qv = load_in(q, base + tid);
            vv = load_in(v, base + tid);
        }
        const float nk = block_sum<NW>(kv * kv, red);
        const float nu = block_sum<NW>(uv * uv, red);
        if (tid < D) {
            kh[tid] = nk > 0.f ? kv / sqrtf(nk) : 0.f;
            uh[tid] = nu > 0.f ? uv / sqrtf(nu) : 0.f;
            pq[tid] = phi(qv);
            zk[tid] += phi(kv);
        }
        __syncthreads();

        // Eq. (9): z = A u^, delta = 1 + u^'z, A -= z z' / delta
        float zi = 0.f;
        if (tid < D) {
            for (int j = 0; j < D; ++j) zi = fmaf(sA[tid * P + j], uh[j], zi);
            z[tid] = zi;
        }
        const float delta = 1.f + block_sum<NW>(tid < D ? uh[tid] * zi : 0.f, red);
        const float invd = 1.f / delta;
        for (int idx = tid; idx < DD; idx += NT) {
            const int i = idx / D, j = idx % D;
            sA[i * P + j] -= (z[i] * z[j]) * invd;
        }
        __syncthreads();

        // Eq. (10): alpha^ from the new A; residual from the old S; rank-1 write
        float yi = 0.f, ri = 0.f;
        if (tid < D) {
            for (int j = 0; j < D; ++j) {
                yi = fmaf(sA[tid * P + j], kh[j], yi);
                ri = fmaf(sS[tid * P + j], kh[j], ri);
            }
        }
        const float ny = block_sum<NW>(yi * yi, red);
        if (tid < D) {
            al[tid] = ny > 0.f ? yi / sqrtf(ny) : 0.f;
            ev[tid] = vv - ri;
        }
        __syncthreads();
        for (int idx = tid; idx < DD; idx += NT) {
            const int i = idx / D, j = idx % D;
            sS[i * P + j] = fmaf(ev[i], al[j], sS[i * P + j]);
        }

        // Eq. (11): o = S phi(q) / max(phi(q)' zkey, eps)
        const float den = fmaxf(block_sum<NW>(tid < D ? pq[tid] * zk[tid] : 0.f, red), eps);
        if (tid < D) {
            float s = 0.f;
            for (int j = 0; j < D; ++j) s = fmaf(sS[tid * P + j], pq[j], s);
            o[base + tid] = s / den;
        }
        __syncthreads();
    }

    for (int idx = tid; idx < DD; idx += NT) {
        const int i = idx / D, j = idx % D;
        if (S_out) S_out[bh * DD + idx] = sS[i * P + j];
        if (A_out) A_out[bh * DD + idx] = sA[i * P + j];
    }
    if (zk_out && tid < D) zk_out[bh * D + tid] = zk[tid];
}

template <int D, typename Tin>
hipError_t launch_ref(const FwdArgs &a)
{
    hipLaunchKernelGGL((vla_fwd_ref<D, Tin>), dim3(a.B * a.H), dim3(256), 0, a.stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u,
                       a.T, a.lambda0, a.eps, a.o, a.S_out, a.A_out, a.zk_out,
                       a.S0, a.A0, a.zk0);
    return hipGetLastError();
}

hipError_t launch_forward_ref(const FwdArgs &a)
{
    const bool bf = a.dtype == 1;
#define VLA_REF_CASE(DV) \
    case DV: return bf ? launch_ref<DV, uint16_t>(a) : launch_ref<DV, float>(a);
    switch (a.d) {
        VLA_REF_CASE(16)
        VLA_REF_CASE(32)
    default: return hipErrorInvalidValue;
    }
#undef VLA_REF_CASE
}

}  // namespace vla
