// vla_ref_kernel.hip -- the VLA recurrence for the small head dimensions
// d_h in {16, 32}, forward and decode step.
//
// One wave owns one (batch, head) for the whole sequence and keeps A and S in
// registers: lane l holds columns [c0, c0 + EPL) of row l / LPR of both (LPR =
// 64 / d lanes per row, EPL = d / LPR entries each), so a matrix-vector product
// is EPL multiply-adds and a DPP sum over the row's lanes, and a rank-1 update is
// EPL multiply-adds.  Token vectors pass between lanes through LDS; with one
// wave, LDS instructions complete in program order, so no barrier is needed
// anywhere.  At these sizes a head is a few kilobytes of state and the sequence
// is a chain of short dependent steps: what matters is the latency of one token,
// which this keeps to a handful of wave-wide sums.  The state is read into
// registers before anything is written, so a decode step may update it in
// place.  Source: "Variational Linear Attention" (arXiv 2605.11196), section
// 3.3, Eqs. (9)-(11); initial A_0 = I / lambda0 from section 3.2.
#include "vla_common.h"
#include "vla_chunk_parts.h"

namespace vla {
namespace {

using chunk::dpp;
using chunk::sfor;
using chunk::sum_row16;
using chunk::wave_lds_order;

// sum over the whole wave, the same value in every lane: the four 16-lane rows
// are summed by DPP, then their totals read out
__device__ __forceinline__ float wave_sum(float x)
{
    x = sum_row16(x);
    auto at = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
    return (at(0) + at(16)) + (at(32) + at(48));
}

// sum over the LPR adjacent lanes of a matrix row
template <int LPR>
__device__ __forceinline__ float row_sum(float x)
{
    static_assert(LPR == 2 || LPR == 4, "lanes per row");
    x += dpp<0xB1>(x);                        // quad_perm [1, 0, 3, 2]
    if constexpr (LPR == 4) x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    return x;
}

template <int D, typename Tin>
__global__ void __launch_bounds__(64)
vla_fwd_ref(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
            const Tin *__restrict__ u, int T, float lambda0, float eps, float *__restrict__ o,
            float *S_out, float *A_out, float *zk_out, const float *S0, const float *A0,
            const float *zk0)
{
    constexpr int LPR = 64 / D, EPL = D / LPR, DD = D * D;
    static_assert(EPL % 4 == 0, "vector reads");
    __shared__ __align__(16) float kh[D], uh[D], pq[D], zv[D], al[D];

    const int lane = threadIdx.x, row = lane / LPR, part = lane % LPR, c0 = part * EPL;
    const bool lead = part == 0;   // the lane that speaks for its row
    const bool col = lane < D;     // lane j < d: entry j of the token vectors
    const size_t bh = blockIdx.x;

    float a[EPL], s[EPL];
    sfor<EPL>([&](auto e) {
        const size_t idx = bh * DD + (size_t)row * D + c0 + e;
        s[e] = S0 ? S0[idx] : 0.f;
        a[e] = A0 ? A0[idx] : (row == c0 + e ? 1.f / lambda0 : 0.f);
    });
    float zk = col && zk0 ? zk0[bh * D + lane] : 0.f;

    auto read_vec = [&](const float *p, float (&x)[EPL]) {
        sfor<EPL / 4>([&](auto h) {
            const chunk::f4 y = chunk::ld4(p + c0 + 4 * h);
            sfor<4>([&](auto r) { x[4 * h + r] = y[int(r)]; });
        });
    };

    // token t's entries: lanes j < d take q, k, u at column j; every lane v at its row
    float qn = 0.f, kn = 0.f, un = 0.f, vn = 0.f;
    auto load = [&](int t) {
        const size_t base = (bh * (size_t)T + t) * D;
        if (col) {
            qn = load_in(q, base + lane);
            kn = load_in(k, base + lane);
            un = load_in(u, base + lane);
        }
        vn = load_in(v, base + row);
    };
    if (T > 0) load(0);
    for (int t = 0; t < T; ++t) {
        const float qv = qn, kv = kn, uv = un, vv = vn;
        if (t + 1 < T) load(t + 1);   // the next token's loads in flight meanwhile

        // normalisation, phi, key sum and the readout's denominator (Eq. (11))
        const float nk = wave_sum(kv * kv), nu = wave_sum(uv * uv);
        if (col) {
            kh[lane] = nk > 0.f ? kv / sqrtf(nk) : 0.f;
            uh[lane] = nu > 0.f ? uv / sqrtf(nu) : 0.f;
            pq[lane] = phi(qv);
            zk += phi(kv);   // inclusive key sum
        }
        const float pv = col ? phi(qv) : 0.f;
        const float den = fmaxf(wave_sum(pv * zk), eps);
        wave_lds_order();

        // Eq. (9): z = A u^, delta = 1 + u^'z, A -= z z' / delta
        float x[EPL];
        read_vec(uh, x);
        float zi = 0.f;
        sfor<EPL>([&](auto e) { zi = fmaf(a[e], x[e], zi); });
        zi = row_sum<LPR>(zi);
        const float delta = 1.f + wave_sum(lead ? uh[row] * zi : 0.f);
        if (lead) zv[row] = zi;
        wave_lds_order();
        read_vec(zv, x);
        const float zs = zi / delta;
        sfor<EPL>([&](auto e) { a[e] = fmaf(-zs, x[e], a[e]); });

        // Eq. (10): alpha^ from the new A, the residual from the old S, the write
        read_vec(kh, x);
        float yi = 0.f, ri = 0.f;
        sfor<EPL>([&](auto e) {
            yi = fmaf(a[e], x[e], yi);
            ri = fmaf(s[e], x[e], ri);
        });
        yi = row_sum<LPR>(yi);
        ri = row_sum<LPR>(ri);
        const float ny = wave_sum(lead ? yi * yi : 0.f);
        if (lead) al[row] = ny > 0.f ? yi / sqrtf(ny) : 0.f;
        wave_lds_order();
        read_vec(al, x);
        const float ei = vv - ri;
        sfor<EPL>([&](auto e) { s[e] = fmaf(ei, x[e], s[e]); });

        // Eq. (11): o = S phi(q) / den
        read_vec(pq, x);
        float oi = 0.f;
        sfor<EPL>([&](auto e) { oi = fmaf(s[e], x[e], oi); });
        oi = row_sum<LPR>(oi);
        if (lead) o[(bh * (size_t)T + t) * D + row] = oi / den;
        wave_lds_order();
    }

    sfor<EPL>([&](auto e) {
        const size_t idx = bh * DD + (size_t)row * D + c0 + e;
        if (S_out) S_out[idx] = s[e];
        if (A_out) A_out[idx] = a[e];
    });
    if (zk_out && col) zk_out[bh * D + lane] = zk;
}

template <int D, typename Tin>
hipError_t launch_ref(const FwdArgs &a)
{
    hipLaunchKernelGGL((vla_fwd_ref<D, Tin>), dim3(a.B * a.H), dim3(64), 0, a.stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u,
                       a.T, a.lambda0, a.eps, a.o, a.S_out, a.A_out, a.zk_out,
                       a.S0, a.A0, a.zk0);
    return hipGetLastError();
}

}  // namespace

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
