// vla_chunk_kernel.hip -- chunked matrix-core kernels of the VLA recurrence for
// d_h in {64, 96, 128}: the blocked chains of vla_chunk_parts.h arranged in time.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9)-(11); A_0 = I / lambda0 (section 3.2).
//
// One workgroup per head with both chains, NA waves each, so that every SIMD
// holds a wave of each chain; it serves single decode steps (T = 1, state
// updated in place) and T = 0 (state copy).  Longer sequences use the two-pass
// form of vla_twopass.hip, which spreads a head over many compute units.
// Period p has two segments separated by LDS barriers:
//   segment 1:  penalty waves: Z0, Y0, Grams of chunk p; key-sum prefix of
//                              chunk p.
//               memory waves:  S K^, S Phi, 1/|w|, Grams of chunk p-1.
//   segment 2:  penalty waves: factorise, update A, W of chunk p (into LDS).
//               memory waves:  (I+N)^-1, E, readout, update S for chunk p-1;
//                              readout denominators of chunk p; staging of p+1.
#include "vla_chunk_parts.h"

namespace vla {
namespace {

using namespace chunk;

// ---------------------------------------------------------------- fused kernel
template <int D, typename Tin>
__global__ void __launch_bounds__(128 * Cfg<D>::NA)
vla_fwd_fused(const Tin *__restrict__ q, const Tin *__restrict__ k,
              const Tin *__restrict__ v, const Tin *__restrict__ u,
              int T, float lambda0, float eps,
              float *__restrict__ o, float *S_out, float *A_out, float *zk_out,
              const float *S0, const float *A0, const float *zk0)
{
    using Hd = Head<D, Tin>;
    constexpr int NA = Cfg<D>::NA, BPW = Cfg<D>::BPW, C = Cfg<D>::C;
    __shared__ __align__(16) Lds<D> L;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const bool awave = w < NA;
    const size_t bh = blockIdx.x;
    const size_t DD = (size_t)D * D;
    const int NC = (T + C - 1) / C;

    // memory waves stage the inputs; penalty-wave threads 0..D-1 own the key sums
    Hd hd(L, q, k, v, u, o, T, eps, bh, tid & 63, awave ? w : w - NA, tid - 64 * NA, !awave,
          awave ? tid : -1);
    typename Hd::State st;
    if (hd.kcol >= 0 && zk0) hd.zk_run = zk0[bh * D + hd.kcol];
    if (awave) {
        hd.load_state(st, A0 ? A0 + bh * DD : nullptr, 1.f / lambda0);
    } else {
        hd.load_state(st, S0 ? S0 + bh * DD : nullptr, 0.f);
        if (NC > 0) {
            hd.template prefetch<true, true>(0);
            hd.template stage1<true, true>(0);
            hd.template prefetch<true, true>(1);
        }
    }
    vmem_drain();
    __syncthreads();

    if (awave) {
        WToLds<D> wl{L, 0, hd.g, hd.n};
        for (int p = 0; p <= NC; ++p) {
            hd.pp = p;
            VLA_PROBE(p, 0);
            if (p < NC) {
                hd.a_products(st, p);
                hd.stage2(p);
            }
            VLA_PROBE(p, 1);
            lds_barrier();
            VLA_PROBE(p, 2);
            if (p < NC) {
                wl.sp = p & 1;
                hd.a_update(st, p, wl);
            }
            VLA_PROBE(p, 3);
            lds_barrier();
        }
    } else {
        f4 sk[BPW], sq[BPW], invn4 = {0.f, 0.f, 0.f, 0.f};
        Raw1<Tin> vraw[BPW][4];
        for (int p = 0; p <= NC; ++p) {
            const int cq = p - 1;   // chunk of this period's memory-chain work
            hd.pp = p;
            VLA_PROBE(p, 0);
            if (p >= 1) {
                hd.s_products(st, cq, sk, sq);
                hd.s_grams(cq, invn4);
            }
            VLA_PROBE(p, 1);
            lds_barrier();
            VLA_PROBE(p, 2);
            if (p >= 1) hd.s_update(st, cq, sk, sq, invn4, vraw, L.wt[cq & 1]);
            VLA_PROBE(p, 10);
            if (p < NC) {
                hd.stage3(p);
                hd.load_v(p, vraw);   // used in the next period
            }
            if (p + 1 < NC) {
                hd.template stage1<true, true>(p + 1);
                hd.template prefetch<true, true>(p + 2);
            }
            VLA_PROBE(p, 3);
            lds_barrier();
        }
    }

    float *const out = awave ? A_out : S_out;
    if (out) hd.store_state(st, out + bh * DD);
    if (hd.kcol >= 0 && zk_out) zk_out[bh * D + hd.kcol] = hd.zk_run;
    VLA_PROBE_FLUSH();
}

template <int D, typename Tin>
hipError_t launch_chunk(const FwdArgs &a)
{
    const int BH = a.B * a.H;
    hipLaunchKernelGGL((vla_fwd_fused<D, Tin>), dim3(BH), dim3(128 * Cfg<D>::NA), 0, a.stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u,
                       a.T, a.lambda0, a.eps, a.o, a.S_out, a.A_out, a.zk_out, a.S0, a.A0, a.zk0);
    return hipGetLastError();
}

}  // namespace

bool chunk_supported(int d) { return d == 64 || d == 96 || d == 128; }

hipError_t launch_forward_chunk(const FwdArgs &a)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch_chunk<64, uint16_t>(a) : launch_chunk<64, float>(a);
    case 96: return bf ? launch_chunk<96, uint16_t>(a) : launch_chunk<96, float>(a);
    case 128: return bf ? launch_chunk<128, uint16_t>(a) : launch_chunk<128, float>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
