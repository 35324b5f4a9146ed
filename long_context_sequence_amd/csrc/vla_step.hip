// vla_step.hip -- one decode token of the VLA recurrence for d_h in {64, 96, 128}:
// the state (S, A, zkey) of every head is read, advanced by one token and
// written back in place.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9)-(11), for a single token t:
//   z = A u^,  delta = 1 + u^'z,  A <- A - z z' / delta                  (9)
//   y = A k^ (the new A),  alpha^ = y / |y|,  e = v - S k^,  S <- S + e alpha^'  (10)
//   zkey <- zkey + phi(k),  o = S phi(q) / max(phi(q)' zkey, eps)     (11)
// Both products with A use the old A (A_new k^ = A k^ - z (z'k^) / delta), and
// both products with S use the old S (S_new phi(q) = S phi(q) + e (alpha^'phi(q))),
// so each state is read once and written once.
//
// One workgroup per head, 1024 threads: the TPR adjacent threads of a row hold
// its 16-byte granules round-robin (thread g of the row holds granules g, g+TPR,
// g+2 TPR, ...), so that one load or store instruction of a wave covers whole
// 128-byte lines of TPR/2 ... rows (a thread holding consecutive columns makes
// each instruction touch every line at a quarter of its width, which halves
// the rate at which one CU writes the state back); the row products are
// reductions over adjacent lanes; the d-vectors live in LDS, and the scalars
// (delta, z'k^, |y|, y'phi(q), the denominator) are formed by every wave the
// same way from them.  Each thread writes back exactly the elements it read.
#include "vla_chunk_parts.h"
#include "vla_reduce.h"

namespace vla {
namespace {

using namespace chunk;

template <int D>
struct StepCfg {
    static constexpr int TPR = D == 64 ? 16 : 8;   // threads per row
    static constexpr int EPT = D / TPR;            // columns per thread (4, 12, 16)
    static constexpr int NG = EPT / 4;             // granules per thread
    static constexpr int ACTIVE = D * TPR;         // threads holding a row slice
    static_assert(EPT % 4 == 0 && ACTIVE <= 1024, "row slices of whole 16-byte granules");
};

template <int D, typename Tin>
__global__ void __launch_bounds__(1024)
vla_decode(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
           const Tin *__restrict__ u, float eps, float *S, float *A, float *zkey, float *__restrict__ o)
{
    using Cf = StepCfg<D>;
    constexpr int TPR = Cf::TPR, EPT = Cf::EPT, NV = (D + 63) / 64;
    __shared__ __align__(16) float qf[D], kf[D], vf[D], uf[D], zkf[D];
    __shared__ __align__(16) float zs[D], ws[D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int bh = blockIdx.x;
    const size_t DD = (size_t)D * D;
    const bool act = tid < Cf::ACTIVE;
    const int row = act ? tid / TPR : 0, g = tid % TPR;
    // column of element e = 4 h + r of this thread (granule g + TPR h)
    auto col = [&](int e) { return 4 * (g + TPR * (e >> 2)) + (e & 3); };

    // the token's vectors first (their wait then leaves the state loads in flight)
    float xq = 0.f, xk = 0.f, xv = 0.f, xu = 0.f, xz = 0.f;
    if (tid < D) {
        const size_t off = (size_t)bh * D + tid;
        xq = load_in(q, off);
        xk = load_in(k, off);
        xv = load_in(v, off);
        xu = load_in(u, off);
        xz = zkey[off];
    }
    float a[EPT], s[EPT];
    float *Ah = A + bh * DD + (size_t)row * D + 4 * g, *Sh = S + bh * DD + (size_t)row * D + 4 * g;
    if (act) {
        sfor<Cf::NG>([&](auto h) {
            const f4 x = ld4(Ah + 4 * TPR * h), y = ld4(Sh + 4 * TPR * h);
            sfor<4>([&](auto r) {
                a[4 * h + r] = x[int(r)];
                s[4 * h + r] = y[int(r)];
            });
        });
    }
    if (tid < D) {           // phi(q) and the new key sum zkey + phi(k) are kept
        qf[tid] = phi_fast(xq);
        kf[tid] = xk;
        vf[tid] = xv;
        uf[tid] = xu;
        zkf[tid] = xz + phi_fast(xk);
    }
    __syncthreads();

    // |k|^2, |u|^2 (every wave alike)
    float pk = 0.f, pu = 0.f;
    sfor<NV>([&](auto c) {
        const int j = lane + 64 * c;
        if (j < D) {
            pk = fmaf(kf[j], kf[j], pk);
            pu = fmaf(uf[j], uf[j], pu);
        }
    });
    pk = wave_sum(pk);
    pu = wave_sum(pu);
    const float ik = pk > 0.f ? rsqrtf(pk) : 0.f, iu = pu > 0.f ? rsqrtf(pu) : 0.f;

    // row products: z = A u^, w = A k^ (old A), r = S k^, p = S phi(q) (old S),
    // with the raw u and k and the inverse norms applied to the sums
    float pz = 0.f, pw = 0.f, pr = 0.f, pp = 0.f;
    sfor<EPT>([&](auto e) {
        const int j = col(e);
        const float uj = uf[j], kj = kf[j];
        pz = fmaf(a[e], uj, pz);
        pw = fmaf(a[e], kj, pw);
        pr = fmaf(s[e], kj, pr);
        pp = fmaf(s[e], qf[j], pp);
    });
    pz = row_sum<TPR>(pz) * iu, pw = row_sum<TPR>(pw) * ik;
    pr = row_sum<TPR>(pr) * ik, pp = row_sum<TPR>(pp);
    if (act && tid % TPR == 0) {
        zs[row] = pz;
        ws[row] = pw;
    }
    __syncthreads();

    // the scalars of the token (every wave alike)
    float du = 0.f, dk = 0.f;
    sfor<NV>([&](auto c) {
        const int j = lane + 64 * c;
        if (j < D) {
            du = fmaf(uf[j], zs[j], du);
            dk = fmaf(zs[j], kf[j], dk);
        }
    });
    const float delta = fmaf(wave_sum(du), iu, 1.f), zk = wave_sum(dk) * ik;
    const float ci = zk / delta, id = 1.f / delta;
    float yy = 0.f, yq = 0.f, dn = 0.f;
    sfor<NV>([&](auto c) {
        const int j = lane + 64 * c;
        if (j < D) {
            const float yj = ws[j] - zs[j] * ci, fq = qf[j];
            yy = fmaf(yj, yj, yy);
            yq = fmaf(yj, fq, yq);
            dn = fmaf(fq, zkf[j], dn);
        }
    });
    yy = wave_sum(yy);
    const float iy = yy > 0.f ? rsqrtf(yy) : 0.f;
    const float aq = wave_sum(yq) * iy;                       // alpha^' phi(q)
    const float rden = 1.f / fmaxf(wave_sum(dn), eps);

    if (act) {
        const float zi = pz, ei = vf[row] - pr;
        sfor<EPT>([&](auto e) {
            const int j = col(e);
            a[e] = fmaf(-zi * zs[j], id, a[e]);                  // A - z z' / delta
            s[e] = fmaf(ei, (ws[j] - zs[j] * ci) * iy, s[e]);    // S + e alpha^'
        });
        sfor<Cf::NG>([&](auto h) {
            st4(Ah + 4 * TPR * h, f4{a[4 * h], a[4 * h + 1], a[4 * h + 2], a[4 * h + 3]});
            st4(Sh + 4 * TPR * h, f4{s[4 * h], s[4 * h + 1], s[4 * h + 2], s[4 * h + 3]});
        });
        if (tid % TPR == 0) o[(size_t)bh * D + row] = (pp + ei * aq) * rden;
    }
    if (tid < D) zkey[(size_t)bh * D + tid] = zkf[tid];
}

template <int D, typename Tin>
hipError_t launch(const FwdArgs &a)
{
    const int BH = a.B * a.H;
    hipLaunchKernelGGL((vla_decode<D, Tin>), dim3(BH), dim3(1024), 0, a.stream, (const Tin *)a.q,
                       (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u, a.eps, a.S_out,
                       a.A_out, a.zk_out, a.o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const FwdArgs &a)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch<64, uint16_t>(a) : launch<64, float>(a);
    case 96: return bf ? launch<96, uint16_t>(a) : launch<96, float>(a);
    case 128: return bf ? launch<128, uint16_t>(a) : launch<128, float>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
