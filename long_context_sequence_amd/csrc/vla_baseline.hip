// vla_baseline.hip -- the two baselines on the same inputs, d_h in {64, 96, 128}:
//
//   linear attention  the recurrent form of the "Linear Attention" wiki article:
//                     S <- S + v phi(k)',  z <- z + phi(k),
//                     o = S phi(q) / (phi(q)' z)   (no floor; phi > 0)
//   DeltaNet          section 3.5 of "Variational Linear Attention": alpha^
//                     replaced by a scalar gate beta on the unit key and no A,
//                     i.e. the delta rule of the kexue.fm article's "linear
//                     version" with eta = beta:
//                     e = v - S k^,  S <- S + beta e k^',  o by Eq. (11).
//
// Both are the memory chain of the VLA forward (E = (V - S K^)(I + N)^-1,
// S <- S + E Alpha^', o = (S Phi + E P) / den) with other per-chunk records:
//   DeltaNet          Alpha^ = beta K^, N = (beta K^'K^) strictly upper;
//   linear attention  Alpha^ = Phi(K), K^ = 0 (so N = 0 and E = V).
// So a baseline is two small kernels that write those records (no chain: every
// chunk is independent once the key sum at its start is known) and the
// forward's memory-pass kernel.
//
//   keysum   per (head, group of GC chunks): sum of phi(k) over the group (fp64).
//   prep     per (head, group): the key sum at the group start (zkey_0 plus the
//            earlier groups' sums, fp64), then chunk pairs in order: staging,
//            key-sum prefix and 1/den per token, and the C x C factors on the
//            matrix cores (N, P, and for a pair the cross factors Alpha^_a'K^_b,
//            stored solved by chunk b's triangle as the forward's records hold
//            it, and Alpha^_a'Phi_b), (I + N)^-1 by back substitution.
//   memory   the forward's memory pass on those records.
#include "vla_chunk_parts.h"
#include "vla_record.h"

namespace vla {
namespace {

using namespace chunk;
using rec::CH;
using rec::Rec;

constexpr int GC = 16;   // chunks per group (even: pairs never straddle groups)

template <int D, typename Tin>
__global__ void __launch_bounds__(256)
vla_bl_keysum(const Tin *__restrict__ k, int T, int NG, double *__restrict__ gsum)
{
    constexpr int CPT = D / 16;
    __shared__ double red[16][D];
    const int bh = blockIdx.x / NG, gi = blockIdx.x % NG;
    const int tid = threadIdx.x, tl = tid >> 4, cc = tid & 15;
    const int t0 = gi * GC * CH, t1 = min(T, t0 + GC * CH);
    const Tin *kh = k + (size_t)bh * T * D;
    double acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[i] = 0.0;
    for (int t = t0 + tl; t < t1; t += 16) {
        RawVec<Tin, CPT> r;
        r.load(kh + (size_t)t * D + cc * CPT);
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc[i] += (double)phi_fast(r.get(i));
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) red[tl][cc * CPT + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
        for (int r = 0; r < 16; ++r) s += red[r][tid];
        gsum[((size_t)bh * NG + gi) * D + tid] = s;
    }
}

template <int D>
struct BLds {
    static constexpr int C = CH, LD = D + 4, LT = C + 4;
    float al[2][C * LD];     // Alpha^ [token][key] of the pair's two chunks
    float kh[2][C * LD];     // k^ (DeltaNet)
    float ph[2][C * LD];     // phi(q)
    float zk[2][C * LD];     // phi(k), then the inclusive key sum
    float nt[4][C * LT];     // per wave: scratch for (I + N)^-1
};

// X = Al' Y over all keys (C x C, accumulator layout: lane 16g + n, register r
// holds X[4g + r][n]); Al, Y token-major in LDS with row stride LD.
template <int D>
__device__ __forceinline__ f4 ctc(const float *al, const float *y, int g, int n)
{
    constexpr int LD = D + 4;
    f4 x = {0.f, 0.f, 0.f, 0.f};
    sfor<D / 16>([&](auto b) {
        x = mma4(ld4(&al[n * LD + 16 * b + 4 * g]), ld4(&y[n * LD + 16 * b + 4 * g]), x);
    });
    return x;
}

// (I + N)^-1 from N (accumulator layout; only c < t is used) to the record's
// transposed layout at tt, by back substitution four columns at a time (one
// wave, its scratch nt).
__device__ __forceinline__ void tinv_out(f4 nx, int g, int n, float *nt, float *tt, float (&X)[4])
{
    constexpr int LT = CH + 4;
    sfor<4>([&](auto r) { nt[(4 * g + r) * LT + n] = 4 * g + r < n ? -nx[int(r)] : 0.f; });
    wave_lds_order();
    float NNr[16];
    sfor<4>([&](auto q4) {
        const f4 a = ld4(&nt[n * LT + 4 * q4]);
        sfor<4>([&](auto r) { NNr[4 * q4 + r] = a[int(r)]; });
    });
    sfor<4>([&](auto c) { X[c] = n == 4 * c + g ? 1.f : 0.f; });
    asm volatile(VLA_TINV_BLOCK
                 : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3])
                 : "v"(NNr[1]), "v"(NNr[2]), "v"(NNr[3]), "v"(NNr[4]), "v"(NNr[5]),
                   "v"(NNr[6]), "v"(NNr[7]), "v"(NNr[8]), "v"(NNr[9]), "v"(NNr[10]),
                   "v"(NNr[11]), "v"(NNr[12]), "v"(NNr[13]), "v"(NNr[14]), "v"(NNr[15]));
    sfor<4>([&](auto c) { tt[swz16(4 * c + g, n >> 2) + (n & 3)] = X[c]; });
}

// Workgroup (head, group of GC chunks), 4 waves.  DELTA selects DeltaNet,
// otherwise linear attention.
template <int D, typename Tin, bool DELTA>
__global__ void __launch_bounds__(256)
vla_bl_prep(const Tin *__restrict__ q, const Tin *__restrict__ k, int T, int NG, float beta,
            float eps, const float *zk0, const double *__restrict__ gsum, float *__restrict__ rec,
            float *zk_out)
{
    using R = Rec<D>;
    constexpr int CPT = D / 16, LD = D + 4, RS = R::SIZE;
    __shared__ __align__(16) BLds<D> L;
    const int bh = blockIdx.x / NG, gi = blockIdx.x % NG;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tl = tid >> 4, cc = tid & 15;   // staging: token tl, columns [cc CPT, +CPT)
    const int NC = (T + CH - 1) / CH;
    const int c0 = gi * GC, c1 = min(NC, c0 + GC);
    const size_t tok0 = (size_t)bh * T;
    float *rh = rec + (size_t)bh * NC * RS;

    // key sum at the group start, one column per thread (Kahan-compensated
    // running sum inside the group)
    float zrun = 0.f, zcmp = 0.f;
    if (tid < D) {
        double z = zk0 ? (double)zk0[bh * D + tid] : 0.0;
        for (int i = 0; i < gi; ++i) z += gsum[((size_t)bh * NG + i) * D + tid];
        zrun = (float)z;
    }

    // chunk c into LDS slot s (and its k^, phi(q) rows into the record)
    auto stage = [&](int c, int s) {
        const int t = c * CH + tl;
        const bool ok = t < T;
        RawVec<Tin, CPT> rq, rk;
        const size_t off = (tok0 + (size_t)(ok ? t : T - 1)) * D + (size_t)cc * CPT;
        rq.load(q + off);
        rk.load(k + off);
        float ik = 0.f;
        if constexpr (DELTA) {
            float pk = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) pk = fmaf(rk.get(i), rk.get(i), pk);
            const float nk = sum_row16(pk);
            ik = ok && nk > 0.f ? rsqrtf(nk) : 0.f;
        }
        float *rkh = rh + (size_t)c * RS + R::KH, *rph = rh + (size_t)c * RS + R::PH;
        const int e0 = tl * LD + cc * CPT;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int col = cc * CPT + i;
            const float pq = phi_fast(rq.get(i));
            const float pk = ok ? phi_fast(rk.get(i)) : 0.f;
            const float kv = rk.get(i) * ik;   // 0 unless DeltaNet
            L.ph[s][e0 + i] = pq;
            L.zk[s][e0 + i] = pk;
            L.kh[s][e0 + i] = kv;
            L.al[s][e0 + i] = DELTA ? beta * kv : pk;
            rkh[swzd<D>(tl, col >> 2) + (col & 3)] = kv;
            rph[swzd<D>(tl, col >> 2) + (col & 3)] = pq;
        }
    };
    // key-sum prefix of slot s (one column per thread), then 1/den per token
    auto keys_den = [&](int c, int s) {
        if (tid < D) {
            float loc = 0.f;
#pragma unroll
            for (int tt = 0; tt < CH; ++tt) {
                loc += L.zk[s][tt * LD + tid];
                L.zk[s][tt * LD + tid] = zrun + loc;
            }
            const float y = loc - zcmp, ts = zrun + y;
            zcmp = (ts - zrun) - y;
            zrun = ts;
        }
        __syncthreads();
        const int e0 = tl * LD + cc * CPT;
        float pd = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) pd = fmaf(L.ph[s][e0 + i], L.zk[s][e0 + i], pd);
        pd = sum_row16(pd);
        if (cc == 0) rh[(size_t)c * RS + R::RD + tl] = DELTA ? 1.f / fmaxf(pd, eps) : 1.f / pd;
    };
    // Alpha^ [key][token] of slot s into chunk c's record (own key blocks)
    auto alpha_out = [&](int c, int s) {
        for (int b = w; b < D / 16; b += 4) {
            f4 a;
            sfor<4>([&](auto r) { a[int(r)] = L.al[s][(4 * g + r) * LD + 16 * b + n]; });
            st4(&rh[(size_t)c * RS + R::AH + swz16(16 * b + n, g)], a);
        }
    };
    const f4 eye4 = {n == 4 * g ? 1.f : 0.f, n == 4 * g + 1 ? 1.f : 0.f, n == 4 * g + 2 ? 1.f : 0.f,
                     n == 4 * g + 3 ? 1.f : 0.f};
    // the C x C factors of chunk c in slot s: (I + N)^-1 (wave wt) and P (wave wp);
    // with ydst (DeltaNet, chunk b of a pair), wave wt also leaves the pair's key
    // cross factor solved by chunk b's triangle (its scratch and wave wt + 1's)
    auto factors = [&](int c, int s, int wt, int wp, float *ydst = nullptr) {
        float *rc = rh + (size_t)c * RS;
        if (w == wt) {
            if constexpr (DELTA) {
                float X[4];
                tinv_out(ctc<D>(L.al[s], L.kh[s], g, n), g, n, L.nt[w], rc + R::TT, X);
                if (ydst) solved_cross(ctc<D>(L.al[0], L.kh[1], g, n), X, g, n, L.nt[w], L.nt[w + 1], ydst);
            } else {
                st4(&rc[R::TT + swz16(n, g)], eye4);
            }
        }
        if (w == wp) {
            f4 p = ctc<D>(L.al[s], L.ph[s], g, n);
            sfor<4>([&](auto r) { p[int(r)] = 4 * g + r <= n ? p[int(r)] : 0.f; });
            st4(&rc[R::PT + swz16(n, g)], p);
        }
    };

    for (int c = c0; c < c1; c += 2) {
        const bool pair = c + 1 < c1;
        stage(c, 0);
        if (pair) stage(c + 1, 1);
        __syncthreads();
        keys_den(c, 0);
        if (pair) keys_den(c + 1, 1);
        alpha_out(c, 0);
        if (pair) alpha_out(c + 1, 1);
        factors(c, 0, 0, 1);
        if (pair) {
            float *rc = rh + (size_t)c * RS;
            factors(c + 1, 1, 2, 3, rc + R::QK);
            if (!DELTA && w == 0) st4(&rc[R::QK + swz16(n, g)], f4{0.f, 0.f, 0.f, 0.f});   // unused
            if (w == 1) st4(&rc[R::QP + swz16(n, g)], ctc<D>(L.al[0], L.ph[1], g, n));
        }
        __syncthreads();
    }
    if (gi == NG - 1 && zk_out && tid < D) zk_out[bh * D + tid] = zrun;
}

struct BPlan {
    int NC = 0, NG = 0;
    size_t rec = 0, gsum = 0, bytes = 0;
};

BPlan make_bplan(int BH, int T, int D)
{
    BPlan p;
    p.NC = (T + CH - 1) / CH;
    p.NG = (p.NC + GC - 1) / GC;
    const size_t rs = 48 * (size_t)D + 4 * CH * CH + CH;   // Rec<D>::SIZE
    p.rec = 0;
    size_t off = (BH * (size_t)p.NC * rs * sizeof(float) + 255) & ~(size_t)255;
    p.gsum = off;
    off += ((size_t)BH * p.NG * D * sizeof(double) + 255) & ~(size_t)255;
    p.bytes = p.NC > 0 ? off : 0;
    return p;
}

template <int D, typename Tin>
hipError_t launch_bl(const FwdArgs &a, bool delta, float beta)
{
    const int BH = a.B * a.H;
    const BPlan p = make_bplan(BH, a.T, D);
    char *ws = static_cast<char *>(a.ws);
    float *rec = reinterpret_cast<float *>(ws + p.rec);
    double *gsum = reinterpret_cast<double *>(ws + p.gsum);
    const Tin *q = (const Tin *)a.q, *k = (const Tin *)a.k;
    hipLaunchKernelGGL((vla_bl_keysum<D, Tin>), dim3(BH * p.NG), dim3(256), 0, a.stream, k, a.T,
                       p.NG, gsum);
    if (delta)
        hipLaunchKernelGGL((vla_bl_prep<D, Tin, true>), dim3(BH * p.NG), dim3(256), 0, a.stream,
                           q, k, a.T, p.NG, beta, a.eps, a.zk0, gsum, rec, a.zk_out);
    else
        hipLaunchKernelGGL((vla_bl_prep<D, Tin, false>), dim3(BH * p.NG), dim3(256), 0, a.stream,
                           q, k, a.T, p.NG, beta, a.eps, a.zk0, gsum, rec, a.zk_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_memory_pass(a, rec, !delta);
}

}  // namespace

size_t baseline_workspace_bytes(int BH, int T, int d) { return make_bplan(BH, T, d).bytes; }

hipError_t launch_baseline(const FwdArgs &a, bool delta, float beta)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch_bl<64, uint16_t>(a, delta, beta) : launch_bl<64, float>(a, delta, beta);
    case 96: return bf ? launch_bl<96, uint16_t>(a, delta, beta) : launch_bl<96, float>(a, delta, beta);
    case 128: return bf ? launch_bl<128, uint16_t>(a, delta, beta) : launch_bl<128, float>(a, delta, beta);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
