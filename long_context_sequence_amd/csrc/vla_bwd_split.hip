// vla_bwd_split.hip -- the reverse sweep of the gradients for d_h in {64, 96, 128}
// as two chains running side by side, each with one barrier per token.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9)-(11); the pages print no backward, so this is the chain rule through
// those equations in reverse order (the conventions are stated at vla_backward
// in include/vla.h).  The forward's two chains meet only at alpha^ (Eq. (10)).
// In reverse the adjoint of S (dS) never needs the adjoint of A, and the
// adjoint of A needs from the memory side only g_alpha = dL/dalpha^_t.
//
// The adjoint of A in conjugated form.  With z = A_{t-1} u^ and delta = 1 +
// u^'z, Eq. (9) reads A_t = (I - z u^'/delta) A_{t-1}, so the map that carries
// the adjoint Sigma (= dA + dA') from A_t back to A_{t-1} is
// M_t = I - u^ z'/delta = A_{t-1}^-1 A_t: Sigma_{t-1} = M_t Sigma'_t M_t', where
// Sigma'_t = Sigma_t + gy k^' + k^ gy' adds the gate's share (gy = dL/dy_t for
// y_t = A_t k^_t).  In the frame Q_t = A_t Sigma_t A_t the transport cancels:
//     Q_{t-1} = Q_t + p y' + y p',   p = A_t gy,
// and the gradient with respect to u^_t, which the chain rule assembles from
// Sigma'_t z, z'Sigma'_t z and A_{t-1}, collapses to -Q_{t-1} u^_t (checked
// in fp64 against the per-token recurrence, to rounding).  At the end
// Sigma_0 = A_0^-1 Q_0 A_0^-1.  So the penalty side is an accumulation with
// plain fp32 multiply-adds (the conjugated quantities carry no cancellation;
// an fp32 model of this gives 2e-6 relative error in dL/du at T = 4096, where
// an fp32 Sigma gave 7e-3) next to A_t itself (A_{t-1} = A_t + z z'/delta).
//
// Two workgroups per head:
//
//   memory     dS and dS' (row slices), per token t from T - 1 down:
//              dS += g phi(q)'/den (g = dL/do_t); ge = dS alpha^ (= dL/dv_t),
//              g_alpha = dS'e; dS -= ge k^'.  It writes dv and g_alpha and
//              publishes how far it is.
//   penalty    A, Q and S' (row slices), a few tokens behind: p = A_t gy,
//              Q u^, S_t'g, S_t'ge; Q += p y' + y p'; A_{t-1} = A_t + z z'/delta;
//              S_{t-1}' = S_t' - alpha^ e'.  From these it writes du, dq and dk
//              (both chains' shares) and the key-sum adjoint.
//
// Layout: (D / RB) * TPR row threads, thread (rows i0, i0 + 1, columns [c0,
// c0 + EPT)) holding that block of each d x d matrix (row products are DPP
// sums over TPR adjacent lanes; a token vector's entries are read from LDS
// once for the block's two rows, which halves the LDS traffic of one row per
// thread, the bound of this sweep), and two service waves (SplitCfg): the copy
// wave brings the token vectors into LDS (direct copies LA tokens ahead into
// rings of RING slots, transforms two tokens ahead into working slots), the
// gradient wave forms each token's gradients from the row results.  Per token one barrier:
// the row products of step 1 of token t go through LDS, then step 2 of token t
// and step 1 of token t - 1 (thread-local dependencies only) share the next
// interval, while the gradient wave forms token t + 1's gradients (row results
// in three LDS slots, transformed vectors in four: the gradient's token, the two
// steps' tokens and the one being transformed).
#include "vla_bwd.h"
#include "vla_chunk_parts.h"
#include "vla_record.h"
#include "vla_reduce.h"
#include "vla_sweep.h"

namespace vla {
namespace {

using namespace chunk;

template <int D>
struct SplitCfg {
    // eight threads per pair of rows, then the two service waves
    static constexpr int TPR = 8, EPT = D / TPR, RB = 2, NR = D / RB * TPR, NWR = NR / 64;
    static constexpr int NT = NR + 128, WCOPY = NWR, WGRAD = NWR + 1;
    static constexpr int NV = (D + 63) / 64;
    static constexpr int W = 64 * NV;   // ring row: what NV wave-wide 4-byte copies fill
    static_assert(EPT % 4 == 0 && NR % 64 == 0 && NT <= 1024, "row blocks of whole granules");
};

// Token vectors reach LDS by direct copies (4 bytes per lane, 256 bytes per
// copy), LA tokens ahead of the interval whose step 2 they feed,
// into rings of RING slots.  At the end of each interval the copy wave waits
// for its copies of the token three ahead (the next interval transforms it and
// the one after uses it), so LA - 3 tokens of copies stay in flight: as many as
// the wait count can express (63 copies) for a chain that issues cpt copies
// per token, at most LA_MAX.  (A copy takes a couple of microseconds to land,
// several intervals.)
#ifndef VLA_BWD_LA_MAX
#define VLA_BWD_LA_MAX 12
#endif
constexpr int LA_MAX = VLA_BWD_LA_MAX;
// d = 128 keeps six tokens in eight slots (with the larger rings, LDS offsets
// past 64 KB, its loop runs out of registers)
template <int D> constexpr int RING = D == 128 ? 8 : 16;
constexpr int lookahead(int cpt, int d)
{
    const int la = 3 + 63 / cpt < LA_MAX ? 3 + 63 / cpt : LA_MAX;
    return d == 128 && la > 6 ? 6 : la;
}
static_assert(LA_MAX + 2 <= RING<64>, "tokens in use at once: t + 1 down to t - LA");

// The memory workgroup publishes its progress every PUB tokens; a waiting wave
// polls at most SPIN_LIMIT times (each poll sleeps 256 cycles; about a second
// in all).
constexpr int PUB = 16, SPIN_LIMIT = 1 << 20;

// element j of a raw ring row: fp32 as stored, or bf16 (two per word)
template <typename Tin>
__device__ __forceinline__ float raw_get(const float *row, int j)
{
    if constexpr (sizeof(Tin) == 4) {
        return row[j];
    } else {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(row)[j] << 16);
    }
}

// One stream of per-token vectors: token x's bytes at base + x * stride (+ 256
// per copy) into ring row x mod RING, NC copies per token.  The copy wave's
// wait counts are the exact number of copies per token: padding a stream with
// repeated copies would not do, since the compiler merges identical copies.
template <int NC, int R>
struct Stream {
    Buf buf;
    unsigned stride;
    float *ring;
    int row;   // ring row width (floats)
    __device__ __forceinline__ void issue(int x, int lane) const
    {
        float *dst = ring + (x & (R - 1)) * row;
        const unsigned vo = (unsigned)x * stride + 4u * (unsigned)lane;
        sfor<NC>([&](auto i) { buf.lds4(dst + 64 * i, vo + 256u * i); });
    }
};

// copies per token: a d-vector of floats, of inputs, the 8 scalars
template <int D> constexpr int NCF = (D + 63) / 64;
template <int D, typename Tin> constexpr int NCI = (D * (int)sizeof(Tin) + 255) / 256;

template <int D>
__device__ __forceinline__ Stream<NCF<D>, RING<D>> fstream(const float *base, unsigned bytes,
                                                           unsigned stride, float *ring)
{
    return Stream<NCF<D>, RING<D>>{Buf(base, bytes), stride, ring, SplitCfg<D>::W};
}

template <int D, typename Tin>
__device__ __forceinline__ Stream<NCI<D, Tin>, RING<D>> istream(const Tin *base, int T, float *ring)
{
    return Stream<NCI<D, Tin>, RING<D>>{Buf(base, (unsigned)(T * D * sizeof(Tin))),
                                        D * (unsigned)sizeof(Tin), ring, SplitCfg<D>::W};
}

template <int D>
__device__ __forceinline__ Stream<1, RING<D>> scstream(const float *base, unsigned bytes, unsigned stride,
                                                       float *ring)
{
    return Stream<1, RING<D>>{Buf(base, bytes), stride, ring, 64};
}

// ------------------------------------------------------------- memory chain
template <int D>
struct SLds {
    static constexpr int W = SplitCfg<D>::W, R = RING<D>;
    float g[R][W], al[R][W], e[R][W], rq[R][W], rk[R][W];
    float sc[R][64];
    float pq[4][D], kh[4][D];
    float r1[3][2][D];   // ge, g_alpha
};

template <int D, typename Tin>
__device__ __forceinline__ void
bwd_s(SLds<D> &L, int bh, const Tin *__restrict__ q, const Tin *__restrict__ k, int T, float eps,
      const float *__restrict__ dO, const float *dS_T, float *__restrict__ dv, float *dS0,
      const float *__restrict__ rec, float *__restrict__ galpha, int *progress)
{
    using Cf = SplitCfg<D>;
    using K = rec::Keep<D>;
    constexpr int TPR = Cf::TPR, EPT = Cf::EPT, RB = Cf::RB, NV = Cf::NV, RS = K::RS;
    // streams: dL/do, alpha^, e (floats), q, k (inputs), the scalars
    constexpr int CPT = 3 * NCF<D> + 2 * NCI<D, Tin> + 1;   // copies per token
    constexpr int LA = lookahead(CPT, D);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool rows = w < Cf::NWR;
    const int i0 = rows ? tid / TPR * RB : 0, c0 = (tid % TPR) * EPT;
    const bool leader = rows && tid % TPR == 0;
    const size_t DD = (size_t)D * D, tok0 = (size_t)bh * T;
    const float *rh = rec + tok0 * RS;

    // dS and dS' (row blocks) from dL/dS_T
    float gS[RB][EPT], gSt[RB][EPT];
    sfor<RB>([&](auto h) {
        sfor<EPT>([&](auto e) {
            const size_t off = bh * DD + (size_t)(i0 + h) * D + c0 + e;
            const size_t toff = bh * DD + (size_t)(c0 + e) * D + i0 + h;
            gS[h][e] = rows && dS_T ? dS_T[off] : 0.f;
            gSt[h][e] = rows && dS_T ? dS_T[toff] : 0.f;
        });
    });

    const unsigned recb = (unsigned)(T * RS * 4);
    const auto s_g = fstream<D>(dO + tok0 * D, (unsigned)(T * D * 4), D * 4u, &L.g[0][0]);
    const auto s_al = fstream<D>(rh + K::AL, recb - K::AL * 4u, RS * 4u, &L.al[0][0]);
    const auto s_e = fstream<D>(rh + K::E, recb - K::E * 4u, RS * 4u, &L.e[0][0]);
    const auto s_q = istream<D, Tin>(q + tok0 * D, T, &L.rq[0][0]);
    const auto s_k = istream<D, Tin>(k + tok0 * D, T, &L.rk[0][0]);
    const auto s_sc = scstream<D>(rh + K::SC, recb - K::SC * 4u, RS * 4u, &L.sc[0][0]);
    auto issue = [&](int x) {
        if (w == Cf::WCOPY) {
            s_g.issue(x, lane);
            s_al.issue(x, lane);
            s_e.issue(x, lane);
            s_q.issue(x, lane);
            s_k.issue(x, lane);
            s_sc.issue(x, lane);
        }
    };
    // q: phi(q); k: k^ = k / |k| (two tokens ahead)
    auto transform = [&](int x) {
        if (w != Cf::WCOPY) return;
        const int rs = x & (RING<D> - 1), ws = x & 3;
        const float ik = L.sc[rs][3];
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                L.pq[ws][j] = phi_fast(raw_get<Tin>(L.rq[rs], j));
                L.kh[ws][j] = raw_get<Tin>(L.rk[rs], j) * ik;
            }
        });
    };

    // step 1: the readout's share of dS, then dS alpha^ and dS'e
    auto step1 = [&](int t) {
        const int v = t & 3, r = t & (RING<D> - 1), s = t % 3;
        const float iden = 1.f / fmaxf(L.sc[r][2], eps);
        float gi[RB], pqi[RB], pge[RB], pga[RB];
        sfor<RB>([&](auto h) {
            gi[h] = L.g[r][i0 + h] * iden;
            pqi[h] = L.pq[v][i0 + h] * iden;
            pge[h] = pga[h] = 0.f;
        });
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float pqj = L.pq[v][j], gj = L.g[r][j], alj = L.al[r][j], ej = L.e[r][j];
            sfor<RB>([&](auto h) {
                gS[h][e] = fmaf(gi[h], pqj, gS[h][e]);
                gSt[h][e] = fmaf(pqi[h], gj, gSt[h][e]);
                pge[h] = fmaf(gS[h][e], alj, pge[h]);
                pga[h] = fmaf(gSt[h][e], ej, pga[h]);
            });
        });
        sfor<RB>([&](auto h) {
            pge[h] = row_sum<TPR>(pge[h]);
            pga[h] = row_sum<TPR>(pga[h]);
        });
        if (leader) {
            sfor<RB>([&](auto h) {
                L.r1[s][0][i0 + h] = pge[h];
                L.r1[s][1][i0 + h] = pga[h];
            });
        }
    };
    // step 2: dS -= ge k^'
    auto step2 = [&](int t) {
        const int v = t & 3, s = t % 3;
        float khi[RB], gei[RB];
        sfor<RB>([&](auto h) {
            khi[h] = L.kh[v][i0 + h];
            gei[h] = L.r1[s][0][i0 + h];
        });
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float khj = L.kh[v][j], gej = L.r1[s][0][j];
            sfor<RB>([&](auto h) {
                gS[h][e] = fmaf(-gei[h], khj, gS[h][e]);
                gSt[h][e] = fmaf(-khi[h], gej, gSt[h][e]);
            });
        });
    };
    // gradient wave: token t's dv and g_alpha
    auto grads = [&](int t) {
        const int s = t % 3;
        const size_t o = (tok0 + t) * D;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                dv[o + j] = L.r1[s][0][j];
                galpha[o + j] = L.r1[s][1][j];
            }
        });
    };
    // gradient wave: tokens >= t are out (dv and g_alpha written): publish t to
    // the penalty workgroup
    auto publish = [&](int t) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) __hip_atomic_store(progress + bh, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    for (int i = 0; i < LA && i < T; ++i) issue(T - 1 - i);
    // drain every load so far as a wait the compiler sees (otherwise it waits
    // for every load in flight at the top of each iteration)
    vmem_drain();
    __syncthreads();
    if (T > 0) transform(T - 1);
    if (T > 1) transform(T - 2);
    __syncthreads();
    if (rows && T > 0) step1(T - 1);
    lds_barrier();
    for (int t = T - 1; t >= 0; --t) {
        if (t >= LA) issue(t - LA);
        if (t >= 2) transform(t - 2);
        if (w == Cf::WGRAD && t + 1 < T) {
            grads(t + 1);
            if ((t + 1) % PUB == 0) publish(t + 1);
        }
        if (rows) {
            step2(t);
            if (t >= 1) step1(t - 1);
        }
        if (w == Cf::WCOPY) {   // this wave's copies of token t - 3 done
            if (t >= LA) vm_wait<(LA - 3) * CPT>();
            else vmem_drain();
        }
        lds_barrier();
    }
    if (w == Cf::WGRAD && T > 0) {
        grads(0);
        publish(0);
    }

    if (rows && dS0) {
        sfor<RB>([&](auto h) {
            float *dst = dS0 + bh * DD + (size_t)(i0 + h) * D + c0;
            sfor<EPT / 4>([&](auto q) {
                st4(dst + 4 * q, f4{gS[h][4 * q], gS[h][4 * q + 1], gS[h][4 * q + 2], gS[h][4 * q + 3]});
            });
        });
    }
}

// ------------------------------------------------------------ penalty chain
template <int D>
struct ALds {
    static constexpr int W = SplitCfg<D>::W, R = RING<D>;
    float ga[R][W], gv[R][W], g[R][W], al[R][W], z[R][W], e[R][W], zt[R][W];
    float rq[R][W], rk[R][W], ru[R][W];
    float sc[R][64];
    float gy[4][D], y[4][D], kh[4][D], uh[4][D], pq[4][D], dpq[4][D], dpk[4][D];
    float ts[4][4];       // per working slot: y'u^, e'ge, k^'alpha^
    float r1[3][4][D];    // A_t gy, Q_t u^, S_t'g, S_t'ge
    int lost;             // the copy wave gave up waiting
};

template <int D, typename Tin>
__device__ __forceinline__ void
bwd_a(ALds<D> &L, int bh, const Tin *__restrict__ q, const Tin *__restrict__ k,
      const Tin *__restrict__ u, int T, float lambda0, float eps, const float *__restrict__ S_T,
      const float *__restrict__ A_T, const float *__restrict__ dO, const float *dzk_T,
      float *__restrict__ dq, float *__restrict__ dk, const float *__restrict__ dv,
      float *__restrict__ du, bool qin, float *qb, float *dA0, bool a0given, float *dzk0,
      const float *__restrict__ rec, const float *__restrict__ galpha, const int *progress)
{
    using Cf = SplitCfg<D>;
    using K = rec::Keep<D>;
    constexpr int TPR = Cf::TPR, EPT = Cf::EPT, RB = Cf::RB, NV = Cf::NV, RS = K::RS;
    // streams: g_alpha, dL/dv, dL/do, alpha^, z, e, zkey_t (floats), q, k, u
    // (inputs), the scalars
    constexpr int CPT = 7 * NCF<D> + 3 * NCI<D, Tin> + 1;   // copies per token
    constexpr int LA = lookahead(CPT, D);
    static_assert((LA - 3) * CPT < 64, "wait count fits vmcnt");

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool rows = w < Cf::NWR;
    const int i0 = rows ? tid / TPR * RB : 0, c0 = (tid % TPR) * EPT;
    const bool leader = rows && tid % TPR == 0;
    const size_t DD = (size_t)D * D, tok0 = (size_t)bh * T;
    const float *rh = rec + tok0 * RS;

    // A_T, Q_T = A_T Sigma_T A_T (formed beforehand when dL/dA_T is given) and
    // S_T' (row blocks)
    float A[RB][EPT], Q[RB][EPT], St[RB][EPT];
    sfor<RB>([&](auto h) {
        sfor<EPT>([&](auto e) {
            const size_t off = bh * DD + (size_t)(i0 + h) * D + c0 + e;
            const size_t toff = bh * DD + (size_t)(c0 + e) * D + i0 + h;
            A[h][e] = rows ? A_T[off] : 0.f;
            Q[h][e] = rows && qin ? qb[off] : 0.f;
            St[h][e] = rows ? S_T[toff] : 0.f;
        });
    });
    float gzk[NV];   // gradient wave: the key-sum adjoint, entries lane + 64 c
    sfor<NV>([&](auto c) {
        const int j = lane + 64 * c;
        gzk[c] = dzk_T && j < D ? dzk_T[(size_t)bh * D + j] : 0.f;
    });

    const unsigned recb = (unsigned)(T * RS * 4), vb = (unsigned)(T * D * 4);
    const auto s_ga = fstream<D>(galpha + tok0 * D, vb, D * 4u, &L.ga[0][0]);
    const auto s_gv = fstream<D>(dv + tok0 * D, vb, D * 4u, &L.gv[0][0]);
    const auto s_g = fstream<D>(dO + tok0 * D, vb, D * 4u, &L.g[0][0]);
    const auto s_al = fstream<D>(rh + K::AL, recb - K::AL * 4u, RS * 4u, &L.al[0][0]);
    const auto s_z = fstream<D>(rh + K::Z, recb - K::Z * 4u, RS * 4u, &L.z[0][0]);
    const auto s_e = fstream<D>(rh + K::E, recb - K::E * 4u, RS * 4u, &L.e[0][0]);
    const auto s_zt = fstream<D>(rh + K::ZK, recb - K::ZK * 4u, RS * 4u, &L.zt[0][0]);
    const auto s_q = istream<D, Tin>(q + tok0 * D, T, &L.rq[0][0]);
    const auto s_k = istream<D, Tin>(k + tok0 * D, T, &L.rk[0][0]);
    const auto s_u = istream<D, Tin>(u + tok0 * D, T, &L.ru[0][0]);
    const auto s_sc = scstream<D>(rh + K::SC, recb - K::SC * 4u, RS * 4u, &L.sc[0][0]);

    // Tokens >= seen are out of the memory workgroup (its last published
    // value, read with acquire ordering).  A wait gives up after SPIN_LIMIT
    // polls (the memory workgroup, already running, publishes within
    // microseconds); from then on the wave waits no more and the head's
    // outputs are NaN, so a failure shows instead of hanging.
    int seen = T;
    bool lost = false;
    auto await = [&](int x) {
        for (int n = 0; seen > x && !lost; ++n) {
            seen = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(progress + bh, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT));
            if (seen > x) {
                if (n >= SPIN_LIMIT) lost = true;
                __builtin_amdgcn_s_sleep(4);
            }
        }
    };
    auto issue = [&](int x) {
        if (w == Cf::WCOPY) {
            await(x);   // g_alpha and dL/dv of token x must be out
            if (lost && lane == 0) L.lost = 1;
            s_ga.issue(x, lane);
            s_gv.issue(x, lane);
            s_g.issue(x, lane);
            s_al.issue(x, lane);
            s_z.issue(x, lane);
            s_e.issue(x, lane);
            s_zt.issue(x, lane);
            s_q.issue(x, lane);
            s_k.issue(x, lane);
            s_u.issue(x, lane);
            s_sc.issue(x, lane);
        }
    };
    // gy = (g_alpha - alpha^ (alpha^'g_alpha)) / |y|; y = A_t k^ = alpha^ |y|;
    // k^, u^; phi(q), phi'(q), phi'(k); the token's y'u^, e'ge, k^'alpha^
    auto transform = [&](int x) {
        if (w != Cf::WCOPY) return;
        const int rs = x & (RING<D> - 1), ws = x & 3;
        const float iy = L.sc[rs][1], ik = L.sc[rs][3], iu = L.sc[rs][4];
        const float ny = iy > 0.f ? 1.f / iy : 0.f;   // |y| (0 with a zero key)
        float aga = 0.f, yu = 0.f, ege = 0.f, kal = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const float al = L.al[rs][j];
                aga = fmaf(al, L.ga[rs][j], aga);
                yu = fmaf(al * ny, raw_get<Tin>(L.ru[rs], j) * iu, yu);
                ege = fmaf(L.e[rs][j], L.gv[rs][j], ege);
                kal = fmaf(raw_get<Tin>(L.rk[rs], j) * ik, al, kal);
            }
        });
        aga = wave_sum(aga);
        yu = wave_sum(yu);
        ege = wave_sum(ege);
        kal = wave_sum(kal);
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const float al = L.al[rs][j], xq = raw_get<Tin>(L.rq[rs], j), xk = raw_get<Tin>(L.rk[rs], j);
                L.gy[ws][j] = (L.ga[rs][j] - al * aga) * iy;
                L.y[ws][j] = al * ny;
                L.kh[ws][j] = xk * ik;
                L.uh[ws][j] = raw_get<Tin>(L.ru[rs], j) * iu;
                L.pq[ws][j] = phi_fast(xq);
                L.dpq[ws][j] = dphi(xq);
                L.dpk[ws][j] = dphi(xk);
            }
        });
        if (lane == 0) {
            L.ts[ws][0] = yu;
            L.ts[ws][1] = ege;
            L.ts[ws][2] = kal;
        }
    };

    // step 1: A_t gy, Q_t u^, S_t'g, S_t'ge
    auto step1 = [&](int t) {
        const int v = t & 3, r = t & (RING<D> - 1), s = t % 3;
        float pr[4][RB];
        sfor<4>([&](auto c) { sfor<RB>([&](auto h) { pr[c][h] = 0.f; }); });
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float gyj = L.gy[v][j], uhj = L.uh[v][j], gj = L.g[r][j], gvj = L.gv[r][j];
            sfor<RB>([&](auto h) {
                pr[0][h] = fmaf(A[h][e], gyj, pr[0][h]);
                pr[1][h] = fmaf(Q[h][e], uhj, pr[1][h]);
                pr[2][h] = fmaf(St[h][e], gj, pr[2][h]);
                pr[3][h] = fmaf(St[h][e], gvj, pr[3][h]);
            });
        });
        sfor<4>([&](auto c) { sfor<RB>([&](auto h) { pr[c][h] = row_sum<TPR>(pr[c][h]); }); });
        if (leader) {
            sfor<4>([&](auto c) { sfor<RB>([&](auto h) { L.r1[s][c][i0 + h] = pr[c][h]; }); });
        }
    };
    // step 2: Q += p y' + y p'; A_{t-1} = A_t + z z'/delta; S_{t-1}' = S_t' - alpha^ e'
    auto step2 = [&](int t) {
        const int v = t & 3, r = t & (RING<D> - 1), s = t % 3;
        const float id = 1.f / L.sc[r][0];
        float pi[RB], yi[RB], zi[RB], ali[RB];
        sfor<RB>([&](auto h) {
            pi[h] = L.r1[s][0][i0 + h];
            yi[h] = L.y[v][i0 + h];
            zi[h] = L.z[r][i0 + h];
            ali[h] = L.al[r][i0 + h];
        });
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float yj = L.y[v][j], pj = L.r1[s][0][j], zj = L.z[r][j], ej = L.e[r][j];
            sfor<RB>([&](auto h) {
                Q[h][e] = fmaf(pi[h], yj, Q[h][e]);
                Q[h][e] = fmaf(yi[h], pj, Q[h][e]);
                A[h][e] = fmaf(zi[h] * zj, id, A[h][e]);
                St[h][e] = fmaf(-ali[h], ej, St[h][e]);
            });
        });
    };
    // gradient wave: token t's du, dq and dk (both chains' shares).  With
    // p = A_t gy, w = Q_{t-1} u^ = Q_t u^ + p (y'u^) + y (p'u^) and
    // gkh = alpha^ (e'ge) - S_t'ge + p, every reduction it needs is one of
    // p'u^, c1'phi(q), k^'c2, k^'p, u^'Q_t u^ (one round) or a token scalar:
    //     k^'gkh = (e'ge)(k^'alpha^) - k^'c2 + k^'p,  u^'w = u^'Q_t u^ + 2 (y'u^)(p'u^)
    auto grads = [&](int t) {
        const int v = t & 3, r = t & (RING<D> - 1), s = t % 3;
        const float dn = L.sc[r][2], iden = 1.f / fmaxf(dn, eps), ik = L.sc[r][3], iu = L.sc[r][4];
        const float yu = L.ts[v][0], ege = L.ts[v][1], kal = L.ts[v][2];
        float s1 = 0.f, a1 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const float p = L.r1[s][0][j], uhj = L.uh[v][j], khj = L.kh[v][j];
                s1 = fmaf(p, uhj, s1);                      // p'u^
                a1 = fmaf(L.r1[s][2][j], L.pq[v][j], a1);   // g'S_t phi(q)
                b1 = fmaf(khj, L.r1[s][3][j], b1);          // k^'S_t'ge
                b2 = fmaf(khj, p, b2);                      // k^'p
                b3 = fmaf(uhj, L.r1[s][1][j], b3);          // u^'Q_t u^
            }
        });
        s1 = wave_sum(s1);
        a1 = wave_sum(a1);
        b1 = wave_sum(b1);
        b2 = wave_sum(b2);
        b3 = wave_sum(b3);
        const float gden = dn >= eps ? -a1 * iden * iden : 0.f;
        const float a3 = fmaf(ege, kal, b2 - b1), a4 = fmaf(2.f * yu, s1, b3);
        const float bad = L.lost ? __builtin_nanf("") : 0.f;
        const size_t o = (tok0 + t) * D;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const float p = L.r1[s][0][j], khj = L.kh[v][j], uhj = L.uh[v][j];
                const float wq = fmaf(L.y[v][j], s1, fmaf(p, yu, L.r1[s][1][j]));
                const float gkh = fmaf(L.al[r][j], ege, p - L.r1[s][3][j]);
                const float gpq = fmaf(L.r1[s][2][j], iden, gden * L.zt[r][j]);
                gzk[c] = fmaf(gden, L.pq[v][j], gzk[c]);
                dq[o + j] = gpq * L.dpq[v][j] + bad;
                dk[o + j] = fmaf(ik, gkh - khj * a3, gzk[c] * L.dpk[v][j]) + bad;
                du[o + j] = -iu * (wq - uhj * a4) + bad;
            }
        });
    };

    if (tid == 0) L.lost = 0;
    __syncthreads();
    for (int i = 0; i < LA && i < T; ++i) issue(T - 1 - i);
    vmem_drain();
    __syncthreads();
    if (T > 0) transform(T - 1);
    if (T > 1) transform(T - 2);
    __syncthreads();
    if (rows && T > 0) step1(T - 1);
    lds_barrier();
    for (int t = T - 1; t >= 0; --t) {
        if (t >= LA) issue(t - LA);
        if (t >= 2) transform(t - 2);
        if (w == Cf::WGRAD && t + 1 < T) grads(t + 1);
        if (rows) {
            step2(t);
            if (t >= 1) step1(t - 1);
        }
        if (w == Cf::WCOPY) {
            if (t >= LA) vm_wait<(LA - 3) * CPT>();
            else vmem_drain();
        }
        lds_barrier();
    }
    if (w == Cf::WGRAD && T > 0) grads(0);

    if (w == Cf::WGRAD && dzk0) {
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) dzk0[(size_t)bh * D + j] = gzk[c];
        });
    }
    // dL/dA_0 = Sigma_0 / 2 = A_0^-1 Q_0 A_0^-1 / 2: here for the default
    // A_0 = I / lambda0; with a given A_0, Q_0 goes to qb for vla_bwd_sandwich
    if (rows && dA0) {
        const float sc = a0given ? 1.f : 0.5f * lambda0 * lambda0;
        sfor<RB>([&](auto h) {
            float *dst = (a0given ? qb : dA0) + bh * DD + (size_t)(i0 + h) * D + c0;
            sfor<EPT / 4>([&](auto q) {
                st4(dst + 4 * q, f4{sc * Q[h][4 * q], sc * Q[h][4 * q + 1], sc * Q[h][4 * q + 2],
                                    sc * Q[h][4 * q + 3]});
            });
        });
    }
}

// Resets the role tickets and every head's progress (T: no token out yet).
__global__ void __launch_bounds__(256) vla_bwd_sync_init(int *sync, int BH, int T)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i <= BH; i += gridDim.x * 256) sync[i] = i == 0 ? 0 : T;
}

// 2 BH workgroups.  Each takes a ticket when it starts: tickets 0 .. BH - 1
// run the memory chains of heads 0 .. BH - 1, the rest the penalty chains.  A
// penalty workgroup waits only on the memory workgroup of its head, which took
// its ticket earlier and so is already running and never waits itself: the
// launch finishes whatever the number of resident workgroups.
template <int D, typename Tin>
__global__ void __launch_bounds__(SplitCfg<D>::NT)
vla_bwd_sweep(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ u, int T,
              float lambda0, float eps, const float *__restrict__ S_T, const float *__restrict__ A_T,
              const float *__restrict__ dO, const float *dS_T, const float *dzk_T,
              float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
              float *__restrict__ du, float *dS0, float *dA0, float *dzk0, bool qin, bool a0given,
              float *qb, const float *__restrict__ rec, float *__restrict__ galpha, int *sync, int BH)
{
    __shared__ __align__(16) union {
        SLds<D> s;
        ALds<D> a;
    } L;
    __shared__ int ticket;
    if (threadIdx.x == 0) ticket = __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int tk = ticket;
    if (tk < BH)
        bwd_s<D, Tin>(L.s, tk, q, k, T, eps, dO, dS_T, dv, dS0, rec, galpha, sync + 1);
    else
        bwd_a<D, Tin>(L.a, tk - BH, q, k, u, T, lambda0, eps, S_T, A_T, dO, dzk_T, dq, dk, dv, du, qin,
                      qb, dA0, a0given, dzk0, rec, galpha, sync + 1);
}

// ----------------------------------------------- conjugation of the final adjoints
// One workgroup per head, thread (row i, columns [c0, c0 + EPT)): out = L M L
// with L, M symmetric d x d, through LDS (L and L M).
//   mode 0 (before the sweep): Q_T = A_T Sigma_T A_T, Sigma_T = dA_T + dA_T'
//   mode 1 (after it): dL/dA_0 = A_0^-1 Q_0 A_0^-1 / 2, with A_0^-1 by the
//          symmetric sweep (fp64)
template <int D>
struct ConjLds {
    float l[D][D + 1];
    float lm[D][D + 1];
    double rowbuf[2][4 * D + 16];
};

template <int D>
__global__ void __launch_bounds__(D * 8)
vla_bwd_sandwich(int mode, const float *__restrict__ lmat, const float *__restrict__ dA_T,
                 float *qb, float *__restrict__ dA0)
{
    constexpr int TPR = 8, EPT = D / TPR;
    __shared__ __align__(16) ConjLds<D> L;
    const int bh = blockIdx.x, tid = threadIdx.x, i = tid / TPR, c0 = (tid % TPR) * EPT;
    const size_t base = (size_t)bh * D * D;
    const float *lh = lmat + base;
    if (mode == 0) {
        sfor<EPT>([&](auto e) { L.l[i][c0 + e] = lh[(size_t)i * D + c0 + e]; });
    } else {
        double m[EPT];
        sfor<EPT>([&](auto e) { m[e] = (double)lh[(size_t)i * D + c0 + e]; });
        sweep_all<D, EPT>(m, i, c0, L.rowbuf);   // -A_0^-1
        sfor<EPT>([&](auto e) { L.l[i][c0 + e] = (float)-m[e]; });
    }
    __syncthreads();
    // L M, row i, columns [c0, c0 + EPT): M from global (Sigma_T or Q_0)
    float acc[EPT];
    sfor<EPT>([&](auto e) { acc[e] = 0.f; });
    for (int a = 0; a < D; ++a) {
        const float la = L.l[i][a];
        sfor<EPT>([&](auto e) {
            const int c = c0 + e;
            const float mv = mode == 0 ? dA_T[base + (size_t)a * D + c] + dA_T[base + (size_t)c * D + a]
                                       : qb[base + (size_t)a * D + c];
            acc[e] = fmaf(la, mv, acc[e]);
        });
    }
    sfor<EPT>([&](auto e) { L.lm[i][c0 + e] = acc[e]; });
    __syncthreads();
    // (L M) L
    sfor<EPT>([&](auto e) { acc[e] = 0.f; });
    for (int a = 0; a < D; ++a) {
        const float x = L.lm[i][a];
        sfor<EPT>([&](auto e) { acc[e] = fmaf(x, L.l[a][c0 + e], acc[e]); });
    }
    sfor<EPT>([&](auto e) {
        if (mode == 0) qb[base + (size_t)i * D + c0 + e] = acc[e];
        else dA0[base + (size_t)i * D + c0 + e] = 0.5f * acc[e];
    });
}

template <int D>
hipError_t sandwich(int mode, int BH, const float *lmat, const float *dA_T, float *qb, float *dA0,
                    hipStream_t stream)
{
    hipLaunchKernelGGL(vla_bwd_sandwich<D>, dim3(BH), dim3(D * 8), 0, stream, mode, lmat, dA_T, qb, dA0);
    return hipGetLastError();
}

template <int D, typename Tin>
hipError_t launch(const BwdArgs &a, const float *rec, const float *S_T, const float *A_T, float *galpha,
                  int *sync, float *qb)
{
    const int BH = a.B * a.H;
    const bool qin = a.dA_T != nullptr, a0given = a.A0 != nullptr && a.dA0 != nullptr;
    hipError_t e;
    if (qin && (e = sandwich<D>(0, BH, A_T, a.dA_T, qb, nullptr, a.stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(vla_bwd_sync_init, dim3((BH + 256) / 256), dim3(256), 0, a.stream, sync, BH, a.T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((vla_bwd_sweep<D, Tin>), dim3(2 * BH), dim3(SplitCfg<D>::NT), 0, a.stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.u, a.T, a.lambda0, a.eps, S_T,
                       A_T, a.dO, a.dS_T, a.dzk_T, a.dq, a.dk, a.dv, a.du, a.dS0, a.dA0, a.dzk0, qin,
                       a0given, qb, rec, galpha, sync, BH);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a0given) return sandwich<D>(1, BH, a.A0, nullptr, qb, a.dA0, a.stream);
    return hipSuccess;
}

}  // namespace

hipError_t launch_backward_split(const BwdArgs &a, const float *rec, const float *S_T,
                                 const float *A_T, float *galpha, int *sync, float *qb)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch<64, uint16_t>(a, rec, S_T, A_T, galpha, sync, qb)
                       : launch<64, float>(a, rec, S_T, A_T, galpha, sync, qb);
    case 96: return bf ? launch<96, uint16_t>(a, rec, S_T, A_T, galpha, sync, qb)
                       : launch<96, float>(a, rec, S_T, A_T, galpha, sync, qb);
    case 128: return bf ? launch<128, uint16_t>(a, rec, S_T, A_T, galpha, sync, qb)
                        : launch<128, float>(a, rec, S_T, A_T, galpha, sync, qb);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
