// vla_bwd.hip -- reverse mode of the VLA recurrence: gradients of a loss with
// respect to q, k, v, u and the initial state, given the adjoints of o and of the
// final state, for d_h in {16, 32, 64, 96, 128}.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9)-(11) (the forward); the pages train the layer end to end but print
// no backward, so this is the chain rule through those equations, step by step
// in reverse order, with the conventions stated at vla_backward in
// include/vla.h.
//
// This kernel serves d in {16, 32} (both phases below).  For d in {64, 96, 128}
// the two-pass forward (vla_twopass.hip) keeps the per-token records and the
// reverse sweep runs as two chains side by side (vla_bwd_split.hip); T = 0 at
// every d takes a copy kernel (vla_bwd_empty: the initial state's gradients are
// the final state's adjoints).
//
// One workgroup per head, D * TPR threads: thread (row i, columns [c0, c0+EPT))
// holds that slice of row i of every d x d matrix, so a matrix-vector product is
// a sum over TPR adjacent lanes (DPP), and rank-1 updates are local.
//
// The reverse sweep needs, per token, z = A_{t-1} u^, alpha^, e, the key sum
// zkey_t and the scalars delta, 1/|y|, phi(q)'zkey, 1/|k|, 1/|u|, and the
// final states S_T, A_T; phase 1 computes them.  The key sum is kept rather
// than rebuilt by subtraction: zkey_t grows like t, and subtracting phi(k) from
// a sum formed in another order would leave the early tokens' zkey_t, small
// against zkey_T, with most of the rounding of zkey_T.
//
// Phase 1 runs the forward one token at a time (states S, A in registers) and
// keeps those per-token values in the workspace.  One barrier per token: the token
// vectors rotate through three LDS slots (staged by the last wave one token
// ahead, raw loads two tokens ahead) and the row products through two.  The
// per-token barriers are LDS-only (global loads stay in flight across them;
// global data crosses between the phases only, behind a full barrier).
//
// Phase 2 walks back from t = T-1 with the adjoints dS (held twice, as rows of
// dS and of dS'), Sigma = dA + dA' (dA only ever acts through its symmetric
// part) and S' (rows of S', so that the products S'g and S'ge are row sums).
// Sigma is stored in fp64 (its rank-2 update terms and products stay fp32, each
// term rounded symmetrically): its entries stay large while the sensitivities
// they carry down the chain shrink (dL/dA_0 falls roughly as 1/T^2), so fp32
// storage would round away most of dA0 and du at T in the thousands;
// S_{t-1} = S_t - e alpha^' and A_{t-1} = A_t + z z' / delta are rebuilt from the
// stored vectors, the same rank-1 terms the forward added (S and A stay of the
// order of their initial values, so their rebuilds keep relative accuracy).
// Per token:
//   A  dS += g phi(q)'/den;  ge = dS alpha^, galpha = dS'e, c1 = S_t'g
//   B  gy = (galpha - alpha^ (alpha^'galpha)) / |y|;  dS -= ge k^';
//      c2 = S_t'ge;  Sigma += gy k^' + k^ gy';  A_t gy;  Sigma z
//   C  gdelta = z'Sigma z / (2 delta^2), gz = -Sigma z / delta + gdelta u^;
//      A <- A_{t-1}, A_{t-1} gz;  Sigma += gz u^' + u^ gz';  S' <- S_{t-1}'
//   D  (wave 0) the token's dq, dk, dv, du from those vectors, the key-sum
//      adjoint and the normalisation Jacobians.
// C of token t and A of token t - 1 share a barrier interval (A needs dS after
// B of t and S_{t-1}' after C of t, both local), so a token costs two
// barriers: ... | B(t) | C(t), A(t-1) | B(t-1) | ...; wave 0's D of token t
// runs at the start of the next interval.  Token vectors rotate through three
// LDS slots and row results through two, so D of token t never races the
// staging of token t - 2 or the row results of token t - 1.

#include "vla_bwd.h"
#include "vla_chunk_parts.h"
#include "vla_record.h"
#include "vla_reduce.h"

namespace vla {
namespace {

using namespace chunk;

// Threads per row (TPR): every wave repeats the token's scalar work (dot
// products, norms, the step scalars), so fewer, wider threads cost less issue;
// four per row at d <= 32, the sizes this kernel serves.  The last wave loads
// and stages the token vectors.
template <int D> struct BwdCfg {
    static_assert(D <= 32, "d >= 64 runs the split sweep (vla_bwd_split.hip)");
    static constexpr int TPR = 4, EPT = D / TPR;
    static constexpr int TRP = D + 1;   // row pitch of tr
};


template <int D>
struct BwdLds {
    // phase 1: token vectors (three slots) and row products z, w (two slots)
    float fk[3][D], fu[3][D], fq[3][D], fv[3][D], fpk[3][D];
    float fsc[3][4];
    float zw[2][2][D];
    // phase 2: token vectors and scalars (three slots) ...
    float g[3][D], pq[3][D], kh[3][D], uh[3][D], z[3][D], al[3][D], e[3][D], zt[3][D];
    float dpq[3][D], dpk[3][D];
    float sc[3][8];
    // ... and the row results of steps A, B, C (two slots)
    float r1[2][3][D], r2[2][3][D], r3[2][D];
    // S -> S' between the phases (and S' itself above d = 64)
    float tr[D * BwdCfg<D>::TRP];
};

template <int D, typename Tin>
__global__ void __launch_bounds__(D * BwdCfg<D>::TPR)
vla_bwd(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
        const Tin *__restrict__ u, int T, float lambda0, float eps,
        const float *S0, const float *A0, const float *zk0, const float *__restrict__ dO,
        const float *dS_T, const float *dA_T, const float *dzk_T, float *__restrict__ dq,
        float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ du, float *dS0,
        float *dA0, float *dzk0, float *__restrict__ rec)
{
    using Cf = BwdCfg<D>;
    constexpr int TPR = Cf::TPR, EPT = Cf::EPT, NT = D * TPR, NW = NT / 64;
    using K = rec::Keep<D>;
    constexpr int NV = (D + 63) / 64, RS = K::RS, P = Cf::TRP;
    static_assert(RS == backward_record_floats(D), "record size");
    static_assert(EPT % 4 == 0 && NT % 64 == 0 && NT <= 1024, "row slices of whole granules");
    __shared__ __align__(16) BwdLds<D> L;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = tid / TPR, c0 = (tid % TPR) * EPT;
    const bool leader = tid % TPR == 0;
    const int bh = blockIdx.x;
    const size_t DD = (size_t)D * D, tok0 = (size_t)bh * T;
    float *rh = rec + tok0 * RS;   // this head's per-token records
    const int T1 = T;              // tokens of phase 1

    // ------------------------------------------------------------ phase 1
    float S[EPT], A[EPT];
    {
        const size_t off = bh * DD + (size_t)row * D + c0;
        sfor<EPT / 4>([&](auto h) {
            const f4 x = S0 ? ld4(S0 + off + 4 * h) : f4{0.f, 0.f, 0.f, 0.f};
            f4 y;
            if (A0) {
                y = ld4(A0 + off + 4 * h);
            } else {
                sfor<4>([&](auto r) { y[int(r)] = row == c0 + 4 * h + r ? 1.f / lambda0 : 0.f; });
            }
            sfor<4>([&](auto r) {
                S[4 * h + r] = x[int(r)];
                A[4 * h + r] = y[int(r)];
            });
        });
    }
    float zk[NV];   // wave 0: zkey, entries lane + 64 c
    sfor<NV>([&](auto c) {
        const int j = lane + 64 * c;
        zk[c] = zk0 && j < D ? zk0[(size_t)bh * D + j] : 0.f;
    });

    // the last wave stages token vectors: raw values in registers two tokens
    // ahead, normalised into LDS one token ahead
    // (kept as loaded, bf16 as its bit pattern, so that the loads stay in
    // flight until the staging a token later)
    Raw1<Tin> xq[NV], xk[NV], xu[NV], xv[NV];
    auto p1_load = [&](int t) {
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const size_t o = (tok0 + t) * D + j;
                xq[c].load(q, o);
                xk[c].load(k, o);
                xu[c].load(u, o);
                xv[c].load(v, o);
            }
        });
    };
    auto p1_stage = [&](int slot) {
        float nk = 0.f, nu = 0.f;
        sfor<NV>([&](auto c) {
            if (lane + 64 * c < D) {
                nk = fmaf(xk[c].get(), xk[c].get(), nk);
                nu = fmaf(xu[c].get(), xu[c].get(), nu);
            }
        });
        nk = wave_sum(nk);
        nu = wave_sum(nu);
        const float ik = nk > 0.f ? rsqrtf(nk) : 0.f, iu = nu > 0.f ? rsqrtf(nu) : 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                L.fk[slot][j] = xk[c].get() * ik;
                L.fu[slot][j] = xu[c].get() * iu;
                L.fq[slot][j] = phi_fast(xq[c].get());
                L.fv[slot][j] = xv[c].get();
                L.fpk[slot][j] = phi_fast(xk[c].get());
            }
        });
        if (lane == 0) {
            L.fsc[slot][0] = ik;
            L.fsc[slot][1] = iu;
        }
    };
    if (w == NW - 1 && T1 > 0) {
        p1_load(0);
        p1_stage(0);
        if (T1 > 1) p1_load(1);
    }
    // drain what the prologue issued, as a wait the compiler sees: otherwise it
    // waits for every load in flight at the top of each iteration
    vmem_drain();
    __syncthreads();

    for (int t = 0; t < T1; ++t) {
        const int s3 = t % 3, s2 = t & 1;
        float *rt = rh + (size_t)t * RS;
        // z = A u^, w = A k^ (old A), r = S k^ (old S)
        float pz = 0.f, pw = 0.f, pr = 0.f;
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float uj = L.fu[s3][j], kj = L.fk[s3][j];
            pz = fmaf(A[e], uj, pz);
            pw = fmaf(A[e], kj, pw);
            pr = fmaf(S[e], kj, pr);
        });
        pz = row_sum<TPR>(pz);
        pw = row_sum<TPR>(pw);
        pr = row_sum<TPR>(pr);
        const float ei = L.fv[s3][row] - pr;
        if (leader) {
            L.zw[s2][0][row] = pz;
            L.zw[s2][1][row] = pw;
            rt[K::Z + row] = pz;
            rt[K::E + row] = ei;
        }
        if (w == NW - 1 && t + 1 < T1) {
            p1_stage((t + 1) % 3);
            if (t + 2 < T1) p1_load(t + 2);
        }
        lds_barrier();

        // delta = 1 + u^'z, z'k^, and y = A_t k^ = w - z (z'k^) / delta
        float a = 0.f, b = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const float zj = L.zw[s2][0][j];
                a = fmaf(L.fu[s3][j], zj, a);
                b = fmaf(zj, L.fk[s3][j], b);
            }
        });
        const float delta = 1.f + wave_sum(a), ci = wave_sum(b) / delta, id = 1.f / delta;
        float yy = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const float yj = L.zw[s2][1][j] - L.zw[s2][0][j] * ci;
                yy = fmaf(yj, yj, yy);
            }
        });
        yy = wave_sum(yy);
        const float iy = yy > 0.f ? rsqrtf(yy) : 0.f;
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float zj = L.zw[s2][0][j];
            A[e] = fmaf(-pz * zj, id, A[e]);                               // Eq. (9)
            S[e] = fmaf(ei, (L.zw[s2][1][j] - zj * ci) * iy, S[e]);        // Eq. (10)
        });
        if (w == 0) {
            float dn = 0.f;
            sfor<NV>([&](auto c) {
                const int j = lane + 64 * c;
                if (j < D) {
                    rt[K::AL + j] = (L.zw[s2][1][j] - L.zw[s2][0][j] * ci) * iy;
                    zk[c] += L.fpk[s3][j];
                    rt[K::ZK + j] = zk[c];
                    dn = fmaf(L.fq[s3][j], zk[c], dn);
                }
            });
            dn = wave_sum(dn);
            if (lane == 0) {
                const f4 s01 = {delta, iy, dn, L.fsc[s3][0]};
                st4(rt + K::SC, s01);
                st4(rt + K::SC + 4, f4{L.fsc[s3][1], 0.f, 0.f, 0.f});
            }
        }
    }

    // ------------------------------------------------------------ phase 2
    __syncthreads();
    // S' rows: through LDS into registers
    sfor<EPT>([&](auto e) { L.tr[row * P + c0 + e] = S[e]; });
    __syncthreads();
    float St[EPT], gS[EPT], gSt[EPT];   // S', dS, dS' (row slices)
    auto st_get = [&](auto e) -> float { return St[e]; };
    auto st_set = [&](auto e, float x) { St[e] = x; };
    double Sg[EPT];                     // Sigma (row slice)
    sfor<EPT>([&](auto e) { St[e] = L.tr[(c0 + e) * P + row]; });
    {
        const size_t off = bh * DD + (size_t)row * D + c0;
        sfor<EPT>([&](auto e) {
            const size_t tr_off = bh * DD + (size_t)(c0 + e) * D + row;
            gS[e] = dS_T ? dS_T[off + e] : 0.f;
            gSt[e] = dS_T ? dS_T[tr_off] : 0.f;
            Sg[e] = dA_T ? (double)dA_T[off + e] + (double)dA_T[tr_off] : 0.0;
        });
    }
    float gzk[NV];
    sfor<NV>([&](auto c) {
        const int j = lane + 64 * c;
        gzk[c] = dzk_T && j < D ? dzk_T[(size_t)bh * D + j] : 0.f;
    });

    // A token's vectors are loaded (raw, a token ahead) and staged into LDS in
    // nine groups: dO; q; k; u; z; alpha^; e; zkey_t; the scalars (also loaded
    // by the k and u groups, for 1/|k|, 1/|u|).  The last wave owns them all
    // and alone calls p2_load, p2_stage.
    const bool stager = w == NW - 1;
    float yg[NV], yz[NV], ya[NV], ye[NV], yw[NV];
    Raw1<Tin> yq[NV], yk[NV], yu[NV];
    f4 ys0, ys1;
    auto p2_load = [&](int t) {
        const float *rt = rh + (size_t)t * RS;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                const size_t o = (tok0 + t) * D + j;
                yg[c] = dO[o];
                yq[c].load(q, o);
                yk[c].load(k, o);
                yu[c].load(u, o);
                yz[c] = rt[K::Z + j];
                ya[c] = rt[K::AL + j];
                ye[c] = rt[K::E + j];
                yw[c] = rt[K::ZK + j];
            }
        });
        {
            ys0 = ld4(rt + K::SC);
            ys1 = ld4(rt + K::SC + 4);
        }
    };
    auto p2_stage = [&](int slot) {
        const float ik = ys0[3], iu = ys1[0];
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                L.g[slot][j] = yg[c];
                {
                    const float qj = yq[c].get();
                    L.pq[slot][j] = phi_fast(qj);
                    L.dpq[slot][j] = dphi(qj);
                }
                {
                    const float kj = yk[c].get();
                    L.kh[slot][j] = kj * ik;
                    L.dpk[slot][j] = dphi(kj);
                }
                L.uh[slot][j] = yu[c].get() * iu;
                L.z[slot][j] = yz[c];
                L.al[slot][j] = ya[c];
                L.e[slot][j] = ye[c];
                L.zt[slot][j] = yw[c];
            }
        });
        if (lane == 0) {
            st4(&L.sc[slot][0], ys0);
            st4(&L.sc[slot][4], ys1);
        }
    };
    if (stager && T > 0) {
        p2_load(T - 1);
        p2_stage((T - 1) % 3);
        if (T > 1) p2_load(T - 2);
    }
    vmem_drain();
    __syncthreads();

    // Token t's vectors sit in LDS slot t % 3, its row results in slot t % 2.
    // Step A: the readout's share of dS, then dS alpha^, dS'e, S_t'g.
    auto step_a = [&](int t) {
        const int v3 = t % 3, s = t & 1;
        const float iden = 1.f / fmaxf(L.sc[v3][2], eps);
        float pge = 0.f, pga = 0.f, pc1 = 0.f;
        const float gi = L.g[v3][row] * iden, pqi = L.pq[v3][row] * iden;
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float gj = L.g[v3][j];
            gS[e] = fmaf(gi, L.pq[v3][j], gS[e]);
            gSt[e] = fmaf(pqi, gj, gSt[e]);
            pge = fmaf(gS[e], L.al[v3][j], pge);
            pga = fmaf(gSt[e], L.e[v3][j], pga);
            pc1 = fmaf(st_get(e), gj, pc1);
        });
        pge = row_sum<TPR>(pge);
        pga = row_sum<TPR>(pga);
        pc1 = row_sum<TPR>(pc1);
        if (leader) {
            L.r1[s][0][row] = pge;
            L.r1[s][1][row] = pga;
            L.r1[s][2][row] = pc1;
        }
    };
    // Step B: gy; dS -= ge k^'; S_t'ge; Sigma += gy k^' + k^ gy'; A_t gy; Sigma z.
    auto step_b = [&](int t) {
        const int v3 = t % 3, s = t & 1;
        const float iy = L.sc[v3][1];
        float aga = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) aga = fmaf(L.al[v3][j], L.r1[s][1][j], aga);
        });
        aga = wave_sum(aga);
        float pc2 = 0.f, paty = 0.f, psz = 0.f;
        const float khi = L.kh[v3][row], ge_i = L.r1[s][0][row];
        const float gyi = (L.r1[s][1][row] - L.al[v3][row] * aga) * iy;
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float gej = L.r1[s][0][j], khj = L.kh[v3][j];
            const float gyj = (L.r1[s][1][j] - L.al[v3][j] * aga) * iy;
            gS[e] = fmaf(-ge_i, khj, gS[e]);
            gSt[e] = fmaf(-khi, gej, gSt[e]);
            pc2 = fmaf(st_get(e), gej, pc2);
            Sg[e] += (double)sym_sum(gyi, khj, khi, gyj);
            paty = fmaf(A[e], gyj, paty);
            psz = fmaf((float)Sg[e], L.z[v3][j], psz);
        });
        pc2 = row_sum<TPR>(pc2);
        paty = row_sum<TPR>(paty);
        psz = row_sum<TPR>(psz);
        if (leader) {
            L.r2[s][0][row] = pc2;
            L.r2[s][1][row] = paty;
            L.r2[s][2][row] = psz;
        }
    };
    // Step C: gdelta, gz; A_{t-1} and A_{t-1} gz; Sigma += gz u^' + u^ gz';
    // S_{t-1}'.  Returns gdelta.
    auto step_c = [&](int t) -> float {
        const int v3 = t % 3, s = t & 1;
        const float id = 1.f / L.sc[v3][0];
        float zsz = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) zsz = fmaf(L.z[v3][j], L.r2[s][2][j], zsz);
        });
        const float gdel = 0.5f * wave_sum(zsz) * id * id;
        float pagz = 0.f;
        const float zi = L.z[v3][row], uhi = L.uh[v3][row], ali = L.al[v3][row];
        const float gzi = fmaf(-L.r2[s][2][row], id, gdel * uhi);
        sfor<EPT>([&](auto e) {
            const int j = c0 + e;
            const float zj = L.z[v3][j], uhj = L.uh[v3][j];
            const float gzj = fmaf(-L.r2[s][2][j], id, gdel * uhj);
            A[e] = fmaf(zi * zj, id, A[e]);
            pagz = fmaf(A[e], gzj, pagz);
            Sg[e] += (double)sym_sum(gzi, uhj, uhi, gzj);
            st_set(e, fmaf(-ali, L.e[v3][j], st_get(e)));
        });
        pagz = row_sum<TPR>(pagz);
        if (leader) L.r3[s][row] = pagz;
        return gdel;
    };
    // Step D (wave 0): the token's gradients from the row results.
    auto step_d = [&](int t, float gdel) {
        const int v3 = t % 3, s = t & 1;
        const float dn = L.sc[v3][2], iden = 1.f / fmaxf(dn, eps);
        float a1 = 0.f, a2 = 0.f;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                a1 = fmaf(L.r1[s][2][j], L.pq[v3][j], a1);   // g'S_t phi(q)
                a2 = fmaf(L.e[v3][j], L.r1[s][0][j], a2);    // e'ge
            }
        });
        a1 = wave_sum(a1);
        a2 = wave_sum(a2);
        const float gden = dn >= eps ? -a1 * iden * iden : 0.f;
        float gkh[NV], guh[NV], a3 = 0.f, a4 = 0.f;
        const size_t o = (tok0 + t) * D;
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            gkh[c] = guh[c] = 0.f;
            if (j < D) {
                const float gpq = fmaf(L.r1[s][2][j], iden, gden * L.zt[v3][j]);
                dq[o + j] = gpq * L.dpq[v3][j];
                dv[o + j] = L.r1[s][0][j];
                gzk[c] = fmaf(gden, L.pq[v3][j], gzk[c]);
                gkh[c] = fmaf(L.al[v3][j], a2, L.r2[s][1][j] - L.r2[s][0][j]);
                guh[c] = fmaf(gdel, L.z[v3][j], L.r3[s][j]);
                a3 = fmaf(L.kh[v3][j], gkh[c], a3);
                a4 = fmaf(L.uh[v3][j], guh[c], a4);
            }
        });
        a3 = wave_sum(a3);
        a4 = wave_sum(a4);
        const float ik = L.sc[v3][3], iu = L.sc[v3][4];
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) {
                dk[o + j] = fmaf(ik, gkh[c] - L.kh[v3][j] * a3, gzk[c] * L.dpk[v3][j]);
                du[o + j] = iu * (guh[c] - L.uh[v3][j] * a4);
            }
        });
    };

    // Two barriers per token: B(t) | C(t) with A(t - 1) |.  Wave 0 forms token
    // t + 1's gradients at the start of iteration t, while the others begin B(t).
    if (T > 0) step_a(T - 1);
    lds_barrier();
    float gdel_d = 0.f;
    for (int t = T - 1; t >= 0; --t) {
        if (stager && t > 0) {   // token t - 1 into slot (t - 1) % 3
            p2_stage((t - 1) % 3);
            if (t > 1) p2_load(t - 2);
        }
        if (w == 0 && t + 1 < T) step_d(t + 1, gdel_d);
        step_b(t);
        lds_barrier();
        gdel_d = step_c(t);
        if (t > 0) step_a(t - 1);
        lds_barrier();
    }
    if (w == 0 && T > 0) step_d(0, gdel_d);

    // gradients of the initial state
    {
        const size_t off = bh * DD + (size_t)row * D + c0;
        sfor<EPT / 4>([&](auto h) {
            if (dS0) st4(dS0 + off + 4 * h, f4{gS[4 * h], gS[4 * h + 1], gS[4 * h + 2], gS[4 * h + 3]});
            if (dA0)
                st4(dA0 + off + 4 * h, f4{(float)(0.5 * Sg[4 * h]), (float)(0.5 * Sg[4 * h + 1]),
                                          (float)(0.5 * Sg[4 * h + 2]), (float)(0.5 * Sg[4 * h + 3])});
        });
    }
    if (w == 0 && dzk0) {
        sfor<NV>([&](auto c) {
            const int j = lane + 64 * c;
            if (j < D) dzk0[(size_t)bh * D + j] = gzk[c];
        });
    }
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// head sizes whose records come from the two-pass forward (vla_twopass.hip
// instantiates it for d = 64, 96, 128); the others run phase 1
constexpr bool records_from_forward(int d) { return d == 64 || d == 96 || d == 128; }

// Workspace: the per-token records; for d in {64, 96, 128} also the two-pass
// forward's workspace, its final S, A, zkey, the gate adjoints dL/dalpha^ that
// the memory chain's sweep hands to the penalty chain's, their
// synchronisation words and one d x d matrix per head for the penalty
// adjoint's conjugated form at the ends of the sweep.
struct BwdPlan {
    size_t rec = 0, fwd = 0, st = 0, ga = 0, sync = 0, qb = 0, bytes = 0;
};
BwdPlan bwd_plan(int BH, int T, int d)
{
    BwdPlan p;
    if (T <= 0) return p;
    size_t off = up256((size_t)BH * T * backward_record_floats(d) * sizeof(float));
    if (records_from_forward(d)) {
        p.fwd = off;
        off = up256(off + twopass_workspace_bytes(BH, T, d));
        p.st = off;
        off = up256(off + (size_t)BH * (2 * (size_t)d * d + d) * sizeof(float));
        p.ga = off;
        off = up256(off + (size_t)BH * T * d * sizeof(float));
        p.sync = off;
        off = up256(off + ((size_t)BH + 1) * sizeof(int));
        p.qb = off;
        off = up256(off + (size_t)BH * d * d * sizeof(float));
    }
    p.bytes = off;
    return p;
}

// T = 0: no token to go through, so the initial state's gradients are the final
// state's adjoints, dA0 symmetrised as (G + G')/2 (A_0 is a symmetric matrix);
// missing adjoints are zero.  A grid-stride pass over the B H d^2 entries.
__global__ void __launch_bounds__(256)
vla_bwd_empty(int BH, int D, const float *dS_T, const float *dA_T, const float *dzk_T, float *dS0,
              float *dA0, float *dzk0)
{
    const size_t DD = (size_t)D * D, n = (size_t)BH * DD;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        if (dS0) dS0[e] = dS_T ? dS_T[e] : 0.f;
        if (dA0) {
            const size_t h = e / DD, r = e % DD, i = r / D, j = r % D;
            dA0[e] = dA_T ? (float)(0.5 * ((double)dA_T[e] + (double)dA_T[h * DD + j * D + i])) : 0.f;
        }
        if (dzk0 && e < (size_t)BH * D) dzk0[e] = dzk_T ? dzk_T[e] : 0.f;
    }
}

hipError_t launch_empty(const BwdArgs &a)
{
    const size_t n = (size_t)a.B * a.H * a.d * a.d;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(vla_bwd_empty, dim3(blocks), dim3(256), 0, a.stream, a.B * a.H, a.d, a.dS_T, a.dA_T,
                       a.dzk_T, a.dS0, a.dA0, a.dzk0);
    return hipGetLastError();
}

// both phases in the one kernel (per-token forward, then the reverse sweep)
template <int D, typename Tin>
hipError_t launch_phase1(const BwdArgs &a, dim3 grid, dim3 block, float *rec)
{
    static_assert(!records_from_forward(D), "phase 1 serves d in {16, 32}");
    hipLaunchKernelGGL((vla_bwd<D, Tin>), grid, block, 0, a.stream, (const Tin *)a.q,
                       (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u, a.T, a.lambda0, a.eps,
                       a.S0, a.A0, a.zk0, a.dO, a.dS_T, a.dA_T, a.dzk_T, a.dq, a.dk, a.dv, a.du,
                       a.dS0, a.dA0, a.dzk0, rec);
    return hipGetLastError();
}

template <int D, typename Tin>
hipError_t launch(const BwdArgs &a)
{
    const int BH = a.B * a.H;
    const BwdPlan p = bwd_plan(BH, a.T, D);
    char *ws = static_cast<char *>(a.ws);
    float *rec = reinterpret_cast<float *>(ws + p.rec);
    if (a.T <= 0) return launch_empty(a);
    if constexpr (records_from_forward(D)) {
        // the forward on the matrix-core kernels, keeping the per-token records;
        // its o goes to dq (overwritten below), its final state to the workspace
        float *stS = reinterpret_cast<float *>(ws + p.st), *stA = stS + (size_t)BH * D * D;
        float *stZ = stA + (size_t)BH * D * D;
        FwdArgs f{a.q, a.k, a.v, a.u, a.dtype, a.B, a.H, a.T, D, a.lambda0, a.eps,
                  a.dq, stS, stA, stZ, a.S0, a.A0, a.zk0, a.stream,
                  ws + p.fwd, twopass_workspace_bytes(BH, a.T, D)};
        f.keep = rec;
        const hipError_t e = launch_forward_twopass(f, 3);
        if (e != hipSuccess) return e;
        const float *frec = reinterpret_cast<const float *>(ws + p.fwd + twopass_records_offset(BH, a.T, D));
        return launch_backward_split(a, rec, frec, stS, stA,
                                     reinterpret_cast<float *>(ws + p.ga),
                                     reinterpret_cast<int *>(ws + p.sync),
                                     reinterpret_cast<float *>(ws + p.qb));
    } else {
        return launch_phase1<D, Tin>(a, dim3(BH), dim3(D * BwdCfg<D>::TPR), rec);
    }
}

}  // namespace

size_t backward_workspace_bytes(int BH, int T, int d)
{
    return bwd_plan(BH, T, d).bytes;
}

hipError_t launch_backward(const BwdArgs &a)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 16: return bf ? launch<16, uint16_t>(a) : launch<16, float>(a);
    case 32: return bf ? launch<32, uint16_t>(a) : launch<32, float>(a);
    case 64: return bf ? launch<64, uint16_t>(a) : launch<64, float>(a);
    case 96: return bf ? launch<96, uint16_t>(a) : launch<96, float>(a);
    case 128: return bf ? launch<128, uint16_t>(a) : launch<128, float>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
