// vla_twopass.hip -- forward pass of the VLA recurrence for d_h in {64, 96, 128}
// as two passes over the sequence, so that the work of one head spreads over
// many compute units.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.2
// (A_0 = I / lambda0 and unit u, so that A_t is the inverse of
// A_0^-1 + sum_{s<=t} u^_s u^_s') and section 3.3, Eqs. (9)-(11).
//
// The penalty chain (Eq. 9) reads only the inputs, and A_t is the inverse of
//     M_t = A_0^-1 + sum_{s<=t} u^_s u^_s'.
// The sequence is cut into segments of whole chunks, and the chain of each
// segment starts from the inverse of M at its first token, formed directly:
//
//   gram     per (head, segment but the last): sum of u^ u^' over the segment
//            (fp32 matrix-core products of 16 tokens, summed in fp64) and the sum
//            of phi(k) (fp64).
//   inverse  per (head, segment > 0): M at the segment start in fp64 and its
//            inverse by the symmetric sweep operator (fp64), stored as fp32, and
//            the key sum at the segment start.
//   penalty  per (head, segment): the blocked penalty chain of vla_chunk_parts.h
//            from that A; for every chunk of 16 tokens it writes the operands
//            the memory chain needs to a record: alpha^ (d x C, key-major),
//            (I + N)^-1 and P = (Alpha^'Phi) o Up (C x C, transposed), 1 / den,
//            and k^ and phi(q) (C x d, token-major).  The key sum and den follow
//            Eq. (11).
//   memory   per (head, group of 16-row value blocks): the memory chain from the
//            records and v, two chunks per step (the second one's products
//            with S corrected by cross factors the penalty pass also records):
//                R = V - S K^,  E = R (I + N)^-1,
//                o = (S Phi + E P) / den,  S <- S + E Alpha^'.
//            Records and v reach LDS through direct copies, two or three steps
//            ahead (as many stages as LDS holds).
//            Rows of S do not interact, so the value rows of a head are split
//            over workgroups, and the key columns of a block over the waves of a
//            workgroup (partial products summed through LDS in a fixed order).
//
// All four run on the caller's stream; the workspace holds the records, the
// Grams and the segment starts (its size is twopass_workspace_bytes).
#include "vla_chunk_parts.h"
#include "vla_record.h"
#include "vla_sweep.h"

namespace vla {
namespace {

using namespace chunk;

using rec::CH;
using rec::Rec;

using rec::Keep;   // the per-token records kept for the gradients

// Value blocks per memory workgroup and the ways each block's key tiles are
// split over its waves (VBW x KS waves per workgroup).  The stages of a
// workgroup fill most of the LDS, so one workgroup runs per compute unit; the
// splits are chosen so that the B H (d / 16) / VBW workgroups fit one round
// on 256 compute units at the workloads' head counts (d = 96: 128 heads x 2;
// d = 128: 64 heads x 4), since a second round would run the whole chain
// again: at d = 128 four value blocks of one key split each in two rounds
// took 8.7 ms, two blocks of two key splits in one round 4.8 ms.
template <int D> struct MemCfg;
template <> struct MemCfg<64> { static constexpr int VBW = 2, KS = 2; };
template <> struct MemCfg<96> { static constexpr int VBW = 3, KS = 2; };
template <> struct MemCfg<128> { static constexpr int VBW = 2, KS = 2; };

// ------------------------------------------------------------------- gram
// Workgroup (head, segment j < S - 1, part pp < P): the part's share of
// G_j = sum of u^ u^' and z_j = sum of phi(k) over segment j (the segment's
// chunks split in P runs, so that the launch has enough workgroups).  Tokens go
// in blocks of GB = 64; thread (token tl, part cc) stages columns [cc CPT, +CPT)
// of u^ of tokens tl + 16 s (s < 4) of a block, transposed ([i][token]), while
// the loads of the next block are in flight.  G is symmetric: only its tiles
// (a, b) with a <= b are formed, wave w taking tiles w, w + 4, ..., and stored
// with their mirror images.  Each block's fp32 matrix-core partial sums are
// added to fp64 accumulators.
template <int D, typename Tin>
__global__ void __launch_bounds__(256)
vla_gram(const Tin *__restrict__ k, const Tin *__restrict__ u, int T, int S, int SC, int P,
         double *__restrict__ gram, double *__restrict__ zks)
{
    constexpr int NB = D / 16, NTILE = NB * (NB + 1) / 2, TPW = (NTILE + 3) / 4;
    constexpr int CPT = D / 16, GB = 64, LT = GB + 4;
    __shared__ __align__(16) float ut[2][D * LT];
    __shared__ double zred[256 * CPT];

    const int S1 = S - 1;
    const int pp = blockIdx.x % P, j = (blockIdx.x / P) % S1, bh = blockIdx.x / (P * S1);
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tl = tid >> 4, cc = tid & 15;
    const int PC = (SC + P - 1) / P;                 // chunks per part
    const int cb = j * SC + pp * PC, ce = min(j * SC + SC, cb + PC);
    const int t0 = cb * CH, t1 = min(T, ce * CH);   // the part's tokens (may be none)
    const int NBK = t1 > t0 ? (t1 - t0 + GB - 1) / GB : 0;
    const Tin *uh = u + (size_t)bh * T * D, *kh = k + (size_t)bh * T * D;

    // tile index -> (a, b), a <= b
    int ta[TPW], tb[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        int idx = w + 4 * t, a = 0;
        while (idx >= NB - a && a < NB - 1) { idx -= NB - a; ++a; }
        ta[t] = a;
        tb[t] = a + idx;
    }

    RawVec<Tin, CPT> ru[4], rk[4];
    double zacc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) zacc[i] = 0.0;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    double gacc[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) gacc[t][r] = 0.0;

    const Buf ub(uh, (unsigned)T * D * sizeof(Tin)), kb(kh, (unsigned)T * D * sizeof(Tin));
    auto prefetch = [&](int blk) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int t = t0 + blk * GB + 16 * s2 + tl;
            const unsigned off = ((unsigned)(t < t1 ? t : t1 - 1) * D + cc * CPT) * sizeof(Tin);
            ru[s2].load(ub, off);
            rk[s2].load(kb, off);
        }
    };
    auto stage = [&](int blk) {
        float *dst = ut[blk & 1];
        float zblk[CPT];   // this block's phi(k), four tokens per column in fp32
#pragma unroll
        for (int i = 0; i < CPT; ++i) zblk[i] = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const bool ok = t0 + blk * GB + 16 * s2 + tl < t1;
            float pu = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) pu = fmaf(ru[s2].get(i), ru[s2].get(i), pu);
            const float nu = sum_row16(pu);
            const float iu = ok && nu > 0.f ? rsqrtf(nu) : 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) dst[(cc * CPT + i) * LT + 16 * s2 + tl] = ru[s2].get(i) * iu;
            if (ok) {
#pragma unroll
                for (int i = 0; i < CPT; ++i) zblk[i] += phi_fast(rk[s2].get(i));
            }
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) zacc[i] += (double)zblk[i];
    };

    if (NBK > 0) {
        prefetch(0);
        stage(0);
        if (NBK > 1) prefetch(1);
    }
    vmem_drain();
    __syncthreads();
    for (int blk = 0; blk < NBK; ++blk) {
        const float *src = ut[blk & 1];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            if (w + 4 * t < NTILE) {
                f4 acc = zero;
#pragma unroll
                for (int s2 = 0; s2 < GB / 16; ++s2) {
                    const f4 af = ld4(&src[(16 * ta[t] + n) * LT + 16 * s2 + 4 * g]);
                    const f4 bf = ld4(&src[(16 * tb[t] + n) * LT + 16 * s2 + 4 * g]);
                    acc = mma4(af, bf, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) gacc[t][r] += (double)acc[r];
            }
        }
        if (blk + 1 < NBK) {
            stage(blk + 1);
            if (blk + 2 < NBK) prefetch(blk + 2);
        }
        lds_barrier();
    }

    // full symmetric matrix: off-diagonal tiles are written twice
    double *G = gram + (((size_t)bh * S1 + j) * P + pp) * D * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        if (w + 4 * t < NTILE) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                G[(size_t)(16 * ta[t] + 4 * g + r) * D + 16 * tb[t] + n] = gacc[t][r];
            if (ta[t] != tb[t]) {
                double2 *Gt = reinterpret_cast<double2 *>(&G[(size_t)(16 * tb[t] + n) * D + 16 * ta[t] + 4 * g]);
                Gt[0] = make_double2(gacc[t][0], gacc[t][1]);
                Gt[1] = make_double2(gacc[t][2], gacc[t][3]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) zred[tid * CPT + i] = zacc[i];
    __syncthreads();
    if (tid < D) {
        const int pc = tid / CPT, pi = tid % CPT;
        double z = 0.0;
        for (int t2 = 0; t2 < CH; ++t2) z += zred[(t2 * 16 + pc) * CPT + pi];
        zks[(((size_t)bh * S1 + j) * P + pp) * D + tid] = z;
    }
}

// ------------------------------------------------------------------- prefix
// With many segments per head (few heads), the inverse of segment j would sum
// the Gram parts of all j earlier segments, O(S^2) reads per head.  Thread e
// (an entry of G, or of the key sum past the d^2 entries) runs once through a
// head's parts in order and leaves in part 0 of segment j the sum over segments
// 0 .. j; the parts of eight segments are read before their sums are written.
template <int D>
__global__ void __launch_bounds__(256)
vla_gram_prefix(int S, int P, double *__restrict__ gram, double *__restrict__ zks)
{
    constexpr int DD = D * D, NE = DD + D, NBLK = (NE + 255) / 256, SB = 8;
    const int bh = blockIdx.x / NBLK, e = (blockIdx.x % NBLK) * 256 + threadIdx.x;
    if (e >= NE) return;
    const int S1 = S - 1;
    double *b = e < DD ? gram + (size_t)bh * S1 * P * DD + e : zks + (size_t)bh * S1 * P * D + (e - DD);
    const size_t stride = e < DD ? (size_t)DD : (size_t)D;   // between consecutive parts
    double acc = 0.0;
    for (int j0 = 0; j0 < S1; j0 += SB) {
        double x[SB];
        sfor<SB>([&](auto v) {
            double t = 0.0;
            if (j0 + v < S1)
                for (int pp = 0; pp < P; ++pp) t += b[((size_t)(j0 + v) * P + pp) * stride];
            x[v] = t;
        });
        sfor<SB>([&](auto v) {
            if (j0 + v < S1) {
                acc += x[v];
                b[(size_t)(j0 + v) * P * stride] = acc;
            }
        });
    }
}

// ------------------------------------------------------------------- inverse
// (sweep_tiles, vla_sweep.h)

// Workgroup (head, segment j >= 1): A at the segment start = M^-1 with
// M = A_0^-1 + sum_{i<j} G_i, and the key sum at the segment start.  With
// `prefixed` the sums over the earlier segments are ready in part 0 of segment
// j - 1 (vla_gram_prefix); otherwise the parts are summed here.  With a
// caller-given A_0 (or zkey_0) the workgroup of segment 1 also copies it to slot
// 0, which the penalty pass reads instead, so that the final state may overwrite
// the initial one.
// The matrix lives in fp64 matrix-core tiles (sweep_tiles, vla_sweep.h): D / 16
// waves, wave I holding tile row I.
template <int D>
__global__ void __launch_bounds__(4 * D)
vla_seginv(int S, int P, float lambda0, const float *A0, const float *zk0,
           const double *__restrict__ gram, const double *__restrict__ zks,
           float *__restrict__ aseg, float *__restrict__ zseg, bool prefixed)
{
    constexpr int NB = D / 16;
    __shared__ __align__(16) double rowbuf[2][4 * D + 16];
    const int S1 = S - 1;
    const int bh = blockIdx.x / S1, j = blockIdx.x % S1 + 1;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int I = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t DD = (size_t)D * D;
    // element (row, column) of tile (I, J), register r
    auto rc = [&](int J, int r) { return (size_t)(16 * I + g + 4 * r) * D + 16 * J + n; };

    Tiles64<D> t;
    if (A0) {
        const float *a0 = A0 + bh * DD;
        sfor<NB>([&](auto J) { sfor<4>([&](auto r) { t[J][int(r)] = (double)a0[rc(J, r)]; }); });
        if (j == 1)
            sfor<NB>([&](auto J) { sfor<4>([&](auto r) { aseg[(size_t)bh * S * DD + rc(J, r)] = a0[rc(J, r)]; }); });
        sweep_tiles<D>(t, I, lane, rowbuf);   // -A_0^-1
        sfor<NB>([&](auto J) { t[J] = -t[J]; });
    } else {
        sfor<NB>([&](auto J) {
            sfor<4>([&](auto r) { t[J][int(r)] = 16 * I + g + 4 * r == 16 * J + n ? (double)lambda0 : 0.0; });
        });
    }
    // G parts of the segments before j, in order, PF parts in flight (as many
    // as the registers allow: four at d = 64, two otherwise)
    constexpr int PF = D == 64 ? 4 : 2;
    const int NPART = prefixed ? 1 : j * P;
    const double *gb = gram + (size_t)bh * S1 * P * DD + (prefixed ? (size_t)(j - 1) * P * DD : 0);
    auto load_part = [&](int s2, Tiles64<D> &x) {
        const double *G = gb + (size_t)s2 * DD;
        sfor<NB>([&](auto J) { sfor<4>([&](auto r) { x[J][int(r)] = G[rc(J, r)]; }); });
    };
    int s = 0;
    for (; s + PF <= NPART; s += PF) {
        Tiles64<D> x[PF];
        sfor<PF>([&](auto i) { load_part(s + i, x[i]); });
        sfor<PF>([&](auto i) { sfor<NB>([&](auto J) { t[J] += x[i][J]; }); });
    }
    for (; s < NPART; ++s) {
        Tiles64<D> x0;
        load_part(s, x0);
        sfor<NB>([&](auto J) { t[J] += x0[J]; });
    }
    sweep_tiles<D>(t, I, lane, rowbuf);   // -M^-1
    float *A = aseg + ((size_t)bh * S + j) * DD;
    sfor<NB>([&](auto J) { sfor<4>([&](auto r) { A[rc(J, r)] = (float)(-t[J][int(r)]); }); });
    if (tid < D) {
        double z = zk0 ? (double)zk0[bh * D + tid] : 0.0;
        const double *zb = zks + (size_t)bh * S1 * P * D + (prefixed ? (size_t)(j - 1) * P * D : 0) + tid;
        int s2 = 0;
        for (; s2 + 4 <= NPART; s2 += 4) {
            double x[4];
            sfor<4>([&](auto v) { x[v] = zb[(size_t)(s2 + v) * D]; });
            sfor<4>([&](auto v) { z += x[v]; });
        }
        for (; s2 < NPART; ++s2) z += zb[(size_t)s2 * D];
        zseg[((size_t)bh * S + j) * D + tid] = (float)z;
        if (zk0 && j == 1) zseg[(size_t)bh * S * D + tid] = zk0[bh * D + tid];
    }
}

// ------------------------------------------------------------------- penalty
// LDS of a penalty workgroup (the members the steps of Head use).
template <int D>
struct PLds {
    // the small, often-read arrays first, so that their offsets fit the 16-bit
    // immediate offsets of LDS instructions
    static constexpr int C = Cfg<D>::C, NA = Cfg<D>::NA, LD = Cfg<D>::LD, LT = Cfg<D>::LT;
    float gp[NA][2][C * LT]; // per wave: partials of I + U^'Z0 and Z0'K^
    float nq[NA][2][C * LT]; // per wave: partials of W'K^ and W'Phi
    float nrm[NA][C];        // per wave: partial |w_t|^2
    union {                  // L^-1 scratch of the factorisation / (I+N)^-1 scratch
        float lit[NA][C * LT];
        float tit[NA][C * LT];
    };
    float inv[NA][C];
    float hms[256];          // A operand of W' (per lane), from wave 0
    float mx[256];           // A operand of -(I + G)^-1 (per lane), from wave 0
    float wt[D * LT];        // W [i][token] of the last updated chunk
    float z0t[2][D * LT];    // Z0 [i][token], by chunk parity
    float uh[C * LD];        // u^ [token][i] of the chunk whose Z0 is formed next
    float kh[2][C * LD];     // k^, by chunk parity
    float ph[2][C * LD];     // phi(q), by chunk parity
    float zk[2][C * LD];     // phi(k), then the inclusive key sum, by chunk parity
};

// Staging of the penalty pass by its last NWS waves, LPT lanes per token (lane
// cc of token tl holds columns [cc CP, +CP)): raw q, k, u of a chunk into
// registers, then k^, u^, phi(q), phi(k) into LDS, k^ and phi(q) also to the
// chunk's record; later the readout denominators of the chunk.  With six waves
// (d = 96) four of them stage, 16 lanes per token, so that the raw inputs held
// across the update phase take half the registers.
__device__ __forceinline__ float sum_row8(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x;
}

template <int D, typename Tin, bool SAVE = false>
struct PenStage {
    static constexpr int LPT = Cfg<D>::NA >= 6 ? 16 : 8;   // lanes per token
    static constexpr int NWS = LPT * CH / 64;              // staging waves
    static constexpr int LD = Cfg<D>::LD, CP = D / LPT;
    int tl, cc;
    bool on;
    RawVec<Tin, CP> rq, rk, ru;
    __device__ __forceinline__ explicit PenStage(int ts)
        : tl((ts / LPT) & (CH - 1)), cc(ts % LPT), on(ts >= 0 && ts < LPT * CH)
    {
    }
    __device__ __forceinline__ static float row_sum(float x)
    {
        if constexpr (LPT == 16) return sum_row16(x);
        else return sum_row8(x);
    }
    // rows past T re-read row T-1 (stage zeroes k^, u^ and phi(k) there); the
    // views cover one head's T x d inputs
    __device__ __forceinline__ void prefetch(const Buf &qb, const Buf &kb, const Buf &ub, int T, int cq)
    {
        if (!on) return;
        const int t = cq * CH + tl;
        const unsigned off = ((unsigned)(t < T ? t : T - 1) * D + (unsigned)(cc * CP)) * sizeof(Tin);
        rq.load(qb, off);
        rk.load(kb, off);
        ru.load(ub, off);
    }
    __device__ __forceinline__ void stage(PLds<D> &L, int cq, int T, float *rkh, float *rph,
                                          float *kept = nullptr)
    {
        if (!on) return;
        const int slot = cq & 1;
        const bool ok = cq * CH + tl < T;
        float pk = 0.f, pu = 0.f;
#pragma unroll
        for (int i = 0; i < CP; ++i) {
            pk = fmaf(rk.get(i), rk.get(i), pk);
            pu = fmaf(ru.get(i), ru.get(i), pu);
        }
        const float nk = row_sum(pk), nu = row_sum(pu);
        const float ik = ok && nk > 0.f ? rsqrtf(nk) : 0.f;
        const float iu = ok && nu > 0.f ? rsqrtf(nu) : 0.f;
        if constexpr (SAVE) {
            if (cc == 0 && ok) {
                float *kt = kept + (size_t)(cq * CH + tl) * Keep<D>::RS + Keep<D>::SC;
                kt[3] = ik;
                kt[4] = iu;
            }
        }
        const int e0 = tl * LD + cc * CP;
#pragma unroll
        for (int i = 0; i < CP; ++i) {
            const int col = cc * CP + i;
            const float kv = rk.get(i) * ik, pq = phi_fast(rq.get(i));
            L.kh[slot][e0 + i] = kv;
            L.uh[e0 + i] = ru.get(i) * iu;
            L.ph[slot][e0 + i] = pq;
            L.zk[slot][e0 + i] = ok ? phi_fast(rk.get(i)) : 0.f;
            rkh[swzd<D>(tl, col >> 2) + (col & 3)] = kv;
            rph[swzd<D>(tl, col >> 2) + (col & 3)] = pq;
        }
    }
    // 1 / max(phi(q)' zkey, eps) per token of chunk cq (key sums in LDS) to rrd
    __device__ __forceinline__ void den(const PLds<D> &L, int cq, float eps, float *rrd,
                                        int T = 0, float *kept = nullptr) const
    {
        if (!on) return;
        const int slot = cq & 1, e0 = tl * LD + cc * CP;
        float pd = 0.f;
#pragma unroll
        for (int i = 0; i < CP; ++i) pd = fmaf(L.ph[slot][e0 + i], L.zk[slot][e0 + i], pd);
        pd = row_sum(pd);
        if (cc == 0) rrd[tl] = __builtin_amdgcn_rcpf(fmaxf(pd, eps));
        if constexpr (SAVE) {
            if (cq * CH + tl < T) {
                float *kt = kept + (size_t)(cq * CH + tl) * Keep<D>::RS;
                if constexpr (CP % 4 == 0) {
#pragma unroll
                    for (int i = 0; i < CP; i += 4)
                        st4(kt + Keep<D>::ZK + cc * CP + i, ld4(&L.zk[slot][e0 + i]));
                } else {
#pragma unroll
                    for (int i = 0; i < CP; ++i) kt[Keep<D>::ZK + cc * CP + i] = L.zk[slot][e0 + i];
                }
                if (cc == 0) kt[Keep<D>::SC + 2] = pd;
            }
        }
    }
};

// The penalty pass's W sink, which also keeps z_t and delta_t of each token
// (rows of L^-1 Z0' and the pivots of I + G) in the per-token records.
template <int D>
struct KeepW : WToLds<D, PLds<D>> {
    static constexpr bool KEEPS_Z = true;
    float *kept;   // this head's per-token records
    int tok, T;    // first token of the chunk, tokens
    __device__ __forceinline__ void zcols(int b, f4 q2, f4 inv4)
    {
        const int g = this->g, n = this->n;
        sfor<4>([&](auto r) {
            const int t = tok + 4 * g + r;
            if (t < T) {
                float *kt = kept + (size_t)t * Keep<D>::RS;
                kt[Keep<D>::Z + 16 * b + n] = q2[int(r)];
                if (b == 0 && n == 0) kt[Keep<D>::SC] = 1.f / inv4[int(r)];
            }
        });
    }
};

// X = Alpha^'Y (C x C) with Alpha^ = W diag(1/|w|) of the last updated chunk
// (W [i][token] and the |w|^2 partials in LDS) and Y (C x d, token-major in LDS,
// row stride LD) of the next one: register r of lane 16 g + n holds X[4 g + r][n]
// (stored as is, st4 at swz16(n, g), the record holds X').  One wave.
template <int D>
__device__ __forceinline__ f4 cross_factor(const PLds<D> &L, const float *y, int g, int n, float invm)
{
    constexpr int NB = D / 16, LD = Cfg<D>::LD, LT = Cfg<D>::LT;
    f4 x = {0.f, 0.f, 0.f, 0.f};
    sfor<NB>([&](auto b) {
        f4 aw;
        sfor<4>([&](auto r) { aw[int(r)] = L.wt[(16 * b + 4 * g + r) * LT + n] * invm; });
        x = mma4(aw, ld4(&y[n * LD + 16 * b + 4 * g]), x);
    });
    return x;
}

// Workgroup (head, segment j): the penalty chain over chunks [j SC, (j+1) SC)
// from A at the segment start, writing each chunk's record.  Two phases per
// chunk p, each ended by a barrier:
//   factorisation   all: Y0 of own blocks; wave 0: factorise I + G of chunk p;
//                   all: alpha^ of chunk p-1 to the record (1/|w| from the
//                   partials); wave 1: (I+N)^-1 and P of chunk p-1; cross
//                   factors of chunk p-1 (if even) with chunk p; key-sum
//                   prefix of chunk p; stage chunk p+1 (k^ and phi(q) also to
//                   its record), prefetch p+2
//   update          all: W, downdate A, |w|^2, W'K^ and W'Phi partials of
//                   chunk p; Z0 and the G partials of chunk p+1 from the new A
//                   (own blocks only, so no barrier in between); 1/den of
//                   chunk p.
//
// With SAVE, the per-token quantities the gradients need (Keep) also go to
// `kept`: z and delta from the factorisation, alpha^ and 1/|y| with the record,
// 1/|k|, 1/|u| and phi(q)'zkey from the staging.
template <int D, typename Tin, bool SAVE = false>
__global__ void __launch_bounds__(64 * Cfg<D>::NA)
vla_pen(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ u,
        int T, int S, int SC, float lambda0, float eps,
        const float *A0, const float *zk0, const float *aseg, const float *zseg,
        float *__restrict__ rec, float *A_out, float *zk_out, float *kept_all = nullptr)
{
    using Hd = Head<D, PLds<D>>;
    constexpr int BPW = Cfg<D>::BPW, LT = Cfg<D>::LT, RS = Rec<D>::SIZE, NA = Cfg<D>::NA;
    __shared__ __align__(16) PLds<D> L;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x / S, j = blockIdx.x % S;
    const size_t DD = (size_t)D * D;
    const int NC = (T + CH - 1) / CH;
    const int c0 = j * SC, c1 = min(NC, c0 + SC);

    // serial work spread over the waves.  Wave 0 factorises I + G and the waves
    // from 2 on own the key sums.  Six waves (d = 96): wave 1 forms the C x C
    // factors of the record and the key cross factors, the last wave the phi(q)
    // cross factors, and the last four stage the inputs.  Four waves: two
    // workgroups share a compute unit, and the dispatcher puts wave i of one on
    // the SIMD of wave i - 1 (mod 4) of the other (measured), so the roles are
    // spread to even out those pairs: waves 1 and 3 stage the inputs, and wave 2
    // forms the C x C factors and both cross factors besides its key sums.
    constexpr int NWS = PenStage<D, Tin, SAVE>::NWS;
    constexpr bool FOUR = NA == 4;
    const int lane = tid & 63;
    Hd hd(L, lane, w, tid - 128);
    PenStage<D, Tin, SAVE> ps(FOUR ? (w == 1 ? lane : (w == 3 ? 64 + lane : -1)) : tid - 64 * (NA - NWS));
    const int wfac = FOUR ? 2 : 1;   // the wave of the record's C x C factors
    float *kept = SAVE ? kept_all + (size_t)bh * T * Keep<D>::RS : nullptr;
    typename Hd::State st;
    const float *a_init;
    if (j > 0)
        a_init = aseg + ((size_t)bh * S + j) * DD;
    else
        a_init = A0 ? (S > 1 ? aseg + (size_t)bh * S * DD : A0 + bh * DD) : nullptr;
    hd.load_state(st, a_init, 1.f / lambda0);
    if (hd.kcol >= 0) {
        if (j > 0)
            hd.zk_run = zseg[((size_t)bh * S + j) * D + hd.kcol];
        else if (zk0)
            hd.zk_run = S > 1 ? zseg[(size_t)bh * S * D + hd.kcol] : zk0[bh * D + hd.kcol];
    }
    const size_t hoff = (size_t)bh * T * D;
    const unsigned hbytes = (unsigned)T * D * sizeof(Tin);
    const Buf qb(q + hoff, hbytes), kb(k + hoff, hbytes), ub(u + hoff, hbytes);
    float *rb = rec + ((size_t)bh * NC + c0) * RS;   // record of chunk p below
    ps.prefetch(qb, kb, ub, T, c0);
    ps.stage(L, c0, T, rb + Rec<D>::KH, rb + Rec<D>::PH, kept);
    if (c0 + 1 < c1) ps.prefetch(qb, kb, ub, T, c0 + 1);
    vmem_drain();
    __syncthreads();
    hd.z_products(st, c0);
    lds_barrier();

    auto sink = [&]() {
        if constexpr (SAVE) return KeepW<D>{{L, hd.g, hd.n}, kept, 0, T};
        else return WToLds<D, PLds<D>>{L, hd.g, hd.n};
    };
    auto wl = sink();
    // alpha^ of the last updated chunk (record at rp, first token tp) from W in
    // L.wt and the |w|^2 partials: the own blocks
    auto alpha_out = [&](float *rp, int tp, f4 invn4) {
        sfor<BPW>([&](auto bb) {
            const int b = w * BPW + bb;
            const f4 a = ld4(&L.wt[(16 * b + hd.n) * LT + 4 * hd.g]) * invn4;
            st4(&rp[Rec<D>::AH + swz16(16 * b + hd.n, hd.g)], a);
            if constexpr (SAVE) {
                sfor<4>([&](auto r) {
                    const int t = tp + 4 * hd.g + r;
                    if (t < T) {
                        float *kt = kept + (size_t)t * Keep<D>::RS;
                        kt[Keep<D>::AL + 16 * b + hd.n] = a[int(r)];
                        if (b == 0 && hd.n == 0) kt[Keep<D>::SC + 1] = invn4[int(r)];
                    }
                });
            }
        });
    };
    // Alpha^'K^ of an even chunk with the next, kept by wave wfac until the
    // next chunk's (I + N)^-1 exists; the record gets it solved (solved_cross)
    f4 qk = {0.f, 0.f, 0.f, 0.f};
    // the C x C factors of chunk c (record at rc), with the solved key cross
    // factor of the pair (c - 1, c) when chunk c - 1 is an even chunk of the segment
    auto factors = [&](float *rc, int c, f4 invn4) {
        if (w == wfac) {
            const bool pair = c - 1 >= c0 && ((c - 1) & 1) == 0;
            hd.prep_tp(rc + Rec<D>::TT, rc + Rec<D>::PT, invn4, qk, pair ? rc - RS + Rec<D>::QK : nullptr);
        }
    };
    for (int p = c0; p < c1; ++p, rb += RS) {
        f4 y[BPW];
        hd.y_products(st, p, y);
        if (w == 0) hd.template factorize<!SAVE>();
        if (p > c0) {
            const f4 invn4 = hd.inv_norms4();
            alpha_out(rb - RS, (p - 1) * CH, invn4);
            factors(rb - RS, p - 1, invn4);
            if (((p - 1) & 1) == 0) {   // cross factors of an even chunk with the next
                if (FOUR ? w == 2 : w == 1) {   // wave wfac
                    const float invm = hd.inv_norm_n();
                    qk = cross_factor<D>(L, L.kh[p & 1], hd.g, hd.n, invm);
                    if constexpr (FOUR)
                        st4(&(rb - RS + Rec<D>::QP)[swz16(hd.n, hd.g)],
                            cross_factor<D>(L, L.ph[p & 1], hd.g, hd.n, invm));
                } else if (!FOUR && w == NA - 1) {
                    st4(&(rb - RS + Rec<D>::QP)[swz16(hd.n, hd.g)],
                        cross_factor<D>(L, L.ph[p & 1], hd.g, hd.n, hd.inv_norm_n()));
                }
            }
        }
        hd.stage2(p);
        if (p + 1 < c1) {
            ps.stage(L, p + 1, T, rb + RS + Rec<D>::KH, rb + RS + Rec<D>::PH, kept);
            if (p + 2 < c1) ps.prefetch(qb, kb, ub, T, p + 2);
        }
        lds_barrier();
        if constexpr (SAVE) wl.tok = p * CH;
        hd.downdate(st, p, y, wl);
        if (p + 1 < c1) hd.z_products(st, p + 1);
        ps.den(L, p, eps, rb + Rec<D>::RD, T, kept);
        lds_barrier();
    }
    if (c1 > c0) {   // the last chunk's alpha^ and C x C factors
        const f4 invn4 = hd.inv_norms4();
        alpha_out(rb - RS, (c1 - 1) * CH, invn4);
        factors(rb - RS, c1 - 1, invn4);
    }
    if (j == S - 1) {
        if (A_out) hd.store_state(st, A_out + bh * DD);
        if (hd.kcol >= 0 && zk_out) zk_out[bh * D + hd.kcol] = hd.zk_run;
    }
}

// ------------------------------------------------------------------- memory
// Staging of the memory pass: per pair of chunks, the two records (as stored)
// and the workgroup's columns of v for the 32 tokens (token-major), copied
// from device memory straight into LDS in 1 KB pieces (16 bytes per lane),
// the same number of pieces per wave.
template <int D, typename Tin>
struct MemStage {
    static constexpr int VBW = MemCfg<D>::VBW, KS = MemCfg<D>::KS, NW = VBW * KS;
    static constexpr int RS = Rec<D>::SIZE;
    static constexpr int NR = (2 * RS * 4 + 1023) / 1024;      // pieces of the records
    static constexpr int ROWB = 16 * VBW * (int)sizeof(Tin);   // bytes of v per token
    static constexpr int NV = 32 * ROWB / 1024;                // pieces of v
    static constexpr int NI = (NR + NV + NW - 1) / NW * NW;    // pieces per pair
    static constexpr int NIW = NI / NW;                        // per wave
    static constexpr int VOFF = 256 * (NI - NV);               // v, in floats from the stage start
    static constexpr int SIZE = 256 * NI;                      // floats per stage
    static constexpr int NS = 3 * SIZE * 4 + 2 * NW * 4096 <= 160 * 1024 ? 3 : 2;   // stages
    static_assert(NV * 1024 == 32 * ROWB && 2 * SIZE * 4 + 2 * NW * 4096 <= 160 * 1024, "LDS");
};

// Operands of one chunk for one memory wave, read from its stage: k^ and phi(q)
// of token n, keys 16 rho + 4 g + [0, 4) (rho = the wave's key tiles);
// alpha^[16 rho + n][4 g + r]; the transposed C x C factors at row n; 1/den of
// token n; v of token 4 g + r, value 16 b + n.
template <int NT>
struct MemOps {
    f4 ak[NT], ap[NT], aw[NT], ta, pa;
    float rd, v[4];
};

// Workgroup (head, value group): VBW value blocks of 16 rows; wave w takes block
// w / KS and key tiles [NT (w % KS), +NT).  The state tiles are S' in MFMA
// accumulator layout (register r of lane 16 g + n of tile rho holds
// S[16 b + n][16 rho + 4 g + r]).
//
// The chain runs over pairs of chunks (a, b) from S at the start of a:
//   (S K_a)', (S K_b)' (token x value) and S Phi_a, S Phi_b (value x token)
//   partials of the own key tiles -> LDS                           | barrier
//   sum the KS partials (same order in every wave);
//   E_a' = T_a'(V_a - S K^_a)';
//   E_b' = T_b'(V_b - S K^_b - E_a Alpha^_a'K^_b)'   (S after a, applied to K^_b),
//   formed as T_b'(V_b - S K^_b)' + X_ab' E_a' with the record's solved cross
//   factor X_ab = -(Alpha^_a'K^_b) T_b, so only the last product waits for E_a;
//   key split 0: o_a = (S Phi_a + E_a P_a) / den, key split 1:
//   o_b = (S Phi_b + E_a Alpha^_a'Phi_b + E_b P_b) / den  (value x token, so
//   that a lane stores four consecutive values of one token; formed in the
//   next step, once the S Phi partials of the other waves have crossed its
//   barrier);
//   S' += Alpha^_a E_a' + Alpha^_b E_b'.
// An odd last chunk takes the single-chunk form of the same step.
//
// Pair p is staged in LDS stage p mod NS.  Every wave copies its pieces of pair
// p + NS after the barrier of step p (all reads of stage p mod NS are done by
// then), spread over the step, and waits for its pieces of pair p + 1 before
// the barrier of step p, so that the barrier publishes them.
//
// With SAVE, the errors e_t also go to the per-token records (Keep): key split
// 0 writes chunk a's, key split 1 chunk b's, the others store through an empty
// view, so that every wave issues the same number of stores.
//
// With LIN (records of cumulative-sum linear attention: k^ = 0 and
// (I + N)^-1 = I), the errors are the values themselves, so the products with
// K^ and the triangular solves are skipped.
template <int D, typename Tin, bool SAVE = false, bool LIN = false>
__global__ void __launch_bounds__(64 * MemCfg<D>::VBW * MemCfg<D>::KS)
vla_mem(const Tin *__restrict__ v, int T, int BH, const float *__restrict__ rec, const float *S0,
        float *__restrict__ o, float *S_out, float *kept_all = nullptr)
{
    using MS = MemStage<D, Tin>;
    using R = Rec<D>;
    constexpr int NB = D / 16, VBW = MS::VBW, KS = MS::KS, NW = MS::NW, NT = NB / KS;
    constexpr int NG = NB / VBW, RS = R::SIZE, NS = MS::NS, NIW = MS::NIW;
    static_assert(NT * KS == NB && NG * VBW == NB && KS >= 2, "block split");
    // the stages: three separate arrays, or two with no third allocated (at
    // d = 128 with fp32 inputs the two fill the LDS to the byte)
    float *stg[3];
    if constexpr (NS == 3) {
        __shared__ __align__(16) float stg0[MS::SIZE];
        __shared__ __align__(16) float stg1[MS::SIZE];
        __shared__ __align__(16) float stg2[MS::SIZE];
        stg[0] = stg0;
        stg[1] = stg1;
        stg[2] = stg2;
    } else {
        __shared__ __align__(16) float stg0[MS::SIZE];
        __shared__ __align__(16) float stg1[MS::SIZE];
        stg[0] = stg0;
        stg[1] = stg1;
        stg[2] = stg0;
    }
    __shared__ __align__(16) float red[2][NW][4][256];   // per step parity and wave: partials

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int vbl = w / KS, ks = w % KS;
    // the NG workgroups of a head share an XCD (blockIdx mod 8) and its L2
    int bh, vg;
    const int x = blockIdx.x;
    if (BH % 8 == 0) {
        const int s = x >> 3;
        bh = (s / NG) * 8 + (x & 7);
        vg = s % NG;
    } else {
        bh = x / NG;
        vg = x % NG;
    }
    const int b = vg * VBW + vbl;
    const int rho0 = ks * NT;
    const int NC = (T + CH - 1) / CH, NP = NC / 2, NPT = (NC + 1) / 2;
    const size_t DD = (size_t)D * D;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    const Buf rbuf(rec + (size_t)bh * NC * RS, (unsigned)(NC * RS * 4));
    const Buf vbuf(v + (size_t)bh * T * D, (unsigned)T * D * (unsigned)sizeof(Tin));
    float *oh = o + (size_t)bh * T * D;
    float *kept = SAVE ? kept_all + (size_t)bh * T * Keep<D>::RS : nullptr;
    // the errors of chunk c (this wave's value block) to the records; rows past
    // T are dropped
    auto keep_e = [&](int c, bool mine, f4 e) {
        const Buf kb_(kept, mine ? (unsigned)T * Keep<D>::RS * 4u : 0u);
        sfor<4>([&](auto r) {
            kb_.st32(e[int(r)], 4u * ((unsigned)(c * CH + 4 * g + r) * Keep<D>::RS + Keep<D>::E + 16 * b + n));
        });
    };

    f4 st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        st[t] = S0 ? ld4(&S0[bh * DD + (size_t)(16 * b + n) * D + 16 * (rho0 + t) + 4 * g]) : zero;

    // this wave's pieces [I0, I1) of pair pm into stage s (pieces w, w + NW, ...)
    constexpr int NRP = MS::NI - MS::NV;   // pieces of records
    auto stage_pieces = [&](auto I0, auto I1, int pm, float *s) {
        pm = min(pm, NPT - 1);
        auto rpiece = [&](int j) {
            rbuf.lds16(s + 256 * j, (unsigned)(1024 * j + 16 * lane), (unsigned)pm * 2 * RS * 4);
        };
        auto vpiece = [&](int j) {
            // byte b of the pair's v slice (tokens of ROWB bytes back to back; a
            // 16-byte granule never straddles two tokens, ROWB being a multiple of 16)
            const unsigned b = 1024u * (unsigned)(j - NRP) + 16u * (unsigned)lane;
            const unsigned tp = b / MS::ROWB, cb = b % MS::ROWB;   // token in the pair, byte in its row
            const unsigned off = ((32u * (unsigned)pm + tp) * D + 16u * VBW * (unsigned)vg) * sizeof(Tin) + cb;
            vbuf.lds16(s + 256 * j, off);
        };
        sfor<decltype(I1)::value - decltype(I0)::value>([&](auto i0) {
            constexpr int i = decltype(I0)::value + decltype(i0)::value;
            const int j = w + NW * i;
            if constexpr (NW * (i + 1) <= NRP) rpiece(j);
            else if constexpr (NW * i >= NRP) vpiece(j);
            else if (j < NRP) rpiece(j);
            else vpiece(j);
        });
    };
    auto stage_pair = [&](int pm, float *s) { stage_pieces(ic<0>{}, ic<NIW>{}, pm, s); };
    // the pieces of one step, spread over six points of its second half, so
    // that the copies of the four waves do not queue up at once
    auto stage_part = [&](auto K, int pm, float *s) {
        constexpr int k = decltype(K)::value;
        __builtin_amdgcn_sched_barrier(0);
        stage_pieces(ic<k * NIW / 6>{}, ic<(k + 1) * NIW / 6>{}, pm, s);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto ops = [&](const float *s, int xc, MemOps<NT> &m) {   // chunk xc (0 or 1) of a stage
        const float *c = s + xc * RS;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (!LIN) m.ak[t] = ld4(c + R::KH + swzd<D>(n, 4 * (rho0 + t) + g));
            m.ap[t] = ld4(c + R::PH + swzd<D>(n, 4 * (rho0 + t) + g));
            m.aw[t] = ld4(c + R::AH + swz16(16 * (rho0 + t) + n, g));
        }
        if constexpr (!LIN) m.ta = ld4(c + R::TT + swz16(n, g));
        m.pa = ld4(c + R::PT + swz16(n, g));
        m.rd = c[R::RD + n];
        const Tin *vs = reinterpret_cast<const Tin *>(s + MS::VOFF);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            m.v[r] = load_in(vs, (16 * xc + 4 * g + r) * (16 * VBW) + 16 * vbl + n);
    };
    auto sk_part = [&](const f4 (&a)[NT]) {   // (S K)' partial: token x value
        f4 acc = zero;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = mma(a[t][r], st[t][r], acc);
        }
        return acc;
    };
    auto sq_part = [&](const f4 (&a)[NT]) {   // S Phi partial: value x token
        f4 acc = zero;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = mma(st[t][r], a[t][r], acc);
        }
        return acc;
    };
    auto reduce = [&](int sl, int slot) {
        f4 s = ld4(&red[sl][vbl * KS][slot][lane * 4]);
#pragma unroll
        for (int s2 = 1; s2 < KS; ++s2) s += ld4(&red[sl][vbl * KS + s2][slot][lane * 4]);
        return s;
    };
    auto errors = [&](const MemOps<NT> &m, f4 sk) {   // E' = T'(V - S K^)'
        f4 vm;   // v past T reads as 0 (and k^ is 0 there)
#pragma unroll
        for (int r = 0; r < 4; ++r) vm[r] = m.v[r] - sk[r];
        return mma4(m.ta, vm, zero);
    };
    auto values = [&](const MemOps<NT> &m) {   // E' = V' (linear attention)
        f4 vm;
#pragma unroll
        for (int r = 0; r < 4; ++r) vm[r] = m.v[r];
        return vm;
    };
    // o of chunk c (value x token) from this wave when it writes it (others
    // store through an empty view, so that every store is unconditional)
    auto store_o = [&](int c, bool mine, f4 ob, float rd) {
        const Buf ob_(oh + (size_t)c * CH * D, mine ? (unsigned)(T - c * CH) * D * 4u : 0u);
        ob_.st128(ob * rd, 4u * (n * D + 16 * b + 4 * g));   // rows past T dropped
    };
    auto update = [&](const MemOps<NT> &m, f4 e) {   // S' += Alpha^ E'
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int t = 0; t < NT; ++t) st[t] = mma(m.aw[t][r], e[r], st[t]);
        }
    };
    // the wait before the barrier of a step: this wave's pieces of the next
    // pair (behind them: the step's store, and for three stages the copies and
    // the store of one more step)
    constexpr int NST = SAVE ? 5 : 1;   // stores per step
    auto wait_next = [&]() {
        if constexpr (NS == 3) vm_wait<NIW + 2 * NST>();
        else vm_wait<NST>();
    };
    // The readout of a pair needs the S Phi partials of the other waves, which
    // are formed after the barrier of the pair's step (off the chain from S to
    // S) and published by the barrier of the next step: the readout of pair p
    // happens in step p + 1.  What it needs of pair p is carried along.
    struct Carry {
        f4 ea, eb, pa, pb, qp;
        float rd;
    } cy = {zero, zero, zero, zero, zero, 0.f};
    auto readout = [&](int sl) {   // the carried pair, partials in red[sl]
        if (ks == 0) return mma4(cy.ea, cy.pa, reduce(sl, 2));
        return mma4(cy.eb, cy.pb, mma4(cy.ea, cy.qp, reduce(sl, 3)));
    };
    auto step2 = [&](int pm, float *s) {
        const int sl = pm & 1;
        MemOps<NT> ma, mb;
        ops(s, 0, ma);
        ops(s, 1, mb);
        const f4 qp = ld4(s + R::QP + swz16(n, g));
        f4 qk = zero;
        if constexpr (!LIN) {
            qk = ld4(s + R::QK + swz16(n, g));
            st4(&red[sl][w][0][lane * 4], sk_part(ma.ak));
            st4(&red[sl][w][1][lane * 4], sk_part(mb.ak));
        }
        // the S Phi partials are formed before the barrier and go to LDS after
        // it (read one step later)
        const f4 sqa = sq_part(ma.ap), sqb = sq_part(mb.ap);
        wait_next();
        lds_barrier();
        stage_part(ic<0>{}, pm + NS, s);
        // T_b'(V_b - S K^_b)' does not wait for E_a; the record's key cross
        // factor is already solved (Y = -T_b'(Alpha^_a'K^_b)')
        const f4 xb = LIN ? zero : errors(mb, reduce(sl, 1));
        const f4 ea = LIN ? values(ma) : errors(ma, reduce(sl, 0));
        stage_part(ic<1>{}, pm + NS, s);
        const f4 ob = readout(sl ^ 1);   // pair pm - 1 (nothing at pm = 0)
        stage_part(ic<2>{}, pm + NS, s);
        const f4 eb = LIN ? values(mb) : mma4(qk, ea, xb);
        stage_part(ic<3>{}, pm + NS, s);
        update(ma, ea);
        stage_part(ic<4>{}, pm + NS, s);
        update(mb, eb);
        st4(&red[sl][w][2][lane * 4], sqa);
        st4(&red[sl][w][3][lane * 4], sqb);
        stage_part(ic<5>{}, pm + NS, s);
        // the step's only store, after its copies (so the waits above count
        // one store and the copies of a step)
        const int cp = 2 * (pm - 1) + (ks == 0 ? 0 : 1);
        store_o(max(cp, 0), pm > 0 && ks < 2, ob, cy.rd);
        if constexpr (SAVE) keep_e(2 * pm + (ks == 0 ? 0 : 1), ks < 2, ks == 0 ? ea : eb);
        cy = Carry{ea, eb, ma.pa, mb.pa, qp, ks == 0 ? ma.rd : mb.rd};
    };

    stage_pair(0, stg[0]);
    stage_pair(1, stg[1]);
    if constexpr (NS == 3) stage_pair(2, stg[NS - 1]);
    vm_wait<0>();
    lds_barrier();
    int pm = 0;
    if constexpr (NS == 3) {
        for (; pm + 3 <= NP; pm += 3) {
            step2(pm, stg[0]);
            step2(pm + 1, stg[1]);
            step2(pm + 2, stg[NS - 1]);
        }
        if (pm < NP) step2(pm, stg[0]);
        if (pm + 1 < NP) step2(pm + 1, stg[1]);
    } else {
        for (; pm + 2 <= NP; pm += 2) {
            step2(pm, stg[0]);
            step2(pm + 1, stg[1]);
        }
        if (pm < NP) step2(pm, stg[0]);
    }
    if (NP > 0) {   // the readout of the last pair
        lds_barrier();
        store_o(2 * (NP - 1) + (ks == 0 ? 0 : 1), ks < 2, readout((NP - 1) & 1), cy.rd);
    }
    if (NC & 1) {   // the last chunk alone (staged as pair NP)
        const int c = NC - 1, sl = NP & 1, k = NP % NS;
        const float *s = stg[k];
        MemOps<NT> m;
        ops(s, 0, m);
        if constexpr (!LIN) st4(&red[sl][w][0][lane * 4], sk_part(m.ak));
        st4(&red[sl][w][2][lane * 4], sq_part(m.ap));
        lds_barrier();
        const f4 e = LIN ? values(m) : errors(m, reduce(sl, 0));
        store_o(c, ks == 0, mma4(e, m.pa, reduce(sl, 2)), m.rd);
        if constexpr (SAVE) keep_e(c, ks == 0, e);
        update(m, e);
    }
    vm_wait<0>();   // no copy into LDS outlives the workgroup
    if (S_out) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            st4(&S_out[bh * DD + (size_t)(16 * b + n) * D + 16 * (rho0 + t) + 4 * g], st[t]);
    }
}

// ------------------------------------------------------------------- host
inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    int NC = 0, S = 1, SC = 0, P = 1;   // chunks, segments, chunks per segment, gram parts
    size_t rec = 0, gram = 0, zks = 0, aseg = 0, zseg = 0, bytes = 0;
};

// Segments: enough penalty workgroups to fill the device (two per compute unit
// at d = 64, whose LDS allows two; one otherwise), at least two chunks each.
Plan make_plan(int BH, int T, int D)
{
    Plan p;
    p.NC = (T + CH - 1) / CH;
    if (p.NC == 0) return p;
    const int target = D == 64 ? 512 : 256;
    int S = (target + BH - 1) / BH;
    const int smax = p.NC / 2 > 1 ? p.NC / 2 : 1;
    S = S < smax ? S : smax;
    p.SC = (p.NC + S - 1) / S;
    p.SC += p.SC & 1;   // segments start at even chunks (pairs of the memory pass)
    p.S = (p.NC + p.SC - 1) / p.SC;
    if (p.S > 1) {   // gram parts: at most one round of workgroups (LDS allows
                     // 3, 2, 1 per compute unit at d = 64, 96, 128), each at
                     // least 4 chunks
        const int round = 256 * (D == 64 ? 3 : D == 96 ? 2 : 1);
        const int want = round / (BH * (p.S - 1));
        const int most = p.SC / 4 > 1 ? p.SC / 4 : 1;
        p.P = want < 1 ? 1 : (want < most ? want : most);
    }
    const int rs = 48 * D + 4 * CH * CH + CH;   // Rec<D>::SIZE
    size_t off = 0;
    p.rec = off;
    off = up256(off + (size_t)BH * p.NC * rs * sizeof(float));
    if (p.S > 1) {
        p.gram = off;
        off = up256(off + (size_t)BH * (p.S - 1) * p.P * D * D * sizeof(double));
        p.zks = off;
        off = up256(off + (size_t)BH * (p.S - 1) * p.P * D * sizeof(double));
        p.aseg = off;
        off = up256(off + (size_t)BH * p.S * D * D * sizeof(float));
        p.zseg = off;
        off = up256(off + (size_t)BH * p.S * D * sizeof(float));
    }
    p.bytes = off;
    return p;
}

template <int D, typename Tin>
hipError_t launch(const FwdArgs &a, int phases)
{
    const int BH = a.B * a.H;
    const Plan p = make_plan(BH, a.T, D);
    char *ws = static_cast<char *>(a.ws);
    float *rec = reinterpret_cast<float *>(ws + p.rec);
    double *gram = reinterpret_cast<double *>(ws + p.gram);
    double *zks = reinterpret_cast<double *>(ws + p.zks);
    float *aseg = reinterpret_cast<float *>(ws + p.aseg);
    float *zseg = reinterpret_cast<float *>(ws + p.zseg);
    const Tin *q = (const Tin *)a.q, *k = (const Tin *)a.k, *v = (const Tin *)a.v,
              *u = (const Tin *)a.u;
    if (phases & 1) {
        if (p.S > 1) {
            hipLaunchKernelGGL((vla_gram<D, Tin>), dim3(BH * (p.S - 1) * p.P), dim3(256), 0, a.stream,
                               k, u, a.T, p.S, p.SC, p.P, gram, zks);
            // prefix sums over the segments once a head has many (a launch
            // more than the direct sums cost with a few)
            const bool prefixed = (p.S - 1) * p.P > 16;
            if (prefixed)
                hipLaunchKernelGGL((vla_gram_prefix<D>), dim3(BH * ((D * D + D + 255) / 256)), dim3(256), 0,
                                   a.stream, p.S, p.P, gram, zks);
            hipLaunchKernelGGL((vla_seginv<D>), dim3(BH * (p.S - 1)), dim3(4 * D), 0, a.stream, p.S,
                               p.P, a.lambda0, a.A0, a.zk0, gram, zks, aseg, zseg, prefixed);
        }
        if (a.keep)
            hipLaunchKernelGGL((vla_pen<D, Tin, true>), dim3(BH * p.S), dim3(64 * Cfg<D>::NA), 0,
                               a.stream, q, k, u, a.T, p.S, p.SC, a.lambda0, a.eps, a.A0, a.zk0,
                               aseg, zseg, rec, a.A_out, a.zk_out, a.keep);
        else
            hipLaunchKernelGGL((vla_pen<D, Tin>), dim3(BH * p.S), dim3(64 * Cfg<D>::NA), 0, a.stream,
                               q, k, u, a.T, p.S, p.SC, a.lambda0, a.eps, a.A0, a.zk0, aseg, zseg,
                               rec, a.A_out, a.zk_out, nullptr);
    }
    if (phases & 2) {
        constexpr int NG = (D / 16) / MemCfg<D>::VBW;
        if (a.keep)
            hipLaunchKernelGGL((vla_mem<D, Tin, true>), dim3(BH * NG),
                               dim3(64 * MemCfg<D>::VBW * MemCfg<D>::KS), 0, a.stream, v, a.T, BH,
                               rec, a.S0, a.o, a.S_out, a.keep);
        else
            hipLaunchKernelGGL((vla_mem<D, Tin>), dim3(BH * NG),
                               dim3(64 * MemCfg<D>::VBW * MemCfg<D>::KS), 0, a.stream, v, a.T, BH,
                               rec, a.S0, a.o, a.S_out, nullptr);
    }
    return hipGetLastError();
}

template <int D, typename Tin>
hipError_t launch_mem_only(const FwdArgs &a, const float *rec, bool lin)
{
    constexpr int NG = (D / 16) / MemCfg<D>::VBW;
    const int BH = a.B * a.H;
    const dim3 grid(BH * NG), block(64 * MemCfg<D>::VBW * MemCfg<D>::KS);
    if (lin)
        hipLaunchKernelGGL((vla_mem<D, Tin, false, true>), grid, block, 0, a.stream,
                           (const Tin *)a.v, a.T, BH, rec, a.S0, a.o, a.S_out, nullptr);
    else
        hipLaunchKernelGGL((vla_mem<D, Tin>), grid, block, 0, a.stream, (const Tin *)a.v, a.T, BH,
                           rec, a.S0, a.o, a.S_out, nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_memory_pass(const FwdArgs &a, const float *rec, bool lin)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch_mem_only<64, uint16_t>(a, rec, lin) : launch_mem_only<64, float>(a, rec, lin);
    case 96: return bf ? launch_mem_only<96, uint16_t>(a, rec, lin) : launch_mem_only<96, float>(a, rec, lin);
    case 128: return bf ? launch_mem_only<128, uint16_t>(a, rec, lin) : launch_mem_only<128, float>(a, rec, lin);
    default: return hipErrorInvalidValue;
    }
}

bool chunk_supported(int d) { return d == 64 || d == 96 || d == 128; }

// The passes address a head's records, per-token records, inputs and o with
// 32-bit byte offsets (buffer resources); each must stay below 2^31 bytes.
template <int D>
static bool fits(long long T, bool keep)
{
    const long long lim = 1LL << 31, NC = (T + CH - 1) / CH;
    if (NC * Rec<D>::SIZE * 4 >= lim || T * D * 4 >= lim) return false;
    return !keep || T * Keep<D>::RS * 4 < lim;
}

bool twopass_size_ok(int T, int d, bool keep)
{
    switch (d) {
    case 64: return fits<64>(T, keep);
    case 96: return fits<96>(T, keep);
    case 128: return fits<128>(T, keep);
    default: return (long long)T * d * 4 < (1LL << 31) &&
                    (!keep || (long long)T * (4 * d + 8) * 4 < (1LL << 31));
    }
}

size_t twopass_workspace_bytes(int BH, int T, int d)
{
    return make_plan(BH, T, d).bytes;
}

size_t twopass_records_offset(int BH, int T, int d)
{
    return make_plan(BH, T, d).rec;
}

hipError_t launch_forward_twopass(const FwdArgs &a, int phases)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch<64, uint16_t>(a, phases) : launch<64, float>(a, phases);
    case 96: return bf ? launch<96, uint16_t>(a, phases) : launch<96, float>(a, phases);
    case 128: return bf ? launch<128, uint16_t>(a, phases) : launch<128, float>(a, phases);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
