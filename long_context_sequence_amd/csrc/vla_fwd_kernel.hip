// vla_fwd_kernel.hip -- register-resident gfx950 kernel of the VLA recurrence
// for d_h in {64, 96, 128}.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9) (Sherman-Morrison downdate of A), (10) (gated delta write of S) and
// (11) (ELU+1 readout with the running key sum); A_0 = I / lambda0 (section 3.2).
//
// Mapping.  One workgroup owns one (batch, head) for all T tokens.  It has
// 2*NH wavefronts, NH = d/16: "A-waves" 0..NH-1 carry the penalty chain (Eq. 9
// and the gate of Eq. 10) and "S-waves" NH..2NH-1 carry the memory chain (the
// write of Eq. 10 and the readout of Eq. 11), so every SIMD runs one wave of
// each chain and overlaps the stalls of one with the arithmetic of the other.
// Wave h of a chain owns rows 16h .. 16h+15 of its matrix; lane l = 16g + n
// (g = lane group = 16-lane DPP row, n = row within it) holds row 16h + n and
// the columns of group g:
//     columns 16g + m            for m = 0..15
//     columns 64 + SW1 g + m     for m = 0..SW1-1   (SW1 = (d-64)/4)
// i.e. CPL = 16 + SW1 matrix entries per lane, in VGPRs for the whole sequence.
// A "lane-distributed" vector keeps element 16g + n in lane 16g + n (and
// element 64 + SW1 g + n in a second register), so column j of the whole 16-lane
// row is one DPP row_newbcast away: every multiply-add of the matrix-vector
// products and rank-1 updates is a single v_fmac_f32 with a DPP-broadcast
// source.  Row sums over the four lane groups use the gfx950 permlane32/16 swaps.
//
// Per token, the only cross-wave exchange is an LDS all-gather of z (the
// Sherman-Morrison vector) and y (= A k^) plus four dot-product partials, behind
// one s_barrier.  The penalty chain runs one token ahead of the memory chain and
// the readout one token behind it:
//     iteration t:  A-waves: apply z_{t-1}; z_t = A u^_t, w_t = A k^_t;
//                            y_{t-1} = w_{t-1} - z_{t-1} (z_{t-1}'k^_{t-1})/delta
//                            (Eq. 9 applied to k^, i.e. A_{t-1} k^ from A_{t-2} k^)
//                   S-waves: apply e_{t-2} alpha^_{t-2}; S k^_{t-1}, S phi(q_{t-1});
//                            e_{t-1}; readout o_{t-2}
//
// State-independent work (k^, u^, phi(q), the key-sum prefix and the readout
// denominator) is done per tile of TT tokens in a prologue and kept in an LDS
// ring of RING token records; the raw inputs of the next tile are prefetched
// into registers while the current tile runs.
#include <utility>

#include "vla_common.h"

namespace vla {
namespace {

template <typename F, int... Is>
__device__ __forceinline__ void sfor_impl(F &&f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void sfor(F &&f)
{
    sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// acc += x[lane M of this 16-lane row] * y.
// The broadcast source x must not be written by a VALU instruction right before
// this (DPP read-after-VALU-write hazard, invisible to the compiler inside asm):
// every x used here comes straight from an LDS load.
template <int M>
__device__ __forceinline__ void fmac_bc(float &acc, float x, float y)
{
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(x), "v"(y), "n"(M));
}

// acc = x[lane M of this 16-lane row] * y (same hazard rule as fmac_bc).
template <int M>
__device__ __forceinline__ void fmul_bc(float &acc, float x, float y)
{
    asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "=v"(acc)
        : "v"(x), "v"(y), "n"(M));
}

// One pass over a lane's CPL matrix entries:
//     mv[m] += x[col m] * mult                  (rank-1 update of the row)
//     acc1   = sum_m y1[col m] * mv[m]          (two matrix-vector products with
//     acc2   = sum_m y2[col m] * mv[m]           the updated row)
// where x, y1, y2 are lane-distributed vectors (registers ..0: columns 16g + m,
// registers ..1: columns 64 + SW1 g + m).  Each asm block covers 8 columns in the
// order update(i+1), acc1(i), acc2(i): an entry is read three instructions after
// its update and an accumulator three instructions after its previous write.
// Inside a block the DPP sources (x, y1, y2) are never written, so no wait states
// are needed; every DPP source comes straight from an LDS load.
#define VLA_MAC(D, S, M, L) "v_fmac_f32_dpp " D ", " S ", " M " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n\t"
#define VLA_MUL(D, S, M, L) "v_mul_f32_dpp " D ", " S ", " M " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n\t"
// operands: %0..%7 entries, %8 acc1, %9 acc2, %10 x, %11 mult, %12 y1, %13 y2
#define VLA_CHUNK(A0, L0, L1, L2, L3, L4, L5, L6, L7)                                   \
    VLA_MAC("%0", "%10", "%11", L0) VLA_MAC("%1", "%10", "%11", L1)                     \
    A0("%8", "%12", "%0", L0) A0("%9", "%13", "%0", L0)                                  \
    VLA_MAC("%2", "%10", "%11", L2) VLA_MAC("%8", "%12", "%1", L1) VLA_MAC("%9", "%13", "%1", L1) \
    VLA_MAC("%3", "%10", "%11", L3) VLA_MAC("%8", "%12", "%2", L2) VLA_MAC("%9", "%13", "%2", L2) \
    VLA_MAC("%4", "%10", "%11", L4) VLA_MAC("%8", "%12", "%3", L3) VLA_MAC("%9", "%13", "%3", L3) \
    VLA_MAC("%5", "%10", "%11", L5) VLA_MAC("%8", "%12", "%4", L4) VLA_MAC("%9", "%13", "%4", L4) \
    VLA_MAC("%6", "%10", "%11", L6) VLA_MAC("%8", "%12", "%5", L5) VLA_MAC("%9", "%13", "%5", L5) \
    VLA_MAC("%7", "%10", "%11", L7) VLA_MAC("%8", "%12", "%6", L6) VLA_MAC("%9", "%13", "%6", L6) \
    VLA_MAC("%8", "%12", "%7", L7) VLA_MAC("%9", "%13", "%7", L7)

// FIRST: the accumulators start here (multiply instead of multiply-add).
// HI: columns use DPP lanes 8..15 of the row instead of 0..7.
template <bool FIRST, bool HI>
__device__ __forceinline__ void pass_chunk(float *e, float &acc1, float &acc2, float x,
                                           float mult, float y1, float y2)
{
    if constexpr (FIRST && !HI) {
        asm volatile(VLA_CHUNK(VLA_MUL, 0, 1, 2, 3, 4, 5, 6, 7)
                     : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]),
                       "+v"(e[6]), "+v"(e[7]), "=&v"(acc1), "=&v"(acc2)
                     : "v"(x), "v"(mult), "v"(y1), "v"(y2));
    } else if constexpr (!HI) {
        asm volatile(VLA_CHUNK(VLA_MAC, 0, 1, 2, 3, 4, 5, 6, 7)
                     : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]),
                       "+v"(e[6]), "+v"(e[7]), "+v"(acc1), "+v"(acc2)
                     : "v"(x), "v"(mult), "v"(y1), "v"(y2));
    } else {
        static_assert(!FIRST, "a pass starts at columns 0..7");
        asm volatile(VLA_CHUNK(VLA_MAC, 8, 9, 10, 11, 12, 13, 14, 15)
                     : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]),
                       "+v"(e[6]), "+v"(e[7]), "+v"(acc1), "+v"(acc2)
                     : "v"(x), "v"(mult), "v"(y1), "v"(y2));
    }
}

template <int CPL, int SW1>
__device__ __forceinline__ void row_pass(float (&mv)[CPL], float x0, float x1, float mult,
                                         float y10, float y11, float y20, float y21,
                                         float &acc1, float &acc2)
{
    pass_chunk<true, false>(&mv[0], acc1, acc2, x0, mult, y10, y20);
    pass_chunk<false, true>(&mv[8], acc1, acc2, x0, mult, y10, y20);
    if constexpr (SW1 >= 8) pass_chunk<false, false>(&mv[16], acc1, acc2, x1, mult, y11, y21);
    if constexpr (SW1 == 16) pass_chunk<false, true>(&mv[24], acc1, acc2, x1, mult, y11, y21);
}

// v_permlane32_swap / v_permlane16_swap with the two wait states a VALU write
// of either operand needs before the swap reads it.  Issued from asm so that the
// compiler does not pad them with the long wait it assumes after the DPP
// multiply-add asm blocks.  After permlane32: a = [a_lo, b_lo], b = [a_hi, b_hi]
// (32-lane halves); after permlane16: a = [a0, b0, a2, b2], b = [a1, b1, a3, b3]
// (16-lane rows).
__device__ __forceinline__ void pl32_swap(float &a, float &b)
{
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void pl16_swap(float &a, float &b)
{
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// x, y <- their sums over lanes l, l^16, l^32, l^48 (the four lane groups), in
// every lane, bit-identical across lanes.
__device__ __forceinline__ void sum2_groups(float &x, float &y)
{
    pl32_swap(x, y);
    float X = x + y, X2 = X;        // rows: x02 x13 y02 y13
    pl16_swap(X, X2);
    float Q = X + X2, Q2 = Q;       // rows: x x y y
    pl32_swap(Q, Q2);
    x = Q;
    y = Q2;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a DPP row (xor 1, xor 2, half-mirror, mirror).
__device__ __forceinline__ float sum_row16(float x)
{
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror
    x += dpp<0x140>(x);   // row_mirror
    return x;
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <int D>
struct FastCfg {
    static constexpr int NH = D / 16;            // wavefronts per chain
    static constexpr int NHP = (NH + 3) / 4 * 4; // partials row padded to 16 bytes
    static constexpr int NT = 128 * NH;          // A-waves + S-waves
    static constexpr int SW1 = (D - 64) / 4;     // second column segment per lane group
    static constexpr int CPL = 16 + SW1;         // matrix columns per lane
    static constexpr int TT = 32;                // tokens per prologue tile
    static constexpr int RING = 64;              // token records in LDS (power of 2, >= TT + 2)
                                                 // plus one alias record in front (see below)
    static constexpr int RS = 4 * D + 4;         // record stride in floats: k^, u^, phi(q), v
    static constexpr int KH = 0, UH = D, PQ = 2 * D, VV = 3 * D;   // record fields
    static constexpr int ZS = D + 4;             // stride of the key-sum scratch rows
    static constexpr int PT = 16 * TT;           // prologue threads: 16 per token
    static constexpr int CPT = D / 16;           // prologue columns per thread (4, 6, 8)
};

// CPT consecutive inputs of one token, held in registers.
template <typename Tin, int N> struct RawVec;
template <int N> struct RawVec<float, N> {   // N in {4, 6, 8}; 8-byte aligned
    float2 x[N / 2];
    __device__ __forceinline__ void load(const float *p, bool ok)
    {
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            x[i] = ok ? reinterpret_cast<const float2 *>(p)[i] : make_float2(0.f, 0.f);
    }
    __device__ __forceinline__ float get(int i) const { return (i & 1) ? x[i >> 1].y : x[i >> 1].x; }
};
template <int N> struct RawVec<uint16_t, N> {   // N in {4, 6, 8}; 4-byte aligned
    uint32_t x[N / 2];
    __device__ __forceinline__ void load(const uint16_t *p, bool ok)
    {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) x[i] = ok ? reinterpret_cast<const uint32_t *>(p)[i] : 0u;
    }
    __device__ __forceinline__ float get(int i) const
    {
        return (i & 1) ? bf16_hi(x[i >> 1]) : bf16_lo(x[i >> 1]);
    }
};

// phi = ELU + 1 with the hardware exp2 path (relative error ~1e-6 here).
__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <int D, typename Tin>
__global__ void __launch_bounds__(FastCfg<D>::NT)
vla_fwd_fast(const Tin *__restrict__ q, const Tin *__restrict__ k,
             const Tin *__restrict__ v, const Tin *__restrict__ u,
             int T, float lambda0, float eps,
             float *__restrict__ o, float *S_out, float *A_out, float *zk_out,
             const float *S0, const float *A0, const float *zk0)
{
    using C = FastCfg<D>;
    constexpr int NH = C::NH, NHP = C::NHP, NT = C::NT, SW1 = C::SW1, CPL = C::CPL, TT = C::TT;
    constexpr int RING = C::RING, RS = C::RS, ZS = C::ZS, CPT = C::CPT, PT = C::PT;
    constexpr int KH = C::KH, UH = C::UH, PQ = C::PQ, VV = C::VV;

    // token records: slot s at s_rec[(s + 1) * RS]; s_rec[0 .. RS) repeats the
    // phi(q) field of slot RING-1, so the phi(q) of token t-1 is always one record
    // before the record of token t
    __shared__ __align__(16) float s_rec[(RING + 1) * RS];
    __shared__ __align__(16) float s_zk[TT * ZS];       // phi(k), then the key sum, of a tile
    __shared__ float s_rden[RING];                      // 1 / max(phi(q)' zkey, eps)
    __shared__ __align__(16) float s_z[2][D];           // all-gather of z_t
    __shared__ __align__(16) float s_y[2][D];           // all-gather of y_{t-1}
    __shared__ __align__(16) float s_red[2][4][NHP];    // per-wave dot-product partials
    __shared__ float s_sink[64];                        // target of masked-off exchange writes

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int l = tid & 63, g = l >> 4, n = l & 15;
    const bool awave = w < NH;
    const int wh = awave ? w : w - NH;
    const int row = 16 * wh + n;
    const size_t bh = blockIdx.x;
    const size_t DD = (size_t)D * D;
    // second-segment lane-distributed element (lanes n >= SW1 read a valid dummy
    // element; their values are never broadcast)
    const int l1 = 64 + SW1 * g + (n < SW1 ? n : (SW1 > 0 ? SW1 - 1 : 0));

    float zk_run = 0.f, zk_cmp = 0.f;          // key sum of column tid (tid < D) before
    if (tid < D && zk0) zk_run = zk0[bh * D + tid];   // the tile, Kahan-compensated

    for (int i = tid; i < (RING + 1) * RS; i += NT) s_rec[i] = 0.f;
    for (int i = tid; i < RING; i += NT) s_rden[i] = 0.f;
    for (int i = tid; i < 2 * D; i += NT) {
        (&s_z[0][0])[i] = 0.f;
        (&s_y[0][0])[i] = 0.f;
    }
    for (int i = tid; i < 2 * 4 * NHP; i += NT) (&s_red[0][0][0])[i] = 0.f;

    // prologue thread mapping: 16 threads per token (one DPP row), token tl of the
    // tile, columns [c*CPT, c*CPT+CPT); threads tid >= PT only join the barriers
    const bool pthr = tid < PT;
    const int tl = (tid >> 4) & (TT - 1), c = tid & 15;
    const size_t tok_base = bh * (size_t)T;
    RawVec<Tin, CPT> rq, rk, rv, ru;
    auto prefetch = [&](int t0) {
        if (!pthr) return;
        const int t = t0 + tl;
        const bool ok = t < T;
        const size_t off = (tok_base + (size_t)(ok ? t : 0)) * D + (size_t)c * CPT;
        rq.load(q + off, ok);
        rk.load(k + off, ok);
        rv.load(v + off, ok);
        ru.load(u + off, ok);
    };

    // State-independent work of the tile starting at token t0 (all threads; two
    // barriers).  Leaves k^, u^, phi(q), v of each token in its record and
    // 1/max(phi(q)'zkey, eps) in s_rden, and advances the key sums.
    auto prologue = [&](int t0) {
        const int t = t0 + tl;
        const bool ok = t < T;
        const int slot = t & (RING - 1);
        const int rec = (slot + 1) * RS + c * CPT;
        float pq[CPT];
        if (pthr) {
            float pk = 0.f, pu = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                pk = fmaf(rk.get(i), rk.get(i), pk);
                pu = fmaf(ru.get(i), ru.get(i), pu);
            }
            const float nk = sum_row16(pk), nu = sum_row16(pu);    // |k_t|^2, |u_t|^2
            const float ik = nk > 0.f ? 1.f / sqrtf(nk) : 0.f;
            const float iu = nu > 0.f ? 1.f / sqrtf(nu) : 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                pq[i] = phi_fast(rq.get(i));
                s_rec[rec + KH + i] = rk.get(i) * ik;
                s_rec[rec + UH + i] = ru.get(i) * iu;
                s_rec[rec + PQ + i] = pq[i];
                s_rec[rec + VV + i] = rv.get(i);
                if (slot == RING - 1) s_rec[PQ + c * CPT + i] = pq[i];   // alias record
                s_zk[tl * ZS + c * CPT + i] = ok ? phi_fast(rk.get(i)) : 0.f;
            }
        }
        __syncthreads();
        if (tid < D) {
            // inclusive key sum per column: prefix inside the tile from zero, added
            // to the compensated sum of the earlier tiles
            float loc = 0.f;
#pragma unroll 8
            for (int tt = 0; tt < TT; ++tt) {
                loc += s_zk[tt * ZS + tid];
                s_zk[tt * ZS + tid] = zk_run + loc;
            }
            const float yk = loc - zk_cmp;
            const float ts = zk_run + yk;
            zk_cmp = (ts - zk_run) - yk;
            zk_run = ts;
        }
        __syncthreads();
        if (pthr) {
            float pd = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) pd = fmaf(pq[i], s_zk[tl * ZS + c * CPT + i], pd);
            pd = sum_row16(pd);
            if (c == 0) s_rden[slot] = 1.f / fmaxf(pd, eps);
        }
        // s_rden of a token is first read two iterations later, after two barriers;
        // s_zk is next written after at least one token barrier.
    };

    // Runs every tile: prologue, prefetch of the next tile, then the token
    // iterations (one barrier each), unrolled by two so that buffer parities are
    // compile-time constants.
    auto run = [&](auto &&step) {
        prefetch(0);
        __syncthreads();
        const int ntiles = (T + 2 + TT - 1) / TT;
        for (int tile = 0; tile < ntiles; ++tile) {
            const int t0 = tile * TT;
            prologue(t0);
            if (tile + 1 < ntiles) prefetch(t0 + TT);
            const int tend = min(t0 + TT, T + 2);
            int t = t0;                                    // t0 is even
            for (; t + 1 < tend; t += 2) {
                step(t, std::integral_constant<int, 0>{});
                __syncthreads();
                step(t + 1, std::integral_constant<int, 1>{});
                __syncthreads();
            }
            if (t < tend) {
                step(t, std::integral_constant<int, 0>{});
                __syncthreads();
            }
        }
    };

    float m_[CPL];   // A-waves: rows of A; S-waves: rows of S
    if (awave) {
        // ================================================ penalty chain (A)
        sfor<CPL>([&](auto mm) {
            constexpr int m = decltype(mm)::value;
            const int j = m < 16 ? 16 * g + m : 64 + SW1 * g + (m - 16);
            m_[m] = A0 ? A0[bh * DD + (size_t)row * D + j] : (row == j ? 1.f / lambda0 : 0.f);
        });
        // exchange partials: group 0 u^_t.z_t, 1 k^_t.z_t, 2 |y_{t-1}|^2,
        // 3 y_{t-1}.phi(q_{t-1}) (the record before token t's); element offset of
        // the record entry each group multiplies in, relative to token t's record
        const int o_part = (g == 0 ? UH + row : g == 1 ? KH + row : PQ + row - RS);
        // group 0 lanes write z, group 2 lanes y, lane n == 0 of each group its
        // partial; every other lane writes to the sink
        float *const p_zy = g == 0 ? &s_z[0][row] : g == 2 ? &s_y[0][row] : &s_sink[l];
        const int zy_par = (g == 0 || g == 2) ? D : 0;
        float *const p_red = n == 0 ? &s_red[0][g][wh] : &s_sink[l];
        const int red_par = n == 0 ? 4 * NHP : 0;
        float zr = 0.f, wr = 0.f;   // z_{t-1}, w_{t-1} = A_{t-2} k^_{t-1}

        run([&](int t, auto parity) {
            constexpr int P = decltype(parity)::value;  // t & 1
            constexpr int PB = P ^ 1;                   // buffers written in iteration t-1
            const int st = ((t & (RING - 1)) + 1) * RS; // record of token t
            const float zc0 = s_z[PB][l], zc1 = SW1 ? s_z[PB][l1] : 0.f;   // z_{t-1}
            const float4 ru4 = *reinterpret_cast<const float4 *>(&s_red[PB][0][0]);
            const float4 rk4 = *reinterpret_cast<const float4 *>(&s_red[PB][1][0]);
            float ud = (ru4.x + ru4.y) + (ru4.z + ru4.w);
            float kd = (rk4.x + rk4.y) + (rk4.z + rk4.w);
            if constexpr (NH > 4) {
#pragma unroll
                for (int ww = 4; ww < NH; ++ww) {
                    ud += s_red[PB][0][ww];
                    kd += s_red[PB][1][ww];
                }
            }
            const float invd = fast_rcp(1.f + ud);             // 1 / delta_{t-1}
            const float nc = -(zr * invd);                     // -z_i / delta
            const float yr = wr - zr * (kd * invd);           // y_{t-1} = A_{t-1} k^_{t-1}
            const float u0 = s_rec[st + UH + l], u1 = SW1 ? s_rec[st + UH + l1] : 0.f;
            const float k0 = s_rec[st + KH + l], k1 = SW1 ? s_rec[st + KH + l1] : 0.f;
            const float mem = s_rec[st + o_part];
            float za, wa;
            row_pass<CPL, SW1>(m_, zc0, zc1, nc, u0, u1, k0, k1, za, wa);
            sum2_groups(za, wa);                               // z_t, w_t (rows)
            const float lhs = g < 2 ? za : yr;
            const float rhs = g == 2 ? yr : mem;
            p_red[P * red_par] = sum_row16(lhs * rhs);
            p_zy[P * zy_par] = g == 0 ? za : yr;
            zr = za;
            wr = wa;
        });
    } else {
        // ================================================ memory chain (S)
        sfor<CPL>([&](auto mm) {
            constexpr int m = decltype(mm)::value;
            const int j = m < 16 ? 16 * g + m : 64 + SW1 * g + (m - 16);
            m_[m] = S0 ? S0[bh * DD + (size_t)row * D + j] : 0.f;
        });
        float ep = 0.f, pp = 0.f;   // e_{t-2}, S_{t-3} phi(q_{t-2})
        float *const o_row = o + tok_base * D + row;

        run([&](int t, auto parity) {
            constexpr int P = decltype(parity)::value;
            constexpr int PB = P ^ 1;
            const int sp = (((t - 1) & (RING - 1)) + 1) * RS;   // record of token t-1
            const float yc0 = s_y[PB][l], yc1 = SW1 ? s_y[PB][l1] : 0.f;   // y_{t-2}
            const float4 ry4 = *reinterpret_cast<const float4 *>(&s_red[PB][2][0]);
            const float4 rq4 = *reinterpret_cast<const float4 *>(&s_red[PB][3][0]);
            float yy = (ry4.x + ry4.y) + (ry4.z + ry4.w);
            float yq = (rq4.x + rq4.y) + (rq4.z + rq4.w);
            if constexpr (NH > 4) {
#pragma unroll
                for (int ww = 4; ww < NH; ++ww) {
                    yy += s_red[PB][2][ww];
                    yq += s_red[PB][3][ww];
                }
            }
            const float ny = yy > 0.f ? rsqrtf(yy) : 0.f;     // 1 / |y_{t-2}|
            if (t >= 2 && t - 2 < T)                           // o_{t-2} = S_{t-2} phi(q) / den
                o_row[(size_t)(t - 2) * D] =
                    (pp + ep * (yq * ny)) * s_rden[(t - 2) & (RING - 1)];   // 4 lanes per row
            const float kp0 = s_rec[sp + KH + l], kp1 = SW1 ? s_rec[sp + KH + l1] : 0.f;
            const float q0 = s_rec[sp + PQ + l], q1 = SW1 ? s_rec[sp + PQ + l1] : 0.f;
            const float vrow = s_rec[sp + VV + row];
            const float se = ep * ny;          // alpha^_{t-2,j} e_{t-2,i} = y_j * (e_i / |y|)
            float ra, pa;
            row_pass<CPL, SW1>(m_, yc0, yc1, se, kp0, kp1, q0, q1, ra, pa);
            sum2_groups(ra, pa);
            ep = vrow - ra;    // e_{t-1} = v - S k^ with S before token t-1's write
            pp = pa;
        });
    }

    // ---------------------------------------------------------------- epilogue
    float *const out = awave ? A_out : S_out;
    if (out) {
        sfor<CPL>([&](auto mm) {
            constexpr int m = decltype(mm)::value;
            const int j = m < 16 ? 16 * g + m : 64 + SW1 * g + (m - 16);
            out[bh * DD + (size_t)row * D + j] = m_[m];
        });
    }
    if (zk_out && tid < D) zk_out[bh * D + tid] = zk_run;
}

template <int D, typename Tin>
hipError_t launch_fast(const FwdArgs &a)
{
    hipLaunchKernelGGL((vla_fwd_fast<D, Tin>), dim3(a.B * a.H), dim3(FastCfg<D>::NT), 0, a.stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u,
                       a.T, a.lambda0, a.eps, a.o, a.S_out, a.A_out, a.zk_out,
                       a.S0, a.A0, a.zk0);
    return hipGetLastError();
}

}  // namespace

bool fast_supported(int d) { return d == 64 || d == 96 || d == 128; }

hipError_t launch_forward_fast(const FwdArgs &a)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch_fast<64, uint16_t>(a) : launch_fast<64, float>(a);
    case 96: return bf ? launch_fast<96, uint16_t>(a) : launch_fast<96, float>(a);
    case 128: return bf ? launch_fast<128, uint16_t>(a) : launch_fast<128, float>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
