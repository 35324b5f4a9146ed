// vla_chunk_parts.h -- device parts of the chunked matrix-core kernels of the
// VLA recurrence (d_h in {64, 96, 128}): data layout and the steps of the two
// chains.  The kernels of vla_twopass.hip arrange them in time.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9) (Sherman-Morrison downdate of A), (10) (gated delta write of S) and
// (11) (ELU+1 readout with the running key sum); A_0 = I / lambda0 (section 3.2).
//
// Blocked form.  Tokens are taken in chunks of C = 16.  With A and S the states
// at the start of a chunk, U^, K^, Phi, V (d x C) the chunk's normalised u, k,
// phi(q) and raw v as columns, the C token steps compose exactly (up to rounding):
//
//   penalty chain (Eq. 9).   Z0 = A U^, Y0 = A K^, G = U^' Z0, and the LDL'
//   factorisation I + G = L D L' (L unit lower triangular).  The C downdates
//   of A are one Woodbury step,  A <- A - Z0 (I + G)^-1 Z0',  and the vectors
//   A_t k^_t (A_t after token t's own downdate) are the columns of
//       W = Y0 - Z0 L^-T ((D^-1 L^-1 U^' Y0) o Up),      Up_{ct} = [c <= t],
//   because the downdates up to token t use the leading (t+1) x (t+1) block of
//   I + G, whose factor is the leading block of L D L'.   alpha^_t = w_t / |w_t|.
//
//   memory chain (Eqs. 10, 11).  N_{ct} = alpha^_c' k^_t for c < t (0 otherwise),
//   E = (V - S K^) (I + N)^-1 holds the errors e_t of the token steps, and
//       S <- S + E Alpha^',     S_t phi(q_t) = S phi(q_t) + E ((Alpha^' Phi) o Up)_t.
//
// Mapping.  A chain runs on NA wavefronts (NA = 4 for d = 64, 128 and 6 for
// d = 96).  Each wave owns BPW = d / (16 NA) column blocks of 16 of its stored
// matrix, which is the TRANSPOSE of the state (As = A', Ss = S'), kept in MFMA
// accumulator layout for the whole sequence: tile (rho, b) of block b, register
// r of lane l = 16 g + n holds
//       Xs[16 rho + 4 g + r][16 b + n].
// v_mfma_f32_16x16x4_f32 takes A[m][k] from lane 16 k' + m and B[k][n] from lane
// 16 k' + n (k' = the lane group) and returns D[4 g + r][n] in register r of
// lane 16 g + n.  Used as the B operand with k = 16 rho + 4 g + r, a state tile
// gives the products X' [U^ K^] = (A [U^ K^])' one 16 x 16 tile per block with
// no data movement; the rank-16 updates accumulate into the same registers.
// Every other operand is read from LDS in the layout its product needs.
//
// The 16 x 16 factorisations run in registers with one matrix row per lane of a
// 16-lane DPP row (row_newbcast broadcasts a matrix entry along it); the inverses
// of the unit triangular factors are computed four columns at a time, one per
// lane group.
#pragma once
#include <type_traits>
#include <utility>

#include "vla_common.h"
#include "vla_dpp_blocks.h"

namespace vla {
namespace chunk {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

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
template <int N>
using ic = std::integral_constant<int, N>;

__device__ __forceinline__ f4 mma(float a, float b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four k-steps of a 16 x 16 product, c + sum_s A_s B_s (dependent accumulation
// into one register set issues back to back on gfx950).
__device__ __forceinline__ f4 mma4(const float (&a)[4], const float (&b)[4], f4 c)
{
    c = mma(a[0], b[0], c);
    c = mma(a[1], b[1], c);
    c = mma(a[2], b[2], c);
    return mma(a[3], b[3], c);
}
__device__ __forceinline__ f4 mma4(f4 a, f4 b, f4 c)
{
    c = mma(a[0], b[0], c);
    c = mma(a[1], b[1], c);
    c = mma(a[2], b[2], c);
    return mma(a[3], b[3], c);
}

// 1 / x[lane J of this 16-lane row], after the two wait states a VALU write of x
// needs before a DPP read (x may come straight from an inline-asm FMA).
template <int J>
__device__ __forceinline__ float rcp_bcast(float x)
{
    float r;
    asm volatile("s_nop 1\n\tv_rcp_f32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
                 : "=v"(r)
                 : "v"(x), "n"(J));
    return r;
}

// 16-byte loads and stores (LDS or global)
__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }

// Raw buffer view of device memory: a uniform base and extent in a resource
// descriptor, 32-bit per-lane byte offsets, no 64-bit vector address math.
// Loads past the extent return 0 and stores past it are dropped (every access
// here is whole 16-byte granules inside or outside a row, never straddling the
// end).
struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Buf(const void *base, unsigned bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                              0x00020000))
    {
    }
    __device__ __forceinline__ void st32(float x, unsigned off, unsigned soff = 0) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, soff, 0);
    }
    __device__ __forceinline__ void st128(f4 x, unsigned off, unsigned soff = 0) const
    {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, off, soff, 0);
    }
    // 16 bytes per lane from device memory straight into LDS: lane l's bytes
    // land at lds + 16 l (lds uniform over the wave); bytes past the view read
    // as 0.  Counted by vmcnt like any load.
    __device__ __forceinline__ void lds16(float *lds, unsigned off, unsigned soff = 0) const
    {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, soff, 0, 0);
    }
    // 4 bytes per lane straight into LDS: lane l's bytes land at lds + 4 l
    __device__ __forceinline__ void lds4(float *lds, unsigned off, unsigned soff = 0) const
    {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, off, soff, 0, 0);
    }
};

__device__ __forceinline__ void st4(float *p, f4 x) { *reinterpret_cast<f4 *>(p) = x; }

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a DPP row (xor 1, xor 2, half-mirror, mirror).
__device__ __forceinline__ float sum_row16(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

// Compiler-only ordering point between LDS writes and reads of other lanes of
// the same wave (LDS executes one wave's instructions in order).
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// Wait until this wave's outstanding device-memory operations are done, as a
// real s_waitcnt (vmcnt 0, expcnt and lgkmcnt untouched) that the compiler's
// wait-count tracking sees: after it, registers loaded before a loop no longer
// look pending inside the loop, where every use would otherwise wait for all
// operations issued in the previous iteration.
__device__ __forceinline__ void vmem_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's device-memory operations are outstanding
// (they complete in issue order); expcnt and lgkmcnt untouched.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

// Compiler-only ordering point for memory operations.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier for LDS traffic only.  Unlike __syncthreads() it does not
// wait for outstanding global loads and stores, so prefetches into registers
// stay in flight across it (their consumers wait for them as usual).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One input element kept as loaded (bf16 stays a bit pattern), so that the load
// can stay in flight until the value is used.
template <typename Tin> struct Raw1;
template <> struct Raw1<float> {
    float x;
    __device__ __forceinline__ void load(const float *p, size_t i) { x = p[i]; }
    __device__ __forceinline__ float get() const { return x; }
};
template <> struct Raw1<uint16_t> {
    uint32_t x;
    __device__ __forceinline__ void load(const uint16_t *p, size_t i) { x = p[i]; }
    __device__ __forceinline__ float get() const { return __uint_as_float(x << 16); }
};

// N consecutive inputs of one token, held in registers as loaded (bf16 stays a
// bit pattern), fetched with the widest loads the row offset allows: the
// offset is a multiple of N elements, so a group of V elements with
// N % V == 0 and V * sizeof <= 16 is aligned to its own size.
template <typename Tin, int N>
struct RawVec {
    static constexpr int ES = (int)sizeof(Tin);
    static constexpr int V = (N % 8 == 0 && 8 * ES <= 16) ? 8
                           : (N % 4 == 0 && 4 * ES <= 16) ? 4 : 2;   // elements per load
    static constexpr int NW = N * ES / 4;                              // 32-bit words
    static constexpr int WPL = V * ES / 4;                             // words per load
    uint32_t x[NW];
    __device__ __forceinline__ void load(const Tin *p)
    {
        static_assert(N % 2 == 0 && NW % WPL == 0, "whole loads");
        sfor<NW / WPL>([&](auto i) {
            if constexpr (WPL == 4) {
                const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
                x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
            } else if constexpr (WPL == 2) {
                const uint2 v = reinterpret_cast<const uint2 *>(p)[i];
                x[2 * i] = v.x; x[2 * i + 1] = v.y;
            } else {
                x[i] = reinterpret_cast<const uint32_t *>(p)[i];
            }
        });
    }
    // the same from a buffer view at byte offset `off` (32-bit offsets: no 64-bit
    // address arithmetic per load; bytes past the view read as 0)
    __device__ __forceinline__ void load(const Buf &b, unsigned off)
    {
        static_assert(N % 2 == 0 && NW % WPL == 0, "whole loads");
        sfor<NW / WPL>([&](auto i) {
            const unsigned o = off + 4u * WPL * (unsigned)i;
            if constexpr (WPL == 4) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(b.r, o, 0, 0);
                x[4 * i] = v[0]; x[4 * i + 1] = v[1]; x[4 * i + 2] = v[2]; x[4 * i + 3] = v[3];
            } else if constexpr (WPL == 2) {
                typedef unsigned v2u __attribute__((ext_vector_type(2)));
                const v2u v = __builtin_amdgcn_raw_buffer_load_b64(b.r, o, 0, 0);
                x[2 * i] = v[0]; x[2 * i + 1] = v[1];
            } else {
                x[i] = __builtin_amdgcn_raw_buffer_load_b32(b.r, o, 0, 0);
            }
        });
    }
    __device__ __forceinline__ float get(int i) const
    {
        if constexpr (ES == 4) return __uint_as_float(x[i]);
        else return (i & 1) ? bf16_hi(x[i >> 1]) : bf16_lo(x[i >> 1]);
    }
};

// phi = ELU + 1 with the hardware exp2 path (relative error ~1e-6 here).
__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// 1 / sqrt(x) as the single hardware instruction (v_rsq_f32, about 1 ulp), for
// x > 0 that is a normal float; rsqrtf also rescales denormal x, which costs five
// more instructions.  Used for |w_t|^2 = |A_t k^_t|^2 with unit k^: A_t is the
// inverse of A_0^-1 + sum_{s<=t} u^_s u^_s' (section 3.2), whose eigenvalues are
// at most |A_0^-1| + t, so a nonzero |w_t|^2 is at least (|A_0^-1| + t)^-2, far
// above the denormal range for any sequence length the library accepts.
__device__ __forceinline__ float rsq_normal(float x) { return __builtin_amdgcn_rsqf(x); }

template <int D>
struct Cfg {
    static constexpr int C = 16;                   // tokens per chunk
    static constexpr int NB = D / 16;              // 16-column blocks of a state
    static constexpr int NA = NB % 4 == 0 ? 4 : NB;// waves per chain
    static constexpr int BPW = NB / NA;            // column blocks per wave
    static constexpr int LD = D + 4;               // row stride of [token][i] arrays
    static constexpr int LT = C + 4;               // row stride of [i][token] and C x C arrays
    static constexpr int CPT = D / 16;             // staged columns per thread (16 per token)
};

// Layouts of the per-chunk matrices the memory pass reads through LDS: the
// float offset of granule (16 bytes) c4 of row i of a 16-column matrix, and of
// row t of a D-column matrix.  The granule index is XOR-swizzled with the row,
// so that 16-byte reads of 8 consecutive rows at one column hit distinct banks.
__device__ __forceinline__ constexpr int swz16(int i, int c4) { return 16 * i + 4 * (c4 ^ ((i >> 1) & 3)); }
template <int D>
__device__ __forceinline__ constexpr int swzd(int t, int c4) { return D * t + 4 * (c4 ^ (t & 7)); }

// The key cross factor of a pair of chunks (a, b) as the memory pass applies it:
// there E_b' = T_b'(V_b - S K^_b)' - T_b'(Alpha^_a'K^_b)' E_a', with T_b =
// (I + N_b)^-1, so the record holds Y = -T_b'(Alpha^_a'K^_b)' and the product
// with E_a' is the only one that waits for E_a.  q: register r of lane 16 g + n
// holds (Alpha^_a'K^_b)[4g+r][n] (a 16 x 16 product's result); xi[c]: row n of
// column 4c+g of T_b (as the triangular inverse leaves it).  Y goes to dst as
// the record's 16-column layout stores it; s1, s2: C x (C + 4) LDS scratch.
__device__ __forceinline__ void solved_cross(f4 q, const float (&xi)[4], int g, int n, float *s1,
                                             float *s2, float *dst)
{
    constexpr int LT = 16 + 4;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    sfor<4>([&](auto r) { s1[(4 * g + r) * LT + n] = -q[int(r)]; });   // -(Alpha^_a'K^_b), row-major
    sfor<4>([&](auto c) { s2[n * LT + 4 * c + g] = xi[c]; });          // T_b, row-major
    wave_lds_order();
    const f4 a = ld4(&s1[n * LT + 4 * g]);
    f4 b;
    sfor<4>([&](auto r) { b[int(r)] = s2[(4 * g + r) * LT + n]; });
    // register r of lane 16 g + n: (-(Alpha^_a'K^_b) T_b)[4g+r][n] = Y[n][4g+r]
    st4(&dst[swz16(n, g)], mma4(a, b, zero));
}

// Where the penalty chain leaves W' (key-major: W[i][token]) and the |w|^2
// partials of a chunk: in LDS.
template <int D, typename LdsT>
struct WToLds {
    LdsT &L;
    int g, n;
    __device__ __forceinline__ void block(int b, f4 wt)
    {
        constexpr int LT = Cfg<D>::LT;
        st4(&L.wt[(16 * b + n) * LT + 4 * g], wt);
    }
    __device__ __forceinline__ void norms(int wi, f4 nr)
    {
        if (n == 0) st4(&L.nrm[wi][4 * g], nr);
    }
    // z_t = A_{t-1} u^_t of the chunk's tokens 4g + r at keys 16b + n, and
    // 1/delta_t: nothing to do here (a sink that keeps them overrides this and
    // sets KEEPS_Z, so that the downdate forms them)
    static constexpr bool KEEPS_Z = false;
    __device__ __forceinline__ void zcols(int, f4, f4) {}
};

// Per-thread view of one head's penalty chain: lane coordinates and the steps.
// A wave with chain index wi owns column blocks wi*BPW + bb; LdsT is the
// workgroup's LDS layout (members uh, kh, ph, zk, z0t, wt, gp, nrm, nq,
// lit/tit, inv, hms, mx).
//
// A chunk takes two phases, each ended by a workgroup barrier:
//   factorisation phase   every wave: Y0 = A K^ (y_products); wave 0:
//                         factorise I + G (factorize); work off the chain.
//   update phase          every wave: W, the downdate of A and the |w|^2 and
//                         W'K^, W'Phi partials of the chunk (downdate), then Z0
//                         and the G partials of the next chunk with the new A
//                         (z_products), which need only the wave's own blocks.
// 1/|w| is applied where the partials are used (prep_tp, the record's alpha^,
// the cross factors), in the next chunk's factorisation phase.
template <int D, typename LdsT>
struct Head {
    using Cf = Cfg<D>;
    static constexpr int C = Cf::C, NB = Cf::NB, NA = Cf::NA, BPW = Cf::BPW;
    static constexpr int LD = Cf::LD, LT = Cf::LT;
    typedef f4 State[BPW][NB];

    LdsT &L;
    int g, n, wi;                       // lane group, lane in group, wave index within the chain
    int kcol;                           // key-sum column of this thread, or -1
    float zk_run = 0.f, zk_cmp = 0.f;   // its Kahan-compensated key sum

    // phi(k), then the key sums, of chunk cq
    __device__ __forceinline__ float *zkb(int cq) const { return L.zk[cq & 1]; }

    __device__ __forceinline__ Head(LdsT &L_, int lane, int wi_, int kcol_)
        : L(L_), g(lane >> 4), n(lane & 15), wi(wi_), kcol(kcol_ >= 0 && kcol_ < D ? kcol_ : -1)
    {
    }

    // ------------------------------------------------------------ state I/O
    // The d x d state is row-major in memory; the tiles hold its transpose.
    __device__ __forceinline__ void load_state(State &st, const float *src, float diag) const
    {
        sfor<BPW>([&](auto bb) {
            const int row = 16 * (wi * BPW + bb) + n;
            sfor<NB>([&](auto rho) {
                const int col = 16 * rho + 4 * g;
                if (src) {
                    st[bb][rho] = ld4(&src[(size_t)row * D + col]);
                } else {
                    f4 x;
                    sfor<4>([&](auto r) { x[int(r)] = row == col + r ? diag : 0.f; });
                    st[bb][rho] = x;
                }
            });
        });
    }
    __device__ __forceinline__ void store_state(const State &st, float *dst) const
    {
        sfor<BPW>([&](auto bb) {
            const int row = 16 * (wi * BPW + bb) + n;
            sfor<NB>([&](auto rho) { st4(&dst[(size_t)row * D + 16 * rho + 4 * g], st[bb][rho]); });
        });
    }

    // inclusive key sum per column: prefix inside the chunk, added to the
    // compensated sum of the earlier chunks
    __device__ __forceinline__ void stage2(int cq)
    {
        if (kcol < 0) return;
        float *zk = zkb(cq);
        float f[C];
#pragma unroll
        for (int tt = 0; tt < C; ++tt) f[tt] = zk[tt * LD + kcol];
        float loc = 0.f;
#pragma unroll
        for (int tt = 0; tt < C; ++tt) {
            loc += f[tt];
            zk[tt * LD + kcol] = zk_run + loc;
        }
        const float yk = loc - zk_cmp;
        const float tsum = zk_run + yk;
        zk_cmp = (tsum - zk_run) - yk;
        zk_run = tsum;
    }

    // 1/|w_t| of the last updated chunk from the waves' |w|^2 partials: for
    // t = 4g + r (rows of the C x C factors) and for t = n (this lane's token)
    __device__ __forceinline__ f4 inv_norms4() const
    {
        f4 ns4 = ld4(&L.nrm[0][4 * g]);
        sfor<NA - 1>([&](auto w2) { ns4 += ld4(&L.nrm[w2 + 1][4 * g]); });
        f4 r4;
        sfor<4>([&](auto r) { r4[int(r)] = ns4[int(r)] > 0.f ? rsq_normal(ns4[int(r)]) : 0.f; });
        return r4;
    }
    __device__ __forceinline__ float inv_norm_n() const
    {
        float ns = L.nrm[0][n];
        sfor<NA - 1>([&](auto w2) { ns += L.nrm[w2 + 1][n]; });
        return ns > 0.f ? rsq_normal(ns) : 0.f;
    }

    // ------------------------------------------------------------ penalty chain
    // Z0' of the own blocks of chunk cq into L.z0t[cq & 1] (Z0 [i][token]), and
    // this wave's partials (rows i of its blocks) of U^'Z0 and of U^'A K^ = Z0'K^
    // (A symmetric), so that the product A K^ is off the path to the
    // factorisation.  U^ of chunk cq is in L.uh.
    __device__ __forceinline__ void z_products(const State &st, int cq)
    {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        const float *ub = L.uh, *kb = L.kh[cq & 1];
        float *z0t = L.z0t[cq & 1];
        f4 z[BPW];
        sfor<BPW>([&](auto bb) { z[bb] = zero; });
        sfor<NB>([&](auto rho) {
            const f4 au = ld4(&ub[n * LD + 16 * rho + 4 * g]);
            sfor<4>([&](auto r) {
                sfor<BPW>([&](auto bb) { z[bb] = mma(au[int(r)], st[bb][rho][int(r)], z[bb]); });
            });
        });
        // z[bb] register r = Z0[16b + n][4g + r]
        sfor<BPW>([&](auto bb) { st4(&z0t[(16 * (wi * BPW + bb) + n) * LT + 4 * g], z[bb]); });
        wave_lds_order();
        f4 gu = zero, gk = zero;
        sfor<BPW>([&](auto bb) {
            const int b = wi * BPW + bb;
            const f4 au = ld4(&ub[n * LD + 16 * b + 4 * g]);    // U^_n[16b + 4g + r]
            f4 bz;                                              // Z0_n[16b + 4g + r]
            sfor<4>([&](auto r) { bz[int(r)] = z0t[(16 * b + 4 * g + r) * LT + n]; });
            const f4 bk = ld4(&kb[n * LD + 16 * b + 4 * g]);    // K^_n[16b + 4g + r]
            gu = mma4(au, bz, gu);
            gk = mma4(bz, bk, gk);
        });
        if (wi == 0) sfor<4>([&](auto r) { gu[int(r)] += 4 * g + r == n ? 1.f : 0.f; });
        sfor<4>([&](auto r) {
            L.gp[wi][0][(4 * g + r) * LT + n] = gu[int(r)];
            L.gp[wi][1][(4 * g + r) * LT + n] = gk[int(r)];
        });
    }

    // Y0' = (A K^)' of the own blocks of chunk cq, with the state before the
    // chunk's downdate.
    __device__ __forceinline__ void y_products(const State &st, int cq, f4 (&y)[BPW]) const
    {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        const float *kb = L.kh[cq & 1];
        sfor<BPW>([&](auto bb) { y[bb] = zero; });
        sfor<NB>([&](auto rho) {
            const f4 ak = ld4(&kb[n * LD + 16 * rho + 4 * g]);
            sfor<4>([&](auto r) {
                sfor<BPW>([&](auto bb) { y[bb] = mma(ak[int(r)], st[bb][rho][int(r)], y[bb]); });
            });
        });
    }

    // Wave 0: factorise I + G = L D L' from the waves' partials and leave L^-1
    // (both ways round in L.lit[0]), 1/d (L.inv[0]) and the A operand of W',
    // H = -(D^-1 L^-1 U^'Y0) o Up (L.hms), in LDS.  With EXPL, the two C x C
    // matrices the downdate applies to Z0' are formed here once instead:
    // M = -(I + G)^-1 = -L^-T D^-1 L^-1 (L.mx) and H' L^-1 (L.hms), each as the
    // A operand a lane needs with the contraction index 4 g + c, so that every
    // wave takes two products per block in place of three.
    template <bool EXPL>
    __device__ __forceinline__ void factorize()
    {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        float Mr[16], gub[4];
        sfor<4>([&](auto r) {
            float a = L.gp[0][0][(4 * g + r) * LT + n];
            sfor<NA - 1>([&](auto w2) { a += L.gp[w2 + 1][0][(4 * g + r) * LT + n]; });
            L.lit[0][(4 * g + r) * LT + n] = a;
        });
        sfor<4>([&](auto c) {
            float a = L.gp[0][1][(4 * c + g) * LT + n];
            sfor<NA - 1>([&](auto w2) { a += L.gp[w2 + 1][1][(4 * c + g) * LT + n]; });
            gub[c] = a;
        });
        wave_lds_order();
        sfor<4>([&](auto q4) {
            const f4 a = ld4(&L.lit[0][n * LT + 4 * q4]);
            sfor<4>([&](auto r) { Mr[4 * q4 + r] = a[int(r)]; });
        });
        wave_lds_order();
        // LDL' (column by column, Crout order): lane n holds row n.  LDr[j] =
        // L[n][j] d_j (d_j in lane j), NLr[j] = -L[n][j] for n > j, 0
        // otherwise; 1/d_j to LDS.  Column j+1's terms k < j are issued
        // around the inversion of pivot j (software pipelining); only its
        // k = j term waits for it.
        float LDr[16], NLr[16];
        float ca = Mr[0], cb = 0.f;
        float invn = 0.f;
        sfor<16>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            if constexpr (j > 0) ldl_block<j, j - 1, 1>(ca, LDr, NLr);
            const float acc = ca + cb;
            const float inv = rcp_bcast<j>(acc);
            constexpr int E = j, E1 = E < 2 ? E : 2;
            float na = 0.f, nb = 0.f;
            if constexpr (j + 1 < 16) {
                na = Mr[j + 1];
                if constexpr (E1 > 0) ldl_early<j + 1, 0, E1>(na, nb, LDr, NLr);
            }
            LDr[j] = acc;
            NLr[j] = n > j ? -(acc * inv) : 0.f;
            invn = n == j ? inv : invn;   // lane n keeps 1 / d_n
            if constexpr (j + 1 < 16 && E > E1) ldl_early<j + 1, E1, E - E1>(na, nb, LDr, NLr);
            ca = na;
            cb = nb;
        });
        L.inv[0][n] = invn;   // every lane group holds the same values
        float X[4];
        sfor<4>([&](auto c) { X[c] = n == 4 * c + g ? 1.f : 0.f; });
        asm volatile(VLA_LINV_BLOCK
                     : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3])
                     : "v"(NLr[0]), "v"(NLr[1]), "v"(NLr[2]), "v"(NLr[3]), "v"(NLr[4]),
                       "v"(NLr[5]), "v"(NLr[6]), "v"(NLr[7]), "v"(NLr[8]), "v"(NLr[9]),
                       "v"(NLr[10]), "v"(NLr[11]), "v"(NLr[12]), "v"(NLr[13]), "v"(NLr[14]));
        sfor<4>([&](auto c) { L.lit[0][(4 * c + g) * LT + n] = X[c]; });
        wave_lds_order();
        const f4 inv4 = ld4(&L.inv[0][4 * g]);
        f4 hm = mma4(X, gub, zero);
        sfor<4>([&](auto r) { hm[int(r)] = 4 * g + r <= n ? -(hm[int(r)] * inv4[int(r)]) : 0.f; });
        if constexpr (EXPL) {
            // register c of lane 16 g + n: L^-1 [4g+c][n]
            const f4 lit = ld4(&L.lit[0][n * LT + 4 * g]);
            // (H' L^-1)' = L^-T H: register c of lane 16 g + n is (H' L^-1)[n][4g+c]
            st4(&L.hms[4 * (16 * g + n)], mma4(lit, hm, zero));
            // M[4g+c][n], read as M[n][4g+c] (M is symmetric)
            st4(&L.mx[4 * (16 * g + n)], mma4(lit * -inv4, lit, zero));
        } else {
            st4(&L.hms[4 * (16 * g + n)], hm);
        }
    }

    // After the factorisation of chunk cq: W' (to `wout`), the downdate
    // As <- As - Z0 (I + G)^-1 Z0' of the own blocks, the |w|^2 partials, and
    // this wave's partials of W'K^ and W'Phi (unnormalised alpha^, rows t of
    // its blocks' keys) into L.nq.
    // With a sink that keeps z_t, the products go through L^-1 Z0' (whose rows
    // are the z_t); otherwise through M and H' L^-1 from factorize<true>.
    template <class WOut>
    __device__ __forceinline__ void downdate(State &st, int cq, const f4 (&y)[BPW], WOut &&wout)
    {
        constexpr bool EXPL = !std::decay_t<WOut>::KEEPS_Z;
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        const float *z0t = L.z0t[cq & 1];
        float X[4];
        f4 inv4, lit, hm;
        if constexpr (EXPL) {
            lit = ld4(&L.mx[4 * (16 * g + n)]);    // M [n][4g+c]
            hm = ld4(&L.hms[4 * (16 * g + n)]);    // (H' L^-1) [n][4g+c]
        } else {
            sfor<4>([&](auto c) { X[c] = L.lit[0][(4 * c + g) * LT + n]; });   // L^-1 [n][4c+g]
            inv4 = ld4(&L.inv[0][4 * g]);                          // 1 / d_{4g+r}
            lit = ld4(&L.lit[0][n * LT + 4 * g]);                  // L^-1 [4g+r][n]
            hm = ld4(&L.hms[4 * (16 * g + n)]);
        }
        f4 nr = zero;
        sfor<BPW>([&](auto bb) {
            const int b = wi * BPW + bb;
            f4 nx, wt;
            if constexpr (EXPL) {
                const f4 zb = ld4(&z0t[(16 * b + n) * LT + 4 * g]);   // Z0'[4g+c][16b+n]
                nx = mma4(lit, zb, zero);           // -(I + G)^-1 Z0'
                wt = mma4(hm, zb, y[bb]);           // W'
            } else {
                float zb[4];   // Z0'[4c+g][16b+n]
                sfor<4>([&](auto c) { zb[c] = z0t[(16 * b + n) * LT + 4 * c + g]; });
                const f4 q2 = mma4(X, zb, zero);    // L^-1 Z0': row t is z_t
                const f4 q1 = q2 * -inv4;           // -D^-1 L^-1 Z0' (the sign rides on the multiply)
                nx = mma4(lit, q1, zero);           // -(I + G)^-1 Z0'
                wt = mma4(hm, q2, y[bb]);           // W'
                wout.zcols(b, q2, inv4);
            }
            f4 az[NB];
            sfor<NB>([&](auto rho) { az[rho] = ld4(&z0t[(16 * rho + n) * LT + 4 * g]); });
            sfor<4>([&](auto r) {      // As <- As - Z0 (I + G)^-1 Z0'
                sfor<NB>([&](auto rho) { st[bb][rho] = mma(az[rho][int(r)], nx[int(r)], st[bb][rho]); });
            });
            wout.block(b, wt);
            nr += wt * wt;
        });
        sfor<4>([&](auto r) { nr[int(r)] = sum_row16(nr[int(r)]); });
        wout.norms(wi, nr);
        wave_lds_order();
        const float *kb = L.kh[cq & 1], *pb = L.ph[cq & 1];
        f4 gn = zero, gq = zero;
        sfor<BPW>([&](auto bb) {
            const int b = wi * BPW + bb;
            f4 aw;   // W_n[16b + 4g + r]
            sfor<4>([&](auto r) { aw[int(r)] = L.wt[(16 * b + 4 * g + r) * LT + n]; });
            gn = mma4(aw, ld4(&kb[n * LD + 16 * b + 4 * g]), gn);
            gq = mma4(aw, ld4(&pb[n * LD + 16 * b + 4 * g]), gq);
        });
        sfor<4>([&](auto r) {
            L.nq[wi][0][(4 * g + r) * LT + n] = gn[int(r)];
            L.nq[wi][1][(4 * g + r) * LT + n] = gq[int(r)];
        });
    }

    // The two C x C factors of the memory chain from the waves' partials in
    // L.nq (rows scaled by 1/|w|, invn4 from inv_norms4): (I + N)^-1 and
    // (Alpha^'Phi) o Up, each stored transposed (X'[m][t] = X[t][m], rows as
    // swz16 places them), so that lane 16 g + n reads X[4 g + r][n] as four
    // consecutive floats at swz16(n, g).  One wave computes them.
    // With ydst, also the solved key cross factor of the pair (previous chunk,
    // this one) from qk, the previous chunk's Alpha^'K^ (solved_cross; wave wi + 1's
    // scratch, unused otherwise).
    __device__ __forceinline__ void prep_tp(float *tt, float *pt, f4 invn4, f4 qk = {}, float *ydst = nullptr)
    {
        float NNr[16];
        f4 qa;
        sfor<4>([&](auto r) {   // -N[4g+r][n] (strictly upper), rows through LDS
            float a = L.nq[0][0][(4 * g + r) * LT + n];
            sfor<NA - 1>([&](auto w2) { a += L.nq[w2 + 1][0][(4 * g + r) * LT + n]; });
            const float sc = 4 * g + r < n ? -invn4[int(r)] : 0.f;   // a select, not a branch
            L.tit[wi][(4 * g + r) * LT + n] = a * sc;
        });
        wave_lds_order();
        sfor<4>([&](auto q4) {
            const f4 a = ld4(&L.tit[wi][n * LT + 4 * q4]);
            sfor<4>([&](auto r) { NNr[4 * q4 + r] = a[int(r)]; });
        });
        sfor<4>([&](auto r) {
            float a = L.nq[0][1][(4 * g + r) * LT + n];
            sfor<NA - 1>([&](auto w2) { a += L.nq[w2 + 1][1][(4 * g + r) * LT + n]; });
            qa[int(r)] = a * (4 * g + r <= n ? invn4[int(r)] : 0.f);
        });
        st4(&pt[swz16(n, g)], qa);
        float X[4];
        sfor<4>([&](auto c) { X[c] = n == 4 * c + g ? 1.f : 0.f; });
        asm volatile(VLA_TINV_BLOCK
                     : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3])
                     : "v"(NNr[1]), "v"(NNr[2]), "v"(NNr[3]), "v"(NNr[4]), "v"(NNr[5]),
                       "v"(NNr[6]), "v"(NNr[7]), "v"(NNr[8]), "v"(NNr[9]), "v"(NNr[10]),
                       "v"(NNr[11]), "v"(NNr[12]), "v"(NNr[13]), "v"(NNr[14]), "v"(NNr[15]));
        sfor<4>([&](auto c) { tt[swz16(4 * c + g, n >> 2) + (n & 3)] = X[c]; });   // column 4c+g of (I+N)^-1
        if (ydst) solved_cross(qk, X, g, n, L.tit[wi], L.tit[wi + 1], ydst);
    }

};

}  // namespace chunk
}  // namespace vla
