// vla_fwd_kernel.hip -- register-resident gfx950 kernel of the VLA recurrence
// for d_h in {64, 96, 128}.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9) (Sherman-Morrison downdate of A), (10) (gated delta write of S) and
// (11) (ELU+1 readout with the running key sum); A_0 = I / lambda0 (section 3.2).
//
// Mapping.  One workgroup owns one (batch, head) for all T tokens, with
// NW = d/16 wavefronts.  Wave w owns rows 16w .. 16w+15 of both A and S; lane
// l = 16g + n (g = lane group = 16-lane DPP row, n = row within it) holds row
// 16w + n and the columns of group g:
//     columns 16g + m            for m = 0..15
//     columns 64 + SW1 g + m     for m = 0..SW1-1   (SW1 = (d-64)/4)
// so each lane keeps CPL = 16 + SW1 entries of A and of S in VGPRs for the
// whole sequence.  A "lane-distributed" vector keeps element 16g + n in lane
// 16g + n (and element 64 + SW1 g + n in a second register), so the value of
// column j for the whole 16-lane row is one DPP row_newbcast away: every
// multiply-add of a matrix-vector product or rank-1 update is a single
// v_fmac_f32 with a DPP-broadcast source operand.  Row results are summed over
// the four lane groups with the gfx950 permlane32/permlane16 swaps.
//
// Per token, the only cross-wave exchange is one LDS all-gather of z (the
// Sherman-Morrison vector) and of y (= A k^), plus four dot-product partials,
// behind a single s_barrier.  The penalty chain runs one token ahead of the
// memory chain and the readout one token behind it:
//     iteration t:  A-pass of token t   (apply z_{t-1}; z_t = A u^_t, w_t = A k^_t)
//                   S-pass of token t-1 (apply e_{t-2} alpha^_{t-2}; S k^_{t-1},
//                                        S phi(q_{t-1}); e_{t-1})
//                   readout of token t-2
// using A_t k^ = A_{t-1} k^ - z (z'k^)/delta (Eq. 9 applied to k^), so that
// y_t = A_t k^_t needs only row-local data and two scalars.
//
// State-independent work (k^, u^, phi(q), the key-sum prefix and the readout
// denominator) is done per tile of TT tokens in a prologue and kept in an LDS
// ring of TT+8 token slots; the raw inputs of the next tile are prefetched into
// registers while the current tile runs.
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
// this (DPP read-after-VALU-write hazard): every x used here comes straight from
// an LDS load.
template <int M>
__device__ __forceinline__ void fmac_bc(float &acc, float x, float y)
{
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(x), "v"(y), "n"(M));
}

// Sum over lanes l, l^16, l^32, l^48 (the four lane groups); every lane gets the
// same bits.
__device__ __forceinline__ float sum_groups(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
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

template <int D>
struct FastCfg {
    static constexpr int NW = D / 16;            // wavefronts per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int SW1 = (D - 64) / 4;     // second column segment per lane group
    static constexpr int CPL = 16 + SW1;         // matrix columns per lane
    static constexpr int TT = D > 96 ? 32 : 64;  // tokens per prologue tile
    static constexpr int RING = TT + 8;          // LDS token slots (>= TT + 2)
    static constexpr int RS = D + 4;             // padded LDS row stride (floats)
    static constexpr int CPT = D * TT / NT;      // prologue columns per thread
    static constexpr int NCH = D / CPT;          // prologue column chunks per token
};

// 16 (fp32) or 8/16 (bf16) consecutive inputs of one token, held in registers.
template <typename Tin, int N> struct RawVec;
template <int N> struct RawVec<float, N> {
    float4 x[N / 4];
    __device__ __forceinline__ void load(const float *p, bool ok)
    {
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            x[i] = ok ? reinterpret_cast<const float4 *>(p)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ float get(int i) const
    {
        const float4 &v = x[i >> 2];
        switch (i & 3) {
        case 0: return v.x;
        case 1: return v.y;
        case 2: return v.z;
        default: return v.w;
        }
    }
};
template <int N> struct RawVec<uint16_t, N> {
    uint4 x[N / 8];
    __device__ __forceinline__ void load(const uint16_t *p, bool ok)
    {
#pragma unroll
        for (int i = 0; i < N / 8; ++i)
            x[i] = ok ? reinterpret_cast<const uint4 *>(p)[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    __device__ __forceinline__ float get(int i) const
    {
        const uint4 &v = x[i >> 3];
        uint32_t wd;
        switch ((i >> 1) & 3) {
        case 0: wd = v.x; break;
        case 1: wd = v.y; break;
        case 2: wd = v.z; break;
        default: wd = v.w; break;
        }
        return (i & 1) ? bf16_hi(wd) : bf16_lo(wd);
    }
};

template <int D, typename Tin>
__global__ void __launch_bounds__(FastCfg<D>::NT)
vla_fwd_fast(const Tin *__restrict__ q, const Tin *__restrict__ k,
             const Tin *__restrict__ v, const Tin *__restrict__ u,
             int T, float lambda0, float eps,
             float *__restrict__ o, float *S_out, float *A_out, float *zk_out,
             const float *S0, const float *A0, const float *zk0)
{
    using C = FastCfg<D>;
    constexpr int NW = C::NW, NT = C::NT, SW1 = C::SW1, CPL = C::CPL, TT = C::TT;
    constexpr int RING = C::RING, RS = C::RS, CPT = C::CPT, NCH = C::NCH;

    __shared__ __align__(16) float s_kh[RING * RS];   // k^ per token slot
    __shared__ __align__(16) float s_uh[RING * RS];   // u^
    __shared__ __align__(16) float s_pq[RING * RS];   // phi(q)
    __shared__ __align__(16) float s_v[RING * RS];    // v
    __shared__ __align__(16) float s_zk[TT * RS];     // phi(k), then the key sum, of a tile
    __shared__ float s_rden[RING];                    // 1 / max(phi(q)' zkey, eps)
    __shared__ float s_part[2][NCH][TT];              // prologue partial sums
    __shared__ float s_z[2][D];                       // all-gather of z_t
    __shared__ float s_y[2][D];                       // all-gather of y_{t-1}
    __shared__ float s_red[2][4][NW];                 // per-wave dot-product partials

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g = l >> 4, n = l & 15;
    const int row = 16 * w + n;
    const size_t bh = blockIdx.x;
    const size_t DD = (size_t)D * D;
    // lane-distributed second-segment element of this lane (lanes n >= SW1 read a
    // valid dummy; their values are never broadcast)
    const int l1 = 64 + SW1 * g + (n < SW1 ? n : (SW1 > 0 ? SW1 - 1 : 0));

    // ---------------------------------------------------------------- state
    float a[CPL], s[CPL];
    sfor<CPL>([&](auto mm) {
        constexpr int m = decltype(mm)::value;
        const int j = m < 16 ? 16 * g + m : 64 + SW1 * g + (m - 16);
        const size_t idx = bh * DD + (size_t)row * D + j;
        a[m] = A0 ? A0[idx] : (row == j ? 1.f / lambda0 : 0.f);
        s[m] = S0 ? S0[idx] : 0.f;
    });
    float zk_run = 0.f, zk_cmp = 0.f;          // key-sum column tid (tid < D), Kahan
    if (tid < D && zk0) zk_run = zk0[bh * D + tid];

    for (int i = tid; i < RING * RS; i += NT) {
        s_kh[i] = 0.f;
        s_uh[i] = 0.f;
        s_pq[i] = 0.f;
        s_v[i] = 0.f;
    }
    for (int i = tid; i < RING; i += NT) s_rden[i] = 0.f;
    for (int i = tid; i < 2 * D; i += NT) {
        (&s_z[0][0])[i] = 0.f;
        (&s_y[0][0])[i] = 0.f;
    }
    for (int i = tid; i < 2 * 4 * NW; i += NT) (&s_red[0][0][0])[i] = 0.f;

    // prologue thread mapping: token tl of the tile, columns [ch*CPT, ch*CPT+CPT)
    const int tl = tid % TT, ch = tid / TT;
    const size_t tok_base = bh * (size_t)T;
    RawVec<Tin, CPT> rq, rk, rv, ru;
    auto prefetch = [&](int t0) {
        const int t = t0 + tl;
        const bool ok = t < T;
        const size_t off = (tok_base + (size_t)(ok ? t : 0)) * D + (size_t)ch * CPT;
        rq.load(q + off, ok);
        rk.load(k + off, ok);
        rv.load(v + off, ok);
        ru.load(u + off, ok);
    };
    prefetch(0);
    __syncthreads();

    // carried row values (lane's row 16w+n; identical in the four lane groups)
    float zr = 0.f, wr = 0.f;   // z_{t-1}, w_{t-1} = A_{t-2} k^_{t-1}
    float ep = 0.f, pp = 0.f;   // e_{t-2}, (S_{t-3} phi(q_{t-2}))

    const int ntiles = (T + 2 + TT - 1) / TT;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int t0 = tile * TT;
        // ------------------------------------------- tile prologue (no state)
        {
            const int t = t0 + tl;
            const bool ok = t < T;
            const int slot = t % RING;
            float pk = 0.f, pu = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                pk = fmaf(rk.get(i), rk.get(i), pk);
                pu = fmaf(ru.get(i), ru.get(i), pu);
            }
            s_part[0][ch][tl] = pk;
            s_part[1][ch][tl] = pu;
            __syncthreads();
            float nk = 0.f, nu = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < NCH; ++c2) {
                nk += s_part[0][c2][tl];
                nu += s_part[1][c2][tl];
            }
            const float ik = nk > 0.f ? 1.f / sqrtf(nk) : 0.f;
            const float iu = nu > 0.f ? 1.f / sqrtf(nu) : 0.f;
            const int base = slot * RS + ch * CPT;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                s_kh[base + i] = rk.get(i) * ik;
                s_uh[base + i] = ru.get(i) * iu;
                s_pq[base + i] = phi(rq.get(i));
                s_v[base + i] = rv.get(i);
                s_zk[tl * RS + ch * CPT + i] = ok ? phi(rk.get(i)) : 0.f;
            }
            __syncthreads();
            if (tid < D) {   // inclusive running key sum down the tile, per column
                for (int tt = 0; tt < TT; ++tt) {
                    const float x = s_zk[tt * RS + tid];
                    const float yk = x - zk_cmp;
                    const float ts = zk_run + yk;
                    zk_cmp = (ts - zk_run) - yk;
                    zk_run = ts;
                    s_zk[tt * RS + tid] = zk_run;
                }
            }
            __syncthreads();
            float pd = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                pd = fmaf(s_pq[base + i], s_zk[tl * RS + ch * CPT + i], pd);
            s_part[0][ch][tl] = pd;
            __syncthreads();
            if (ch == 0) {
                float dsum = 0.f;
#pragma unroll
                for (int c2 = 0; c2 < NCH; ++c2) dsum += s_part[0][c2][tl];
                s_rden[slot] = 1.f / fmaxf(dsum, eps);
            }
            // s_rden[slot] is first read two iterations later, after two barriers.
        }
        if (tile + 1 < ntiles) prefetch(t0 + TT);

        const int tend = min(t0 + TT, T + 2);
        for (int t = t0; t < tend; ++t) {
            const int pb = (t + 1) & 1, cb = t & 1;
            const int st = t % RING;                  // slot of token t
            const int sp = (t + RING - 1) % RING;     // slot of token t-1

            // ---- P1: results of the exchange for token t-1
            const float zc0 = s_z[pb][l], zc1 = SW1 ? s_z[pb][l1] : 0.f;   // z_{t-1}
            const float yc0 = s_y[pb][l], yc1 = SW1 ? s_y[pb][l1] : 0.f;   // y_{t-2}
            float ud = 0.f, kd = 0.f, yy = 0.f, yq = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                ud += s_red[pb][0][ww];    // u^_{t-1}' z_{t-1}
                kd += s_red[pb][1][ww];    // k^_{t-1}' z_{t-1}
                yy += s_red[pb][2][ww];    // |y_{t-2}|^2
                yq += s_red[pb][3][ww];    // y_{t-2}' phi(q_{t-2})
            }
            const float invd = 1.f / (1.f + ud);              // 1 / delta_{t-1}
            const float nc = -(zr * invd);                     // -z_i / delta
            const float yr = wr - zr * (kd * invd);           // y_{t-1} = A_{t-1} k^_{t-1}
            const float ny = yy > 0.f ? rsqrtf(yy) : 0.f;     // 1 / |y_{t-2}|
            if (t >= 2 && t - 2 < T && g == 0) {               // readout of token t-2
                const float aq = yq * ny;                      // alpha^' phi(q)
                o[(tok_base + (size_t)(t - 2)) * D + row] = (pp + ep * aq) * s_rden[(t - 2) % RING];
            }

            // ---- P2: A-pass of token t
            const float u0 = s_uh[st * RS + l], u1 = SW1 ? s_uh[st * RS + l1] : 0.f;
            const float k0 = s_kh[st * RS + l], k1 = SW1 ? s_kh[st * RS + l1] : 0.f;
            float za = 0.f, wa = 0.f;
            sfor<CPL>([&](auto mm) {
                constexpr int m = decltype(mm)::value;
                if constexpr (m < 16) {
                    fmac_bc<m>(a[m], zc0, nc);
                    fmac_bc<m>(za, u0, a[m]);
                    fmac_bc<m>(wa, k0, a[m]);
                } else {
                    fmac_bc<m - 16>(a[m], zc1, nc);
                    fmac_bc<m - 16>(za, u1, a[m]);
                    fmac_bc<m - 16>(wa, k1, a[m]);
                }
            });
            const float zn = sum_groups(za), wn = sum_groups(wa);

            // ---- P3: S-pass of token t-1
            const float kp0 = s_kh[sp * RS + l], kp1 = SW1 ? s_kh[sp * RS + l1] : 0.f;
            const float q0 = s_pq[sp * RS + l], q1 = SW1 ? s_pq[sp * RS + l1] : 0.f;
            const float vrow = s_v[sp * RS + row];
            const float se = ep * ny;          // alpha^_{t-2,j} e_{t-2,i} = y_j * (e_i / |y|)
            float ra = 0.f, pa = 0.f;
            sfor<CPL>([&](auto mm) {
                constexpr int m = decltype(mm)::value;
                if constexpr (m < 16) {
                    fmac_bc<m>(s[m], yc0, se);
                    fmac_bc<m>(ra, kp0, s[m]);
                    fmac_bc<m>(pa, q0, s[m]);
                } else {
                    fmac_bc<m - 16>(s[m], yc1, se);
                    fmac_bc<m - 16>(ra, kp1, s[m]);
                    fmac_bc<m - 16>(pa, q1, s[m]);
                }
            });
            const float rn = sum_groups(ra), pn = sum_groups(pa);

            // ---- P4: exchange (one s_barrier)
            // group 0: u^_t'z_t, group 1: k^_t'z_t, group 2: |y_{t-1}|^2,
            // group 3: y_{t-1}'phi(q_{t-1}), each summed over this wave's 16 rows
            const float rhs_mem = g == 0 ? s_uh[st * RS + row]
                                : g == 1 ? s_kh[st * RS + row] : s_pq[sp * RS + row];
            const float lhs = g < 2 ? zn : yr;
            const float rhs = g == 2 ? yr : rhs_mem;
            const float part = sum_row16(lhs * rhs);
            if (n == 0) s_red[cb][g][w] = part;
            if (g == 0) {
                s_z[cb][row] = zn;
                s_y[cb][row] = yr;
            }
            zr = zn;
            wr = wn;
            ep = vrow - rn;    // e_{t-1} = v - S_{t-2} k^  (S before token t-1's write)
            pp = pn;
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- epilogue
    sfor<CPL>([&](auto mm) {
        constexpr int m = decltype(mm)::value;
        const int j = m < 16 ? 16 * g + m : 64 + SW1 * g + (m - 16);
        const size_t idx = bh * DD + (size_t)row * D + j;
        if (A_out) A_out[idx] = a[m];
        if (S_out) S_out[idx] = s[m];
    });
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
