// vla_sweep.h -- the symmetric sweep operator (fp64) that inverts a symmetric
// positive definite d x d matrix in place: on fp64 matrix-core tiles for the
// segment inverses of the forward (sweep_tiles), and with one matrix row per
// group of threads for the initial-state adjoint of the gradients (sweep_all).
#pragma once
#include "vla_chunk_parts.h"

namespace vla {
namespace chunk {

// 4 x 4 block inverse for the sweeps: lanes e < 16 each form entry (r, c) =
// (e >> 2, e & 3) of B^-1 = adj(B) / det(B), with B[r][c] = bb[r * stride + c] +
// [r == c] (the published rows hold B - I), and write it to dst[4 r + c].  Every
// lane forms det(B) from the 2 x 2 minors of rows 0-1 and 2-3, and its entry from
// the 3 x 3 minor of B without row c and column r.
__device__ __forceinline__ void block_inverse4(const double *bb, int stride, int e, double *dst)
{
    auto B = [&](int r, int c) { return bb[r * stride + c] + (r == c ? 1.0 : 0.0); };
    double a[16];
    sfor<16>([&](auto q) { a[q] = B(q / 4, q % 4); });
    const double s0 = a[0] * a[5] - a[4] * a[1], s1 = a[0] * a[6] - a[4] * a[2];
    const double s2 = a[0] * a[7] - a[4] * a[3], s3 = a[1] * a[6] - a[5] * a[2];
    const double s4 = a[1] * a[7] - a[5] * a[3], s5 = a[2] * a[7] - a[6] * a[3];
    const double d5 = a[10] * a[15] - a[14] * a[11], d4 = a[9] * a[15] - a[13] * a[11];
    const double d3 = a[9] * a[14] - a[13] * a[10], d2 = a[8] * a[15] - a[12] * a[11];
    const double d1 = a[8] * a[14] - a[12] * a[10], d0 = a[8] * a[13] - a[12] * a[9];
    const double det = s0 * d5 - s1 * d4 + s2 * d3 + s3 * d2 - s4 * d1 + s5 * d0;
    const int r = e >> 2, c = e & 3;
    double mm[3][3];
    sfor<3>([&](auto t) {
        const int row = int(t) + (int(t) >= c ? 1 : 0);
        sfor<3>([&](auto u) { mm[t][u] = B(row, int(u) + (int(u) >= r ? 1 : 0)); });
    });
    const double minor = mm[0][0] * (mm[1][1] * mm[2][2] - mm[1][2] * mm[2][1]) -
                         mm[0][1] * (mm[1][0] * mm[2][2] - mm[1][2] * mm[2][0]) +
                         mm[0][2] * (mm[1][0] * mm[2][1] - mm[1][1] * mm[2][0]);
    dst[4 * r + c] = ((r + c) & 1 ? -minor : minor) / det;
}

// In-place symmetric sweep of all pivots, four at a time: M -> -M^-1 (M
// symmetric positive definite, so no pivoting is needed).  Thread (row i,
// columns [c0, c0 + EPT)) holds its entries in m.  For the pivot block K of
// rows/columns 4s .. 4s+3 with diagonal block B, rows K of the current matrix
// are published with B replaced by B - I (R, 4 x D), together with B^-1; then
//     m <- m - (R' B^-1) R
// gives every entry of the block sweep except the diagonal of B's block, which
// is 2 too large.  One barrier per block (row buffers double-buffered); the
// first 16 lanes of the publishing threads form B^-1 (block_inverse4).  Only
// compile-time indices into m, so that it stays in registers.
template <int D, int EPT>
__device__ __forceinline__ void sweep_all(double (&m)[EPT], int i, int c0, double (*rowbuf)[4 * D + 16])
{
    static_assert(EPT % 2 == 0 && D % 4 == 0, "row slices are read as pairs");
    auto publish = [&](int s, int slot) {
        const int k = 4 * s;
        if (i >= k && i < k + 4) {
            double *rw = rowbuf[slot] + (i - k) * D;
            sfor<EPT>([&](auto e) { rw[c0 + e] = c0 + e == i ? m[e] - 1.0 : m[e]; });
            wave_lds_order();   // rows K sit in one wave (threads 4 TPR s .. 4 TPR s + 4 TPR - 1)
            // B^-1, one entry per lane in the first 16 publishing lanes
            const int e = (i - k) * (D / EPT) + c0 / EPT;
            if (e < 16) block_inverse4(rowbuf[slot] + k, D, e, rowbuf[slot] + 4 * D);
        }
    };
    publish(0, 0);
    __syncthreads();
    for (int sb = 0; sb < D / 4; ++sb) {
        const double *rb = rowbuf[sb & 1];
        // B^-1 is the same for every thread: one lane per wave reads it, and it
        // reaches the others as scalars (LDS bandwidth is this loop's bound)
        double bi[16];
        {
            double2 x[8];
            if ((threadIdx.x & 63) == 0) {
                sfor<8>([&](auto q) { x[q] = *reinterpret_cast<const double2 *>(&rb[4 * D + 2 * q]); });
            } else {
                sfor<8>([&](auto q) { x[q] = make_double2(0.0, 0.0); });
            }
            auto bcast = [](double v) {
                const unsigned long long b = __double_as_longlong(v);
                const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
                const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
                return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
            };
            sfor<8>([&](auto q) {
                bi[2 * q] = bcast(x[q].x);
                bi[2 * q + 1] = bcast(x[q].y);
            });
        }
        double ui[4] = {0.0, 0.0, 0.0, 0.0};   // row i of R' B^-1
#pragma unroll
        for (int a2 = 0; a2 < 4; ++a2) {
            const double ra = rb[a2 * D + i];
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) ui[b2] = fma(ra, bi[4 * a2 + b2], ui[b2]);
        }
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) {
            sfor<EPT / 2>([&](auto h) {
                const double2 x = *reinterpret_cast<const double2 *>(&rb[b2 * D + c0 + 2 * h]);
                m[2 * h] = fma(-ui[b2], x.x, m[2 * h]);
                m[2 * h + 1] = fma(-ui[b2], x.y, m[2 * h + 1]);
            });
        }
        const int k = 4 * sb;
        if (i >= k && i < k + 4) {   // the lanes holding the block diagonal
            const int ed = i - c0;
            sfor<EPT>([&](auto e) { m[e] -= e == ed ? 2.0 : 0.0; });
        }
        if (sb + 1 < D / 4) publish(sb + 1, (sb + 1) & 1);
        __syncthreads();
    }
}


typedef double dbl4 __attribute__((ext_vector_type(4)));

// fp64 matrix-core tile of a D x D matrix: wave I of a workgroup of D / 16 waves
// holds tile row I, and register i of lane l of tile (I, J) is
//     M[16 I + l / 16 + 4 i][16 J + l % 16],
// the accumulator layout of v_mfma_f64_16x16x4f64 (which takes A[m][k] from lane
// 16 k + m and B[k][n] from lane 16 k + n).
template <int D>
using Tiles64 = dbl4[D / 16];

// The symmetric sweep of sweep_all on tiles: M -> -M^-1 for symmetric positive
// definite M, four pivots per step.  The rows K = 4s .. 4s + 3 of the pivot
// block sit in tile row s / 4, in register s % 4 of the four lane groups (row
// 4 (s % 4) + g in group g); that wave publishes them with the diagonal block B
// replaced by B - I, and B^-1, and after one barrier every wave applies
//     M <- M - (R' B^-1) R
// to its tiles as a rank-4 matrix-core update (A operand -(R' B^-1) for the
// tile row's 16 rows, B operand R for each tile column), then takes 2 off the
// diagonal of B's block (the update leaves it 2 too large).  Register indices
// are compile-time (the steps of a tile row are unrolled), so the tiles stay in
// registers.
template <int D>
__device__ __forceinline__ void sweep_tiles(Tiles64<D> &t, int I, int lane, double (*rowbuf)[4 * D + 16])
{
    constexpr int NB = D / 16;
    const int g = lane >> 4, n = lane & 15;
    auto publish = [&](int Is, auto Q, double *rw) {   // pivot block 4 Is + Q (Q compile-time)
        constexpr int q = decltype(Q)::value;
        if (I != Is) return;   // wave-uniform
        sfor<NB>([&](auto J) {
            double x = t[J][q];
            if (int(J) == Is && n == 4 * q + g) x -= 1.0;   // B - I on the diagonal
            rw[g * D + 16 * J + n] = x;
        });
        wave_lds_order();
        if (lane < 16) block_inverse4(rw + 16 * Is + 4 * q, D, lane, rw + 4 * D);
    };
    publish(0, ic<0>{}, rowbuf[0]);
    __syncthreads();
    for (int Is = 0; Is < NB; ++Is) {
        sfor<4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            const double *R = rowbuf[q & 1];
            // U[16 I + n][g] = sum_a R[a][16 I + n] B^-1[a][g]
            double ra[4], bi[4];
            sfor<4>([&](auto a) {
                ra[a] = R[a * D + 16 * I + n];
                bi[a] = R[4 * D + 4 * a + g];
            });
            double nu = 0.0;
            sfor<4>([&](auto a) { nu = fma(-ra[a], bi[a], nu); });
            sfor<NB>([&](auto J) {
                t[J] = __builtin_amdgcn_mfma_f64_16x16x4f64(nu, R[g * D + 16 * J + n], t[J], 0, 0, 0);
            });
            if (I == Is) {
                sfor<NB>([&](auto J) {
                    if (int(J) == Is && n == 4 * q + g) t[J][q] -= 2.0;
                });
            }
            if constexpr (q < 3) {
                publish(Is, ic<q + 1>{}, rowbuf[(q + 1) & 1]);
            } else {
                if (Is + 1 < NB) publish(Is + 1, ic<0>{}, rowbuf[0]);
            }
            __syncthreads();
        });
    }
}

}  // namespace chunk
}  // namespace vla
