// vla_scan.hip -- the memory chain of the forward (Eqs. (10), (11)) as a
// parallel scan over chunks, d_h in {64, 96, 128}: the pages' own parallel form,
// built to be measured against the chained memory pass.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.4,
// Eq. (12): the write of Eq. (10) is an affine map of S, so the states are a
// scan of those maps.  As printed, Eq. (12) multiplies on the wrong side:
// Eq. (10) gives S_t = S_{t-1} (I - k^ alpha^') + v alpha^', a right
// multiplication, so a map is a pair (F, G): S -> S F + G, and applying
// (F1, G1) and then (F2, G2) is (F1 F2, G1 F2 + G2).  Over a chunk of 16 tokens
// the maps compose to F = I - K^ T Alpha^', G = V T Alpha^' (T = (I + N)^-1 of
// the chunked form, K^, V, Alpha^ with the chunk's tokens as columns).
//
//   penalty pass  the forward's first pass: per-chunk records (alpha^, T, P,
//                 1/den, k^, phi(q); vla_record.h), final A and zkey
//   vla_scan_maps (F_c, G_c) per chunk from its record and v; identity maps up
//                 to a power of two n; S_0 folded into G_0 (G_0 <- S_0 F_0 + G_0)
//   vla_scan_level  log2 n up-sweep and log2 n down-sweep levels of the
//                 work-efficient (Blelloch) scan; one workgroup per combine, two
//                 d x d x d products on fp32 matrix cores
//   vla_scan_apply  S at each chunk start (the G of the exclusive prefix; S_0 for
//                 the first chunk), then the chunk's readout
//                 E = (V - S K^) T, o = (S Phi + E P) / den; final S = the total's G
//
// Work: the combines cost 2 (n - 1) x 4 d^3 FLOP per head against the chain's
// 6 d^2 per token, which is the point of the comparison.
#include "vla_chunk_parts.h"
#include "vla_common.h"
#include "vla_record.h"

namespace vla {
namespace {

using namespace chunk;
using rec::CH;
using rec::Rec;

// map slots of a head: n chunk maps, then the total
__host__ __device__ inline size_t slot_floats(int n, int d) { return (size_t)(n + 1) * 2 * d * d; }

// ------------------------------------------------------------------- maps
// Thread (row i, columns [j0, j0 + 16)) of both maps: d^2 / 16 threads.
template <int D, typename Tin>
__global__ void __launch_bounds__(D * D / 16)
vla_scan_maps(const Tin *__restrict__ v, int T, int NC, int n, const float *__restrict__ recs,
              const float *S0, float *__restrict__ maps)
{
    constexpr int RS = Rec<D>::SIZE, P = D + 1, DD = D * D, NT = DD / 16;
    __shared__ float tinv[CH][CH + 1];            // T[t][s]
    __shared__ __align__(16) float al[CH][D + 4];   // alpha^_s[j] (rows 16-byte aligned)
    __shared__ float kh[CH][P], vv[CH][P];        // k^_t[i], v_t[i]
    __shared__ float xk[D][CH + 1], xv[D][CH + 1];   // (K^ T)[i][s], (V T)[i][s]
    __shared__ float f0[D * P];                   // F_0 (first chunk with S_0)

    const int bh = blockIdx.x / n, c = blockIdx.x % n, tid = threadIdx.x;
    float *F = maps + (size_t)bh * slot_floats(n, D) + (size_t)c * 2 * DD, *G = F + DD;
    if (c >= NC) {   // identity map
        for (int idx = tid * 4; idx < DD; idx += 4 * NT) {
            f4 x;
            sfor<4>([&](auto r) { x[int(r)] = (idx + r) / D == (idx + r) % D ? 1.f : 0.f; });
            st4(F + idx, x);
            st4(G + idx, f4{0.f, 0.f, 0.f, 0.f});
        }
        return;
    }
    const float *r = recs + ((size_t)bh * NC + c) * RS;
    if (tid < CH * CH) {
        const int t = tid >> 4, s = tid & 15;
        tinv[t][s] = r[Rec<D>::TT + swz16(s, t >> 2) + (t & 3)];   // stored transposed
    }
    for (int idx = tid; idx < CH * D; idx += NT) {
        const int s = idx / D, j = idx % D;
        al[s][j] = r[Rec<D>::AH + swz16(j, s >> 2) + (s & 3)];
        kh[s][j] = r[Rec<D>::KH + swzd<D>(s, j >> 2) + (j & 3)];
        const int tok = c * CH + s;
        vv[s][j] = tok < T ? load_in(v, ((size_t)bh * T + tok) * D + j) : 0.f;
    }
    __syncthreads();
    for (int idx = tid; idx < D * CH; idx += NT) {
        const int i = idx / CH, s = idx % CH;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            a = fmaf(kh[t][i], tinv[t][s], a);
            b = fmaf(vv[t][i], tinv[t][s], b);
        }
        xk[i][s] = a;
        xv[i][s] = b;
    }
    __syncthreads();
    // one pass over the chunk's tokens s
    const int i = tid / (D / 16), j0 = (tid % (D / 16)) * 16;
    float fr[16], gr[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        fr[jj] = i == j0 + jj ? 1.f : 0.f;
        gr[jj] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < CH; ++s) {
        const float xa = -xk[i][s], xb = xv[i][s];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const f4 av = ld4(&al[s][j0 + 4 * h]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                fr[4 * h + r] = fmaf(xa, av[r], fr[4 * h + r]);
                gr[4 * h + r] = fmaf(xb, av[r], gr[4 * h + r]);
            }
        }
    }
    if (c == 0 && S0) {   // G_0 <- S_0 F_0 + G_0
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) f0[i * P + j0 + jj] = fr[jj];
        __syncthreads();
        const float *s0 = S0 + (size_t)bh * DD + (size_t)i * D;
        for (int m = 0; m < D; ++m) {
            const float sm = s0[m];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) gr[jj] = fmaf(sm, f0[m * P + j0 + jj], gr[jj]);
        }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        st4(F + i * D + j0 + 4 * h, f4{fr[4 * h], fr[4 * h + 1], fr[4 * h + 2], fr[4 * h + 3]});
        st4(G + i * D + j0 + 4 * h, f4{gr[4 * h], gr[4 * h + 1], gr[4 * h + 2], gr[4 * h + 3]});
    }
}

// ------------------------------------------------------------------- scan
// One combine per workgroup: L then R, out = (F_L F_R, G_L F_R + G_R).
//   up-sweep (pair i = (k + 1) 2 span - 1, j = i - span): L = slot j, R = slot i,
//     out to slot i; at the last level (one pair, i = n - 1) out goes to the
//     total slot and slot n - 1 becomes the identity;
//   down-sweep: L = slot i (the prefix before the pair), R = slot j (the left
//     half's total): out to slot i, and slot j <- L.
// Wave w (d / 16 waves) forms row block w of both products: lane (n, g) holds
// rows 16 w + n of F_L and G_L, columns KG g .. KG g + KG - 1 (KG = d / 4), and
// k-step s contracts over key KG g + s (A operand from registers, B = F_R from
// LDS, rows padded to d + 1).
template <int D, bool DOWN, bool LAST>
__global__ void __launch_bounds__(4 * D)
vla_scan_level(float *maps, int n, int span)
{
    constexpr int P = D + 1, DD = D * D, NT = 4 * D, KG = D / 4, TN = D / 16;
    __shared__ float fr[D * P];

    const int per = n / (2 * span);
    const int bh = blockIdx.x / per, k = blockIdx.x % per;
    const int i = (k + 1) * 2 * span - 1, j = i - span;
    float *base = maps + (size_t)bh * slot_floats(n, D);
    float *Si = base + (size_t)i * 2 * DD, *Sj = base + (size_t)j * 2 * DD;
    const float *FL = DOWN ? Si : Sj, *FR = DOWN ? Sj : Si;
    const float *GL = FL + DD, *GR = FR + DD;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nn = lane & 15, g = lane >> 4;
    for (int idx = tid * 4; idx < DD; idx += 4 * NT) {
        const f4 x = ld4(FR + idx);
        const int row = idx / D, col = idx % D;
        sfor<4>([&](auto r) { fr[row * P + col + r] = x[int(r)]; });
    }
    float af[KG], ag[KG];
    {
        const float *fl = FL + (16 * w + nn) * D + KG * g, *gl = GL + (16 * w + nn) * D + KG * g;
        sfor<KG / 4>([&](auto h) {
            const f4 x = ld4(fl + 4 * h), y = ld4(gl + 4 * h);
            sfor<4>([&](auto r) {
                af[4 * h + r] = x[int(r)];
                ag[4 * h + r] = y[int(r)];
            });
        });
    }
    f4 accF[TN], accG[TN];
    sfor<TN>([&](auto tn) {
        accF[tn] = f4{0.f, 0.f, 0.f, 0.f};
        sfor<4>([&](auto r) { accG[tn][int(r)] = GR[(16 * w + 4 * g + r) * D + 16 * tn + nn]; });
    });
    __syncthreads();   // every read of slot j and of slot i is done before either is written

    sfor<KG>([&](auto s) {
        sfor<TN>([&](auto tn) {
            const float b = fr[(KG * g + s) * P + 16 * tn + nn];
            accF[tn] = mma(af[s], b, accF[tn]);
            accG[tn] = mma(ag[s], b, accG[tn]);
        });
    });

    float *out = LAST ? base + (size_t)n * 2 * DD : Si;
    sfor<TN>([&](auto tn) {
        sfor<4>([&](auto r) {
            const int row = 16 * w + 4 * g + r, col = 16 * tn + nn;
            out[row * D + col] = accF[tn][int(r)];
            out[DD + row * D + col] = accG[tn][int(r)];
        });
    });
    if (LAST) {   // slot n - 1 <- identity (this is slot i)
        for (int idx = tid * 4; idx < DD; idx += 4 * NT) {
            f4 x;
            sfor<4>([&](auto r) { x[int(r)] = (idx + r) / D == (idx + r) % D ? 1.f : 0.f; });
            st4(Si + idx, x);
            st4(Si + DD + idx, f4{0.f, 0.f, 0.f, 0.f});
        }
    }
    if (DOWN) {   // slot j <- L (the rows this lane holds)
        float *fj = Sj + (16 * w + nn) * D + KG * g, *gj = Sj + DD + (16 * w + nn) * D + KG * g;
        sfor<KG / 4>([&](auto h) {
            st4(fj + 4 * h, f4{af[4 * h], af[4 * h + 1], af[4 * h + 2], af[4 * h + 3]});
            st4(gj + 4 * h, f4{ag[4 * h], ag[4 * h + 1], ag[4 * h + 2], ag[4 * h + 3]});
        });
    }
}

// ------------------------------------------------------------------- apply
// Workgroup (head, chunk): S at the chunk start, then the chunk's outputs.
// Thread (row i, tokens 4 q .. 4 q + 3): 4 d threads.
template <int D, typename Tin>
__global__ void __launch_bounds__(4 * D)
vla_scan_apply(const Tin *__restrict__ v, int T, int NC, int n, const float *__restrict__ recs,
               const float *S0, const float *__restrict__ maps, float *__restrict__ o,
               float *S_out)
{
    constexpr int RS = Rec<D>::SIZE, P = D + 1, DD = D * D, NT = 4 * D;
    __shared__ float sm[D * P];                     // S at the chunk start
    __shared__ __align__(16) float kt[D][CH], pt[D][CH];   // k^_t[m], phi(q_t)[m] as [m][t]
    __shared__ float vv[CH][P];
    __shared__ float tinv[CH][CH + 1], pm[CH][CH + 1], rd[CH];
    __shared__ float wv[D][CH + 1], ev[D][CH + 1];   // V - S K^, E

    const int bh = blockIdx.x / NC, c = blockIdx.x % NC, tid = threadIdx.x;
    const float *slots = maps + (size_t)bh * slot_floats(n, D);
    const float *Sst = c == 0 ? (S0 ? S0 + (size_t)bh * DD : nullptr)
                              : slots + (size_t)c * 2 * DD + DD;   // G of the exclusive prefix
    for (int idx = tid * 4; idx < DD; idx += 4 * NT) {
        const f4 x = Sst ? ld4(Sst + idx) : f4{0.f, 0.f, 0.f, 0.f};
        const int row = idx / D, col = idx % D;
        sfor<4>([&](auto r) { sm[row * P + col + r] = x[int(r)]; });
    }
    const float *r = recs + ((size_t)bh * NC + c) * RS;
    for (int idx = tid; idx < CH * D; idx += NT) {
        const int s = idx / D, j = idx % D;
        kt[j][s] = r[Rec<D>::KH + swzd<D>(s, j >> 2) + (j & 3)];
        pt[j][s] = r[Rec<D>::PH + swzd<D>(s, j >> 2) + (j & 3)];
        const int tok = c * CH + s;
        vv[s][j] = tok < T ? load_in(v, ((size_t)bh * T + tok) * D + j) : 0.f;
    }
    if (tid < CH * CH) {
        const int t = tid >> 4, s = tid & 15;
        tinv[t][s] = r[Rec<D>::TT + swz16(s, t >> 2) + (t & 3)];
        pm[t][s] = r[Rec<D>::PT + swz16(s, t >> 2) + (t & 3)];
        if (tid < CH) rd[tid] = r[Rec<D>::RD + tid];
    }
    __syncthreads();
    const int i = tid >> 2, q0 = (tid & 3) * 4;
    float sk[4] = {0.f, 0.f, 0.f, 0.f}, sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int m = 0; m < D; ++m) {   // one S entry against the four tokens' k^, phi(q)
        const float sv = sm[i * P + m];
        const f4 kv = ld4(&kt[m][q0]), pv = ld4(&pt[m][q0]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            sk[tt] = fmaf(sv, kv[tt], sk[tt]);
            sp[tt] = fmaf(sv, pv[tt], sp[tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) wv[i][q0 + tt] = vv[q0 + tt][i] - sk[tt];
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = q0 + tt;
        float e = 0.f;
#pragma unroll
        for (int s = 0; s < CH; ++s) e = fmaf(wv[i][s], tinv[s][t], e);
        ev[i][t] = e;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = q0 + tt, tok = c * CH + t;
        float a = sp[tt];
#pragma unroll
        for (int s = 0; s < CH; ++s) a = fmaf(ev[i][s], pm[s][t], a);
        if (tok < T) o[((size_t)bh * T + tok) * D + i] = a * rd[t];
    }
    if (c == 0 && S_out) {   // S_T = the G of the total map (S_0 folded into G_0)
        const float *tg = slots + (size_t)n * 2 * DD + DD;
        for (int idx = tid * 4; idx < DD; idx += 4 * NT)
            st4(S_out + (size_t)bh * DD + idx, ld4(tg + idx));
    }
}

int scan_slots(int NC)
{
    int n = 2;
    while (n < NC) n *= 2;
    return n;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int D, typename Tin>
hipError_t launch(const FwdArgs &a)
{
    const int BH = a.B * a.H, NC = (a.T + CH - 1) / CH, n = scan_slots(NC);
    hipError_t e = launch_forward_twopass(a, 1);   // records, A_out, zkey_out
    if (e != hipSuccess) return e;
    const float *recs = reinterpret_cast<const float *>(static_cast<const char *>(a.ws) +
                                                        twopass_records_offset(BH, a.T, D));
    float *maps = reinterpret_cast<float *>(static_cast<char *>(a.ws) +
                                            up256(twopass_workspace_bytes(BH, a.T, D)));
    const Tin *v = static_cast<const Tin *>(a.v);
    hipLaunchKernelGGL((vla_scan_maps<D, Tin>), dim3(BH * n), dim3(D * D / 16), 0, a.stream, v, a.T,
                       NC, n, recs, a.S0, maps);
    for (int span = 1; span < n; span *= 2) {
        const int grid = BH * (n / (2 * span));
        if (2 * span == n)
            hipLaunchKernelGGL((vla_scan_level<D, false, true>), dim3(grid), dim3(4 * D), 0, a.stream,
                               maps, n, span);
        else
            hipLaunchKernelGGL((vla_scan_level<D, false, false>), dim3(grid), dim3(4 * D), 0,
                               a.stream, maps, n, span);
    }
    for (int span = n / 2; span >= 1; span /= 2)
        hipLaunchKernelGGL((vla_scan_level<D, true, false>), dim3(BH * (n / (2 * span))), dim3(4 * D),
                           0, a.stream, maps, n, span);
    hipLaunchKernelGGL((vla_scan_apply<D, Tin>), dim3(BH * NC), dim3(4 * D), 0, a.stream, v, a.T, NC,
                       n, recs, a.S0, maps, a.o, a.S_out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs &a)
{
    return a.dtype == 1 ? launch<D, uint16_t>(a) : launch<D, float>(a);
}

}  // namespace

bool scan_supported(int d) { return d == 64 || d == 96 || d == 128; }

size_t scan_workspace_bytes(int BH, int T, int d)
{
    if (!scan_supported(d) || T <= 0) return 0;
    const int n = scan_slots((T + CH - 1) / CH);
    return up256(twopass_workspace_bytes(BH, T, d)) +
           up256((size_t)BH * slot_floats(n, d) * sizeof(float));
}

hipError_t launch_forward_scan(const FwdArgs &a)
{
    if (a.T < 1) return hipErrorInvalidValue;
    switch (a.d) {
    case 64: return launch_d<64>(a);
    case 96: return launch_d<96>(a);
    case 128: return launch_d<128>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
