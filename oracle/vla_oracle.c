/*
 * vla_oracle.c -- plain fp64 CPU reference of the Variational Linear Attention
 * (VLA) per-head forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle for the HIP
 * library: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code with the GPU path and the GPU path never
 * calls it.
 *
 * Source: "Variational Linear Attention: Stable Associative Memory for
 * Long-Context Transformers" (arXiv 2605.11196), section 3.2 (lambda0 and the
 * initial A_0 = I / lambda0), section 3.3, Eqs. (9), (10) and (11).
 *
 * Per token t = 1..T, for one attention head of dimension d:
 *   normalise      k^_t = k_t / |k_t|,  u^_t = u_t / |u_t|
 *   Eq. (9)        z_t = A_{t-1} u^_t,  delta_t = 1 + u^_t' z_t,
 *                  A_t = A_{t-1} - z_t z_t' / delta_t
 *   Eq. (10)       e_t = v_t - S_{t-1} k^_t,  alpha^_t = A_t k^_t / |A_t k^_t|,
 *                  S_t = S_{t-1} + e_t alpha^_t'
 *   Eq. (11)       zkey_t = sum_{s<=t} phi(k_s),  phi = ELU + 1,
 *                  o_t = S_t phi(q_t) / max(phi(q_t)' zkey_t, eps)
 *
 * Readings where the pages leave a detail open (each is also listed in the
 * design notes):
 *   - u is unit-normalised here as well as k (section 3.2 states that u is unit
 *     length; normalising an already-unit u changes nothing);
 *   - a zero vector normalises to the zero vector (so u = 0 leaves A unchanged,
 *     k = 0 or A k^ = 0 leaves S unchanged);
 *   - phi in the key sum of Eq. (11) is applied to the raw key k_s, not k^_s;
 *   - ELU uses alpha = 1: phi(x) = x + 1 for x > 0, exp(x) otherwise.
 *
 * Storage: every matrix is d x d row-major, S[i*d + j] with i the value index
 * and j the key index (o = S phi(q)); token arrays are [T][d] row-major.
 * Everything is computed in fp64, one token at a time, in the order above.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define VLA_ORACLE_OK 0
#define VLA_ORACLE_EINVAL 1
#define VLA_ORACLE_ENOMEM 2

/* phi(x) = ELU(x) + 1 with the standard ELU (alpha = 1). */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* out = x / |x|, or the zero vector when |x| = 0. */
static void normalise(const double *x, double *out, int d)
{
    double n2 = 0.0;
    for (int i = 0; i < d; ++i) n2 += x[i] * x[i];
    if (n2 > 0.0) {
        double n = sqrt(n2);
        for (int i = 0; i < d; ++i) out[i] = x[i] / n;
    } else {
        for (int i = 0; i < d; ++i) out[i] = 0.0;
    }
}

/* y = M x for a d x d row-major M. */
static void matvec(const double *M, const double *x, double *y, int d)
{
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += M[(size_t)i * d + j] * x[j];
        y[i] = s;
    }
}

static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += a[i] * b[i];
    return s;
}

/*
 * One head, T tokens.
 *
 * q, k, v, u : [T][d] inputs (exact stored values widened to fp64).
 * S0, A0     : [d][d] initial state, or NULL for the defaults S_0 = 0 and
 *              A_0 = I / lambda0.
 * zkey0      : [d] initial key sum, or NULL for 0.
 * o          : [T][d] output (may be NULL when T == 0).
 * S, A, zkey : final state out ([d][d], [d][d], [d]); required.
 * Optional per-token traces (NULL to skip):
 *   tr_delta [T], tr_alpha [T][d], tr_e [T][d], tr_z [T][d],
 *   tr_den [T], tr_A [T][d][d] (A_t), tr_S [T][d][d] (S_t).
 *
 * Returns 0, or nonzero on bad arguments / allocation failure.
 */
int vla_oracle_forward(int T, int d, double lambda0, double eps,
                       const double *q, const double *k, const double *v, const double *u,
                       const double *S0, const double *A0, const double *zkey0,
                       double *o, double *S, double *A, double *zkey,
                       double *tr_delta, double *tr_alpha, double *tr_e, double *tr_z,
                       double *tr_den, double *tr_A, double *tr_S)
{
    if (T < 0 || d < 1 || !(lambda0 > 0.0) || !(eps > 0.0) || !S || !A || !zkey)
        return VLA_ORACLE_EINVAL;
    if (T > 0 && (!q || !k || !v || !u || !o))
        return VLA_ORACLE_EINVAL;

    const size_t dd = (size_t)d * d;

    /* Initial state (section 3.2: A_0 = I / lambda0; S_0 = 0; empty key sum). */
    if (S0) memcpy(S, S0, dd * sizeof(double));
    else memset(S, 0, dd * sizeof(double));
    if (A0) {
        memcpy(A, A0, dd * sizeof(double));
    } else {
        memset(A, 0, dd * sizeof(double));
        for (int i = 0; i < d; ++i) A[(size_t)i * d + i] = 1.0 / lambda0;
    }
    if (zkey0) memcpy(zkey, zkey0, (size_t)d * sizeof(double));
    else memset(zkey, 0, (size_t)d * sizeof(double));

    double *work = (double *)malloc(8 * (size_t)d * sizeof(double));
    if (!work) return VLA_ORACLE_ENOMEM;
    double *kh = work, *uh = work + d, *z = work + 2 * d, *y = work + 3 * d;
    double *al = work + 4 * d, *e = work + 5 * d, *pq = work + 6 * d, *num = work + 7 * d;

    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * d, *kt = k + (size_t)t * d;
        const double *vt = v + (size_t)t * d, *ut = u + (size_t)t * d;

        normalise(kt, kh, d);
        normalise(ut, uh, d);

        /* Eq. (9): Sherman-Morrison rank-1 downdate of the inverse penalty. */
        matvec(A, uh, z, d);
        const double delta = 1.0 + dot(uh, z, d);
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j)
                A[(size_t)i * d + j] -= z[i] * z[j] / delta;

        /* Eq. (10): gate from the updated A_t, residual from S_{t-1}. */
        matvec(A, kh, y, d);
        normalise(y, al, d);
        matvec(S, kh, e, d);
        for (int i = 0; i < d; ++i) e[i] = vt[i] - e[i];
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j)
                S[(size_t)i * d + j] += e[i] * al[j];

        /* Eq. (11): inclusive key sum and normalised readout from S_t. */
        for (int i = 0; i < d; ++i) {
            pq[i] = phi(qt[i]);
            zkey[i] += phi(kt[i]);
        }
        double den = dot(pq, zkey, d);
        if (den < eps) den = eps;
        matvec(S, pq, num, d);
        for (int i = 0; i < d; ++i) o[(size_t)t * d + i] = num[i] / den;

        if (tr_delta) tr_delta[t] = delta;
        if (tr_den) tr_den[t] = den;
        if (tr_alpha) memcpy(tr_alpha + (size_t)t * d, al, (size_t)d * sizeof(double));
        if (tr_e) memcpy(tr_e + (size_t)t * d, e, (size_t)d * sizeof(double));
        if (tr_z) memcpy(tr_z + (size_t)t * d, z, (size_t)d * sizeof(double));
        if (tr_A) memcpy(tr_A + (size_t)t * dd, A, dd * sizeof(double));
        if (tr_S) memcpy(tr_S + (size_t)t * dd, S, dd * sizeof(double));
    }
    free(work);
    return VLA_ORACLE_OK;
}
