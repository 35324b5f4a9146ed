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
 * Readings where the pages leave a detail open:
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

/* phi'(x): 1 for x > 0, exp(x) otherwise (phi is continuous with slope 1 at 0). */
static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

/*
 * Reverse mode of the recurrence above, one head, fp64: the gradients of a
 * scalar loss L with respect to the inputs and the initial state, given the
 * adjoints of the outputs.  (The pages state the forward only; the chain rule
 * through Eqs. (9)-(11) is written out here step by step, each forward step
 * undone in the opposite order.)
 *
 * dO      : [T][d] dL/do_t.
 * dS_T, dA_T : [d][d] dL/dS_T, dL/dA_T (entrywise), or NULL for 0.
 * dzk_T   : [d] dL/dzkey_T, or NULL for 0.
 * dq, dk, dv, du : [T][d] outputs (required when T > 0).
 * dS0     : [d][d] dL/dS_0, or NULL to skip.
 * dA0     : [d][d] gradient with respect to A_0 as a symmetric matrix,
 *           (G + G')/2 of the entrywise gradient G, or NULL to skip.
 * dzk0    : [d] dL/dzkey_0, or NULL to skip.
 *
 * The forward runs first (vla_oracle_forward with its per-token traces), so
 * every A_t and S_t is at hand.  Then, for t = T..1, with gS = dL/dS_t,
 * gA = dL/dA_t (entrywise, not symmetrised) and gz = dL/dzkey_t:
 *   Eq. (11)  o = S_t phi(q) / den,  den = max(phi(q)'zkey_t, eps):
 *             gS += g phi(q)' / den;  gphi(q) = S_t' g / den, and where
 *             phi(q)'zkey_t >= eps also gden = -(g'S_t phi(q)) / den^2,
 *             gphi(q) += gden zkey_t, gz += gden phi(q);  the key sum passes
 *             gz to phi(k_t) and on to zkey_{t-1} unchanged.
 *   Eq. (10)  ge = gS alpha^;  galpha^ = gS' e;  gv = ge;
 *             gk^ = -S_{t-1}' ge;  gS <- gS - ge k^'  (= dL/dS_{t-1} so far);
 *             alpha^ = y/|y|:  gy = (galpha^ - alpha^ (alpha^'galpha^)) / |y|;
 *             y = A_t k^:  gA += gy k^';  gk^ += A_t' gy.
 *   Eq. (9)   A_t = A_{t-1} - z z'/delta:  gz_ = -(gA + gA') z / delta,
 *             gdelta = z'gA z / delta^2;  delta = 1 + u^'z:  gz_ += gdelta u^,
 *             gu^ = gdelta z;  z = A_{t-1} u^:  gA += gz_ u^' (now
 *             dL/dA_{t-1}), gu^ += A_{t-1}' gz_.
 *   normalisation x^ = x/|x|:  gx = (gx^ - x^ (x^'gx^)) / |x|; for k also
 *             gphi(k) phi'(k).
 * Conventions where no derivative exists: a zero vector's normalisation passes
 * no gradient (its x^ is 0 whatever the direction), and the denominator floor
 * passes gradient to phi(q)'zkey_t only where that is >= eps (the forward's
 * own branch).
 *
 * Memory: the traces hold 2 T d^2 doubles.  Returns 0, or nonzero on bad
 * arguments / allocation failure.
 */
int vla_oracle_backward(int T, int d, double lambda0, double eps,
                        const double *q, const double *k, const double *v, const double *u,
                        const double *S0, const double *A0, const double *zkey0,
                        const double *dO, const double *dS_T, const double *dA_T,
                        const double *dzk_T,
                        double *dq, double *dk, double *dv, double *du,
                        double *dS0, double *dA0, double *dzk0)
{
    if (T < 0 || d < 1 || !(lambda0 > 0.0) || !(eps > 0.0))
        return VLA_ORACLE_EINVAL;
    if (T > 0 && (!q || !k || !v || !u || !dO || !dq || !dk || !dv || !du))
        return VLA_ORACLE_EINVAL;

    const size_t dd = (size_t)d * d, Tn = T > 0 ? (size_t)T : 1;
    double *trA = (double *)malloc(Tn * dd * sizeof(double));
    double *trS = (double *)malloc(Tn * dd * sizeof(double));
    double *tz = (double *)malloc(Tn * d * sizeof(double));
    double *tal = (double *)malloc(Tn * d * sizeof(double));
    double *te = (double *)malloc(Tn * d * sizeof(double));
    double *tdel = (double *)malloc(Tn * sizeof(double));
    double *tden = (double *)malloc(Tn * sizeof(double));
    double *o = (double *)malloc(Tn * d * sizeof(double));
    double *tzk = (double *)malloc(Tn * d * sizeof(double));
    double *mats = (double *)malloc(5 * dd * sizeof(double));
    double *vec = (double *)malloc(16 * (size_t)d * sizeof(double));
    int rc = VLA_ORACLE_ENOMEM;
    if (!trA || !trS || !tz || !tal || !te || !tdel || !tden || !o || !tzk || !mats || !vec)
        goto out;
    {
        double *Sf = mats, *Af = mats + dd, *Ai = mats + 2 * dd, *Si = mats + 3 * dd;
        double *gA = mats + 4 * dd;
        double *zkf = vec, *kh = vec + d, *uh = vec + 2 * d, *pq = vec + 3 * d;
        double *zk = vec + 4 * d, *g = vec + 5 * d, *c1 = vec + 6 * d, *ge = vec + 7 * d;
        double *gal = vec + 8 * d, *gkh = vec + 9 * d, *y = vec + 10 * d, *gy = vec + 11 * d;
        double *gz = vec + 12 * d, *guh = vec + 13 * d, *gzk = vec + 14 * d;
        double *gS = dS0 ? dS0 : NULL;
        double *gSbuf = NULL;

        rc = vla_oracle_forward(T, d, lambda0, eps, q, k, v, u, S0, A0, zkey0, o, Sf, Af, zkf,
                                tdel, tal, te, tz, tden, trA, trS);
        if (rc != VLA_ORACLE_OK) goto out;

        /* the state before token 1 */
        if (S0) memcpy(Si, S0, dd * sizeof(double));
        else memset(Si, 0, dd * sizeof(double));
        if (A0) {
            memcpy(Ai, A0, dd * sizeof(double));
        } else {
            memset(Ai, 0, dd * sizeof(double));
            for (int i = 0; i < d; ++i) Ai[(size_t)i * d + i] = 1.0 / lambda0;
        }

        if (!gS) {
            gSbuf = (double *)malloc(dd * sizeof(double));
            if (!gSbuf) { rc = VLA_ORACLE_ENOMEM; goto out; }
            gS = gSbuf;
        }
        if (dS_T) memcpy(gS, dS_T, dd * sizeof(double));
        else memset(gS, 0, dd * sizeof(double));
        if (dA_T) memcpy(gA, dA_T, dd * sizeof(double));
        else memset(gA, 0, dd * sizeof(double));
        if (dzk_T) memcpy(gzk, dzk_T, (size_t)d * sizeof(double));
        else memset(gzk, 0, (size_t)d * sizeof(double));
        /* zkey_t = zkey_0 + sum_{s<=t} phi(k_s), for every t */
        for (int i = 0; i < d; ++i) zk[i] = zkey0 ? zkey0[i] : 0.0;
        for (int t = 0; t < T; ++t)
            for (int i = 0; i < d; ++i) {
                zk[i] += phi(k[(size_t)t * d + i]);
                tzk[(size_t)t * d + i] = zk[i];
            }
        (void)zkf;

        for (int t = T - 1; t >= 0; --t) {
            const double *qt = q + (size_t)t * d, *kt = k + (size_t)t * d;
            const double *ut = u + (size_t)t * d;
            const double *At = trA + (size_t)t * dd, *St = trS + (size_t)t * dd;
            const double *Ap = t > 0 ? trA + (size_t)(t - 1) * dd : Ai;
            const double *Sp = t > 0 ? trS + (size_t)(t - 1) * dd : Si;
            const double *z = tz + (size_t)t * d, *al = tal + (size_t)t * d;
            const double *e = te + (size_t)t * d;
            const double delta = tdel[t];
            double nk2 = 0.0, nu2 = 0.0;
            for (int i = 0; i < d; ++i) {
                nk2 += kt[i] * kt[i];
                nu2 += ut[i] * ut[i];
            }
            normalise(kt, kh, d);
            normalise(ut, uh, d);
            for (int i = 0; i < d; ++i) {
                pq[i] = phi(qt[i]);
                g[i] = dO[(size_t)t * d + i];
            }
            memcpy(zk, tzk + (size_t)t * d, (size_t)d * sizeof(double));   /* zkey_t */
            const double dn = dot(pq, zk, d);
            const double den = dn < eps ? eps : dn;

            /* Eq. (11) */
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) gS[(size_t)i * d + j] += g[i] * pq[j] / den;
            for (int j = 0; j < d; ++j) {
                double s = 0.0;
                for (int i = 0; i < d; ++i) s += St[(size_t)i * d + j] * g[i];
                c1[j] = s;
            }
            double gden = 0.0;
            if (dn >= eps) gden = -dot(c1, pq, d) / (den * den);
            for (int j = 0; j < d; ++j) {
                const double gpq = c1[j] / den + gden * zk[j];
                dq[(size_t)t * d + j] = gpq * dphi(qt[j]);
            }
            for (int j = 0; j < d; ++j) gzk[j] += gden * pq[j];

            /* Eq. (10) */
            matvec(gS, al, ge, d);
            for (int j = 0; j < d; ++j) {
                double s = 0.0, r = 0.0;
                for (int i = 0; i < d; ++i) {
                    s += gS[(size_t)i * d + j] * e[i];
                    r += Sp[(size_t)i * d + j] * ge[i];
                }
                gal[j] = s;
                gkh[j] = -r;
            }
            for (int i = 0; i < d; ++i) {
                dv[(size_t)t * d + i] = ge[i];
                for (int j = 0; j < d; ++j) gS[(size_t)i * d + j] -= ge[i] * kh[j];
            }
            matvec(At, kh, y, d);
            const double ny = sqrt(dot(y, y, d));
            if (ny > 0.0) {
                const double aa = dot(al, gal, d);
                for (int i = 0; i < d; ++i) gy[i] = (gal[i] - al[i] * aa) / ny;
            } else {
                memset(gy, 0, (size_t)d * sizeof(double));
            }
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) gA[(size_t)i * d + j] += gy[i] * kh[j];
            for (int j = 0; j < d; ++j) {
                double s = 0.0;
                for (int i = 0; i < d; ++i) s += At[(size_t)i * d + j] * gy[i];
                gkh[j] += s;
            }

            /* Eq. (9) */
            double gdelta = 0.0;
            for (int i = 0; i < d; ++i) {
                double s = 0.0;
                for (int j = 0; j < d; ++j)
                    s += (gA[(size_t)i * d + j] + gA[(size_t)j * d + i]) * z[j];
                gz[i] = -s / delta;
                for (int j = 0; j < d; ++j) gdelta += z[i] * gA[(size_t)i * d + j] * z[j];
            }
            gdelta /= delta * delta;
            for (int i = 0; i < d; ++i) {
                gz[i] += gdelta * uh[i];
                guh[i] = gdelta * z[i];
            }
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) gA[(size_t)i * d + j] += gz[i] * uh[j];
            for (int j = 0; j < d; ++j) {
                double s = 0.0;
                for (int i = 0; i < d; ++i) s += Ap[(size_t)i * d + j] * gz[i];
                guh[j] += s;
            }

            /* normalisation of k and u; phi(k_t) in the key sum */
            const double kk = dot(kh, gkh, d), uu = dot(uh, guh, d);
            const double nk = sqrt(nk2), nu = sqrt(nu2);
            for (int i = 0; i < d; ++i) {
                const double gkn = nk2 > 0.0 ? (gkh[i] - kh[i] * kk) / nk : 0.0;
                dk[(size_t)t * d + i] = gkn + gzk[i] * dphi(kt[i]);
                du[(size_t)t * d + i] = nu2 > 0.0 ? (guh[i] - uh[i] * uu) / nu : 0.0;
            }
        }
        if (dA0)
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j)
                    dA0[(size_t)i * d + j] = 0.5 * (gA[(size_t)i * d + j] + gA[(size_t)j * d + i]);
        if (dzk0) memcpy(dzk0, gzk, (size_t)d * sizeof(double));
        free(gSbuf);
        rc = VLA_ORACLE_OK;
    }
out:
    free(trA); free(trS); free(tz); free(tal); free(te); free(tdel); free(tden);
    free(o); free(tzk); free(mats); free(vec);
    return rc;
}

/*
 * Baselines on the same inputs (test infrastructure, like everything above).
 *
 * Cumulative-sum linear attention, from the "Linear Attention" wiki article,
 * "recurrent form" section: the state gains phi(k_t) v_t' each token, the key
 * sum gains phi(k_t), and the output is phi(q_t)'S_t / phi(q_t)'z_t.  Here S is
 * stored value-major like the VLA state (S[i][j], i value, j key), so
 *     S_t = S_{t-1} + v_t phi(k_t)',   zkey_t = zkey_{t-1} + phi(k_t),
 *     o_t = S_t phi(q_t) / (phi(q_t)' zkey_t).
 * phi = ELU + 1 as in the article's "feature maps" section.  The article's
 * readout has no floor; phi > 0 keeps the denominator positive.
 *
 * q, k, v : [T][d];  S0 [d][d] and zkey0 [d] or NULL (zero);  o [T][d];
 * S [d][d], zkey [d] out;  tr_scale [T] or NULL: per token
 * |S_t|_F |phi(q_t)| / den_t, the size o_t has when nothing cancels.
 * Returns 0 or nonzero on bad arguments.
 */
int vla_oracle_linear_attention(int T, int d, const double *q, const double *k, const double *v,
                                const double *S0, const double *zkey0,
                                double *o, double *S, double *zkey, double *tr_scale)
{
    if (T < 0 || d < 1 || !S || !zkey) return VLA_ORACLE_EINVAL;
    if (T > 0 && (!q || !k || !v || !o)) return VLA_ORACLE_EINVAL;
    const size_t dd = (size_t)d * d;
    if (S0) memcpy(S, S0, dd * sizeof(double));
    else memset(S, 0, dd * sizeof(double));
    if (zkey0) memcpy(zkey, zkey0, (size_t)d * sizeof(double));
    else memset(zkey, 0, (size_t)d * sizeof(double));
    double *work = (double *)malloc(3 * (size_t)d * sizeof(double));
    if (!work) return VLA_ORACLE_ENOMEM;
    double *pk = work, *pq = work + d, *num = work + 2 * d;
    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * d, *kt = k + (size_t)t * d, *vt = v + (size_t)t * d;
        for (int j = 0; j < d; ++j) {
            pk[j] = phi(kt[j]);
            pq[j] = phi(qt[j]);
            zkey[j] += pk[j];
        }
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += vt[i] * pk[j];
        matvec(S, pq, num, d);
        const double den = dot(pq, zkey, d);
        for (int i = 0; i < d; ++i) o[(size_t)t * d + i] = num[i] / den;
        if (tr_scale) tr_scale[t] = sqrt(dot(S, S, d * d) * dot(pq, pq, d)) / den;
    }
    free(work);
    return VLA_ORACLE_OK;
}

/*
 * DeltaNet as the pages' special case of the VLA layer: section 3.5 of
 * "Variational Linear Attention" obtains DeltaNet by replacing alpha^_t with a
 * scalar gate and dropping A_t.  With the gate beta on the unit key, the write
 * of Eq. (10) becomes the delta rule of the kexue.fm article's "linear version"
 * (W_t = W_{t-1} - eta (W_{t-1} k - v) k', eta = beta, k = k^):
 *     e_t = v_t - S_{t-1} k^_t,   S_t = S_{t-1} + beta e_t k^_t',
 * and the readout is Eq. (11) unchanged (raw-key phi sum, max(., eps) floor).
 *
 * q, k, v : [T][d];  S0 [d][d], zkey0 [d] or NULL (zero);  o [T][d];
 * S [d][d], zkey [d] out;  tr_scale [T] or NULL: per token
 * |S_t|_F |phi(q_t)| / den_t.  Returns 0 or nonzero on bad arguments.
 */
int vla_oracle_deltanet(int T, int d, double beta, double eps, const double *q, const double *k,
                        const double *v, const double *S0, const double *zkey0,
                        double *o, double *S, double *zkey, double *tr_scale)
{
    if (T < 0 || d < 1 || !(eps > 0.0) || !S || !zkey) return VLA_ORACLE_EINVAL;
    if (T > 0 && (!q || !k || !v || !o)) return VLA_ORACLE_EINVAL;
    const size_t dd = (size_t)d * d;
    if (S0) memcpy(S, S0, dd * sizeof(double));
    else memset(S, 0, dd * sizeof(double));
    if (zkey0) memcpy(zkey, zkey0, (size_t)d * sizeof(double));
    else memset(zkey, 0, (size_t)d * sizeof(double));
    double *work = (double *)malloc(4 * (size_t)d * sizeof(double));
    if (!work) return VLA_ORACLE_ENOMEM;
    double *kh = work, *e = work + d, *pq = work + 2 * d, *num = work + 3 * d;
    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * d, *kt = k + (size_t)t * d, *vt = v + (size_t)t * d;
        normalise(kt, kh, d);
        matvec(S, kh, e, d);
        for (int i = 0; i < d; ++i) e[i] = vt[i] - e[i];
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += beta * e[i] * kh[j];
        for (int i = 0; i < d; ++i) {
            pq[i] = phi(qt[i]);
            zkey[i] += phi(kt[i]);
        }
        double den = dot(pq, zkey, d);
        if (den < eps) den = eps;
        matvec(S, pq, num, d);
        for (int i = 0; i < d; ++i) o[(size_t)t * d + i] = num[i] / den;
        if (tr_scale) tr_scale[t] = sqrt(dot(S, S, d * d) * dot(pq, pq, d)) / den;
    }
    free(work);
    return VLA_ORACLE_OK;
}
