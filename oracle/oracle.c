/*
 * oracle.c -- plain, slow fp64 CPU oracle for causal linear self-attention.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load, call or run anything under oracle/.  The HIP
 * product path never links, imports or calls this file, and this file shares
 * no code, header, table or helper with it.
 *
 * Everything is computed in double precision, one attention head at a time
 * (the Python wrapper loops over batch and head).  Arrays are row-major:
 *   Q, K, V, dY, Y, dQ, dK, dV : [L][d]
 *   W                          : [M][d]    (FAVOR+ projection, one row per feature)
 *   R0, R, dR                  : [d][M]    (R = sum_i V_i g(K_i)^T)
 *   S0, S, dS                  : [M]       (S = sum_i g(K_i))
 *
 * Sources (page "Sub-Linear Memory: How to Make Performers SLiM"):
 *   - linear self-attention, eq. (2) of Subsection 2.1: the output at l is the
 *     g(Q_l)g(K_i)-weighted average of V_i over i <= l, with g positive;
 *   - prefix-sum form, eq. (3)-(4) of Subsection 2.1: R = PS(V_i g(K_i)^T),
 *     S = PS(g(K_i)), Y_l = R_l g(Q_l) / (S_l . g(Q_l));
 *   - iterative evaluation (the Katharopoulos et al. scheme described in
 *     Subsection 2.1): walk l = 1..L keeping only the current R_l, S_l;
 *   - the gradient of a prefix sum is a prefix sum taken backwards
 *     (Subsection 3.3, the remark after update (20)).
 * The feature maps g are the two the page names in Subsection 2.1: an
 * elementwise map with M = d (here elu(x)+1) and the randomized FAVOR+ map of
 * Choromanski et al., g(x)_m = exp(w_m.x - |x|^2/2)/sqrt(M).
 * Exponential (softmax) attention, eq. (1) of Subsection 2.1, is included only
 * so that tests can check that FAVOR+ approximates it.
 *
 * The loss used for every backward function is <dY, Y> + <dRout, Rout> +
 * <dSout, Sout>, i.e. dY, dRout and dSout are the incoming gradients.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define FEAT_FAVOR 0
#define FEAT_ELU1 1

/* ---------------------------------------------------------------- g(x) --- */

/* One row of the feature map.  FAVOR+: g_m(x) = exp(w_m.x - |x|^2/2)/sqrt(M).
 * elu+1 (M == d): g_j(x) = x_j + 1 for x_j > 0, exp(x_j) otherwise. */
static void feat_row(int kind, int d, int M, const double *x, const double *W, double *phi)
{
    if (kind == FEAT_FAVOR) {
        double xx = 0.0;
        for (int e = 0; e < d; ++e) xx += x[e] * x[e];
        for (int m = 0; m < M; ++m) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += W[(size_t)m * d + e] * x[e];
            phi[m] = exp(s - 0.5 * xx) / sqrt((double)M);
        }
    } else {
        for (int j = 0; j < d; ++j) phi[j] = x[j] > 0.0 ? x[j] + 1.0 : exp(x[j]);
    }
}

/* Vector-Jacobian product of one feature row: dx = (d g/d x)^T dphi.
 * FAVOR+: d g_m/d x = g_m (w_m - x), so dx = sum_m dphi_m g_m (w_m - x).
 * elu+1 : d g_j/d x_j = 1 for x_j > 0, exp(x_j) otherwise. */
static void feat_vjp_row(int kind, int d, int M, const double *x, const double *W,
                         const double *phi, const double *dphi, double *dx)
{
    if (kind == FEAT_FAVOR) {
        for (int e = 0; e < d; ++e) dx[e] = 0.0;
        for (int m = 0; m < M; ++m) {
            double c = dphi[m] * phi[m];
            for (int e = 0; e < d; ++e) dx[e] += c * (W[(size_t)m * d + e] - x[e]);
        }
    } else {
        for (int j = 0; j < d; ++j) dx[j] = dphi[j] * (x[j] > 0.0 ? 1.0 : exp(x[j]));
    }
}

/* Gradient of one FAVOR+ feature row with respect to the projection W,
 * accumulated: g_m(x) depends on W only through w_m, with d g_m/d w_m = g_m x,
 * so dW[m] += dphi_m g_m x.  (elu+1 has no parameters.) */
static void feat_wgrad_row(int d, int M, const double *x, const double *phi, const double *dphi, double *dW)
{
    for (int m = 0; m < M; ++m) {
        const double gm = dphi[m] * phi[m];
        for (int e = 0; e < d; ++e) dW[(size_t)m * d + e] += gm * x[e];
    }
}

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int k = 0; k < n; ++k) s += a[k] * b[k];
    return s;
}

/* Feature map of `rows` rows: Phi[r] = g(X[r]). */
void oracle_featmap(int kind, long rows, int d, int M, const double *X, const double *W, double *Phi)
{
    for (long r = 0; r < rows; ++r) feat_row(kind, d, M, X + (size_t)r * d, W, Phi + (size_t)r * M);
}

/* Feature-map VJP of `rows` rows: dX[r] = J_g(X[r])^T dPhi[r]. */
void oracle_featmap_vjp(int kind, long rows, int d, int M, const double *X, const double *W,
                        const double *dPhi, double *dX)
{
    double *phi = (double *)malloc(sizeof(double) * M);
    for (long r = 0; r < rows; ++r) {
        feat_row(kind, d, M, X + (size_t)r * d, W, phi);
        feat_vjp_row(kind, d, M, X + (size_t)r * d, W, phi, dPhi + (size_t)r * M, dX + (size_t)r * d);
    }
    free(phi);
}

/* W-gradient of `rows` FAVOR+ rows, accumulated into dW [M][d]:
 * dW += sum_r J_W(g(X[r]))^T dPhi[r]. */
void oracle_featmap_wgrad(long rows, int d, int M, const double *X, const double *W, const double *dPhi,
                          double *dW)
{
    double *phi = (double *)malloc(sizeof(double) * M);
    for (long r = 0; r < rows; ++r) {
        feat_row(FEAT_FAVOR, d, M, X + (size_t)r * d, W, phi);
        feat_wgrad_row(d, M, X + (size_t)r * d, phi, dPhi + (size_t)r * M, dW);
    }
    free(phi);
}

static double *feats(int kind, long L, int d, int M, const double *X, const double *W)
{
    double *Phi = (double *)malloc(sizeof(double) * (size_t)L * M);
    oracle_featmap(kind, L, d, M, X, W, Phi);
    return Phi;
}

/* ------------------------------------------- quadratic (masked) form --- */

/* Linear attention by its definition (eq. (2)), one head, O(L^2):
 *   a_{l,i} = g(Q_l).g(K_i) for i <= l (the mask includes the diagonal),
 *   num_l   = R0 g(Q_l) + sum_{i<=l} a_{l,i} V_i,
 *   den_l   = S0.g(Q_l) + sum_{i<=l} a_{l,i},
 *   Y_l     = num_l / den_l.
 * R0, S0 (may be NULL = zero) stand for keys that precede the sequence.
 * Rout = R0 + sum_i V_i g(K_i)^T and Sout = S0 + sum_i g(K_i) (may be NULL).
 * den (may be NULL) receives den_l. */
void oracle_fwd_quadratic(int kind, long L, int d, int M, const double *Q, const double *K,
                          const double *V, const double *W, const double *R0, const double *S0,
                          double *Y, double *den, double *Rout, double *Sout)
{
    double *Fq = feats(kind, L, d, M, Q, W);
    double *Fk = feats(kind, L, d, M, K, W);
    double *num = (double *)malloc(sizeof(double) * d);
    for (long l = 0; l < L; ++l) {
        const double *fq = Fq + (size_t)l * M;
        double dn = 0.0;
        for (int e = 0; e < d; ++e) num[e] = 0.0;
        if (R0)
            for (int e = 0; e < d; ++e) num[e] += dot(R0 + (size_t)e * M, fq, M);
        if (S0) dn += dot(S0, fq, M);
        for (long i = 0; i <= l; ++i) {
            double a = dot(fq, Fk + (size_t)i * M, M);
            dn += a;
            for (int e = 0; e < d; ++e) num[e] += a * V[(size_t)i * d + e];
        }
        for (int e = 0; e < d; ++e) Y[(size_t)l * d + e] = num[e] / dn;
        if (den) den[l] = dn;
    }
    if (Rout) {
        for (int e = 0; e < d; ++e)
            for (int m = 0; m < M; ++m) Rout[(size_t)e * M + m] = R0 ? R0[(size_t)e * M + m] : 0.0;
        for (long i = 0; i < L; ++i)
            for (int e = 0; e < d; ++e)
                for (int m = 0; m < M; ++m)
                    Rout[(size_t)e * M + m] += V[(size_t)i * d + e] * Fk[(size_t)i * M + m];
    }
    if (Sout) {
        for (int m = 0; m < M; ++m) Sout[m] = S0 ? S0[m] : 0.0;
        for (long i = 0; i < L; ++i)
            for (int m = 0; m < M; ++m) Sout[m] += Fk[(size_t)i * M + m];
    }
    free(num);
    free(Fq);
    free(Fk);
}

/* Gradient of the quadratic form for the loss <dY,Y> + <dRout,Rout> + <dSout,Sout>
 * (chain rule through the definition above; dRout, dSout may be NULL = zero):
 *   G_l = dY_l / den_l,   E_l = -(dY_l . Y_l) / den_l,
 *   c_{l,i} = dL/da_{l,i} = G_l . V_i + E_l                      (i <= l)
 *   dg(Q_l) = sum_{i<=l} c_{l,i} g(K_i) + R0^T G_l + E_l S0
 *   dg(K_i) = sum_{l>=i} c_{l,i} g(Q_l) + dRout^T V_i + dSout
 *   dV_i    = sum_{l>=i} a_{l,i} G_l + dRout g(K_i)
 *   dR0     = sum_l G_l g(Q_l)^T + dRout,   dS0 = sum_l E_l g(Q_l) + dSout
 * then dQ, dK through the feature-map VJP, and (FAVOR+, dW not NULL) the
 * gradient of the projection, dW = sum over the Q and K rows of J_W^T dg.
 * dR0, dS0, dW may be NULL. */
void oracle_bwd_quadratic(int kind, long L, int d, int M, const double *Q, const double *K,
                          const double *V, const double *W, const double *R0, const double *S0,
                          const double *dY, const double *dRout, const double *dSout,
                          double *dQ, double *dK, double *dV, double *dR0, double *dS0, double *dW)
{
    double *Fq = feats(kind, L, d, M, Q, W);
    double *Fk = feats(kind, L, d, M, K, W);
    double *Y = (double *)malloc(sizeof(double) * (size_t)L * d);
    double *den = (double *)malloc(sizeof(double) * L);
    double *G = (double *)malloc(sizeof(double) * (size_t)L * d);
    double *E = (double *)malloc(sizeof(double) * L);
    double *dFq = (double *)calloc((size_t)L * M, sizeof(double));
    double *dFk = (double *)calloc((size_t)L * M, sizeof(double));

    oracle_fwd_quadratic(kind, L, d, M, Q, K, V, W, R0, S0, Y, den, NULL, NULL);
    for (long l = 0; l < L; ++l) {
        E[l] = -dot(dY + (size_t)l * d, Y + (size_t)l * d, d) / den[l];
        for (int e = 0; e < d; ++e) G[(size_t)l * d + e] = dY[(size_t)l * d + e] / den[l];
    }
    for (long i = 0; i < L; ++i)
        for (int e = 0; e < d; ++e) dV[(size_t)i * d + e] = 0.0;

    for (long l = 0; l < L; ++l) {
        const double *g = G + (size_t)l * d;
        double *dfq = dFq + (size_t)l * M;
        for (long i = 0; i <= l; ++i) {
            double a = dot(Fq + (size_t)l * M, Fk + (size_t)i * M, M);
            double c = dot(g, V + (size_t)i * d, d) + E[l];
            for (int m = 0; m < M; ++m) {
                dfq[m] += c * Fk[(size_t)i * M + m];
                dFk[(size_t)i * M + m] += c * Fq[(size_t)l * M + m];
            }
            for (int e = 0; e < d; ++e) dV[(size_t)i * d + e] += a * g[e];
        }
        if (R0)
            for (int m = 0; m < M; ++m)
                for (int e = 0; e < d; ++e) dfq[m] += R0[(size_t)e * M + m] * g[e];
        if (S0)
            for (int m = 0; m < M; ++m) dfq[m] += E[l] * S0[m];
    }
    for (long i = 0; i < L; ++i) {
        for (int m = 0; m < M; ++m) {
            double s = dSout ? dSout[m] : 0.0;
            if (dRout)
                for (int e = 0; e < d; ++e) s += dRout[(size_t)e * M + m] * V[(size_t)i * d + e];
            dFk[(size_t)i * M + m] += s;
        }
        if (dRout)
            for (int e = 0; e < d; ++e)
                dV[(size_t)i * d + e] += dot(dRout + (size_t)e * M, Fk + (size_t)i * M, M);
    }
    if (dR0)
        for (int e = 0; e < d; ++e)
            for (int m = 0; m < M; ++m) {
                double s = dRout ? dRout[(size_t)e * M + m] : 0.0;
                for (long l = 0; l < L; ++l) s += G[(size_t)l * d + e] * Fq[(size_t)l * M + m];
                dR0[(size_t)e * M + m] = s;
            }
    if (dS0)
        for (int m = 0; m < M; ++m) {
            double s = dSout ? dSout[m] : 0.0;
            for (long l = 0; l < L; ++l) s += E[l] * Fq[(size_t)l * M + m];
            dS0[m] = s;
        }
    oracle_featmap_vjp(kind, L, d, M, Q, W, dFq, dQ);
    oracle_featmap_vjp(kind, L, d, M, K, W, dFk, dK);
    if (dW && kind == FEAT_FAVOR) {
        memset(dW, 0, sizeof(double) * (size_t)M * d);
        oracle_featmap_wgrad(L, d, M, Q, W, dFq, dW);
        oracle_featmap_wgrad(L, d, M, K, W, dFk, dW);
    }

    free(Fq); free(Fk); free(Y); free(den); free(G); free(E); free(dFq); free(dFk);
}

/* ------------------------------------------------ prefix-sum (linear) --- */

/* Iterative prefix-sum evaluation (eq. (3)-(4), the Katharopoulos et al. scheme
 * of Subsection 2.1): for l = 1..L, R_l = R_{l-1} + V_l g(K_l)^T,
 * S_l = S_{l-1} + g(K_l), Y_l = R_l g(Q_l) / (S_l . g(Q_l)); R_0 = R0, S_0 = S0.
 * Only the current R_l, S_l are kept.  den (may be NULL) receives S_l.g(Q_l). */
void oracle_fwd_prefix(int kind, long L, int d, int M, const double *Q, const double *K,
                       const double *V, const double *W, const double *R0, const double *S0,
                       double *Y, double *den, double *Rout, double *Sout)
{
    double *R = (double *)malloc(sizeof(double) * (size_t)d * M);
    double *S = (double *)malloc(sizeof(double) * M);
    double *fq = (double *)malloc(sizeof(double) * M);
    double *fk = (double *)malloc(sizeof(double) * M);
    for (size_t t = 0; t < (size_t)d * M; ++t) R[t] = R0 ? R0[t] : 0.0;
    for (int m = 0; m < M; ++m) S[m] = S0 ? S0[m] : 0.0;
    for (long l = 0; l < L; ++l) {
        feat_row(kind, d, M, Q + (size_t)l * d, W, fq);
        feat_row(kind, d, M, K + (size_t)l * d, W, fk);
        for (int e = 0; e < d; ++e) {
            double v = V[(size_t)l * d + e];
            for (int m = 0; m < M; ++m) R[(size_t)e * M + m] += v * fk[m];
        }
        for (int m = 0; m < M; ++m) S[m] += fk[m];
        double dn = dot(S, fq, M);
        for (int e = 0; e < d; ++e) Y[(size_t)l * d + e] = dot(R + (size_t)e * M, fq, M) / dn;
        if (den) den[l] = dn;
    }
    if (Rout) memcpy(Rout, R, sizeof(double) * (size_t)d * M);
    if (Sout) memcpy(Sout, S, sizeof(double) * M);
    free(R); free(S); free(fq); free(fk);
}

/* Backward of the iterative form: walk l = L..1 keeping the running gradient
 * GR_l = dL/dR_l (total), which is a prefix sum taken backwards:
 *   GR_l = dRout + sum_{l'>=l} G_{l'} g(Q_{l'})^T   (likewise GS_l with E_{l'}),
 * with G_l = dY_l/den_l, E_l = -(dY_l.Y_l)/den_l.  Per row:
 *   dg(Q_l) = R_l^T G_l + E_l S_l,  dg(K_l) = GR_l^T V_l + GS_l,  dV_l = GR_l g(K_l),
 * and R_{l-1} = R_l - V_l g(K_l)^T is recovered by subtraction from the final
 * state (the reversal the page uses for its slice states).  dR0 = GR_1, dS0 = GS_1.
 * dW (FAVOR+, may be NULL) accumulates the projection gradient of every row's
 * two feature vectors as the walk passes them. */
void oracle_bwd_prefix(int kind, long L, int d, int M, const double *Q, const double *K,
                       const double *V, const double *W, const double *R0, const double *S0,
                       const double *dY, const double *dRout, const double *dSout,
                       double *dQ, double *dK, double *dV, double *dR0, double *dS0, double *dW)
{
    size_t DM = (size_t)d * M;
    double *Y = (double *)malloc(sizeof(double) * (size_t)L * d);
    double *den = (double *)malloc(sizeof(double) * L);
    double *R = (double *)malloc(sizeof(double) * DM);
    double *S = (double *)malloc(sizeof(double) * M);
    double *GR = (double *)malloc(sizeof(double) * DM);
    double *GS = (double *)malloc(sizeof(double) * M);
    double *fq = (double *)malloc(sizeof(double) * M);
    double *fk = (double *)malloc(sizeof(double) * M);
    double *dfq = (double *)malloc(sizeof(double) * M);
    double *dfk = (double *)malloc(sizeof(double) * M);
    double *g = (double *)malloc(sizeof(double) * d);

    oracle_fwd_prefix(kind, L, d, M, Q, K, V, W, R0, S0, Y, den, R, S);
    for (size_t t = 0; t < DM; ++t) GR[t] = dRout ? dRout[t] : 0.0;
    for (int m = 0; m < M; ++m) GS[m] = dSout ? dSout[m] : 0.0;
    if (dW && kind == FEAT_FAVOR) memset(dW, 0, sizeof(double) * (size_t)M * d);

    for (long l = L - 1; l >= 0; --l) {
        const double *x = Q + (size_t)l * d, *k = K + (size_t)l * d, *v = V + (size_t)l * d;
        feat_row(kind, d, M, x, W, fq);
        feat_row(kind, d, M, k, W, fk);
        double El = -dot(dY + (size_t)l * d, Y + (size_t)l * d, d) / den[l];
        for (int e = 0; e < d; ++e) g[e] = dY[(size_t)l * d + e] / den[l];
        /* R, S hold R_l, S_l here */
        for (int m = 0; m < M; ++m) {
            double s = El * S[m];
            for (int e = 0; e < d; ++e) s += R[(size_t)e * M + m] * g[e];
            dfq[m] = s;
        }
        for (int e = 0; e < d; ++e)
            for (int m = 0; m < M; ++m) GR[(size_t)e * M + m] += g[e] * fq[m];
        for (int m = 0; m < M; ++m) GS[m] += El * fq[m];
        for (int m = 0; m < M; ++m) {
            double s = GS[m];
            for (int e = 0; e < d; ++e) s += GR[(size_t)e * M + m] * v[e];
            dfk[m] = s;
        }
        for (int e = 0; e < d; ++e) dV[(size_t)l * d + e] = dot(GR + (size_t)e * M, fk, M);
        feat_vjp_row(kind, d, M, x, W, fq, dfq, dQ + (size_t)l * d);
        feat_vjp_row(kind, d, M, k, W, fk, dfk, dK + (size_t)l * d);
        if (dW && kind == FEAT_FAVOR) {
            feat_wgrad_row(d, M, x, fq, dfq, dW);
            feat_wgrad_row(d, M, k, fk, dfk, dW);
        }
        for (int e = 0; e < d; ++e)
            for (int m = 0; m < M; ++m) R[(size_t)e * M + m] -= v[e] * fk[m];
        for (int m = 0; m < M; ++m) S[m] -= fk[m];
    }
    if (dR0) memcpy(dR0, GR, sizeof(double) * DM);
    if (dS0) memcpy(dS0, GS, sizeof(double) * M);
    free(Y); free(den); free(R); free(S); free(GR); free(GS);
    free(fq); free(fk); free(dfq); free(dfk); free(g);
}

/* --------------------------------------------- sampled rows (big runs) --- */

/* Y_l and den_l by the definition (eq. (2)) for the listed rows only; each row
 * costs O(l (d + M) + d M).  Used where L is too long for the full O(L^2) form. */
void oracle_fwd_rows(int kind, long L, int d, int M, const double *Q, const double *K,
                     const double *V, const double *W, const double *R0, const double *S0,
                     long nrows, const long *rows, double *Yrows, double *denrows)
{
    double *fq = (double *)malloc(sizeof(double) * M);
    double *fk = (double *)malloc(sizeof(double) * M);
    double *num = (double *)malloc(sizeof(double) * d);
    for (long r = 0; r < nrows; ++r) {
        long l = rows[r];
        if (l < 0 || l >= L) continue;
        feat_row(kind, d, M, Q + (size_t)l * d, W, fq);
        double dn = S0 ? dot(S0, fq, M) : 0.0;
        for (int e = 0; e < d; ++e) num[e] = R0 ? dot(R0 + (size_t)e * M, fq, M) : 0.0;
        for (long i = 0; i <= l; ++i) {
            feat_row(kind, d, M, K + (size_t)i * d, W, fk);
            double a = dot(fq, fk, M);
            dn += a;
            for (int e = 0; e < d; ++e) num[e] += a * V[(size_t)i * d + e];
        }
        for (int e = 0; e < d; ++e) Yrows[(size_t)r * d + e] = num[e] / dn;
        if (denrows) denrows[r] = dn;
    }
    free(fq); free(fk); free(num);
}

/* ------------------------------------------- exponential attention --- */

/* Causal exponential self-attention (eq. (1)), no temperature:
 * Y_l = sum_{i<=l} exp(Q_l.K_i) V_i / sum_{i<=l} exp(Q_l.K_i).  The row maximum
 * of Q_l.K_i is subtracted before exp (it cancels in the ratio). */
void oracle_softmax_fwd(long L, int d, const double *Q, const double *K, const double *V, double *Y)
{
    double *s = (double *)malloc(sizeof(double) * L);
    for (long l = 0; l < L; ++l) {
        double mx = -INFINITY, z = 0.0;
        for (long i = 0; i <= l; ++i) {
            s[i] = dot(Q + (size_t)l * d, K + (size_t)i * d, d);
            if (s[i] > mx) mx = s[i];
        }
        for (int e = 0; e < d; ++e) Y[(size_t)l * d + e] = 0.0;
        for (long i = 0; i <= l; ++i) {
            double p = exp(s[i] - mx);
            z += p;
            for (int e = 0; e < d; ++e) Y[(size_t)l * d + e] += p * V[(size_t)i * d + e];
        }
        for (int e = 0; e < d; ++e) Y[(size_t)l * d + e] /= z;
    }
    free(s);
}
