/*
 * path_oracle.c -- plain fp64 CPU oracle for PaTH attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP implementation.
 *
 * Citations name a page and a section of it:
 *   [Notes s2.x]  the reading-notes page "PaTH Attention:通过累积 Householder
 *                 变换编码位置" (cc.laoqi.cc, notes on arXiv 2505.16381v2),
 *                 section 2.x;
 *   [Explainer s3] the explainer page "PaTH Attention: Position Encoding via
 *                 Accumulating Householder Transformations" (gist.science),
 *                 section 3 ("Effizientes Training und Inferenz").
 *
 * What is computed is the plain definition, not a blockwise algorithm:
 *   logit(i, j) = scale * k_j^T H_{j+1} ... H_i q_i  +  sum_{s=j+1..i} log f_s
 * for j <= i, with H_t = I - beta_t w_t w_t^T            [Notes s2.1, s2.5]
 * followed by a causal softmax over j <= i and the value sum o_i.
 * The product is evaluated right to left as a walk: z starts at q_i, the
 * score of key j is read off as k_j . z, and then H_j is applied to z, so
 * that the next key (j-1) sees H_j ... H_i q_i.  This is only associativity
 * of the matrix product in the definition; no block structure is used.
 *
 * The attention scale is an explicit argument (the pages leave it out of
 * their notation [Notes s2.1]); the forget-gate bias is added after scaling
 * and is not scaled.  Positions are 0-based here; the pages count from 1.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* z <- (I - beta w w^T) z.  One Householder-like transition [Notes s2.1, s2.2]. */
static void apply_transition(int d, const double *w, double beta, double *z)
{
    double wz = 0.0;
    for (int e = 0; e < d; ++e) wz += w[e] * z[e];
    for (int e = 0; e < d; ++e) z[e] -= beta * wz * w[e];
}

static double dot(int d, const double *a, const double *b)
{
    double s = 0.0;
    for (int e = 0; e < d; ++e) s += a[e] * b[e];
    return s;
}

/*
 * One query row i of one (batch, head) slice.
 *   q, k, w : [L, d]   v : [L, dv]   beta, logf : [L]  (logf may be NULL: PaTH)
 *   o_row : [dv]   lse : natural-log log-sum-exp of the final logits of row i.
 *   scores : caller scratch of length >= i+1.
 * Definition: [Notes s2.1] (logit, softmax, value sum), [Notes s2.5] (bias).
 */
static void walk_row(int L, int d, int dv, const double *q, const double *k,
                     const double *v, const double *w, const double *beta,
                     const double *logf, double scale, int i, double *z,
                     double *scores, double *o_row, double *lse)
{
    (void)L;
    memcpy(z, q + (size_t)i * d, sizeof(double) * d);
    double bias = 0.0;                 /* sum_{s=j+1..i} log f_s */
    for (int j = i; j >= 0; --j) {
        scores[j] = scale * dot(d, k + (size_t)j * d, z) + bias;
        apply_transition(d, w + (size_t)j * d, beta[j], z);   /* z <- H_j z */
        if (logf) bias += logf[j];
    }
    double m = -INFINITY;
    for (int j = 0; j <= i; ++j) if (scores[j] > m) m = scores[j];
    double l = 0.0;
    for (int e = 0; e < dv; ++e) o_row[e] = 0.0;
    for (int j = 0; j <= i; ++j) {
        double p = exp(scores[j] - m);
        l += p;
        const double *vj = v + (size_t)j * dv;
        for (int e = 0; e < dv; ++e) o_row[e] += p * vj[e];
    }
    for (int e = 0; e < dv; ++e) o_row[e] /= l;
    *lse = m + log(l);
}

/*
 * Forward pass for selected rows of S independent slices.
 *   q, k, w : [S, L, d]   v : [S, L, dv]   beta, logf : [S, L]
 *   rows : [S, nrows] 0-based query positions (each in [0, L))
 *   o : [S, nrows, dv]   lse : [S, nrows]
 * Rows are independent; they are spread over OpenMP threads.
 * Returns 0, or -1 if a row index is out of range (nothing is written then).
 */
int oracle_fwd_rows(int S, int L, int d, int dv,
                    const double *q, const double *k, const double *v,
                    const double *w, const double *beta, const double *logf,
                    double scale, int nrows, const int *rows,
                    double *o, double *lse)
{
    for (long t = 0; t < (long)S * nrows; ++t)
        if (rows[t] < 0 || rows[t] >= L) return -1;
    #pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)d);
        double *scores = (double *)malloc(sizeof(double) * (size_t)L);
        #pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < (long)S * nrows; ++t) {
            long s = t / nrows;
            const size_t off = (size_t)s * L;
            walk_row(L, d, dv, q + off * d, k + off * d, v + off * dv,
                     w + off * d, beta + off, logf ? logf + off : NULL, scale,
                     rows[t], z, scores, o + (size_t)t * dv, lse + t);
        }
        free(z);
        free(scores);
    }
    return 0;
}

/*
 * Keys as a decoding cache holds them after position t has been processed:
 *   out_j = H_t ... H_{j+1} k_j   for j in [0, t]   (out_t = k_t)
 * i.e. every transition after position j is applied to key j, earliest first.
 * This is the cache rewrite of [Notes s2.8] (eq. (1) of the paper) carried
 * out step by step, and equally the prompt-end alignment described there.
 *   k, w : [S, L, d]  beta : [S, L]  out : [S, t+1, d]
 * Returns 0, or -1 if t is out of range.
 */
int oracle_transported_keys(int S, int L, int d, const double *k,
                            const double *w, const double *beta, int t,
                            double *out)
{
    if (t < 0 || t >= L) return -1;
    #pragma omp parallel for schedule(static)
    for (long sj = 0; sj < (long)S * (t + 1); ++sj) {
        long s = sj / (t + 1);
        int j = (int)(sj % (t + 1));
        const size_t off = (size_t)s * L;
        double *z = out + (size_t)sj * d;
        memcpy(z, k + (off + j) * d, sizeof(double) * d);
        for (int u = j + 1; u <= t; ++u)
            apply_transition(d, w + (off + u) * d, beta[off + u], z);
    }
    return 0;
}

/*
 * Gradients of a scalar loss through the forward pass above, given dL/do_i
 * for every row (the loss does not read lse).  The pages give no backward
 * formulas; this is reverse-mode differentiation of the definition as the
 * walk evaluates it, row by row, and its results are checked against finite
 * differences of oracle_fwd_rows.  For one row i:
 *   softmax:  D = do_i . o_i;  ds_j = p_j (do_i . v_j - D);  dv_j += p_j do_i.
 *   walk:     z_j = H_{j+1} ... H_i q_i is the vector key j was scored with
 *             (z_i = q_i, z_{j-1} = H_j z_j).  Going back up from j = 0, with
 *             g the gradient reaching z_{j-1} from the keys below j (zero at
 *             j = 0: z_{-1} is never used):
 *               dk_j    += scale ds_j z_j
 *               dbeta_j += -(w_j . z_j)(w_j . g)
 *               dw_j    += -beta_j ((w_j . g) z_j + (w_j . z_j) g)
 *               g       <- scale ds_j k_j + H_j g      (H_j is symmetric)
 *             and dq_i += g after the last key (j = i).
 *   bias:     the logit of key j carries sum_{s=j+1..i} log f_s, so
 *             dlogf_s += sum_{j<s} ds_j  for 1 <= s <= i.
 * Consequences the tests pin: w_0, beta_0 and log f_0 get no gradient.
 *   q, k, w : [S, L, d]   v, dout : [S, L, dv]   beta, logf : [S, L] (logf may be NULL)
 *   outputs dq, dk, dw : [S, L, d]   dvv : [S, L, dv]   dbeta, dlogf : [S, L]
 *   (dlogf is not written when logf is NULL).  Slices run in parallel.
 */
int oracle_bwd(int S, int L, int d, int dv, const double *q, const double *k,
               const double *v, const double *w, const double *beta,
               const double *logf, double scale, const double *dout,
               double *dq, double *dk, double *dvv, double *dw, double *dbeta,
               double *dlogf)
{
    memset(dq, 0, sizeof(double) * (size_t)S * L * d);
    memset(dk, 0, sizeof(double) * (size_t)S * L * d);
    memset(dw, 0, sizeof(double) * (size_t)S * L * d);
    memset(dvv, 0, sizeof(double) * (size_t)S * L * dv);
    memset(dbeta, 0, sizeof(double) * (size_t)S * L);
    if (logf) memset(dlogf, 0, sizeof(double) * (size_t)S * L);
    #pragma omp parallel
    {
        double *Z = (double *)malloc(sizeof(double) * (size_t)L * d);
        double *sc = (double *)malloc(sizeof(double) * (size_t)L);
        double *ds = (double *)malloc(sizeof(double) * (size_t)L);
        double *o = (double *)malloc(sizeof(double) * (size_t)dv);
        double *g = (double *)malloc(sizeof(double) * (size_t)d);
        double *gn = (double *)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 1)
        for (int s = 0; s < S; ++s) {
            const size_t off = (size_t)s * L;
            const double *qs = q + off * d, *ks = k + off * d, *ws = w + off * d;
            const double *vs = v + off * dv, *bs = beta + off, *fs = logf ? logf + off : NULL;
            double *dqs = dq + off * d, *dks = dk + off * d, *dws = dw + off * d;
            double *dvs = dvv + off * dv, *dbs = dbeta + off, *dfs = logf ? dlogf + off : NULL;
            for (int i = 0; i < L; ++i) {
                const double *doi = dout + (off + i) * dv;
                /* forward walk, keeping the vector each key is scored with */
                memcpy(Z + (size_t)i * d, qs + (size_t)i * d, sizeof(double) * d);
                double bias = 0.0;
                for (int j = i; j >= 0; --j) {
                    double *zj = Z + (size_t)j * d;
                    sc[j] = scale * dot(d, ks + (size_t)j * d, zj) + bias;
                    if (j > 0) {
                        memcpy(zj - d, zj, sizeof(double) * d);
                        apply_transition(d, ws + (size_t)j * d, bs[j], zj - d);
                    }
                    if (fs) bias += fs[j];
                }
                double m = -INFINITY, l = 0.0;
                for (int j = 0; j <= i; ++j) if (sc[j] > m) m = sc[j];
                for (int e = 0; e < dv; ++e) o[e] = 0.0;
                for (int j = 0; j <= i; ++j) {
                    sc[j] = exp(sc[j] - m);      /* unnormalised p_j */
                    l += sc[j];
                    for (int e = 0; e < dv; ++e) o[e] += sc[j] * vs[(size_t)j * dv + e];
                }
                for (int e = 0; e < dv; ++e) o[e] /= l;
                /* softmax backward */
                const double D = dot(dv, doi, o);
                for (int j = 0; j <= i; ++j) {
                    const double p = sc[j] / l;
                    const double *vj = vs + (size_t)j * dv;
                    ds[j] = p * (dot(dv, doi, vj) - D);
                    for (int e = 0; e < dv; ++e) dvs[(size_t)j * dv + e] += p * doi[e];
                }
                /* walk backward, from the farthest key up to the query */
                for (int e = 0; e < d; ++e) g[e] = 0.0;
                for (int j = 0; j <= i; ++j) {
                    const double *zj = Z + (size_t)j * d, *kj = ks + (size_t)j * d;
                    const double *wj = ws + (size_t)j * d;
                    for (int e = 0; e < d; ++e) dks[(size_t)j * d + e] += scale * ds[j] * zj[e];
                    const double a = dot(d, wj, zj), b = dot(d, wj, g);
                    dbs[j] += -a * b;
                    for (int e = 0; e < d; ++e)
                        dws[(size_t)j * d + e] += -bs[j] * (b * zj[e] + a * g[e]);
                    for (int e = 0; e < d; ++e) gn[e] = scale * ds[j] * kj[e] + g[e] - bs[j] * b * wj[e];
                    memcpy(g, gn, sizeof(double) * d);
                }
                for (int e = 0; e < d; ++e) dqs[(size_t)i * d + e] += g[e];
                if (dfs) {
                    double cum = 0.0;
                    for (int j = 0; j < i; ++j) {
                        cum += ds[j];
                        dfs[j + 1] += cum;
                    }
                }
            }
        }
        free(Z); free(sc); free(ds); free(o); free(g); free(gn);
    }
    return 0;
}

/* Threads the parallel regions of this library use from now on (n >= 1). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/*
 * Parameter front-end: the per-token branch that turns a layer input x_t
 * into the transition parameters w_t, beta_t and the forget gate log f_t.
 *   - w_t: a low-rank linear layer, then a causal short convolution of
 *     width 3, then L2 normalisation per head        [Notes s2.1]
 *   - beta_t = 2 sigma(u^T x_t + b), in (0, 2)        [Notes s2.1]
 *   - f_t = sigma(u_f^T x_t + b_f), enters as log f_t [Notes s2.5]
 * The pages fix neither the rank nor the convolution's form; the reading
 * taken here (plainest one consistent with them):
 *   p_t = Wd x_t                 (R outputs)
 *   r_t = Wu p_t                 (H*d channels)
 *   c_t = kc[:,0] r_t + kc[:,1] r_{t-1} + kc[:,2] r_{t-2}
 *         (depthwise, causal, r_s = 0 for s < 0; no activation)
 *   w_t^h = c_t^h / |c_t^h| over the d channels of head h (0 if c_t^h = 0)
 *   beta_t^h = 2 / (1 + exp(-(ub_h . x_t + bb_h)))
 *   logf_t^h = log sigma(uf_h . x_t + bf_h)
 * Weights use the out-by-in layout of a linear layer: Wd [R, Dm],
 * Wu [H*d, R], ub and uf [H, Dm]; kc [H*d, 3]; bb, bf [H].
 * x is [N, L, Dm]; w is written [N, H, L, d], beta and logf [N, H, L].
 * uf, bf and logf may all be NULL (no forget gate).
 */
static double log_sigmoid(double z)
{
    /* log(1 / (1 + e^-z)) without overflow for either sign of z */
    return z >= 0.0 ? -log1p(exp(-z)) : z - log1p(exp(z));
}

int oracle_frontend(int N, int L, int Dm, int R, int H, int d,
                    const double *x, const double *Wd, const double *Wu,
                    const double *kc, const double *ub, const double *bb,
                    const double *uf, const double *bf,
                    double *w, double *beta, double *logf)
{
    if (N < 1 || L < 1 || Dm < 1 || R < 1 || H < 1 || d < 1) return 1;
    const int C = H * d;
    int fail = 0;
    #pragma omp parallel for schedule(static) reduction(|:fail)
    for (int n = 0; n < N; ++n) {
        double *p = malloc(sizeof(double) * (size_t)L * R);
        double *r = malloc(sizeof(double) * (size_t)L * C);
        if (!p || !r) { free(p); free(r); fail = 1; continue; }
        const double *xn = x + (size_t)n * L * Dm;
        for (int t = 0; t < L; ++t) {
            for (int j = 0; j < R; ++j)
                p[(size_t)t * R + j] = dot(Dm, Wd + (size_t)j * Dm, xn + (size_t)t * Dm);
            for (int ch = 0; ch < C; ++ch)
                r[(size_t)t * C + ch] = dot(R, Wu + (size_t)ch * R, p + (size_t)t * R);
        }
        for (int t = 0; t < L; ++t) {
            const double *xt = xn + (size_t)t * Dm;
            for (int h = 0; h < H; ++h) {
                double c[d > 0 ? d : 1];
                double nrm2 = 0.0;
                for (int e = 0; e < d; ++e) {
                    const int ch = h * d + e;
                    double s = 0.0;
                    for (int tau = 0; tau < 3; ++tau)
                        if (t - tau >= 0) s += kc[(size_t)ch * 3 + tau] * r[(size_t)(t - tau) * C + ch];
                    c[e] = s;
                    nrm2 += s * s;
                }
                const double inv = nrm2 > 0.0 ? 1.0 / sqrt(nrm2) : 0.0;
                double *wo = w + (((size_t)n * H + h) * L + t) * d;
                for (int e = 0; e < d; ++e) wo[e] = c[e] * inv;
                const size_t o = ((size_t)n * H + h) * L + t;
                const double zb = dot(Dm, ub + (size_t)h * Dm, xt) + bb[h];
                beta[o] = 2.0 / (1.0 + exp(-zb));
                if (uf && logf) logf[o] = log_sigmoid(dot(Dm, uf + (size_t)h * Dm, xt) + bf[h]);
            }
        }
        free(p);
        free(r);
    }
    return fail;
}
