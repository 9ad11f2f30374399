/*
 * Plain fp64 CPU oracle for the Parallax attention forward (prefill rows and
 * decode rows) and for the prefill backward; at the end of the file, the
 * exact Local Linear Attention solve, the fused input projections, the
 * Walsh-Hadamard output projection and Based linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU kernels are compared against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or helper with the HIP library, and it must never be used as a fallback for
 * the GPU path.
 *
 * What it computes (method: "Parallax: Parameterized Local Linear Attention
 * for Language Modeling", review page, sec. 1 "Key Terms & Definitions" and
 * sec. 3 "Method & Key Results"; tilnote note on Parallax, section on the
 * starting point, Local Linear Attention):
 *
 *   Softmax attention reads the values as a locally constant estimate; Local
 *   Linear Attention (LLA) fits a local linear estimate and needs a per-token
 *   linear solve.  Parallax drops the solve and lets a learned projection
 *   give the probe rho_i = x_i W_R, which reads the key/value covariance as a
 *   correction on top of softmax attention.  Written out, with p_ij the
 *   softmax weights over the visible keys of query i:
 *
 *     kbar_i = sum_j p_ij k_j
 *     c_ij   = rho_i . (k_j - kbar_i)          (no 1/sqrt(d) on this term)
 *     o_i    = sum_j p_ij (1 + c_ij) v_j
 *     lse_i  = log sum_j exp(scale * q_i . k_j)
 *
 *   The rho = (Sigma_kk)^-1 (q - kbar) choice of the probe turns o_i into the
 *   intercept of the p-weighted least-squares fit v ~ a + B (k - q), i.e. the
 *   LLA estimate; Parallax keeps this form with a learned rho.
 *
 * Visible set of query position i (causal; optional sliding window and
 * attention sinks, per the "Sliding-window beats linear attention" review,
 * sec. 1, on windows over preceding tokens and on sink tokens):
 *
 *     j in V(i)  iff  0 <= j <= i  and  (window <= 0 or i - j < window
 *                                         or j < n_sink)
 *
 * Readings taken where the pages are silent: the window counts the query's
 * own key (a window of W keys is i-W < j <= i); sinks stay causal; an empty
 * visible set (only possible for a decode row of length 0, position -1)
 * gives o = 0 and lse = -inf.
 *
 * Algorithm, per row, in the order of the definition: (1) scores and their
 * max, (2) exponentials, their sum and the weights, (3) the weighted key
 * mean, (4) the correction coefficient for each key, (5) the weighted sum of
 * values.  Two plain passes over the visible keys; no tiling, no online
 * rescaling.
 *
 * The CPU tests plant deliberate mistakes in patched copies of this file
 * (tests/oracle_mutants.py) to show that the pins catch each of them; this
 * file itself contains none.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Is key j visible from query position i? */
static int visible(long i, long j, long window, long n_sink)
{
    if (j < 0 || j > i)
        return 0;
    if (window <= 0 || i - j < window || j < n_sink)
        return 1;
    return 0;
}

static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t)
        s += a[t] * b[t];
    return s;
}

/* One output row.  k, v: [n_ctx][d]; q_i, r_i: [d]; work: scratch [2*n_ctx + d]. */
static void one_row(const double *q_i, const double *r_i, long i,
                    const double *k, const double *v, long n_ctx, int d,
                    double scale, long window, long n_sink,
                    double *o_i, double *lse_i, double *work)
{
    double *z = work;            /* scores, then weights p_j       */
    double *c = work + n_ctx;    /* correction coefficients c_j    */
    double *kbar = work + 2 * n_ctx;
    long last = n_ctx - 1;      /* visible() alone decides which keys count */

    /* (1) scores over the visible set and their maximum */
    double m = -INFINITY;
    long n_vis = 0;
    for (long j = 0; j <= last; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        z[j] = scale * dot(q_i, k + j * (long)d, d);
        if (z[j] > m)
            m = z[j];
        ++n_vis;
    }
    for (int t = 0; t < d; ++t)
        o_i[t] = 0.0;
    if (n_vis == 0) {
        *lse_i = -INFINITY;
        return;
    }

    /* (2) exponentials, their sum, normalised weights */
    double ell = 0.0;
    for (long j = 0; j <= last; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        z[j] = exp(z[j] - m);
        ell += z[j];
    }
    *lse_i = m + log(ell);
    for (long j = 0; j <= last; ++j)
        if (visible(i, j, window, n_sink))
            z[j] /= ell;

    /* (3) weighted key mean kbar = sum_j p_j k_j */
    for (int t = 0; t < d; ++t)
        kbar[t] = 0.0;
    for (long j = 0; j <= last; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        double w = z[j];
        for (int t = 0; t < d; ++t)
            kbar[t] += w * k[j * (long)d + t];
    }

    /* (4) correction coefficient c_j = rho . (k_j - kbar) */
    for (long j = 0; j <= last; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        const double *kj = k + j * (long)d;
        double s = 0.0;
        for (int t = 0; t < d; ++t) {
            s += r_i[t] * (kj[t] - kbar[t]);
        }
        c[j] = s;
    }

    /* (5) o = sum_j p_j (1 + c_j) v_j */
    for (long j = 0; j <= last; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        double w = z[j] * (1.0 + c[j]);
        const double *vj = v + j * (long)d;
        for (int t = 0; t < d; ++t)
            o_i[t] += w * vj[t];
    }
}

/*
 * Rows of one (batch, head) slice.
 *   q_rows, r_rows : [n_rows][d]  query and probe of each requested row
 *   pos            : [n_rows]     position i of each row, -1 <= i < n_ctx
 *                                 (-1 = empty visible set, a length-0 decode)
 *   k, v           : [n_ctx][d]   keys and values of the slice
 *   o_rows         : [n_rows][d]  output;  lse_rows: [n_rows]
 * Returns 0, or -1 on an invalid argument (nothing written then).
 */
int parallax_oracle_rows(const double *q_rows, const double *r_rows,
                         const long *pos, long n_rows,
                         const double *k, const double *v, long n_ctx, int d,
                         double scale, long window, long n_sink,
                         double *o_rows, double *lse_rows, int nthreads)
{
    if (n_rows < 0 || n_ctx < 0 || d <= 0 || n_sink < 0)
        return -1;
    for (long n = 0; n < n_rows; ++n)
        if (pos[n] < -1 || pos[n] >= n_ctx)
            return -1;
    if (nthreads < 1)
        nthreads = 1;
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * n_ctx + d + 1));
        if (!work) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long n = 0; n < n_rows; ++n)
                one_row(q_rows + n * (long)d, r_rows + n * (long)d, pos[n],
                        k, v, n_ctx, d, scale, window, n_sink,
                        o_rows + n * (long)d, lse_rows + n, work);
            free(work);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Whole prefill forward over contiguous [B][H][L][d] tensors:
 * o [B][H][L][d], lse [B][H][L].  Returns 0 or -1.
 */
int parallax_oracle_fwd(const double *q, const double *k, const double *v,
                        const double *r, double *o, double *lse,
                        long B, long H, long L, int d,
                        double scale, long window, long n_sink, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0 || n_sink < 0)
        return -1;
    long *pos = (long *)malloc(sizeof(long) * (size_t)(L > 0 ? L : 1));
    if (!pos)
        return -2;
    for (long i = 0; i < L; ++i)
        pos[i] = i;
    int rc = 0;
    for (long bh = 0; bh < B * H && rc == 0; ++bh) {
        long off = bh * L * (long)d;
        rc = parallax_oracle_rows(q + off, r + off, pos, L, k + off, v + off, L, d,
                                  scale, window, n_sink, o + off, lse + bh * L, nthreads);
    }
    free(pos);
    return rc;
}

/*
 * Decode, general form: one query per (sequence, query head) against a
 * contiguous cache of Hkv key/value heads.  Query head h reads kv head
 * h / (Hq / Hkv) (grouped-query attention; Hkv = Hq is the plain case,
 * Hkv = 1 multi-query).  The query sits at position seqlen-1 and sees the
 * keys visible() allows there (causal, optional window and sinks).
 *   q, r   : [B][Hq][d];  k_cache, v_cache: [B][Hkv][Lmax][d]
 *   seqlens: [B] host array or NULL (all Lmax); each clamped to [0, Lmax].
 * o: [B][Hq][d], lse: [B][Hq].  Returns 0 or -1.
 */
int parallax_oracle_decode_ext(const double *q, const double *r,
                               const double *k_cache, const double *v_cache,
                               const int *seqlens, double *o, double *lse,
                               long B, long Hq, long Hkv, long Lmax, int d, double scale,
                               long window, long n_sink, int nthreads)
{
    if (B < 0 || Hq < 0 || Hkv <= 0 || Lmax < 0 || d <= 0 || window < 0 || n_sink < 0 ||
        Hq % Hkv != 0)
        return -1;
    const long g = Hq / Hkv;
    int rc = 0;
    for (long b = 0; b < B && rc == 0; ++b) {
        long n = seqlens ? seqlens[b] : Lmax;
        if (n < 0)
            n = 0;
        if (n > Lmax)
            n = Lmax;
        for (long h = 0; h < Hq && rc == 0; ++h) {
            long hk = h / g;
            long bh = b * Hq + h;
            long p = n - 1;
            const double *kc = k_cache + (b * Hkv + hk) * Lmax * d;
            const double *vc = v_cache + (b * Hkv + hk) * Lmax * d;
            rc = parallax_oracle_rows(q + bh * d, r + bh * d, &p, 1, kc, vc, Lmax, d, scale,
                                      window, n_sink, o + bh * d, lse + bh, nthreads);
        }
    }
    return rc;
}

/* Decode against a contiguous cache with one kv head per query head and
 * no window: the general form with Hkv = H. */
int parallax_oracle_decode(const double *q, const double *r,
                           const double *k_cache, const double *v_cache,
                           const int *seqlens, double *o, double *lse,
                           long B, long H, long Lmax, int d, double scale, int nthreads)
{
    if (H <= 0)
        return (B < 0 || H < 0 || Lmax < 0 || d <= 0) ? -1 : 0;
    return parallax_oracle_decode_ext(q, r, k_cache, v_cache, seqlens, o, lse, B, H, H, Lmax,
                                      d, scale, 0, 0, nthreads);
}

/*
 * Backward of the prefill forward.
 *
 * Gradients of a scalar loss that depends on the outputs through o alone
 * (the log-sum-exp output carries no gradient: dlse = 0), with respect to
 * q, k, v and the probe rho.  This is reverse-mode differentiation of the
 * five forward steps of one_row(), taken in reverse order for each query
 * row i; step (n') is the adjoint of step (n):
 *
 *   (5')  u_j = p_j (1 + c_j),  o = sum_j u_j v_j:
 *           dv_j += u_j dO;          du_j = dO . v_j;
 *           dp_j  = du_j (1 + c_j);  dc_j = du_j p_j
 *   (4')  c_j = rho . (k_j - kbar):
 *           drho += sum_j dc_j (k_j - kbar);  dk_j += dc_j rho;
 *           dkbar = -(sum_j dc_j) rho
 *   (3')  kbar = sum_j p_j k_j:
 *           dp_j += dkbar . k_j;     dk_j += p_j dkbar
 *   (2')  p = softmax(z) over the visible keys:
 *           dz_j = p_j (dp_j - sum_l p_l dp_l)
 *   (1')  z_j = scale q . k_j:
 *           dq += scale sum_j dz_j k_j;  dk_j += scale dz_j q
 *
 * Rows are independent in the forward, so each row's adjoint adds into the
 * key and value gradients of the keys it sees.  Rows are dealt to the
 * threads round-robin; each thread keeps its own dk and dv sums, and these
 * are added in thread order at the end, so a fixed thread count gives a
 * fixed result.
 */

/* Adjoint of one row; adds into dk, dv ([n_ctx][d]) and writes dq_i, dr_i.
 * work: scratch of 4 * n_ctx + 2 * d doubles. */
static void one_row_bwd(const double *q_i, const double *r_i, const double *do_i, long i,
                        const double *k, const double *v, long n_ctx, int d,
                        double scale, long window, long n_sink,
                        double *dq_i, double *dr_i, double *dk, double *dv, double *work)
{
    double *p = work;                 /* softmax weights p_j            */
    double *c = work + n_ctx;         /* correction coefficients c_j    */
    double *dp = work + 2 * n_ctx;    /* adjoint of p_j                 */
    double *dc = work + 3 * n_ctx;    /* adjoint of c_j                 */
    double *kbar = work + 4 * n_ctx;
    double *dkbar = kbar + d;

    for (int t = 0; t < d; ++t)
        dq_i[t] = dr_i[t] = 0.0;

    /* forward steps (1)-(4) again: scores, weights, key mean, corrections */
    double m = -INFINITY;
    long n_vis = 0;
    for (long j = 0; j < n_ctx; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        p[j] = scale * dot(q_i, k + j * (long)d, d);
        if (p[j] > m)
            m = p[j];
        ++n_vis;
    }
    if (n_vis == 0)
        return;
    double ell = 0.0;
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink)) {
            p[j] = exp(p[j] - m);
            ell += p[j];
        }
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink))
            p[j] /= ell;
    for (int t = 0; t < d; ++t)
        kbar[t] = 0.0;
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink))
            for (int t = 0; t < d; ++t)
                kbar[t] += p[j] * k[j * (long)d + t];
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink)) {
            double s = 0.0;
            for (int t = 0; t < d; ++t)
                s += r_i[t] * (k[j * (long)d + t] - kbar[t]);
            c[j] = s;
        }

    /* (5') */
    for (long j = 0; j < n_ctx; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        double u = p[j] * (1.0 + c[j]);
        for (int t = 0; t < d; ++t)
            dv[j * (long)d + t] += u * do_i[t];
        double du = dot(do_i, v + j * (long)d, d);
        dp[j] = du * (1.0 + c[j]);
        dc[j] = du * p[j];
    }

    /* (4') */
    double sum_dc = 0.0;
    for (long j = 0; j < n_ctx; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        const double *kj = k + j * (long)d;
        for (int t = 0; t < d; ++t) {
            dr_i[t] += dc[j] * (kj[t] - kbar[t]);
            dk[j * (long)d + t] += dc[j] * r_i[t];
        }
        sum_dc += dc[j];
    }
    for (int t = 0; t < d; ++t)
        dkbar[t] = -sum_dc * r_i[t];

    /* (3') */
    for (long j = 0; j < n_ctx; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        dp[j] += dot(dkbar, k + j * (long)d, d);
        for (int t = 0; t < d; ++t)
            dk[j * (long)d + t] += p[j] * dkbar[t];
    }

    /* (2') */
    double mean_dp = 0.0;
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink))
            mean_dp += p[j] * dp[j];

    /* (1'), with dz_j formed on the fly */
    for (long j = 0; j < n_ctx; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        double dz = p[j] * (dp[j] - mean_dp);
        const double *kj = k + j * (long)d;
        for (int t = 0; t < d; ++t) {
            dq_i[t] += scale * dz * kj[t];
            dk[j * (long)d + t] += scale * dz * q_i[t];
        }
    }
}

/*
 * Whole prefill backward over contiguous [B][H][L][d] tensors.
 *   q, k, v, r : forward inputs;  dout: gradient of the loss w.r.t. o
 *   dq, dk, dv, dr: outputs, same shape.
 * Returns 0, -1 on an invalid argument, -2 when scratch memory is short.
 */
int parallax_oracle_bwd(const double *q, const double *k, const double *v,
                        const double *r, const double *dout,
                        double *dq, double *dk, double *dv, double *dr,
                        long B, long H, long L, int d,
                        double scale, long window, long n_sink, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0 || n_sink < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    const long sz = L * (long)d;
    double *acc = (double *)calloc((size_t)nthreads * (size_t)(2 * sz) + 1, sizeof(double));
    double *work = (double *)malloc(sizeof(double) * (size_t)nthreads * (size_t)(4 * L + 2 * d + 1));
    int failed = !acc || !work;
    for (long bh = 0; bh < B * H && !failed; ++bh) {
        const long off = bh * sz;
        memset(acc, 0, sizeof(double) * (size_t)nthreads * (size_t)(2 * sz));
#pragma omp parallel for num_threads(nthreads) schedule(static, 1)
        for (long i = 0; i < L; ++i) {
            int tid = 0;
#ifdef _OPENMP
            tid = omp_get_thread_num();
#endif
            double *a = acc + (size_t)tid * (size_t)(2 * sz);
            one_row_bwd(q + off + i * d, r + off + i * d, dout + off + i * d, i,
                        k + off, v + off, L, d, scale, window, n_sink,
                        dq + off + i * d, dr + off + i * d, a, a + sz,
                        work + (size_t)tid * (size_t)(4 * L + 2 * d + 1));
        }
        for (long e = 0; e < sz; ++e) {
            double sk = 0.0, sv = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                sk += acc[(size_t)t * (size_t)(2 * sz) + e];
                sv += acc[(size_t)t * (size_t)(2 * sz) + sz + e];
            }
            dk[off + e] = sk;
            dv[off + e] = sv;
        }
    }
    free(acc);
    free(work);
    return failed ? -2 : 0;
}

/*
 * Exact Local Linear Attention (LLA), the estimator Parallax parameterises
 * (review page "Parallax: Parameterized Local Linear Attention for Language
 * Modeling", sec. 1-2: LLA fits a local linear model around each query and
 * needs a per-token linear solve; tilnote note on Parallax, section on the
 * starting point).  For query i with softmax weights p_j over its visible
 * keys, the p-weighted least-squares fit v ~ a + B (k - q_i) has intercept
 *
 *     a_i = sum_j p_j (1 + rho_i . (k_j - kbar_i)) v_j,
 *     rho_i solving  (Sigma_i + ridge I) rho_i = q_i - kbar_i,
 *     Sigma_i = sum_j p_j (k_j - kbar_i)(k_j - kbar_i)^T,
 *
 * i.e. Parallax's form with the probe obtained by a solve instead of a
 * learned projection.  The solve is done the way a kernel would do it, by
 * conjugate gradients with matrix-free products
 *     Sigma x = sum_j p_j (k_j - kbar) ((k_j - kbar) . x),
 * each of which reads all visible keys again.  CG stops after max_iters
 * iterations or once the residual norm falls below tol times the norm of
 * q - kbar.  ridge >= 0 keeps the system definite for rows with fewer
 * visible keys than d + 1 (the plain solve is singular there).
 *
 *   q_rows: [n_rows][d]; pos: [n_rows]; k, v: [n_ctx][d]
 *   o_rows, rho_rows: [n_rows][d]; iters: [n_rows] CG iterations used
 * Returns 0, -1 on an invalid argument, -2 when scratch memory is short.
 */
static void lla_row(const double *q_i, long i, const double *k, const double *v, long n_ctx,
                    int d, double scale, long window, long n_sink, int max_iters, double tol,
                    double ridge, double *o_i, double *rho, int *iters, double *work)
{
    double *p = work;                /* weights            [n_ctx] */
    double *kbar = work + n_ctx;     /* [d] */
    double *res = kbar + d;          /* CG residual        [d] */
    double *dir = res + d;           /* CG direction       [d] */
    double *Ad = dir + d;            /* Sigma dir          [d] */
    double m = -INFINITY, ell = 0.0;
    for (int t = 0; t < d; ++t)
        o_i[t] = rho[t] = kbar[t] = 0.0;
    *iters = 0;
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink)) {
            p[j] = scale * dot(q_i, k + j * (long)d, d);
            if (p[j] > m)
                m = p[j];
        }
    if (m == -INFINITY)
        return;
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink)) {
            p[j] = exp(p[j] - m);
            ell += p[j];
        }
    for (long j = 0; j < n_ctx; ++j)
        if (visible(i, j, window, n_sink)) {
            p[j] /= ell;
            for (int t = 0; t < d; ++t)
                kbar[t] += p[j] * k[j * (long)d + t];
        }
    /* CG on (Sigma + ridge I) rho = q - kbar, starting from rho = 0 */
    double rr = 0.0;
    for (int t = 0; t < d; ++t) {
        res[t] = q_i[t] - kbar[t];
        dir[t] = res[t];
        rr += res[t] * res[t];
    }
    const double stop = tol * tol * rr;
    for (int it = 0; it < max_iters && rr > stop && rr > 0.0; ++it) {
        for (int t = 0; t < d; ++t)
            Ad[t] = ridge * dir[t];
        for (long j = 0; j < n_ctx; ++j) {
            if (!visible(i, j, window, n_sink))
                continue;
            const double *kj = k + j * (long)d;
            double c = 0.0;
            for (int t = 0; t < d; ++t)
                c += (kj[t] - kbar[t]) * dir[t];
            c *= p[j];
            for (int t = 0; t < d; ++t)
                Ad[t] += c * (kj[t] - kbar[t]);
        }
        const double dAd = dot(dir, Ad, d);
        if (!(dAd > 0.0))
            break;
        const double alpha = rr / dAd;
        double rr_new = 0.0;
        for (int t = 0; t < d; ++t) {
            rho[t] += alpha * dir[t];
            res[t] -= alpha * Ad[t];
            rr_new += res[t] * res[t];
        }
        for (int t = 0; t < d; ++t)
            dir[t] = res[t] + (rr_new / rr) * dir[t];
        rr = rr_new;
        *iters = it + 1;
    }
    /* intercept: sum_j p_j (1 + rho . (k_j - kbar)) v_j */
    for (long j = 0; j < n_ctx; ++j) {
        if (!visible(i, j, window, n_sink))
            continue;
        const double *kj = k + j * (long)d;
        double c = 0.0;
        for (int t = 0; t < d; ++t)
            c += rho[t] * (kj[t] - kbar[t]);
        const double w = p[j] * (1.0 + c);
        for (int t = 0; t < d; ++t)
            o_i[t] += w * v[j * (long)d + t];
    }
}

int parallax_oracle_lla_rows(const double *q_rows, const long *pos, long n_rows,
                             const double *k, const double *v, long n_ctx, int d,
                             double scale, long window, long n_sink, int max_iters, double tol,
                             double ridge, double *o_rows, double *rho_rows, int *iters,
                             int nthreads)
{
    if (n_rows < 0 || n_ctx < 0 || d <= 0 || n_sink < 0 || window < 0 || max_iters < 0 ||
        !(tol >= 0.0) || !(ridge >= 0.0))
        return -1;
    for (long r = 0; r < n_rows; ++r)
        if (pos[r] < -1 || pos[r] >= n_ctx)
            return -1;
    if (nthreads < 1)
        nthreads = 1;
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(n_ctx + 4 * d + 1));
        if (!work) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < n_rows; ++r)
                lla_row(q_rows + r * (long)d, pos[r], k, v, n_ctx, d, scale, window, n_sink,
                        max_iters, tol, ridge, o_rows + r * (long)d, rho_rows + r * (long)d,
                        iters + r, work);
            free(work);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Fused input projections: y = x w^T with w the row-wise stack of W_Q,
 * W_K, W_V and the probe projection W_R, so that row i of y is
 * [q_i | k_i | v_i | rho_i] (review page "Parallax: Parameterized Local
 * Linear Attention for Language Modeling", sec. 1 and sec. 3: the probe is
 * a learned projection of the layer input).  Plain triple loop.
 *   x: [M][K]; w: [N][K]; y: [M][N].  Returns 0 or -1.
 */
int parallax_oracle_project(const double *x, const double *w, double *y, long M, long N,
                            long K, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (long i = 0; i < M; ++i)
        for (long n = 0; n < N; ++n) {
            double s = 0.0;
            for (long t = 0; t < K; ++t)
                s += x[i * K + t] * w[n * K + t];
            y[i * N + n] = s;
        }
    return 0;
}

/*
 * Walsh-Hadamard output projection (review page "Rethinking Attention
 * Output Projection: Structured Hadamard Transforms for Efficient
 * Transformers", sec. 2 "Methodology"): the dense output projection of
 * multi-head attention is replaced by a fixed Walsh-Hadamard transform of
 * the concatenated head outputs followed by a learned per-feature affine
 * map,  out = alpha (.) (Y H) + beta.
 *
 * Readings: H is the Sylvester-ordered Hadamard matrix of order n (n a power
 * of two) scaled by 1/sqrt(n), so that it is orthogonal and preserves the
 * l2 norm of each row, as the page states; alpha and beta are length-n
 * vectors indexed by the output feature.  NULL alpha means all ones, NULL
 * beta all zeros.
 *
 * Steps: (1) build H_n by Sylvester's doubling, H_1 = [1],
 * H_2m = [[H_m, H_m], [H_m, -H_m]]; (2) the plain product Y H_n / sqrt(n);
 * (3) the affine map.
 *   y: [M][n]; out: [M][n].  Returns 0, or -1 for bad sizes.
 */
int parallax_oracle_hadamard(const double *y, const double *alpha, const double *beta,
                             double *out, long M, long n, int nthreads)
{
    if (M < 0 || n < 1 || (n & (n - 1)) != 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    double *h = malloc(sizeof(double) * (size_t)n * (size_t)n);
    if (!h)
        return -1;
    h[0] = 1.0;
    for (long m = 1; m < n; m *= 2)
        for (long i = 0; i < m; ++i)
            for (long j = 0; j < m; ++j) {
                const double e = h[i * n + j];
                h[i * n + j + m] = e;
                h[(i + m) * n + j] = e;
                h[(i + m) * n + j + m] = -e;
            }
    const double norm = 1.0 / sqrt((double)n);
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (long i = 0; i < M; ++i)
        for (long c = 0; c < n; ++c) {
            double s = 0.0;
            for (long t = 0; t < n; ++t)
                s += y[i * n + t] * h[t * n + c];
            s *= norm;
            if (alpha)
                s *= alpha[c];
            if (beta)
                s += beta[c];
            out[i * n + c] = s;
        }
    free(h);
    return 0;
}

/*
 * Based linear attention (review page "Simple linear attention language
 * models balance the recall-throughput tradeoff", "Proposed method"): the
 * linear-attention half of the Based hybrid, whose other half is softmax
 * attention over a small sliding window.  Linear attention replaces
 * exp(scale q.k) by a kernel phi(q).phi(k), so that the causal sum can be
 * carried as a fixed-size state; the feature dimension of phi sets the state
 * size.
 *
 * Reading (the page leaves phi open): phi is the feature map of the
 * second-order Taylor expansion of exp, so that with x = scale * q_i . k_j
 *
 *     w_ij = phi(q_i) . phi(k_j) = 1 + x + x^2 / 2        (> 0 for every x)
 *     o_i  = sum_{j <= i} w_ij v_j / sum_{j <= i} w_ij
 *
 * q and k have the feature dimension dk, v has dv; the sum is causal over
 * all earlier positions (no window).  Written out pairwise, as defined.
 *   q, k: [B][H][L][dk]; v, o: [B][H][L][dv].  Returns 0 or -1.
 */
int parallax_oracle_based(const double *q, const double *k, const double *v, double *o,
                          long B, long H, long L, long dk, long dv, double scale,
                          int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || dk < 1 || dv < 1)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    const long rows = B * H * L;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (long r = 0; r < rows; ++r) {
        const long bh = r / L, i = r % L;
        const double *qi = q + r * dk;
        const double *kb = k + bh * L * dk;
        const double *vb = v + bh * L * dv;
        double *oi = o + r * dv;
        for (long e = 0; e < dv; ++e)
            oi[e] = 0.0;
        double den = 0.0;
        for (long j = 0; j <= i; ++j) {
            double dot = 0.0;
            for (long t = 0; t < dk; ++t)
                dot += qi[t] * kb[j * dk + t];
            const double x = scale * dot;
            const double w = 1.0 + x + 0.5 * x * x;
            den += w;
            for (long e = 0; e < dv; ++e)
                oi[e] += w * vb[j * dv + e];
        }
        if (den > 0.0)
            for (long e = 0; e < dv; ++e)
                oi[e] /= den;
    }
    return 0;
}
