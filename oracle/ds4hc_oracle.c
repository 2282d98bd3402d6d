/*
 * ds4hc_oracle.c -- plain, slow, fp64 CPU oracle of the DeepSeek-V4
 * hyper-connection (HC) op.
 *
 * TEST INFRASTRUCTURE ONLY. It exists to check the HIP library against.
 * Only the test suite, the package's smoke check and the benchmark's CPU
 * baseline may load it. It shares no code, header, table or helper with
 * the HIP path, and the HIP path never calls it.
 *
 * What the op is, per the pages:
 *   - lucebox PR #496 "feat(ds4): add DSpark speculative runtime +
 *     optimizations", PR body: a fused DS4 hyper-connection op
 *     (GGML_OP_DS4_HC) together with a register-resident Sinkhorn kernel.
 *   - lucebox-hub PR #494 "fix(ds4): keep ROCmFPX generation byte-safe",
 *     commit notes: a CPU pool that runs the "HC fn matvecs and hc_post",
 *     and the GPU "HC pre-mix"; comment on the Sinkhorn kernel for
 *     NHC = 4 (n_hc = 4 streams); comment naming "HC-pre" as a cost centre.
 *   - lucebox PR #507 "correct layer-split HC handoff and per-device
 *     state", Implementation: the full HC state is what flows between
 *     layers.
 * The pages name these steps but print no formula. The formulas below
 * are the library's stated reading of them, one function per step:
 *
 *   state X[t] = n streams of d features, flattened index k = i*d + c,
 *   K = n*d, m = 2n + n*n fn outputs.
 *   1. r    = sqrt( (sum_k x_k^2) / K + eps )           (RMS over the
 *                                                        flattened state)
 *   2. xn_k = x_k / r
 *   3. z_j  = sum_k W[j][k] * xn_k + b_j,  j < m        (HC fn matvec)
 *   4. pre_i  = 1/(1+exp(-z_i)),  post_i = 1/(1+exp(-z_{n+i}))  (sigmoid)
 *   5. Z[i][j] = z_{2n + i*n + j};  M[i][j] = exp(Z[i][j] - max_j' Z[i][j'])
 *      then `iters` times: divide every row by its sum, then every
 *      column by its sum (Sinkhorn); H = M.
 *   6. layer_in[c] = sum_i pre_i * X[i][c]              (pre-mix)
 *   7. X'[i][c] = sum_j H[i][j] * X[j][c] + post_i * layer_out[c]  (hc_post)
 *
 * Split over d (lucebox PR #507, Implementation: the HC state crosses the
 * device boundary whole): r is one number per token, so
 * z_j = (sum_k W[j][k] x_k) / r + b_j, and steps 1 and 3 need only the
 * per-token sums S_j = sum_k W[j][k] x_k and Q = sum_k x_k^2, which add
 * over any partition of the columns. ds4hc_oracle_partials computes them
 * for one share of the columns.
 *
 * Readings where the pages are silent (stated constants of the library):
 * eps inside the square root and added to the mean over all K elements;
 * no learned gain; logits ordered pre | post | residual (row-major,
 * i = output stream); plain logistic gates; max subtraction per row
 * before exp; one Sinkhorn iteration = rows then columns; no epsilon in
 * the Sinkhorn divisions; pre-mix and post act on the raw (not normalised)
 * state. Non-finite inputs are not special-cased.
 *
 * All arithmetic is IEEE double, sums run in ascending index order. Inputs
 * arrive as double (every f32, bf16 and f16 value widens to double exactly).
 * Tokens are independent, so the token loop may run on several threads;
 * each token's arithmetic is sequential, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

static int n_logits(int n) { return 2 * n + n * n; }

/* Step 1: r = sqrt(mean of squares over the K flattened elements + eps). */
static double rms_of_state(const double *x, int64_t K, double eps)
{
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k)
        ss += x[k] * x[k];
    return sqrt(ss / (double)K + eps);
}

/* Steps 2-3: z_j = sum_k W[j][k] * (x_k / r) + b_j. W is [m][K] row-major. */
static void fn_matvec(const double *x, int64_t K, double r, const double *W,
                      const double *b, int m, double *z)
{
    for (int j = 0; j < m; ++j) {
        const double *wj = W + (size_t)j * (size_t)K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += wj[k] * (x[k] / r);
        z[j] = acc + b[j];
    }
}

static double logistic(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Step 5 on one n x n logit matrix Z (row-major) -> H (row-major). */
static void sinkhorn_one(int n, int iters, const double *Z, double *H)
{
    for (int i = 0; i < n; ++i) {
        double mx = Z[i * n];
        for (int j = 1; j < n; ++j)
            if (Z[i * n + j] > mx)
                mx = Z[i * n + j];
        for (int j = 0; j < n; ++j)
            H[i * n + j] = exp(Z[i * n + j] - mx);
    }
    for (int it = 0; it < iters; ++it) {
        for (int i = 0; i < n; ++i) {          /* rows */
            double s = 0.0;
            for (int j = 0; j < n; ++j)
                s += H[i * n + j];
            for (int j = 0; j < n; ++j)
                H[i * n + j] /= s;
        }
        for (int j = 0; j < n; ++j) {          /* columns */
            double s = 0.0;
            for (int i = 0; i < n; ++i)
                s += H[i * n + j];
            for (int i = 0; i < n; ++i)
                H[i * n + j] /= s;
        }
    }
}

/* Steps 1-5 for one token: logits z[m] and coefficients pre|post|H [m]. */
static void coefficients_one(int n, int d, const double *x, const double *W,
                             const double *b, double eps, int iters,
                             double *z, double *coeffs)
{
    const int64_t K = (int64_t)n * d;
    const int m = n_logits(n);
    const double r = rms_of_state(x, K, eps);
    fn_matvec(x, K, r, W, b, m, z);
    for (int i = 0; i < n; ++i) {
        coeffs[i] = logistic(z[i]);
        coeffs[n + i] = logistic(z[n + i]);
    }
    sinkhorn_one(n, iters, z + 2 * n, coeffs + 2 * n);
}

/* Step 6 for one token. */
static void premix_one(int n, int d, const double *x, const double *pre, double *layer_in)
{
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int i = 0; i < n; ++i)
            acc += pre[i] * x[(size_t)i * d + c];
        layer_in[c] = acc;
    }
}

/* Step 7 for one token. coeffs = pre|post|H. */
static void post_one(int n, int d, const double *x, const double *coeffs,
                     const double *layer_out, double *x_out)
{
    const double *post = coeffs + n;
    const double *H = coeffs + 2 * n;
    for (int i = 0; i < n; ++i) {
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < n; ++j)
                acc += H[i * n + j] * x[(size_t)j * d + c];
            x_out[(size_t)i * d + c] = acc + post[i] * layer_out[c];
        }
    }
}

static int bad_shape(int64_t T, int n, int d)
{
    return T < 0 || n < 1 || d < 1;
}

/* ---- exported C ABI (host pointers, all double) ---------------------- */

int ds4hc_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void ds4hc_oracle_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* HC-pre: steps 1-6. X [T][n][d], W [m][n*d], b [m].
 * Outputs: layer_in [T][d], coeffs [T][m] (pre|post|H), logits [T][m] or NULL. */
int ds4hc_oracle_pre(int64_t T, int n, int d, const double *X, const double *W,
                     const double *b, double eps, int iters,
                     double *layer_in, double *coeffs, double *logits)
{
    if (bad_shape(T, n, d) || iters < 0 || !X || !W || !b || !layer_in || !coeffs)
        return ORACLE_BAD_ARG;
    const int m = n_logits(n);
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        double z[m];
        const double *x = X + (size_t)t * n * d;
        double *ct = coeffs + (size_t)t * m;
        coefficients_one(n, d, x, W, b, eps, iters, z, ct);
        premix_one(n, d, x, ct, layer_in + (size_t)t * d);
        if (logits)
            memcpy(logits + (size_t)t * m, z, sizeof(double) * (size_t)m);
    }
    return ORACLE_OK;
}

/* Sinkhorn alone: logits_res [T][n][n] -> H [T][n][n]. */
int ds4hc_oracle_sinkhorn(int64_t T, int n, int iters, const double *logits_res, double *H)
{
    if (T < 0 || n < 1 || iters < 0 || !logits_res || !H)
        return ORACLE_BAD_ARG;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t)
        sinkhorn_one(n, iters, logits_res + (size_t)t * n * n, H + (size_t)t * n * n);
    return ORACLE_OK;
}

/* hc_post: step 7. X [T][n][d], coeffs [T][m], layer_out [T][d] -> X_out [T][n][d]. */
int ds4hc_oracle_post(int64_t T, int n, int d, const double *X, const double *coeffs,
                      const double *layer_out, double *X_out)
{
    if (bad_shape(T, n, d) || !X || !coeffs || !layer_out || !X_out)
        return ORACLE_BAD_ARG;
    const int m = n_logits(n);
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t)
        post_one(n, d, X + (size_t)t * n * d, coeffs + (size_t)t * m,
                 layer_out + (size_t)t * d, X_out + (size_t)t * n * d);
    return ORACLE_OK;
}

/* Whole op (steps 1-7) for a layer_out that does not depend on layer_in. */
/* Split-over-d partial sums of one column share: X_share [T][n][ds],
 * W_share [m][n*ds] (W's columns of the share, per stream), out [T][m+1]:
 * out[t][j] = sum_k W_share[j][k] x_k (j < m), out[t][m] = sum_k x_k^2. */
int ds4hc_oracle_partials(int64_t T, int n, int ds, const double *X_share,
                          const double *W_share, double *out)
{
    if (bad_shape(T, n, ds) || !X_share || !W_share || !out)
        return ORACLE_BAD_ARG;
    const int m = n_logits(n);
    const int64_t K = (int64_t)n * ds;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        const double *x = X_share + (size_t)t * (size_t)K;
        double *o = out + (size_t)t * (size_t)(m + 1);
        for (int j = 0; j < m; ++j) {
            const double *wj = W_share + (size_t)j * (size_t)K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += wj[k] * x[k];
            o[j] = acc;
        }
        double q = 0.0;
        for (int64_t k = 0; k < K; ++k)
            q += x[k] * x[k];
        o[m] = q;
    }
    return ORACLE_OK;
}

int ds4hc_oracle_fused(int64_t T, int n, int d, const double *X, const double *W,
                       const double *b, const double *layer_out, double eps, int iters,
                       double *layer_in, double *coeffs, double *X_out)
{
    int rc = ds4hc_oracle_pre(T, n, d, X, W, b, eps, iters, layer_in, coeffs, NULL);
    if (rc != ORACLE_OK)
        return rc;
    return ds4hc_oracle_post(T, n, d, X, coeffs, layer_out, X_out);
}
