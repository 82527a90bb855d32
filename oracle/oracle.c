/*
 * CPU oracle for sparse matrix-vector multiplication and for the storage
 * format conversions -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  It shares no code, header, table or helper with the GPU
 * library: it is a plain, slow, obviously correct statement of what the GPU
 * path must compute, used to check it.
 *
 * What it computes (the pages' definitions restated):
 *
 *   spmv:  y_i = alpha * sum_{k in row i} val[k] * x[col[k]] + beta * y_i
 *          over the stored entries of a CSR matrix (the sparse mat-vec whose
 *          storage variants are compared in "Sparse matrix-vector
 *          multiplication on GPGPU clusters", Sect. 2, and in "Development of
 *          Krylov and AMG linear solvers...", Sect. 2.1, Figs. 1-3).
 *          Duplicated (row, col) entries are summed: the matrix is the sum
 *          of its stored triples.  beta == 0 means y is not read.
 *          Each row sum is accumulated in fp64 with the compensated dot
 *          product "Dot2" of Ogita, Rump and Oishi ("Accurate sum and dot
 *          product", SIAM J. Sci. Comput. 26(6), 2005, Algorithm 5.3): a
 *          TwoProduct error-free split of every product, a TwoSum of the
 *          running sum, and a separately accumulated correction term.  The
 *          result is as accurate as if computed in twice the working
 *          precision and rounded once.  The scale d_i = |alpha| * sum |a*x|
 *          + |beta * y_i| is returned beside it for the tolerance test.
 *
 *   converters (bit-exact references for the GPU-built layouts):
 *     ELLPACK-R  -- rows shifted left into an N x Nmax rectangle stored
 *                   column by column, with the row count padded to a
 *                   multiple of the SIMD width (64 here) and a per-row
 *                   length array ("Sparse matrix-vector multiplication on
 *                   GPGPU clusters", Sect. 2.1, Fig. 1 and footnote 2).
 *     SELL-64    -- the pJDS idea of the same page (Sect. 2.2, Fig. 1 "sort"
 *                   and "pad"): rows sorted by length, longest first, in
 *                   blocks of 64 rows padded to the block's longest row;
 *                   stored slice by slice with a row permutation.
 *     HYB / HEC  -- a regular ELL part of width K plus the remaining
 *                   entries of each row as COO (HYB) or CSR (HEC)
 *                   ("Development of Krylov and AMG linear solvers...",
 *                   Sect. 2.1, Figs. 2-3; "Load-balancing Sparse Matrix
 *                   Vector Product Kernels on GPUs", abstract).
 *   Where the pages leave a convention open the reading taken is:
 *     - ELL-R stride S = 64 * ceil(n / 64); slot (i, j) at j * S + i; pad
 *       slots hold column 0 and value +0.0; padded rows have length 0.
 *       The ELL part of HYB/HEC is stored the same way in blocks of 1024
 *       rows (the Krylov/AMG page sets the ELL stride to 256 or a multiple
 *       of it): slot (i, j) at (i / 1024) * W * 1024 + j * 1024 + i % 1024.
 *     - Windowed sorting (the sort of pJDS applied only inside aligned
 *       windows of sigma rows, so rows move less than sigma and x locality
 *       survives): SELL-64 sorts by (i / sigma, length desc, row asc) and
 *       pads each slice to its longest row; sigma = 1 keeps the row order; the
 *       ELL part of HYB/HEC may sort the rows of every 1024-row block by
 *       (position / sigma, stored length desc, row asc), sigma dividing
 *       1024, with out_perm[p] the row at position p.
 *     - SELL sort key (length descending, row ascending) -- unique, so the
 *       permutation is unique; slice s has width w_s = length of its
 *       longest row (the first one after a whole-matrix sort); entry j of
 *       sorted row r sits at
 *       slice_ptr[r / 64] + 64 * j + r % 64.
 *     - HYB/HEC width K = max{k >= 0 : #{i : len_i >= k} >= ceil(n / 3)}
 *       unless a width is given (clamped to the longest row); the first K
 *       entries of each row (CSR order) go to the ELL part, the rest to the
 *       tail in row order.
 *
 * Values are handled as opaque bytes of the stated element size in the
 * converters, so the references move value bits exactly.
 *
 * Built with -O2 -ffp-contract=off and without fast-math, so that the only
 * fused multiply-add is the explicit fma() of TwoProduct.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* error-free transformations                                              */
/* ---------------------------------------------------------------------- */

/* Knuth's TwoSum: s + e == a + b exactly, s = fl(a + b). */
static void two_sum(double a, double b, double *s, double *e)
{
    double x = a + b;
    double z = x - a;
    *e = (a - (x - z)) + (b - z);
    *s = x;
}

/* TwoProduct via FMA: p + e == a * b exactly, p = fl(a * b). */
static void two_prod(double a, double b, double *p, double *e)
{
    double x = a * b;
    *e = fma(a, b, -x);
    *p = x;
}

/* Dot2 over one CSR row, plus the plain sum of |a * x| for the scale. */
static double row_dot2(int64_t k0, int64_t k1, const int32_t *col,
                       const double *val, const double *x, double *absum)
{
    double s = 0.0, c = 0.0, ab = 0.0;
    for (int64_t k = k0; k < k1; ++k) {
        double p, ep, q;
        two_prod(val[k], x[col[k]], &p, &ep);
        two_sum(s, p, &s, &q);
        c += q + ep;
        ab += fabs(p);
    }
    *absum = ab;
    return s + c;
}

/*
 * y_out[i] = alpha * A x + beta * y_in[i] for every row (or for the rows
 * listed in `rows` when rows != NULL; then y_out/scale_out are indexed by
 * position in that list and y_in by row).  y_in may be NULL when beta == 0.
 * nthreads <= 0 lets OpenMP choose; 1 runs serially.  Returns 0.
 */
int oracle_spmv(int64_t n, const int64_t *rowptr, const int32_t *col,
                const double *val, const double *x, const double *y_in,
                double alpha, double beta, double *y_out, double *scale_out,
                const int64_t *rows, int64_t nrows, int nthreads)
{
    int64_t m = rows ? nrows : n;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
#endif
    for (int64_t t = 0; t < m; ++t) {
        int64_t i = rows ? rows[t] : t;
        double ab;
        double r = row_dot2(rowptr[i], rowptr[i + 1], col, val, x, &ab);
        double yv;
        double sc = fabs(alpha) * ab;
        if (beta == 0.0) {
            yv = alpha * r;
        } else {
            double by = beta * y_in[i];
            yv = alpha * r + by;
            sc += fabs(by);
        }
        y_out[t] = yv;
        if (scale_out)
            scale_out[t] = sc;
    }
    (void)nthreads;
    return 0;
}

/* number of threads OpenMP would use by default (1 without OpenMP) */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* converters                                                              */
/* ---------------------------------------------------------------------- */

static int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

/* longest row */
int64_t oracle_max_len(int64_t n, const int64_t *rowptr)
{
    int64_t w = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t l = rowptr[i + 1] - rowptr[i];
        if (l > w)
            w = l;
    }
    return w;
}

/* stored length of row i in an ELL part of width W */
static int64_t ell_len(const int64_t *rowptr, int64_t i, int64_t W)
{
    int64_t len = rowptr[i + 1] - rowptr[i];
    return len < W ? len : W;
}

/* windowed-sort comparator state: rows of one window, by stored length
 * descending, then row ascending */
static const int64_t *g_ell_rowptr;
static int64_t g_ell_W;
static int cmp_ell_rows(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    int64_t la = ell_len(g_ell_rowptr, a, g_ell_W), lb = ell_len(g_ell_rowptr, b, g_ell_W);
    if (la != lb)
        return la > lb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/*
 * ELLPACK arrays of width W (W >= every row length handled; entries j >= W
 * of a row are skipped, which is how the ELL part of HYB/HEC is built),
 * stored in column-major blocks of B rows: the row at position p holds its
 * entry j in slot (p / B) * W * B + j * B + p % B.  block <= 0 means one
 * block of B = pad64(n) rows (ELLPACK-R's column-by-column layout).  Rows
 * are padded to R = ceil(n / B) * B; out_col/out_val hold W * R slots,
 * out_len R lengths (by position).
 * sigma <= 0: position p holds row p.  sigma > 0 (block > 0, sigma divides
 * B): the rows of each aligned window of sigma positions are ordered by
 * stored length descending, then row ascending; padding rows (>= n) stay
 * last.  out_perm (R entries, may be NULL) receives the row at each
 * position (p itself for padding).
 */
void oracle_ell(int64_t n, const int64_t *rowptr, const int32_t *col,
                const void *val, int vsize, int64_t W, int64_t block,
                int64_t sigma, int32_t *out_col, void *out_val, int32_t *out_len,
                int64_t *out_perm)
{
    int64_t B = block > 0 ? block : pad64(n);
    int64_t R = block > 0 ? (n + block - 1) / block * block : B;
    char *ov = (char *)out_val;
    const char *iv = (const char *)val;
    int64_t *row_at = (int64_t *)malloc((size_t)(R > 0 ? R : 1) * sizeof(int64_t));
    for (int64_t p = 0; p < R; ++p)
        row_at[p] = p;
    if (sigma > 0 && block > 0) {
        g_ell_rowptr = rowptr;
        g_ell_W = W;
        for (int64_t w0 = 0; w0 < n; w0 += sigma) {
            int64_t w1 = w0 + sigma < n ? w0 + sigma : n;  /* real rows of the window */
            qsort(row_at + w0, (size_t)(w1 - w0), sizeof(int64_t), cmp_ell_rows);
        }
    }
    memset(out_col, 0, (size_t)(W * R) * sizeof(int32_t));
    memset(ov, 0, (size_t)(W * R) * (size_t)vsize);
    for (int64_t p = 0; p < R; ++p) {
        int64_t i = row_at[p];
        int64_t len = i < n ? ell_len(rowptr, i, W) : 0;
        out_len[p] = (int32_t)len;
        if (out_perm)
            out_perm[p] = i;
        for (int64_t j = 0; j < len; ++j) {
            int64_t slot = (p / B) * W * B + j * B + p % B;
            int64_t k = rowptr[i] + j;
            out_col[slot] = col[k];
            memcpy(ov + slot * vsize, iv + k * vsize, (size_t)vsize);
        }
    }
    free(row_at);
}

/*
 * Share of the slots that a lane-per-row sweep of the (unsorted) ELL part
 * of width W reads beyond the rows' ends: waves of 64 consecutive rows run
 * to their longest stored row, so the padding read is
 * 1 - sum_i len_i / sum_waves 64 * max len in the wave.
 */
double oracle_ell_pad_fraction(int64_t n, const int64_t *rowptr, int64_t W)
{
    double used = 0, read = 0;
    for (int64_t w0 = 0; w0 < n; w0 += 64) {
        int64_t mx = 0;
        for (int64_t i = w0; i < w0 + 64 && i < n; ++i) {
            int64_t l = ell_len(rowptr, i, W);
            used += (double)l;
            if (l > mx)
                mx = l;
        }
        read += 64.0 * (double)mx;
    }
    return read > 0 ? 1.0 - used / read : 0.0;
}

/* sort key: window (sigma rows; 0 = one window), length descending, then
 * row ascending */
static const int64_t *g_rowptr;
static int64_t g_sigma;
static int cmp_rows(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    if (g_sigma > 0 && a / g_sigma != b / g_sigma)
        return a / g_sigma < b / g_sigma ? -1 : 1;
    int64_t la = g_rowptr[a + 1] - g_rowptr[a];
    int64_t lb = g_rowptr[b + 1] - g_rowptr[b];
    if (la != lb)
        return la > lb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/*
 * SELL-64 layout sizes and permutation.  perm[r] (r < pad64(n)) is the
 * original row at sorted position r (rows >= n are padding, perm = -1 kept
 * out: perm has n entries); slice_ptr has nslices + 1 entries; len_sorted has
 * pad64(n) entries.  sigma <= 0 sorts all rows at once (pJDS); sigma > 0
 * sorts only inside aligned windows of sigma rows.  Returns the total number
 * of slots.
 */
int64_t oracle_sell_layout(int64_t n, const int64_t *rowptr, int64_t sigma, int64_t *perm,
                           int64_t *slice_ptr, int32_t *len_sorted)
{
    int64_t S = pad64(n), ns = S / 64;
    for (int64_t i = 0; i < n; ++i)
        perm[i] = i;
    g_rowptr = rowptr;
    g_sigma = sigma;
    qsort(perm, (size_t)n, sizeof(int64_t), cmp_rows);
    for (int64_t r = 0; r < S; ++r)
        len_sorted[r] = r < n ? (int32_t)(rowptr[perm[r] + 1] - rowptr[perm[r]]) : 0;
    slice_ptr[0] = 0;
    for (int64_t s = 0; s < ns; ++s) {
        /* width = longest row of the slice (its first row unless a window
         * boundary falls inside the slice) */
        int64_t w = 0;
        for (int64_t r = 64 * s; r < 64 * s + 64; ++r)
            if (len_sorted[r] > w)
                w = len_sorted[r];
        slice_ptr[s + 1] = slice_ptr[s] + 64 * w;
    }
    return slice_ptr[ns];
}

/*
 * SELL-64 fill given the layout from oracle_sell_layout.  permuted != 0
 * stores the matrix of the permuted basis, P A P^T with (P v)[r] =
 * v[perm[r]] (the form in which "Sparse matrix-vector multiplication on
 * GPGPU clusters", Sect. 2.2, runs a whole solve): column c becomes the
 * sorted position of row c, inv[c] with perm[inv[c]] = c.  Pads stay 0.
 */
void oracle_sell_fill(int64_t n, const int64_t *rowptr, const int32_t *col,
                      const void *val, int vsize, const int64_t *perm,
                      const int64_t *slice_ptr, int permuted, int32_t *out_col,
                      void *out_val)
{
    int64_t S = pad64(n), ns = S / 64;
    int64_t total = slice_ptr[ns];
    char *ov = (char *)out_val;
    const char *iv = (const char *)val;
    int64_t *inv = NULL;
    if (permuted) {
        inv = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        for (int64_t r = 0; r < n; ++r)
            inv[perm[r]] = r;
    }
    memset(out_col, 0, (size_t)total * sizeof(int32_t));
    memset(ov, 0, (size_t)total * (size_t)vsize);
    for (int64_t r = 0; r < n; ++r) {
        int64_t i = perm[r];
        int64_t len = rowptr[i + 1] - rowptr[i];
        for (int64_t j = 0; j < len; ++j) {
            int64_t slot = slice_ptr[r / 64] + 64 * j + r % 64;
            int64_t k = rowptr[i] + j;
            out_col[slot] = permuted ? (int32_t)inv[col[k]] : col[k];
            memcpy(ov + slot * vsize, iv + k * vsize, (size_t)vsize);
        }
    }
    free(inv);
}

/* HYB/HEC ELL width: the ceil(n/3) rule, or the requested width clamped */
int64_t oracle_hyb_width(int64_t n, const int64_t *rowptr, int64_t requested)
{
    int64_t W = oracle_max_len(n, rowptr);
    if (requested >= 0)
        return requested < W ? requested : W;
    int64_t need = (n + 2) / 3;
    int64_t K = 0;
    for (int64_t k = 1; k <= W; ++k) {
        int64_t cnt = 0;
        for (int64_t i = 0; i < n; ++i)
            if (rowptr[i + 1] - rowptr[i] >= k)
                ++cnt;
        if (cnt >= need)
            K = k;
        else
            break;
    }
    return K;
}

/* the other HYB/HEC width candidate: the smallest k such that at most 1 % of
 * the rows are longer than k (100 * #{i : len_i > k} <= n), so that the ELL
 * part holds the regular rows whole and the tail only the few long ones */
int64_t oracle_regular_width(int64_t n, const int64_t *rowptr)
{
    int64_t W = oracle_max_len(n, rowptr);
    for (int64_t k = 0; k <= W; ++k) {
        int64_t longer = 0;
        for (int64_t i = 0; i < n; ++i)
            if (rowptr[i + 1] - rowptr[i] > k)
                ++longer;
        if (100 * longer <= n)
            return k;
    }
    return W;
}

/* number of tail entries for width K */
int64_t oracle_tail_nnz(int64_t n, const int64_t *rowptr, int64_t K)
{
    int64_t t = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t len = rowptr[i + 1] - rowptr[i];
        if (len > K)
            t += len - K;
    }
    return t;
}

/*
 * Tail of the HYB/HEC split: entries j >= K of every row, in row order and
 * in-row order.  Writes COO row ids (out_row, may be NULL), the CSR row
 * pointer of the tail (out_ptr, n + 1 entries, may be NULL), columns and
 * value bytes.
 */
void oracle_tail(int64_t n, const int64_t *rowptr, const int32_t *col,
                 const void *val, int vsize, int64_t K, int32_t *out_row,
                 int32_t *out_ptr, int32_t *out_col, void *out_val)
{
    char *ov = (char *)out_val;
    const char *iv = (const char *)val;
    int64_t t = 0;
    if (out_ptr)
        out_ptr[0] = 0;
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t k = rowptr[i] + K; k < rowptr[i + 1]; ++k) {
            if (out_row)
                out_row[t] = (int32_t)i;
            out_col[t] = col[k];
            memcpy(ov + t * vsize, iv + k * vsize, (size_t)vsize);
            ++t;
        }
        if (out_ptr)
            out_ptr[i + 1] = (int32_t)t;
    }
}

/* ---------------------------------------------------------------------- */
/* Krylov solvers over the product: the consumers sparse mat-vec serves in */
/* "Development of Krylov and AMG linear solvers for large-scale sparse   */
/* matrices on GPUs" (Sect. 3).  Textbook forms: conjugate gradients      */
/* (Hestenes and Stiefel 1952) for symmetric positive definite A, and     */
/* BiCGSTAB (van der Vorst 1992) for general A.  Stop when the recurred    */
/* residual satisfies ||r|| <= rtol * ||b|| (2-norms) or after max_iter    */
/* iterations.  Products use the Dot2 rows above; inner products are plain */
/* fp64 sums in index order.                                               */
/* ---------------------------------------------------------------------- */

static void solver_matvec(int64_t n, const int64_t *rowptr, const int32_t *col,
                          const double *val, const double *x, double *y)
{
    double ab;
    for (int64_t i = 0; i < n; ++i)
        y[i] = row_dot2(rowptr[i], rowptr[i + 1], col, val, x, &ab);
}

static double solver_dot(int64_t n, const double *a, const double *b)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += a[i] * b[i];
    return s;
}

/* x holds the initial guess on entry and the solution on return.  Returns
 * the iterations taken; *rel_res = ||r|| / ||b|| of the last residual. */
int oracle_cg(int64_t n, const int64_t *rowptr, const int32_t *col, const double *val,
              const double *b, double *x, double rtol, int max_iter, double *rel_res)
{
    double *r = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *q = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double bnorm = sqrt(solver_dot(n, b, b));
    int k = 0;
    solver_matvec(n, rowptr, col, val, x, q);
    for (int64_t i = 0; i < n; ++i) {
        r[i] = b[i] - q[i];
        p[i] = r[i];
    }
    double rr = solver_dot(n, r, r);
    while (sqrt(rr) > rtol * bnorm && k < max_iter) {
        solver_matvec(n, rowptr, col, val, p, q);
        double alpha = rr / solver_dot(n, p, q);
        for (int64_t i = 0; i < n; ++i) {
            x[i] += alpha * p[i];
            r[i] -= alpha * q[i];
        }
        double rr_new = solver_dot(n, r, r);
        double beta = rr_new / rr;
        for (int64_t i = 0; i < n; ++i)
            p[i] = r[i] + beta * p[i];
        rr = rr_new;
        ++k;
    }
    *rel_res = bnorm > 0 ? sqrt(rr) / bnorm : sqrt(rr);
    free(r);
    free(p);
    free(q);
    return k;
}

int oracle_bicgstab(int64_t n, const int64_t *rowptr, const int32_t *col, const double *val,
                    const double *b, double *x, double rtol, int max_iter, double *rel_res)
{
    size_t sz = (size_t)(n > 0 ? n : 1) * sizeof(double);
    double *r = (double *)malloc(sz), *rh = (double *)malloc(sz), *p = (double *)malloc(sz);
    double *v = (double *)malloc(sz), *s = (double *)malloc(sz), *t = (double *)malloc(sz);
    double bnorm = sqrt(solver_dot(n, b, b));
    int k = 0;
    solver_matvec(n, rowptr, col, val, x, t);
    for (int64_t i = 0; i < n; ++i) {
        r[i] = b[i] - t[i];
        rh[i] = r[i];
        p[i] = 0.0;
        v[i] = 0.0;
    }
    double rho = 1.0, alpha = 1.0, omega = 1.0;
    double rr = solver_dot(n, r, r);
    while (sqrt(rr) > rtol * bnorm && k < max_iter) {
        double rho_new = solver_dot(n, rh, r);
        if (rho_new == 0.0)
            break; /* breakdown */
        double beta = (rho_new / rho) * (alpha / omega);
        for (int64_t i = 0; i < n; ++i)
            p[i] = r[i] + beta * (p[i] - omega * v[i]);
        solver_matvec(n, rowptr, col, val, p, v);
        alpha = rho_new / solver_dot(n, rh, v);
        for (int64_t i = 0; i < n; ++i)
            s[i] = r[i] - alpha * v[i];
        solver_matvec(n, rowptr, col, val, s, t);
        double tt = solver_dot(n, t, t);
        omega = tt > 0 ? solver_dot(n, t, s) / tt : 0.0;
        for (int64_t i = 0; i < n; ++i) {
            x[i] += alpha * p[i] + omega * s[i];
            r[i] = s[i] - omega * t[i];
        }
        rr = solver_dot(n, r, r);
        rho = rho_new;
        ++k;
        if (omega == 0.0)
            break; /* s was already the residual of x + alpha p */
    }
    *rel_res = bnorm > 0 ? sqrt(rr) / bnorm : sqrt(rr);
    free(r);
    free(rh);
    free(p);
    free(v);
    free(s);
    free(t);
    return k;
}
