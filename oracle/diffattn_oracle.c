/*
 * Differential-attention oracle: a plain, slow, fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg do. It shares no code, header or constant with the HIP
 * path.
 *
 * Every function writes out the plain definition from the pages:
 *   - "Differential Transformer: Noise-Canceling Attention by Subtraction",
 *     section "The mechanism" (two softmax maps, A1 - lambda*A2, times V) and
 *     section "Making lambda learnable and stable" (lambda re-parameterisation,
 *     lambda_init schedule, per-head norm, (1 - lambda_init) rescale).
 *   - "Differential Transformer: softmax can't say zero, so it subtracts",
 *     section "The mechanism, exactly" (shapes: Q_i, K_i are N x d, V is N x 2d;
 *     both maps are ordinary causal maps reading the same values),
 *     section "The row no longer sums to one" (RMSNorm over the doubled value
 *     width, with a learnable weight, then the fixed (1 - lambda_init) multiply)
 *     and section "DIFF V2: what the authors changed" (paired query heads in
 *     one GQA group, per-token per-head lambda, no per-head norm).
 *
 * Arithmetic: double throughout, libm exp/sqrt, sums taken in index order.
 * No blocking, no online softmax, no fusion: each output row materialises its
 * two softmax rows, differences them and applies the difference to V.
 * Threads (OpenMP) only split independent output rows; they do not change the
 * arithmetic of any row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* lambda_init(l) = 0.8 - 0.6 * exp(-0.3 * (l - 1)), layer index l counted
 * from 1. Source: "Noise-Canceling Attention by Subtraction", section
 * "Making lambda learnable and stable"; the same schedule and its table of
 * values appear in "softmax can't say zero", section "lambda, re-parameterised". */
double oracle_lambda_init(int layer) {
    return 0.8 - 0.6 * exp(-0.3 * ((double)layer - 1.0));
}

/* lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init(l), one value per row
 * of the four [n, dim] vector sets (per head, or n = 1 for one per layer).
 * Source: "Noise-Canceling Attention by Subtraction", section "Making lambda
 * learnable and stable". */
void oracle_lambda(const double* lq1, const double* lk1, const double* lq2,
                   const double* lk2, int n, int dim, int layer, double* out) {
    double li = oracle_lambda_init(layer);
    for (int r = 0; r < n; ++r) {
        double dot1 = 0.0, dot2 = 0.0;
        for (int c = 0; c < dim; ++c) {
            dot1 += lq1[(int64_t)r * dim + c] * lk1[(int64_t)r * dim + c];
            dot2 += lq2[(int64_t)r * dim + c] * lk2[(int64_t)r * dim + c];
        }
        out[r] = exp(dot1) - exp(dot2) + li;
    }
}

/* softmax over the first n entries of s, in place: exp(s_j - max) / sum.
 * Subtracting the maximum leaves the value unchanged in exact arithmetic. */
static void softmax_inplace(double* s, int n) {
    double mx = -INFINITY;
    for (int j = 0; j < n; ++j) if (s[j] > mx) mx = s[j];
    double sum = 0.0;
    for (int j = 0; j < n; ++j) { s[j] = exp(s[j] - mx); sum += s[j]; }
    for (int j = 0; j < n; ++j) s[j] /= sum;
}

/* One output row of DiffAttn:
 *   o = (softmax(scale * q1 K1^T) - lam * softmax(scale * q2 K2^T)) V
 * over the visible keys 0 .. nvis-1 (both maps normalise over the same keys).
 * k1, k2 have row stride ks, v has row stride vs (in elements).
 * work must hold 2*nvis doubles. */
static void diff_row(const double* q1, const double* q2, const double* k1,
                     const double* k2, const double* v, int64_t ks, int64_t vs,
                     int nvis, int d, int dv, double lam, double scale,
                     double* o, double* work) {
    double* a1 = work;
    double* a2 = work + nvis;
    for (int j = 0; j < nvis; ++j) {
        double s1 = 0.0, s2 = 0.0;
        for (int c = 0; c < d; ++c) {
            s1 += q1[c] * k1[(int64_t)j * ks + c];
            s2 += q2[c] * k2[(int64_t)j * ks + c];
        }
        a1[j] = scale * s1;
        a2[j] = scale * s2;
    }
    softmax_inplace(a1, nvis);
    softmax_inplace(a2, nvis);
    for (int c = 0; c < dv; ++c) o[c] = 0.0;
    for (int j = 0; j < nvis; ++j) {
        double w = a1[j] - lam * a2[j];
        for (int c = 0; c < dv; ++c) o[c] += w * v[(int64_t)j * vs + c];
    }
}

/* Number of keys a query row sees. Non-causal: all nk keys. Causal: key j is
 * visible to query i when j <= i + (nk - nq), i.e. the mask is aligned to the
 * last key (nq == nk gives the ordinary j <= i). Returns a prefix length. */
static int visible_keys(int i, int nq, int nk, int causal) {
    if (!causal) return nk;
    int64_t last = (int64_t)i + (int64_t)(nk - nq);
    if (last < 0) return 0;
    if (last >= nk) return nk;
    return (int)(last + 1);
}

/* One head (or one V2 pair): output rows `rows[0..nrows)` (or every row
 * 0..nq-1 when rows == NULL) of the differential map.
 *   q1, q2: [nq, d] row-major; k1, k2: [nk, d]; v: [nk, dv]; out: [nrows, dv].
 *   lam_rows: lambda per query row ([nq]); V1 passes one value repeated,
 *   V2 passes its per-token value for this pair.
 * Returns 0, or -1 if a row would see no key or on allocation failure. */
int oracle_diff_head(const double* q1, const double* q2, const double* k1,
                     const double* k2, const double* v, int nq, int nk, int d,
                     int dv, const double* lam_rows, int causal, double scale,
                     const int32_t* rows, int nrows, double* out) {
    int n_out = rows ? nrows : nq;
    int err = 0;
#pragma omp parallel
    {
        double* work = (double*)malloc(sizeof(double) * 2 * (size_t)(nk > 0 ? nk : 1));
        if (!work) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int r = 0; r < n_out; ++r) {
                int i = rows ? rows[r] : r;
                int nvis = visible_keys(i, nq, nk, causal);
                if (nvis <= 0 || i < 0 || i >= nq) {
#pragma omp atomic write
                    err = -1;
                    continue;
                }
                diff_row(q1 + (int64_t)i * d, q2 + (int64_t)i * d, k1, k2, v, d, dv,
                         nvis, d, dv, lam_rows[i], scale, out + (int64_t)r * dv, work);
            }
            free(work);
        }
    }
    return err;
}

/* Per-head RMSNorm over the dv channels of each row, times the norm weight g
 * (NULL = all ones), then the fixed multiply by (1 - lambda_init):
 *   o <- o / sqrt(mean_c o_c^2 + eps) * g,   o <- o * (1 - lambda_init).
 * Source: "Noise-Canceling Attention by Subtraction", section "Making lambda
 * learnable and stable" items 1 and 2; "softmax can't say zero", section
 * "The row no longer sums to one". */
void oracle_rmsnorm_scale(double* o, int nrows, int dv, const double* g,
                          double eps, double lambda_init) {
    for (int r = 0; r < nrows; ++r) {
        double* row = o + (int64_t)r * dv;
        double ss = 0.0;
        for (int c = 0; c < dv; ++c) ss += row[c] * row[c];
        double inv = 1.0 / sqrt(ss / dv + eps);
        for (int c = 0; c < dv; ++c) {
            row[c] = row[c] * inv * (g ? g[c] : 1.0);
            row[c] = row[c] * (1.0 - lambda_init);
        }
    }
}

/* Gradients of one head's differential map, taken by the chain rule through the
 * definition that oracle_diff_head evaluates (no epilogue; the RMSNorm part is
 * differentiated by the caller). Given go = dL/do for every row, with
 * o_i = sum_j (A1_ij - lam_i A2_ij) v_j and A = softmax over the visible keys:
 *   dL/dA1_ij = go_i . v_j,   dL/dA2_ij = -lam_i (go_i . v_j)
 *   softmax:  dL/dS_ij = A_ij (dL/dA_ij - sum_k A_ik dL/dA_ik)
 *   S = scale q K^T:  dq_i = scale sum_j dL/dS_ij k_j,  dk_j += scale dL/dS_ij q_i
 *   dv_j += (A1_ij - lam_i A2_ij) go_i,   dlam_i = -go_i . (A2 V)_i
 * Shapes as oracle_diff_head (rows are all nq rows); dk1, dk2, dvv are
 * overwritten. Rows are taken in order on one thread (the key-side gradients
 * accumulate over rows). Returns 0, or -1 if a row sees no key or on
 * allocation failure. */
int oracle_diff_head_bwd(const double* q1, const double* q2, const double* k1,
                         const double* k2, const double* v, int nq, int nk, int d,
                         int dv, const double* lam_rows, int causal, double scale,
                         const double* go, double* dq1, double* dq2, double* dk1,
                         double* dk2, double* dvv, double* dlam_rows) {
    double* a1 = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    double* a2 = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    double* da = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    if (!a1 || !a2 || !da) { free(a1); free(a2); free(da); return -1; }
    memset(dk1, 0, sizeof(double) * (size_t)nk * d);
    memset(dk2, 0, sizeof(double) * (size_t)nk * d);
    memset(dvv, 0, sizeof(double) * (size_t)nk * dv);
    int err = 0;
    for (int i = 0; i < nq && !err; ++i) {
        int n = visible_keys(i, nq, nk, causal);
        if (n <= 0) { err = -1; break; }
        const double* q1i = q1 + (int64_t)i * d;
        const double* q2i = q2 + (int64_t)i * d;
        const double* gi = go + (int64_t)i * dv;
        double lam = lam_rows[i];
        for (int j = 0; j < n; ++j) {
            double s1 = 0.0, s2 = 0.0;
            for (int c = 0; c < d; ++c) {
                s1 += q1i[c] * k1[(int64_t)j * d + c];
                s2 += q2i[c] * k2[(int64_t)j * d + c];
            }
            a1[j] = scale * s1;
            a2[j] = scale * s2;
        }
        softmax_inplace(a1, n);
        softmax_inplace(a2, n);
        /* dL/dA (up to the map's factor): go_i . v_j, and the row sums of A * dL/dA */
        double r1 = 0.0, r2 = 0.0, dl = 0.0;
        for (int j = 0; j < n; ++j) {
            double t = 0.0;
            for (int c = 0; c < dv; ++c) t += gi[c] * v[(int64_t)j * dv + c];
            da[j] = t;
            r1 += a1[j] * t;
            r2 += a2[j] * t;
        }
        dl = -r2;   /* go_i . (A2 V)_i = sum_j A2_ij (go_i . v_j) */
        dlam_rows[i] = dl;
        for (int c = 0; c < d; ++c) { dq1[(int64_t)i * d + c] = 0.0; dq2[(int64_t)i * d + c] = 0.0; }
        for (int j = 0; j < n; ++j) {
            double ds1 = a1[j] * (da[j] - r1);
            double ds2 = -lam * a2[j] * (da[j] - r2);
            for (int c = 0; c < d; ++c) {
                dq1[(int64_t)i * d + c] += scale * ds1 * k1[(int64_t)j * d + c];
                dq2[(int64_t)i * d + c] += scale * ds2 * k2[(int64_t)j * d + c];
                dk1[(int64_t)j * d + c] += scale * ds1 * q1i[c];
                dk2[(int64_t)j * d + c] += scale * ds2 * q2i[c];
            }
            double w = a1[j] - lam * a2[j];
            for (int c = 0; c < dv; ++c) dvv[(int64_t)j * dv + c] += w * gi[c];
        }
    }
    free(a1); free(a2); free(da);
    return err;
}

/* Number of OpenMP threads the head loop will use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
