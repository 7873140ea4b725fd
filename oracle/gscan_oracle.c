/*
 * CPU ORACLE for the gated temporal scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this code.  It shares nothing with the HIP library: no headers,
 * no helpers, no tables.  Plain loops in double precision; every input is
 * widened exactly to double by the caller.
 *
 * What it computes (foxhunt design spec "Custom Kernel Optimization - cuBLAS
 * Projections + Batch-Parallel Scans", section Design 1 "Mamba2 Scan"):
 *
 *   Forward, Step 1 (pre-projections):
 *     A_vals[b*K+t, s] = sum_i h_history[b*K+t, i] * W_A[i, s]   (+ a_shift)
 *     B_vals[b*K+t, s] = sum_i h_history[b*K+t, i] * W_B[i, s]
 *     C_vals[b, s]     = sum_i h_s2[b, i] * W_C[i, s]
 *   Forward, Step 2 (per (sample, state) scan, t = 0 first, x starts at 0):
 *     x <- sigmoid(A_vals[b*K+t, s]) * x + B_vals[b*K+t, s]
 *     context[b, s] = C_vals[b, s] * x        (state after all K steps)
 *   Backward, Steps 1-2: replay the projections and the forward scan, then
 *     run the scan in reverse for the loss L = sum_{b,s} d_context * context.
 *   Backward, Step 3: weight gradients contracted over rows:
 *     dW_A = h_history^T @ d_gate, dW_B = h_history^T @ d_x,
 *     dW_C = h_s2^T @ (d_context * x_K)
 *   where d_gate = dL/dA_vals (includes sigmoid'), d_x = dL/dB_vals, and the
 *   operand of dW_C is dL/dC_vals (the spec writes "d_context" for it).
 *
 * a_shift is a constant added to every A value before the sigmoid (0 unless
 * a workload asks for a gate bias); it receives no gradient.
 *
 * Parallelism: OpenMP over fixed blocks of 64 samples.  Each block owns its
 * own weight-gradient partial; partials are summed in block order, so the
 * result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BLOCK 64

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double sigmoid(double a)
{
    return 1.0 / (1.0 + exp(-a));
}

/* out[s] = sum_i row[i] * W[i, s] for s < D  (one row of a projection). */
static void project(const double *row, const double *W, int64_t SH2, int64_t D,
                    double *out)
{
    int64_t i, s;
    for (s = 0; s < D; ++s)
        out[s] = 0.0;
    for (i = 0; i < SH2; ++i)
        for (s = 0; s < D; ++s)
            out[s] += row[i] * W[i * D + s];
}

/* Forward pass: Step 1 projections + Step 2 scan, per sample. */
void oracle_forward(const double *h_history, const double *h_s2,
                    const double *W_A, const double *W_B, const double *W_C,
                    int64_t B, int64_t K, int64_t SH2, int64_t D, double a_shift,
                    double *context)
{
    int64_t b;
#pragma omp parallel for schedule(dynamic, 16)
    for (b = 0; b < B; ++b) {
        double *Cv = (double *)malloc(sizeof(double) * D);
        double *Av = (double *)malloc(sizeof(double) * D);
        double *Bv = (double *)malloc(sizeof(double) * D);
        double *x = (double *)malloc(sizeof(double) * D);
        int64_t t, s;
        project(h_s2 + b * SH2, W_C, SH2, D, Cv);
        for (s = 0; s < D; ++s)
            x[s] = 0.0;
        for (t = 0; t < K; ++t) {
            const double *row = h_history + (b * K + t) * SH2;
            project(row, W_A, SH2, D, Av);
            project(row, W_B, SH2, D, Bv);
            for (s = 0; s < D; ++s) {
                const double g = sigmoid(Av[s] + a_shift);
                x[s] = g * x[s] + Bv[s];
            }
        }
        for (s = 0; s < D; ++s)
            context[b * D + s] = Cv[s] * x[s];
        free(Cv);
        free(Av);
        free(Bv);
        free(x);
    }
}

/*
 * Backward pass for L = sum d_context * context.
 *
 * Replay (Step 1-2): x_0 = 0, g_t = sigmoid(A_t + a_shift),
 *   x_{t+1} = g_t * x_t + B_t, for t = 0..K-1; context = C * x_K.
 * Reverse scan: lam = dL/dx_K = d_context * C;  dC = d_context * x_K.
 *   for t = K-1 down to 0:   (lam is dL/dx_{t+1} on entry)
 *     dB_t = lam
 *     dA_t = lam * x_t * g_t * (1 - g_t)
 *     lam  = g_t * lam         (now dL/dx_t)
 *   The logistic derivative g(1 - g) is formed as sigmoid(a) * sigmoid(-a):
 *   the same number, but 1 - g taken as sigmoid(-a) keeps its relative
 *   precision when the gate saturates towards 1 (1.0 - g would cancel).
 * Step 3: dW_A[i,s] = sum_rows h[r,i] dA[r,s]; dW_B likewise with dB;
 *   dW_C[i,s] = sum_b h_s2[b,i] dC[b,s].
 */
void oracle_backward(const double *h_history, const double *h_s2,
                     const double *W_A, const double *W_B, const double *W_C,
                     int64_t B, int64_t K, int64_t SH2, int64_t D, double a_shift,
                     const double *d_context, double *dW_A, double *dW_B,
                     double *dW_C)
{
    const int64_t nblk = (B + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    const int64_t wsz = SH2 * D;
    double *part = (double *)calloc((size_t)(nblk * 3 * wsz), sizeof(double));
    int64_t blk, i;

#pragma omp parallel for schedule(dynamic, 1)
    for (blk = 0; blk < nblk; ++blk) {
        double *pA = part + blk * 3 * wsz;
        double *pB = pA + wsz;
        double *pC = pB + wsz;
        double *Cv = (double *)malloc(sizeof(double) * D);
        double *Av = (double *)malloc(sizeof(double) * D);
        double *Bv = (double *)malloc(sizeof(double) * D);
        double *xs = (double *)malloc(sizeof(double) * (K + 1) * D); /* x_0..x_K */
        double *gs = (double *)malloc(sizeof(double) * K * D);       /* g_0..g_{K-1} */
        double *gc = (double *)malloc(sizeof(double) * K * D);       /* 1 - g_t */
        double *lam = (double *)malloc(sizeof(double) * D);
        double *dA = (double *)malloc(sizeof(double) * D);
        double *dB = (double *)malloc(sizeof(double) * D);
        double *dC = (double *)malloc(sizeof(double) * D);
        int64_t b;
        const int64_t b_end = (blk + 1) * ORACLE_BLOCK < B ? (blk + 1) * ORACLE_BLOCK : B;
        for (b = blk * ORACLE_BLOCK; b < b_end; ++b) {
            int64_t t, s, ii;
            /* replay */
            project(h_s2 + b * SH2, W_C, SH2, D, Cv);
            for (s = 0; s < D; ++s)
                xs[s] = 0.0;
            for (t = 0; t < K; ++t) {
                const double *row = h_history + (b * K + t) * SH2;
                project(row, W_A, SH2, D, Av);
                project(row, W_B, SH2, D, Bv);
                for (s = 0; s < D; ++s) {
                    const double g = sigmoid(Av[s] + a_shift);
                    gs[t * D + s] = g;
                    gc[t * D + s] = sigmoid(-(Av[s] + a_shift));
                    xs[(t + 1) * D + s] = g * xs[t * D + s] + Bv[s];
                }
            }
            /* reverse scan */
            for (s = 0; s < D; ++s) {
                lam[s] = d_context[b * D + s] * Cv[s];
                dC[s] = d_context[b * D + s] * xs[K * D + s];
            }
            for (t = K - 1; t >= 0; --t) {
                const double *row = h_history + (b * K + t) * SH2;
                for (s = 0; s < D; ++s) {
                    const double g = gs[t * D + s];
                    dB[s] = lam[s];
                    dA[s] = lam[s] * xs[t * D + s] * g * gc[t * D + s];
                    lam[s] = g * lam[s];
                }
                /* Step 3 rows of h_history^T @ d_gate and h_history^T @ d_x */
                for (ii = 0; ii < SH2; ++ii)
                    for (s = 0; s < D; ++s) {
                        pA[ii * D + s] += row[ii] * dA[s];
                        pB[ii * D + s] += row[ii] * dB[s];
                    }
            }
            /* Step 3 row of h_s2^T @ dC */
            for (ii = 0; ii < SH2; ++ii)
                for (s = 0; s < D; ++s)
                    pC[ii * D + s] += h_s2[b * SH2 + ii] * dC[s];
        }
        free(Cv);
        free(Av);
        free(Bv);
        free(xs);
        free(gs);
        free(gc);
        free(lam);
        free(dA);
        free(dB);
        free(dC);
    }

    /* sum the block partials in block order (thread-count independent) */
    for (i = 0; i < wsz; ++i) {
        double a = 0.0, bb = 0.0, c = 0.0;
        for (blk = 0; blk < nblk; ++blk) {
            a += part[blk * 3 * wsz + i];
            bb += part[blk * 3 * wsz + wsz + i];
            c += part[blk * 3 * wsz + 2 * wsz + i];
        }
        dW_A[i] = a;
        dW_B[i] = bb;
        dW_C[i] = c;
    }
    free(part);
}

/*
 * Input gradients: the chain rule through the projections of Step 1 (the
 * spec's backward lists only the weight gradients; these are the gradients
 * a layer below the scan would receive):
 *   d_h_history[b*K+t, i] = sum_s dA_t[s] * W_A[i, s] + dB_t[s] * W_B[i, s]
 *   d_h_s2[b, i]          = sum_s dC[s] * W_C[i, s]
 * with dA_t = dL/dA_vals, dB_t = dL/dB_vals and dC = dL/dC_vals from the same
 * replay and reverse scan as oracle_backward.  Each sample is independent.
 */
void oracle_backward_inputs(const double *h_history, const double *h_s2,
                            const double *W_A, const double *W_B, const double *W_C,
                            int64_t B, int64_t K, int64_t SH2, int64_t D, double a_shift,
                            const double *d_context, double *d_h_history, double *d_h_s2)
{
#pragma omp parallel
    {
        double *Cv = (double *)malloc(sizeof(double) * D);
        double *Av = (double *)malloc(sizeof(double) * D);
        double *Bv = (double *)malloc(sizeof(double) * D);
        double *xs = (double *)malloc(sizeof(double) * (K + 1) * D); /* x_0..x_K */
        double *gs = (double *)malloc(sizeof(double) * K * D);       /* g_0..g_{K-1} */
        double *gc = (double *)malloc(sizeof(double) * K * D);       /* 1 - g_t */
        double *adj = (double *)malloc(sizeof(double) * D); /* dL/dx_{t+1} */
        double *dA = (double *)malloc(sizeof(double) * D);
        double *dB = (double *)malloc(sizeof(double) * D);
        double *dC = (double *)malloc(sizeof(double) * D);
        int64_t b;
#pragma omp for schedule(dynamic, 16)
        for (b = 0; b < B; ++b) {
            int64_t t, s, ii;
            /* replay */
            project(h_s2 + b * SH2, W_C, SH2, D, Cv);
            for (s = 0; s < D; ++s)
                xs[s] = 0.0;
            for (t = 0; t < K; ++t) {
                const double *row = h_history + (b * K + t) * SH2;
                project(row, W_A, SH2, D, Av);
                project(row, W_B, SH2, D, Bv);
                for (s = 0; s < D; ++s) {
                    const double gt = sigmoid(a_shift + Av[s]);
                    gs[t * D + s] = gt;
                    gc[t * D + s] = sigmoid(-(a_shift + Av[s]));
                    xs[(t + 1) * D + s] = gt * xs[t * D + s] + Bv[s];
                }
            }
            /* reverse scan */
            for (s = 0; s < D; ++s) {
                adj[s] = d_context[b * D + s] * Cv[s];
                dC[s] = xs[K * D + s] * d_context[b * D + s];
            }
            for (t = K - 1; t >= 0; --t) {
                double *out = d_h_history + (b * K + t) * SH2;
                for (s = 0; s < D; ++s) {
                    const double gt = gs[t * D + s];
                    dB[s] = adj[s];
                    dA[s] = adj[s] * xs[t * D + s] * gt * gc[t * D + s];
                    adj[s] = gt * adj[s];
                }
                /* row t of d_gate @ W_A^T + d_x @ W_B^T */
                for (ii = 0; ii < SH2; ++ii) {
                    double v = 0.0;
                    for (s = 0; s < D; ++s)
                        v += dA[s] * W_A[ii * D + s] + dB[s] * W_B[ii * D + s];
                    out[ii] = v;
                }
            }
            /* row b of dC @ W_C^T */
            for (ii = 0; ii < SH2; ++ii) {
                double v = 0.0;
                for (s = 0; s < D; ++s)
                    v += dC[s] * W_C[ii * D + s];
                d_h_s2[b * SH2 + ii] = v;
            }
        }
        free(Cv);
        free(Av);
        free(Bv);
        free(xs);
        free(gs);
        free(gc);
        free(adj);
        free(dA);
        free(dB);
        free(dC);
    }
}

/*
 * Batch-parallel bias-gradient reduction (design spec section "IQN Bias
 * Grad Reduce", and the KAN / Q-denoise bias gradients that follow its
 * pattern): out[j] = sum over rows r of grad[r, j], for a row-major
 * [rows, cols] gradient.  The plain definition: one running fp64 sum per
 * column, rows in order.
 */
void oracle_column_sums(const double *grad, int64_t rows, int64_t cols, double *out)
{
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < cols; ++j) {
        double acc = 0.0;
        int64_t r;
        for (r = 0; r < rows; ++r)
            acc += grad[r * cols + j];
        out[j] = acc;
    }
}

/*
 * CIFG matrix-memory update, independent mode (BURT-IMMA CUDA Kernel API
 * Reference, section 2.3 batched_cifg_update with shared_memory_mode =
 * false, which applies section 2.2 cifg_update to every sample):
 *   concat = [h_b ; x_b]                          (length d_model + d_input)
 *   f      = sigmoid(W_f @ concat + b_f)          (length d_model)
 *   C_b[i, j] <- f[i] * C_b[i, j] + (1 - f[i]) * h_b[i] * h_b[j]
 * (the candidate is the rank-1 outer product h h^T; f is broadcast along
 * each row, i.e. over the columns j).  The optional spectral projection of
 * step 5 is not part of this function.  C_in and C_out are [B][d][d],
 * H [B][d], X [B][d_input], W_f [d][d + d_input], b_f [d].  1 - f is
 * evaluated as sigmoid(-a) (no cancellation when the gate saturates).
 */
void oracle_cifg_update(const double *C_in, const double *H, const double *X,
                        const double *W_f, const double *b_f, int64_t B, int64_t d,
                        int64_t d_input, double *C_out)
{
    const int64_t L = d + d_input;
    int64_t b;
#pragma omp parallel for schedule(dynamic, 1)
    for (b = 0; b < B; ++b) {
        double *concat = (double *)malloc(sizeof(double) * L);
        double *f = (double *)malloc(sizeof(double) * d);
        double *fc = (double *)malloc(sizeof(double) * d);
        const double *h = H + b * d;
        int64_t i, j, k;
        /* step 1: concatenate */
        for (k = 0; k < d; ++k)
            concat[k] = h[k];
        for (k = 0; k < d_input; ++k)
            concat[d + k] = X[b * d_input + k];
        /* step 2: forget gate */
        for (i = 0; i < d; ++i) {
            double a = b_f[i];
            for (k = 0; k < L; ++k)
                a += W_f[i * L + k] * concat[k];
            f[i] = sigmoid(a);
            fc[i] = sigmoid(-a);
        }
        /* steps 3-4: rank-1 candidate and the gated update */
        for (i = 0; i < d; ++i)
            for (j = 0; j < d; ++j) {
                const int64_t e = (b * d + i) * d + j;
                C_out[e] = f[i] * C_in[e] + fc[i] * (h[i] * h[j]);
            }
        free(concat);
        free(f);
        free(fc);
    }
}
