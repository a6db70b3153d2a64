/*
 * FLARE / FLARE++ forward operator: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The GPU library
 * never calls it, and the two share no code.
 *
 * Every function works on one (batch, head) problem with fp64 inputs that the
 * caller has widened exactly from the stored fp32 or bf16 values. Loops are
 * written in the order of the definitions; OpenMP only spreads independent
 * rows (latents in the encode, tokens in the decode) over threads, and every
 * sum runs sequentially over its index.
 *
 * Definitions followed (FLARE pages):
 *  - Encode ("2. Implement Encode Stage" of the FLARE skill page; "4. Combine
 *    Encode-Decode into Attention Layer", its encode half): the M latent
 *    queries of a head attend to the N tokens,
 *        l[m][n] = s * <Q[m], K[n]>,  s = 1/sqrt(D),
 *        A_enc[m][n] = softmax over n of l[m][n],
 *        Z[m] = sum_n A_enc[m][n] V[n].
 *  - Decode: the tokens attend back to the latents through the transpose of
 *    the same logits (the "encode-decode factorization" with a token-mixing
 *    matrix of rank at most M, FLARE arXiv abstract),
 *        A_dec[n][m] = softmax over m of l[m][n],
 *        Y[n] = sum_m A_dec[n][m] Z[m].
 *    The FLARE skill page's step 3 instead decodes with separately projected
 *    token queries against Z as keys; the decode follows the transposed-
 *    logit reading (see the readings list of the design notes), and the
 *    page's variant is flare_oracle_attend below.
 *  - FLARE++ (FLARE++ skill page, "Core Mechanism"; FLARE++ arXiv abstract:
 *    the encoder's output corrects the learned queries):
 *        Q' = Q + encode(Q, K, V);  Z = encode(Q', K, V);  Y = decode(Q', K, Z).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double* a, const double* b, int64_t D) {
    double s = 0.0;
    for (int64_t d = 0; d < D; ++d) s += a[d] * b[d];
    return s;
}

/* Encode of one head: Z[M][D] from Q[M][D], K[N][D], V[N][D].
 * Returns 0, or -1 when scratch memory cannot be allocated. */
int flare_oracle_encode(const double* Q, const double* K, const double* V,
                        int64_t N, int64_t M, int64_t D, double* Z) {
    const double s = 1.0 / sqrt((double)D);
    int failed = 0;
#pragma omp parallel
    {
        double* logit = (double*)malloc((size_t)N * sizeof(double));
        if (!logit) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            if (!logit) continue;
            /* logits of latent m against every token, and their maximum */
            double mx = -INFINITY;
            for (int64_t n = 0; n < N; ++n) {
                logit[n] = s * dot(Q + m * D, K + n * D, D);
                if (logit[n] > mx) mx = logit[n];
            }
            /* softmax over the tokens, applied to V */
            double den = 0.0;
            double* z = Z + m * D;
            for (int64_t d = 0; d < D; ++d) z[d] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double e = exp(logit[n] - mx);
                den += e;
                const double* v = V + n * D;
                for (int64_t d = 0; d < D; ++d) z[d] += e * v[d];
            }
            for (int64_t d = 0; d < D; ++d) z[d] /= den;
        }
        free(logit);
    }
    return failed ? -1 : 0;
}

/* Decode of one head for R selected tokens: Y[R][D] from Q[M][D], K[N][D],
 * Z[M][D]; rows[i] names the token of output row i (rows == NULL means all
 * N tokens, R = N). Returns 0, -1 on allocation failure, -2 on a bad row. */
int flare_oracle_decode(const double* Q, const double* K, const double* Z,
                        int64_t N, int64_t M, int64_t D,
                        const int64_t* rows, int64_t R, double* Y) {
    const double s = 1.0 / sqrt((double)D);
    int failed = 0;
#pragma omp parallel
    {
        double* logit = (double*)malloc((size_t)M * sizeof(double));
        if (!logit) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < R; ++i) {
            if (!logit) continue;
            int64_t n = rows ? rows[i] : i;
            if (n < 0 || n >= N) {
#pragma omp atomic write
                failed = 2;
                continue;
            }
            const double* k = K + n * D;
            /* the same logits as the encode, read along the latent axis */
            double mx = -INFINITY;
            for (int64_t m = 0; m < M; ++m) {
                logit[m] = s * dot(Q + m * D, k, D);
                if (logit[m] > mx) mx = logit[m];
            }
            double den = 0.0;
            double* y = Y + i * D;
            for (int64_t d = 0; d < D; ++d) y[d] = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double e = exp(logit[m] - mx);
                den += e;
                const double* z = Z + m * D;
                for (int64_t d = 0; d < D; ++d) y[d] += e * z[d];
            }
            for (int64_t d = 0; d < D; ++d) y[d] /= den;
        }
        free(logit);
    }
    return failed == 1 ? -1 : (failed == 2 ? -2 : 0);
}

/* Token-query decode of one head ("3. Implement Decode Stage" of the FLARE
 * skill page, and the decode half of its step 4): every token's own query
 * q[n] attends to the latent states Z, which serve as keys and values,
 *     l'[n][m] = s * <q[n], Z[m]>,  A[n][m] = softmax over m of l'[n][m],
 *     Y[n] = sum_m A[n][m] Z[m].
 * Y[R][D] from q[N][D] and Z[M][D]; rows as in flare_oracle_decode. */
int flare_oracle_attend(const double* q, const double* Z, int64_t N, int64_t M, int64_t D,
                        const int64_t* rows, int64_t R, double* Y) {
    const double s = 1.0 / sqrt((double)D);
    int failed = 0;
#pragma omp parallel
    {
        double* logit = (double*)malloc((size_t)M * sizeof(double));
        if (!logit) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < R; ++i) {
            if (!logit) continue;
            int64_t n = rows ? rows[i] : i;
            if (n < 0 || n >= N) {
#pragma omp atomic write
                failed = 2;
                continue;
            }
            double mx = -INFINITY;
            for (int64_t m = 0; m < M; ++m) {
                logit[m] = s * dot(q + n * D, Z + m * D, D);
                if (logit[m] > mx) mx = logit[m];
            }
            double den = 0.0;
            double* y = Y + i * D;
            for (int64_t d = 0; d < D; ++d) y[d] = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double e = exp(logit[m] - mx);
                den += e;
                for (int64_t d = 0; d < D; ++d) y[d] += e * Z[m * D + d];
            }
            for (int64_t d = 0; d < D; ++d) y[d] /= den;
        }
        free(logit);
    }
    return failed == 1 ? -1 : (failed == 2 ? -2 : 0);
}

/* FLARE forward of one head: Z = encode(Q, K, V); Y = decode(Q, K, Z).
 * Z_out[M][D] receives Z. */
int flare_oracle_forward(const double* Q, const double* K, const double* V,
                         int64_t N, int64_t M, int64_t D,
                         const int64_t* rows, int64_t R, double* Y, double* Z_out) {
    int rc = flare_oracle_encode(Q, K, V, N, M, D, Z_out);
    if (rc) return rc;
    return flare_oracle_decode(Q, K, Z_out, N, M, D, rows, R, Y);
}

/* FLARE++ forward of one head: Q' = Q + encode(Q, K, V), then the FLARE
 * forward with Q' in place of Q. Qp_out[M][D] receives Q', Z_out[M][D] the
 * second encode's Z. */
int flare_oracle_pp_forward(const double* Q, const double* K, const double* V,
                            int64_t N, int64_t M, int64_t D,
                            const int64_t* rows, int64_t R, double* Y,
                            double* Qp_out, double* Z_out) {
    int rc = flare_oracle_encode(Q, K, V, N, M, D, Qp_out);
    if (rc) return rc;
    for (int64_t i = 0; i < M * D; ++i) Qp_out[i] += Q[i];
    return flare_oracle_forward(Qp_out, K, V, N, M, D, rows, R, Y, Z_out);
}

/* Gradients of one head's FLARE forward (Y = decode(Q, K, encode(Q, K, V)))
 * for an upstream gradient dY[N][D]: dQ[M][D], dK[N][D], dV[N][D]. The
 * forward is the one defined above; the backward is the chain rule through its
 * two softmaxes, written out in fp64 (no algorithmic shortcut):
 *   A[m][n] = softmax_n(l[m][.]),  Z = A V,  Bt[n][m] = softmax_m(l[.][n]),
 *   Y = Bt Z,  l = s Q K^T;
 *   dZ = Bt^T dY,  dV = A^T dZ,
 *   dl[m][n] = A[m][n] (<dZ[m], V[n]> - <dZ[m], Z[m]>)
 *            + Bt[n][m] (<dY[n], Z[m]> - <dY[n], Y[n]>),
 *   dQ = s dl K,  dK = s dl^T Q.
 * (The softmax Jacobian: for p = softmax(x) and an upstream g, dx = p (g -
 * <p, g>); here g is <dZ[m], V[n]> along n for the encode and <dY[n], Z[m]>
 * along m for the decode, and <p, g> is <dZ[m], Z[m]> and <dY[n], Y[n]>.)
 * Returns 0, or -1 when scratch memory cannot be allocated. */
int flare_oracle_backward(const double* Q, const double* K, const double* V, const double* dY,
                          int64_t N, int64_t M, int64_t D, double* dQ, double* dK, double* dV) {
    const double s = 1.0 / sqrt((double)D);
    double* l = (double*)malloc((size_t)M * N * sizeof(double));
    double* A = (double*)malloc((size_t)M * N * sizeof(double));
    double* Bt = (double*)malloc((size_t)M * N * sizeof(double));
    double* Z = (double*)malloc((size_t)M * D * sizeof(double));
    double* Y = (double*)malloc((size_t)N * D * sizeof(double));
    double* dZ = (double*)malloc((size_t)M * D * sizeof(double));
    double* dl = (double*)malloc((size_t)M * N * sizeof(double));
    int rc = 0;
    if (!l || !A || !Bt || !Z || !Y || !dZ || !dl) {
        rc = -1;
        goto done;
    }
    /* forward, keeping the probabilities */
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) l[m * N + n] = s * dot(Q + m * D, K + n * D, D);
    for (int64_t m = 0; m < M; ++m) { /* encode softmax over n */
        double mx = -INFINITY, den = 0.0;
        for (int64_t n = 0; n < N; ++n) mx = fmax(mx, l[m * N + n]);
        for (int64_t n = 0; n < N; ++n) den += (A[m * N + n] = exp(l[m * N + n] - mx));
        for (int64_t n = 0; n < N; ++n) A[m * N + n] /= den;
    }
    for (int64_t n = 0; n < N; ++n) { /* decode softmax over m */
        double mx = -INFINITY, den = 0.0;
        for (int64_t m = 0; m < M; ++m) mx = fmax(mx, l[m * N + n]);
        for (int64_t m = 0; m < M; ++m) den += (Bt[n * M + m] = exp(l[m * N + n] - mx));
        for (int64_t m = 0; m < M; ++m) Bt[n * M + m] /= den;
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t d = 0; d < D; ++d) {
            double z = 0.0;
            for (int64_t n = 0; n < N; ++n) z += A[m * N + n] * V[n * D + d];
            Z[m * D + d] = z;
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t d = 0; d < D; ++d) {
            double y = 0.0;
            for (int64_t m = 0; m < M; ++m) y += Bt[n * M + m] * Z[m * D + d];
            Y[n * D + d] = y;
        }
    /* backward */
    for (int64_t m = 0; m < M; ++m)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t n = 0; n < N; ++n) g += Bt[n * M + m] * dY[n * D + d];
            dZ[m * D + d] = g;
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t m = 0; m < M; ++m) g += A[m * N + n] * dZ[m * D + d];
            dV[n * D + d] = g;
        }
    for (int64_t m = 0; m < M; ++m) {
        const double gz = dot(dZ + m * D, Z + m * D, D);
        for (int64_t n = 0; n < N; ++n) {
            const double gy = dot(dY + n * D, Y + n * D, D);
            dl[m * N + n] = A[m * N + n] * (dot(dZ + m * D, V + n * D, D) - gz) +
                            Bt[n * M + m] * (dot(dY + n * D, Z + m * D, D) - gy);
        }
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t n = 0; n < N; ++n) g += dl[m * N + n] * K[n * D + d];
            dQ[m * D + d] = s * g;
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t m = 0; m < M; ++m) g += dl[m * N + n] * Q[m * D + d];
            dK[n * D + d] = s * g;
        }
done:
    free(l); free(A); free(Bt); free(Z); free(Y); free(dZ); free(dl);
    return rc;
}

/* Gradients of one head's encode alone, Z = encode(Q, K, V) (defined above),
 * for an upstream gradient dZ[M][D]: dQ[M][D], dK[N][D], dV[N][D]. The chain
 * rule through the one softmax, in fp64:
 *   A[m][n] = softmax_n(l[m][.]),  l = s Q K^T,  Z = A V;
 *   dV = A^T dZ,  dl[m][n] = A[m][n] (<dZ[m], V[n]> - <dZ[m], Z[m]>),
 *   dQ = s dl K,  dK = s dl^T Q.
 * Returns 0, or -1 when scratch memory cannot be allocated. */
int flare_oracle_encode_backward(const double* Q, const double* K, const double* V, const double* dZ,
                                 int64_t N, int64_t M, int64_t D, double* dQ, double* dK, double* dV) {
    const double s = 1.0 / sqrt((double)D);
    double* A = (double*)malloc((size_t)M * N * sizeof(double));
    double* Z = (double*)malloc((size_t)M * D * sizeof(double));
    double* dl = (double*)malloc((size_t)M * N * sizeof(double));
    int rc = 0;
    if (!A || !Z || !dl) {
        rc = -1;
        goto done;
    }
    for (int64_t m = 0; m < M; ++m) { /* softmax over n of the logits */
        double mx = -INFINITY, den = 0.0;
        for (int64_t n = 0; n < N; ++n) mx = fmax(mx, s * dot(Q + m * D, K + n * D, D));
        for (int64_t n = 0; n < N; ++n) den += (A[m * N + n] = exp(s * dot(Q + m * D, K + n * D, D) - mx));
        for (int64_t n = 0; n < N; ++n) A[m * N + n] /= den;
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t d = 0; d < D; ++d) {
            double z = 0.0;
            for (int64_t n = 0; n < N; ++n) z += A[m * N + n] * V[n * D + d];
            Z[m * D + d] = z;
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t m = 0; m < M; ++m) g += A[m * N + n] * dZ[m * D + d];
            dV[n * D + d] = g;
        }
    for (int64_t m = 0; m < M; ++m) {
        const double gz = dot(dZ + m * D, Z + m * D, D);
        for (int64_t n = 0; n < N; ++n) dl[m * N + n] = A[m * N + n] * (dot(dZ + m * D, V + n * D, D) - gz);
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t n = 0; n < N; ++n) g += dl[m * N + n] * K[n * D + d];
            dQ[m * D + d] = s * g;
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t m = 0; m < M; ++m) g += dl[m * N + n] * Q[m * D + d];
            dK[n * D + d] = s * g;
        }
done:
    free(A); free(Z); free(dl);
    return rc;
}

/* Gradients of one head's FLARE++ forward (defined above: Q' = Q +
 * encode(Q, K, V), then Y = FLARE(Q', K, V)) for an upstream gradient dY[N][D].
 * The chain rule through the two stages: the FLARE backward with queries Q'
 * gives dQ' and the second stage's dK, dV; the encode backward with dZ = dQ'
 * gives the first stage's; dQ = dQ' + dQ(encode), dK and dV are the sums.
 * Returns 0, or -1 when scratch memory cannot be allocated. */
int flare_oracle_pp_backward(const double* Q, const double* K, const double* V, const double* dY,
                             int64_t N, int64_t M, int64_t D, double* dQ, double* dK, double* dV) {
    double* Qp = (double*)malloc((size_t)M * D * sizeof(double));
    double* dQp = (double*)malloc((size_t)M * D * sizeof(double));
    double* dK1 = (double*)malloc((size_t)N * D * sizeof(double));
    double* dV1 = (double*)malloc((size_t)N * D * sizeof(double));
    int rc = 0;
    if (!Qp || !dQp || !dK1 || !dV1) {
        rc = -1;
        goto done;
    }
    rc = flare_oracle_encode(Q, K, V, N, M, D, Qp);
    if (rc) goto done;
    for (int64_t i = 0; i < M * D; ++i) Qp[i] += Q[i];
    rc = flare_oracle_backward(Qp, K, V, dY, N, M, D, dQp, dK, dV);
    if (rc) goto done;
    rc = flare_oracle_encode_backward(Q, K, V, dQp, N, M, D, dQ, dK1, dV1);
    if (rc) goto done;
    for (int64_t i = 0; i < M * D; ++i) dQ[i] += dQp[i];
    for (int64_t i = 0; i < N * D; ++i) {
        dK[i] += dK1[i];
        dV[i] += dV1[i];
    }
done:
    free(Qp); free(dQp); free(dK1); free(dV1);
    return rc;
}

/* Number of OpenMP threads a parallel region uses (1 without OpenMP). */
int flare_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void flare_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
