/*
 * tpo.c -- plain float64 CPU oracle for one Megatron tensor-parallel layer shard.
 *
 * TEST INFRASTRUCTURE ONLY (see tpo.h).  Straight loops over the
 * definitions, parallelised with OpenMP over independent output rows or
 * (sequence, head) pairs.  No blocking, no fusion, no reordering beyond
 * putting the contiguous index innermost.
 *
 * Sources (page "Megatron-LM: what the tensor parallelism paper actually
 * says"):
 *   - FFN: output = GeLU(x W1) W2, W1 split by columns so GeLU stays local,
 *     W2 split by rows so each shard holds a partial sum that one
 *     all-reduce adds up ("How transformer layers actually decompose").
 *   - Attention: H/N heads per shard, Q/K/V [hidden, hidden] split by the
 *     columns of the shard's heads, output projection split by rows, a
 *     partial output per shard ("The attention heads split").
 *   - The backward is the chain rule through the same steps; the pages
 *     state only that a forward and a backward all-reduce exist (page
 *     "Interactive Paper Explainer", section "One Idea, Two Insertions").
 */
#include "tpo.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int tpo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- GeLU -- */

/* GeLU(u) = u * Phi(u), Phi the standard normal distribution function. */
static double gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }

/* d/du [u * Phi(u)] = Phi(u) + u * phi(u), phi the standard normal density. */
static double gelu_prime(double u)
{
    const double Phi = 0.5 * (1.0 + erf(u / sqrt(2.0)));
    const double phi = exp(-0.5 * u * u) / sqrt(2.0 * acos(-1.0));
    return Phi + u * phi;
}

/* The tanh approximation of GeLU (selected by tpo_dims.gelu = 1):
 * 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3), and its derivative
 * by the chain rule, 0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) dz/du. */
static double gelu_tanh(double u)
{
    const double z = sqrt(2.0 / acos(-1.0)) * (u + 0.044715 * u * u * u);
    return 0.5 * u * (1.0 + tanh(z));
}

static double gelu_tanh_prime(double u)
{
    const double c = sqrt(2.0 / acos(-1.0));
    const double th = tanh(c * (u + 0.044715 * u * u * u));
    const double dz = c * (1.0 + 3.0 * 0.044715 * u * u);
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * dz;
}

/* The FFN activation and its derivative for the form d->gelu selects. */
static double act(const tpo_dims* d, double u) { return d->gelu ? gelu_tanh(u) : gelu(u); }
static double act_prime(const tpo_dims* d, double u) { return d->gelu ? gelu_tanh_prime(u) : gelu_prime(u); }

void tpo_gelu_tanh(const double* u, double* y, long n)
{
    for (long i = 0; i < n; ++i) y[i] = gelu_tanh(u[i]);
}

void tpo_gelu_tanh_prime(const double* u, double* g, long n)
{
    for (long i = 0; i < n; ++i) g[i] = gelu_tanh_prime(u[i]);
}

void tpo_gelu(const double* u, double* y, long n)
{
    for (long i = 0; i < n; ++i) y[i] = gelu(u[i]);
}

void tpo_gelu_prime(const double* u, double* g, long n)
{
    for (long i = 0; i < n; ++i) g[i] = gelu_prime(u[i]);
}

/* ------------------------------------------------------------- checks -- */

static int check_dims(const tpo_dims* d, int shard, int degree)
{
    if (!d || d->batch <= 0 || d->seq <= 0 || d->hidden <= 0 || d->heads <= 0 || d->ffn <= 0)
        return -1;
    if (degree <= 0 || shard < 0 || shard >= degree) return -2;
    if (d->hidden % d->heads) return -3;
    if (d->heads % degree || d->ffn % degree) return -4;
    return 0;
}

static double* zalloc(long n)
{
    double* p = (double*)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    return p;
}

/* ------------------------------------------------------ FFN (MLP) shard -- */

int tpo_mlp_shard_fwd(const tpo_dims* d, int shard, int degree,
                      const double* X, const double* A, const double* b1, const double* B,
                      double* Z_part, double* U, double* Y)
{
    int e = check_dims(d, shard, degree);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, F = d->ffn;
    const long Fs = F / degree, c0 = (long)shard * Fs;

#pragma omp parallel
    {
        double* u = zalloc(Fs);
        double* y = zalloc(Fs);
#pragma omp for schedule(static)
        for (long r = 0; r < T; ++r) {
            /* U[r, c] = sum_k X[r, k] A[k, c0 + c] + b1[c0 + c] */
            for (long c = 0; c < Fs; ++c) u[c] = b1 ? b1[c0 + c] : 0.0;
            for (long k = 0; k < h; ++k) {
                const double x = X[r * h + k];
                const double* a = A + k * F + c0;
                for (long c = 0; c < Fs; ++c) u[c] += x * a[c];
            }
            for (long c = 0; c < Fs; ++c) y[c] = act(d, u[c]);
            if (U) memcpy(U + r * Fs, u, (size_t)Fs * sizeof(double));
            if (Y) memcpy(Y + r * Fs, y, (size_t)Fs * sizeof(double));
            /* Z_part[r, n] = sum_c Y[r, c] B[c0 + c, n] */
            if (Z_part) {
                double* z = Z_part + r * h;
                for (long n = 0; n < h; ++n) z[n] = 0.0;
                for (long c = 0; c < Fs; ++c) {
                    const double yc = y[c];
                    const double* b = B + (c0 + c) * h;
                    for (long n = 0; n < h; ++n) z[n] += yc * b[n];
                }
            }
        }
        free(u);
        free(y);
    }
    return 0;
}

int tpo_mlp_shard_bwd(const tpo_dims* d, int shard, int degree,
                      const double* X, const double* A, const double* b1, const double* B,
                      const double* G,
                      double* dX_part, double* dA, double* db1, double* dB)
{
    int e = check_dims(d, shard, degree);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, F = d->ffn;
    const long Fs = F / degree, c0 = (long)shard * Fs;

    double* U = zalloc(T * Fs);
    double* Y = zalloc(T * Fs);
    double* dU = zalloc(T * Fs);
    if (!U || !Y || !dU) { free(U); free(Y); free(dU); return -9; }
    tpo_mlp_shard_fwd(d, shard, degree, X, A, b1, B, NULL, U, Y);

    /* dY[r, c] = sum_n G[r, n] B[c0 + c, n];  dU = dY * GeLU'(U) */
#pragma omp parallel for schedule(static)
    for (long r = 0; r < T; ++r) {
        const double* g = G + r * h;
        for (long c = 0; c < Fs; ++c) {
            const double* b = B + (c0 + c) * h;
            double s = 0.0;
            for (long n = 0; n < h; ++n) s += g[n] * b[n];
            dU[r * Fs + c] = s * act_prime(d, U[r * Fs + c]);
        }
    }

    /* dB[c0 + c, n] = sum_r Y[r, c] G[r, n] */
    if (dB) {
#pragma omp parallel for schedule(static)
        for (long c = 0; c < Fs; ++c) {
            double* row = dB + (c0 + c) * h;
            for (long n = 0; n < h; ++n) row[n] = 0.0;
            for (long r = 0; r < T; ++r) {
                const double y = Y[r * Fs + c];
                const double* g = G + r * h;
                for (long n = 0; n < h; ++n) row[n] += y * g[n];
            }
        }
    }

    /* dA[k, c0 + c] = sum_r X[r, k] dU[r, c] */
    if (dA) {
#pragma omp parallel for schedule(static)
        for (long k = 0; k < h; ++k) {
            double* row = dA + k * F + c0;
            for (long c = 0; c < Fs; ++c) row[c] = 0.0;
            for (long r = 0; r < T; ++r) {
                const double x = X[r * h + k];
                const double* du = dU + r * Fs;
                for (long c = 0; c < Fs; ++c) row[c] += x * du[c];
            }
        }
    }

    /* db1[c0 + c] = sum_r dU[r, c] */
    if (db1) {
        for (long c = 0; c < Fs; ++c) db1[c0 + c] = 0.0;
        for (long r = 0; r < T; ++r)
            for (long c = 0; c < Fs; ++c) db1[c0 + c] += dU[r * Fs + c];
    }

    /* dX_part[r, k] = sum_c dU[r, c] A[k, c0 + c] */
    if (dX_part) {
#pragma omp parallel for schedule(static)
        for (long r = 0; r < T; ++r) {
            const double* du = dU + r * Fs;
            for (long k = 0; k < h; ++k) {
                const double* a = A + k * F + c0;
                double s = 0.0;
                for (long c = 0; c < Fs; ++c) s += du[c] * a[c];
                dX_part[r * h + k] = s;
            }
        }
    }
    free(U);
    free(Y);
    free(dU);
    return 0;
}

/* ------------------------------------------------------ attention head -- */

void tpo_attn_head_fwd(long s, long dh, long ld, int causal,
                       const double* Q, const double* K, const double* V,
                       double* P, double* O, double* lse)
{
    const double scale = 1.0 / sqrt((double)dh);
    double* row = zalloc(s);
    for (long j = 0; j < s; ++j) {
        const long nk = causal ? j + 1 : s; /* keys 0 .. nk-1 are allowed */
        /* S[j, m] = Q[j] . K[m] / sqrt(d) */
        double mx = -INFINITY;
        for (long m = 0; m < nk; ++m) {
            double acc = 0.0;
            for (long c = 0; c < dh; ++c) acc += Q[j * ld + c] * K[m * ld + c];
            row[m] = acc * scale;
            if (row[m] > mx) mx = row[m];
        }
        /* P[j, m] = exp(S[j, m] - max) / sum over allowed m' */
        double sum = 0.0;
        for (long m = 0; m < nk; ++m) {
            row[m] = exp(row[m] - mx);
            sum += row[m];
        }
        for (long m = 0; m < nk; ++m) row[m] /= sum;
        for (long m = nk; m < s; ++m) row[m] = 0.0;
        if (P) memcpy(P + j * s, row, (size_t)s * sizeof(double));
        if (lse) lse[j] = mx + log(sum);
        /* O[j] = sum_m P[j, m] V[m] */
        if (O) {
            for (long c = 0; c < dh; ++c) O[j * ld + c] = 0.0;
            for (long m = 0; m < nk; ++m) {
                const double p = row[m];
                for (long c = 0; c < dh; ++c) O[j * ld + c] += p * V[m * ld + c];
            }
        }
    }
    free(row);
}

/* Backward of one head, given dO; recomputes P.  dS is formed directly as
 * dS[j, m] = P[j, m] (dP[j, m] - sum_m' P[j, m'] dP[j, m']). */
static void attn_head_bwd(long s, long dh, long ld, int causal,
                          const double* Q, const double* K, const double* V, const double* dO,
                          double* dQ, double* dK, double* dV)
{
    const double scale = 1.0 / sqrt((double)dh);
    double* P = zalloc(s * s);
    double* dS = zalloc(s * s);
    tpo_attn_head_fwd(s, dh, ld, causal, Q, K, V, P, NULL, NULL);

    /* dV[m] = sum_j P[j, m] dO[j] */
    for (long m = 0; m < s; ++m)
        for (long c = 0; c < dh; ++c) dV[m * ld + c] = 0.0;
    for (long j = 0; j < s; ++j)
        for (long m = 0; m < s; ++m) {
            const double p = P[j * s + m];
            if (p == 0.0) continue;
            for (long c = 0; c < dh; ++c) dV[m * ld + c] += p * dO[j * ld + c];
        }

    /* dP[j, m] = dO[j] . V[m];  dS = P * (dP - rowsum(P * dP)) */
    for (long j = 0; j < s; ++j) {
        double rs = 0.0;
        for (long m = 0; m < s; ++m) {
            double dp = 0.0;
            for (long c = 0; c < dh; ++c) dp += dO[j * ld + c] * V[m * ld + c];
            dS[j * s + m] = dp;
            rs += P[j * s + m] * dp;
        }
        for (long m = 0; m < s; ++m) dS[j * s + m] = P[j * s + m] * (dS[j * s + m] - rs);
    }

    /* dQ[j] = sum_m dS[j, m] K[m] / sqrt(d);  dK[m] = sum_j dS[j, m] Q[j] / sqrt(d) */
    for (long j = 0; j < s; ++j)
        for (long c = 0; c < dh; ++c) {
            double acc = 0.0;
            for (long m = 0; m < s; ++m) acc += dS[j * s + m] * K[m * ld + c];
            dQ[j * ld + c] = acc * scale;
        }
    for (long m = 0; m < s; ++m)
        for (long c = 0; c < dh; ++c) {
            double acc = 0.0;
            for (long j = 0; j < s; ++j) acc += dS[j * s + m] * Q[j * ld + c];
            dK[m * ld + c] = acc * scale;
        }
    free(P);
    free(dS);
}

/* ----------------------------------------------------- attention shard -- */

/* Q/K/V[r, j] = sum_k X[r, k] W[k, col0 + j] + b[col0 + j] for the shard's w columns. */
static void project_cols(long T, long h, long w, long col0, const double* X,
                         const double* W, const double* b, double* out)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < T; ++r) {
        double* o = out + r * w;
        for (long j = 0; j < w; ++j) o[j] = b ? b[col0 + j] : 0.0;
        for (long k = 0; k < h; ++k) {
            const double x = X[r * h + k];
            const double* wr = W + k * h + col0;
            for (long j = 0; j < w; ++j) o[j] += x * wr[j];
        }
    }
}

int tpo_attn_shard_fwd(const tpo_dims* d, int shard, int degree,
                       const double* X, const double* Wq, const double* Wk, const double* Wv,
                       const double* bq, const double* bk, const double* bv, const double* Wo,
                       double* Z_part, double* Q, double* K, double* V, double* O, double* lse)
{
    int e = check_dims(d, shard, degree);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, s = d->seq, nb = d->batch;
    const long Hs = d->heads / degree, dh = h / d->heads, w = Hs * dh;
    const long col0 = (long)shard * w;

    double* q = Q ? Q : zalloc(T * w);
    double* k = K ? K : zalloc(T * w);
    double* v = V ? V : zalloc(T * w);
    double* o = O ? O : zalloc(T * w);
    project_cols(T, h, w, col0, X, Wq, bq, q);
    project_cols(T, h, w, col0, X, Wk, bk, k);
    project_cols(T, h, w, col0, X, Wv, bv, v);

#pragma omp parallel for schedule(dynamic, 1)
    for (long bg = 0; bg < nb * Hs; ++bg) {
        const long b = bg / Hs, g = bg % Hs;
        const long off = b * s * w + g * dh;
        tpo_attn_head_fwd(s, dh, w, d->causal, q + off, k + off, v + off, NULL, o + off,
                          lse ? lse + (b * Hs + g) * s : NULL);
    }

    /* Z_part[r, n] = sum_j O[r, j] Wo[col0 + j, n] */
    if (Z_part) {
#pragma omp parallel for schedule(static)
        for (long r = 0; r < T; ++r) {
            double* z = Z_part + r * h;
            for (long n = 0; n < h; ++n) z[n] = 0.0;
            for (long j = 0; j < w; ++j) {
                const double oj = o[r * w + j];
                const double* wo = Wo + (col0 + j) * h;
                for (long n = 0; n < h; ++n) z[n] += oj * wo[n];
            }
        }
    }
    if (!Q) free(q);
    if (!K) free(k);
    if (!V) free(v);
    if (!O) free(o);
    return 0;
}

/* dW[k, col0 + j] = sum_r X[r, k] dP[r, j];  db[col0 + j] = sum_r dP[r, j] */
static void wgrad_cols(long T, long h, long w, long col0, const double* X,
                       const double* dP, double* dW, double* db)
{
#pragma omp parallel for schedule(static)
    for (long k = 0; k < h; ++k) {
        double* row = dW + k * h + col0;
        for (long j = 0; j < w; ++j) row[j] = 0.0;
        for (long r = 0; r < T; ++r) {
            const double x = X[r * h + k];
            const double* g = dP + r * w;
            for (long j = 0; j < w; ++j) row[j] += x * g[j];
        }
    }
    if (db) {
        for (long j = 0; j < w; ++j) db[col0 + j] = 0.0;
        for (long r = 0; r < T; ++r)
            for (long j = 0; j < w; ++j) db[col0 + j] += dP[r * w + j];
    }
}

int tpo_attn_shard_bwd(const tpo_dims* d, int shard, int degree,
                       const double* X, const double* Wq, const double* Wk, const double* Wv,
                       const double* bq, const double* bk, const double* bv, const double* Wo,
                       const double* G,
                       double* dX_part, double* dWq, double* dWk, double* dWv,
                       double* dbq, double* dbk, double* dbv, double* dWo)
{
    int e = check_dims(d, shard, degree);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, s = d->seq, nb = d->batch;
    const long Hs = d->heads / degree, dh = h / d->heads, w = Hs * dh;
    const long col0 = (long)shard * w;

    double* q = zalloc(T * w);
    double* k = zalloc(T * w);
    double* v = zalloc(T * w);
    double* o = zalloc(T * w);
    double* dO = zalloc(T * w);
    double* dq = zalloc(T * w);
    double* dk = zalloc(T * w);
    double* dv = zalloc(T * w);
    tpo_attn_shard_fwd(d, shard, degree, X, Wq, Wk, Wv, bq, bk, bv, Wo, NULL, q, k, v, o, NULL);

    /* dWo[col0 + j, n] = sum_r O[r, j] G[r, n] */
    if (dWo) {
#pragma omp parallel for schedule(static)
        for (long j = 0; j < w; ++j) {
            double* row = dWo + (col0 + j) * h;
            for (long n = 0; n < h; ++n) row[n] = 0.0;
            for (long r = 0; r < T; ++r) {
                const double oj = o[r * w + j];
                const double* g = G + r * h;
                for (long n = 0; n < h; ++n) row[n] += oj * g[n];
            }
        }
    }
    /* dO[r, j] = sum_n G[r, n] Wo[col0 + j, n] */
#pragma omp parallel for schedule(static)
    for (long r = 0; r < T; ++r)
        for (long j = 0; j < w; ++j) {
            const double* wo = Wo + (col0 + j) * h;
            double acc = 0.0;
            for (long n = 0; n < h; ++n) acc += G[r * h + n] * wo[n];
            dO[r * w + j] = acc;
        }

#pragma omp parallel for schedule(dynamic, 1)
    for (long bg = 0; bg < nb * Hs; ++bg) {
        const long b = bg / Hs, g = bg % Hs;
        const long off = b * s * w + g * dh;
        attn_head_bwd(s, dh, w, d->causal, q + off, k + off, v + off, dO + off,
                      dq + off, dk + off, dv + off);
    }

    if (dWq) wgrad_cols(T, h, w, col0, X, dq, dWq, dbq);
    if (dWk) wgrad_cols(T, h, w, col0, X, dk, dWk, dbk);
    if (dWv) wgrad_cols(T, h, w, col0, X, dv, dWv, dbv);

    /* dX_part[r, k] = sum_j dQ[r, j] Wq[k, col0 + j] + dK.. Wk + dV.. Wv */
    if (dX_part) {
#pragma omp parallel for schedule(static)
        for (long r = 0; r < T; ++r)
            for (long kk = 0; kk < h; ++kk) {
                const double* wq = Wq + kk * h + col0;
                const double* wk = Wk + kk * h + col0;
                const double* wv = Wv + kk * h + col0;
                double acc = 0.0;
                for (long j = 0; j < w; ++j)
                    acc += dq[r * w + j] * wq[j] + dk[r * w + j] * wk[j] + dv[r * w + j] * wv[j];
                dX_part[r * h + kk] = acc;
            }
    }
    free(q); free(k); free(v); free(o);
    free(dO); free(dq); free(dk); free(dv);
    return 0;
}

/* ------------------------------------------------ unsharded sublayers -- */
/* Written as whole-matrix products with a naive matmul, independently of
 * the shard code above, so that "sum of partials == full layer" is a real
 * check of the split. */

/* C[M, N] = A[M, K] B[K, N] with explicit strides; trA/trB read the transpose. */
static void mm(long M, long N, long K, const double* A, long lda, int trA,
               const double* B, long ldb, int trB, double* C, long ldc)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < M; ++i)
        for (long j = 0; j < N; ++j) {
            double acc = 0.0;
            for (long k = 0; k < K; ++k) {
                const double a = trA ? A[k * lda + i] : A[i * lda + k];
                const double b = trB ? B[j * ldb + k] : B[k * ldb + j];
                acc += a * b;
            }
            C[i * ldc + j] = acc;
        }
}

int tpo_mlp_full_fwd(const tpo_dims* d, const double* X, const double* A, const double* b1,
                     const double* B, const double* b2, double* Z)
{
    int e = check_dims(d, 0, 1);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, F = d->ffn;
    double* H1 = zalloc(T * F);
    mm(T, F, h, X, h, 0, A, F, 0, H1, F);
    for (long r = 0; r < T; ++r)
        for (long c = 0; c < F; ++c) H1[r * F + c] = act(d, H1[r * F + c] + (b1 ? b1[c] : 0.0));
    mm(T, h, F, H1, F, 0, B, h, 0, Z, h);
    if (b2)
        for (long r = 0; r < T; ++r)
            for (long n = 0; n < h; ++n) Z[r * h + n] += b2[n];
    free(H1);
    return 0;
}

int tpo_mlp_full_bwd(const tpo_dims* d, const double* X, const double* A, const double* b1,
                     const double* B, const double* G,
                     double* dX, double* dA, double* db1, double* dB, double* db2)
{
    int e = check_dims(d, 0, 1);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, F = d->ffn;
    double* Pre = zalloc(T * F);
    double* Act = zalloc(T * F);
    double* dAct = zalloc(T * F);
    mm(T, F, h, X, h, 0, A, F, 0, Pre, F);
    for (long r = 0; r < T; ++r)
        for (long c = 0; c < F; ++c) {
            Pre[r * F + c] += b1 ? b1[c] : 0.0;
            Act[r * F + c] = act(d, Pre[r * F + c]);
        }
    mm(F, h, T, Act, F, 1, G, h, 0, dB, h);          /* dB = Act^T G */
    mm(T, F, h, G, h, 0, B, h, 1, dAct, F);          /* dAct = G B^T */
    for (long i = 0; i < T * F; ++i) dAct[i] *= act_prime(d, Pre[i]);
    mm(h, F, T, X, h, 1, dAct, F, 0, dA, F);         /* dA = X^T dPre */
    mm(T, h, F, dAct, F, 0, A, F, 1, dX, h);         /* dX = dPre A^T */
    if (db1)
        for (long c = 0; c < F; ++c) {
            double acc = 0.0;
            for (long r = 0; r < T; ++r) acc += dAct[r * F + c];
            db1[c] = acc;
        }
    if (db2)
        for (long n = 0; n < h; ++n) {
            double acc = 0.0;
            for (long r = 0; r < T; ++r) acc += G[r * h + n];
            db2[n] = acc;
        }
    free(Pre);
    free(Act);
    free(dAct);
    return 0;
}

/* Full multi-head attention over all H heads: softmax per row, then P V. */
static void full_attn_core(const tpo_dims* d, const double* Qf, const double* Kf,
                           const double* Vf, double* Of, double* Pall)
{
    const long s = d->seq, h = d->hidden, H = d->heads, dh = h / H, nb = d->batch;
    const double scale = 1.0 / sqrt((double)dh);
#pragma omp parallel for schedule(dynamic, 1)
    for (long bg = 0; bg < nb * H; ++bg) {
        const long b = bg / H, g = bg % H;
        double* P = Pall + bg * s * s;
        for (long j = 0; j < s; ++j) {
            const double* qj = Qf + (b * s + j) * h + g * dh;
            double mx = -INFINITY, sum = 0.0;
            for (long m = 0; m < s; ++m) {
                if (d->causal && m > j) { P[j * s + m] = -INFINITY; continue; }
                const double* km = Kf + (b * s + m) * h + g * dh;
                double acc = 0.0;
                for (long c = 0; c < dh; ++c) acc += qj[c] * km[c];
                P[j * s + m] = acc * scale;
                if (P[j * s + m] > mx) mx = P[j * s + m];
            }
            for (long m = 0; m < s; ++m) {
                const double ex = (P[j * s + m] == -INFINITY) ? 0.0 : exp(P[j * s + m] - mx);
                P[j * s + m] = ex;
                sum += ex;
            }
            for (long m = 0; m < s; ++m) P[j * s + m] /= sum;
            double* oj = Of + (b * s + j) * h + g * dh;
            for (long c = 0; c < dh; ++c) {
                double acc = 0.0;
                for (long m = 0; m < s; ++m) acc += P[j * s + m] * Vf[(b * s + m) * h + g * dh + c];
                oj[c] = acc;
            }
        }
    }
}

static void add_bias_rows(long T, long n, double* M, const double* b)
{
    if (!b) return;
    for (long r = 0; r < T; ++r)
        for (long c = 0; c < n; ++c) M[r * n + c] += b[c];
}

int tpo_attn_full_fwd(const tpo_dims* d, const double* X,
                      const double* Wq, const double* Wk, const double* Wv,
                      const double* bq, const double* bk, const double* bv,
                      const double* Wo, const double* bo, double* Z)
{
    int e = check_dims(d, 0, 1);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, s = d->seq;
    double* Qf = zalloc(T * h);
    double* Kf = zalloc(T * h);
    double* Vf = zalloc(T * h);
    double* Of = zalloc(T * h);
    double* Pall = zalloc(d->batch * d->heads * s * s);
    mm(T, h, h, X, h, 0, Wq, h, 0, Qf, h); add_bias_rows(T, h, Qf, bq);
    mm(T, h, h, X, h, 0, Wk, h, 0, Kf, h); add_bias_rows(T, h, Kf, bk);
    mm(T, h, h, X, h, 0, Wv, h, 0, Vf, h); add_bias_rows(T, h, Vf, bv);
    full_attn_core(d, Qf, Kf, Vf, Of, Pall);
    mm(T, h, h, Of, h, 0, Wo, h, 0, Z, h); add_bias_rows(T, h, Z, bo);
    free(Qf); free(Kf); free(Vf); free(Of); free(Pall);
    return 0;
}

/* Backward of the full sublayer.  Uses the identity
 * sum_m' P[j, m'] dP[j, m'] = dO[j] . O[j], a different route from the
 * shard code's direct row sum. */
int tpo_attn_full_bwd(const tpo_dims* d, const double* X,
                      const double* Wq, const double* Wk, const double* Wv,
                      const double* bq, const double* bk, const double* bv,
                      const double* Wo, const double* G,
                      double* dX, double* dWq, double* dWk, double* dWv,
                      double* dbq, double* dbk, double* dbv, double* dWo, double* dbo)
{
    int e = check_dims(d, 0, 1);
    if (e) return e;
    const long T = d->batch * d->seq, h = d->hidden, s = d->seq, H = d->heads, dh = h / H;
    const long nb = d->batch;
    const double scale = 1.0 / sqrt((double)dh);
    double* Qf = zalloc(T * h);
    double* Kf = zalloc(T * h);
    double* Vf = zalloc(T * h);
    double* Of = zalloc(T * h);
    double* dOf = zalloc(T * h);
    double* dQf = zalloc(T * h);
    double* dKf = zalloc(T * h);
    double* dVf = zalloc(T * h);
    double* Pall = zalloc(nb * H * s * s);
    double* tmp = zalloc(T * h);
    mm(T, h, h, X, h, 0, Wq, h, 0, Qf, h); add_bias_rows(T, h, Qf, bq);
    mm(T, h, h, X, h, 0, Wk, h, 0, Kf, h); add_bias_rows(T, h, Kf, bk);
    mm(T, h, h, X, h, 0, Wv, h, 0, Vf, h); add_bias_rows(T, h, Vf, bv);
    full_attn_core(d, Qf, Kf, Vf, Of, Pall);

    mm(h, h, T, Of, h, 1, G, h, 0, dWo, h);     /* dWo = O^T G */
    mm(T, h, h, G, h, 0, Wo, h, 1, dOf, h);     /* dO = G Wo^T */
    if (dbo)
        for (long n = 0; n < h; ++n) {
            double acc = 0.0;
            for (long r = 0; r < T; ++r) acc += G[r * h + n];
            dbo[n] = acc;
        }

#pragma omp parallel for schedule(dynamic, 1)
    for (long bg = 0; bg < nb * H; ++bg) {
        const long b = bg / H, g = bg % H;
        const double* P = Pall + bg * s * s;
        for (long j = 0; j < s; ++j) {
            const long rj = (b * s + j) * h + g * dh;
            double Dj = 0.0; /* dO[j] . O[j] */
            for (long c = 0; c < dh; ++c) Dj += dOf[rj + c] * Of[rj + c];
            for (long m = 0; m < s; ++m) {
                const double p = P[j * s + m];
                if (p == 0.0) continue;
                const long rm = (b * s + m) * h + g * dh;
                double dp = 0.0;
                for (long c = 0; c < dh; ++c) dp += dOf[rj + c] * Vf[rm + c];
                const double ds = p * (dp - Dj) * scale;
                for (long c = 0; c < dh; ++c) {
                    dVf[rm + c] += p * dOf[rj + c];
                    dQf[rj + c] += ds * Kf[rm + c];
                    dKf[rm + c] += ds * Qf[rj + c];
                }
            }
        }
    }

    mm(h, h, T, X, h, 1, dQf, h, 0, dWq, h);
    mm(h, h, T, X, h, 1, dKf, h, 0, dWk, h);
    mm(h, h, T, X, h, 1, dVf, h, 0, dWv, h);
    double* bsum[3] = {dbq, dbk, dbv};
    const double* dsrc[3] = {dQf, dKf, dVf};
    for (int z = 0; z < 3; ++z)
        if (bsum[z])
            for (long n = 0; n < h; ++n) {
                double acc = 0.0;
                for (long r = 0; r < T; ++r) acc += dsrc[z][r * h + n];
                bsum[z][n] = acc;
            }
    mm(T, h, h, dQf, h, 0, Wq, h, 1, dX, h);
    mm(T, h, h, dKf, h, 0, Wk, h, 1, tmp, h);
    for (long i = 0; i < T * h; ++i) dX[i] += tmp[i];
    mm(T, h, h, dVf, h, 0, Wv, h, 1, tmp, h);
    for (long i = 0; i < T * h; ++i) dX[i] += tmp[i];

    free(Qf); free(Kf); free(Vf); free(Of); free(dOf);
    free(dQf); free(dKf); free(dVf); free(Pall); free(tmp);
    return 0;
}

/* -------------------------------------------------------- LayerNorm -- */

void tpo_layernorm(long rows, long cols, double eps, const double* x, double* y)
{
    tpo_layernorm_affine(rows, cols, eps, x, NULL, NULL, y, NULL, NULL);
}

/* Row r: mean = (1/n) sum_c x[r,c], var = (1/n) sum_c (x[r,c] - mean)^2 (biased),
 * rstd = 1/sqrt(var + eps), y[r,c] = gamma[c] * (x[r,c] - mean) * rstd + beta[c]. */
void tpo_layernorm_affine(long rows, long cols, double eps, const double* x, const double* gamma,
                          const double* beta, double* y, double* mean_out, double* rstd_out)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const double* xr = x + r * cols;
        double mean = 0.0, var = 0.0;
        for (long c = 0; c < cols; ++c) mean += xr[c];
        mean /= (double)cols;
        for (long c = 0; c < cols; ++c) var += (xr[c] - mean) * (xr[c] - mean);
        var /= (double)cols;
        const double rstd = 1.0 / sqrt(var + eps);
        for (long c = 0; c < cols; ++c) {
            const double xhat = (xr[c] - mean) * rstd;
            y[r * cols + c] = (gamma ? gamma[c] : 1.0) * xhat + (beta ? beta[c] : 0.0);
        }
        if (mean_out) mean_out[r] = mean;
        if (rstd_out) rstd_out[r] = rstd;
    }
}

/* Chain rule through the row's normalisation, with g = dy * gamma:
 *   dx[c] = rstd * (g[c] - (1/n) sum_k g[k] - xhat[c] * (1/n) sum_k g[k] xhat[k]),
 * the terms coming from xhat's direct dependence on x[c], from the mean and
 * from the variance.  dgamma[c] = sum_r dy[r,c] xhat[r,c], dbeta[c] = sum_r dy[r,c]. */
void tpo_layernorm_bwd(long rows, long cols, double eps, const double* x, const double* gamma,
                       const double* dy, double* dx, double* dgamma, double* dbeta)
{
    double* xh = (double*)malloc(sizeof(double) * (size_t)(rows * cols));
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const double* xr = x + r * cols;
        const double* gr = dy + r * cols;
        double mean = 0.0, var = 0.0;
        for (long c = 0; c < cols; ++c) mean += xr[c];
        mean /= (double)cols;
        for (long c = 0; c < cols; ++c) var += (xr[c] - mean) * (xr[c] - mean);
        var /= (double)cols;
        const double rstd = 1.0 / sqrt(var + eps);
        double sg = 0.0, sgx = 0.0;
        for (long c = 0; c < cols; ++c) {
            const double xhat = (xr[c] - mean) * rstd;
            const double g = gr[c] * (gamma ? gamma[c] : 1.0);
            xh[r * cols + c] = xhat;
            sg += g;
            sgx += g * xhat;
        }
        sg /= (double)cols;
        sgx /= (double)cols;
        for (long c = 0; c < cols; ++c) {
            const double g = gr[c] * (gamma ? gamma[c] : 1.0);
            dx[r * cols + c] = rstd * (g - sg - xh[r * cols + c] * sgx);
        }
    }
    if (dgamma || dbeta) {
#pragma omp parallel for schedule(static)
        for (long c = 0; c < cols; ++c) {
            double sgam = 0.0, sbet = 0.0;
            for (long r = 0; r < rows; ++r) {
                sgam += dy[r * cols + c] * xh[r * cols + c];
                sbet += dy[r * cols + c];
            }
            if (dgamma) dgamma[c] = sgam;
            if (dbeta) dbeta[c] = sbet;
        }
    }
    free(xh);
}
