/*
 * tpo.h -- plain float64 CPU oracle for one Megatron tensor-parallel layer shard.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header or constant with the HIP library and must never sit on the
 * product path.
 *
 * What it computes (all matrices row-major, oriented [in, out] as in x*W):
 *   - the FFN shard of "How transformer layers actually decompose" (page
 *     "Megatron-LM: what the tensor parallelism paper actually says"):
 *     output = GeLU(x W1) W2 with W1 (here A, [h, F]) split by columns and
 *     W2 (here B, [F, h]) split by rows; shard i gives a partial sum;
 *   - the attention shard of "The attention heads split" on the same page:
 *     Q/K/V [h, h] split by the columns of the shard's H/t heads, per-head
 *     softmax attention, output projection Wo [h, h] split by rows;
 *   - the backward of both by the chain rule, and separately coded
 *     unsharded layers for the "partials sum to the full result" check.
 *
 * Readings where the pages are silent: exact erf GeLU, scale 1/sqrt(d),
 * causal mask m <= j (or none), column-parallel biases (b1, bq, bk, bv)
 * added inside the shard, row-parallel biases (b2, bo) added once after
 * the sum (only the unsharded functions take them), LSE = natural log.
 *
 * Every function returns 0 on success and a negative value on a shape error.
 * Outputs are overwritten, never accumulated.
 */
#ifndef TPO_H
#define TPO_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    long batch, seq, hidden, heads, ffn;
    int causal; /* 1: key m allowed for query j iff m <= j; 0: all keys */
    int gelu;   /* FFN activation: 0 the exact GeLU u * Phi(u), 1 its tanh approximation */
} tpo_dims;

/* GeLU(u) = u * Phi(u) and its derivative Phi(u) + u * phi(u), elementwise. */
void tpo_gelu(const double* u, double* y, long n);
void tpo_gelu_prime(const double* u, double* g, long n);
/* The tanh approximation 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) and its derivative. */
void tpo_gelu_tanh(const double* u, double* y, long n);
void tpo_gelu_tanh_prime(const double* u, double* g, long n);

/* ---- FFN (MLP) shard -------------------------------------------------- */
/* X [T,h], A [h,F], b1 [F] or NULL, B [F,h].
 * Out: Z_part [T,h] (b2 not added), U and Y [T,F/t] (pre/post GeLU), may be NULL. */
int tpo_mlp_shard_fwd(const tpo_dims* d, int shard, int degree,
                      const double* X, const double* A, const double* b1, const double* B,
                      double* Z_part, double* U, double* Y);
/* G = dZ [T,h].  Out: dX_part [T,h]; dA [h,F], db1 [F], dB [F,h] are full-size
 * buffers of which only the shard's block (A columns, b1 entries, B rows) is written. */
int tpo_mlp_shard_bwd(const tpo_dims* d, int shard, int degree,
                      const double* X, const double* A, const double* b1, const double* B,
                      const double* G,
                      double* dX_part, double* dA, double* db1, double* dB);

/* ---- attention shard ---------------------------------------------------- */
/* X [T,h], Wq/Wk/Wv/Wo [h,h], bq/bk/bv [h] or NULL.
 * Out: Z_part [T,h] (bo not added); Q, K, V, O [T,w] token-major with
 * w = (H/t)*d (column j = local head j/d, dim j%d); lse [batch, H/t, seq].
 * Q..lse may be NULL. */
int tpo_attn_shard_fwd(const tpo_dims* d, int shard, int degree,
                       const double* X, const double* Wq, const double* Wk, const double* Wv,
                       const double* bq, const double* bk, const double* bv, const double* Wo,
                       double* Z_part, double* Q, double* K, double* V, double* O, double* lse);
/* Out: dX_part [T,h]; dWq/dWk/dWv [h,h] (shard's columns), dbq/dbk/dbv [h]
 * (shard's entries, may be NULL), dWo [h,h] (shard's rows). */
int tpo_attn_shard_bwd(const tpo_dims* d, int shard, int degree,
                       const double* X, const double* Wq, const double* Wk, const double* Wv,
                       const double* bq, const double* bk, const double* bv, const double* Wo,
                       const double* G,
                       double* dX_part, double* dWq, double* dWk, double* dWv,
                       double* dbq, double* dbk, double* dbv, double* dWo);

/* One head's softmax attention on Q, K, V [s, dh] (row stride ld):
 * P [s,s] (may be NULL), O [s,dh] (row stride ld), lse [s] (may be NULL). */
void tpo_attn_head_fwd(long s, long dh, long ld, int causal,
                       const double* Q, const double* K, const double* V,
                       double* P, double* O, double* lse);

/* ---- unsharded sublayers, coded independently of the shard functions --- */
int tpo_mlp_full_fwd(const tpo_dims* d, const double* X, const double* A, const double* b1,
                     const double* B, const double* b2, double* Z);
int tpo_mlp_full_bwd(const tpo_dims* d, const double* X, const double* A, const double* b1,
                     const double* B, const double* G,
                     double* dX, double* dA, double* db1, double* dB, double* db2);
int tpo_attn_full_fwd(const tpo_dims* d, const double* X,
                      const double* Wq, const double* Wk, const double* Wv,
                      const double* bq, const double* bk, const double* bv,
                      const double* Wo, const double* bo, double* Z);
int tpo_attn_full_bwd(const tpo_dims* d, const double* X,
                      const double* Wq, const double* Wk, const double* Wv,
                      const double* bq, const double* bk, const double* bv,
                      const double* Wo, const double* G,
                      double* dX, double* dWq, double* dWk, double* dWv,
                      double* dbq, double* dbk, double* dbv, double* dWo, double* dbo);

/* ---- pre-LN layer composition (LayerNorm before each sublayer, residual after) */
/* LN(x) = (x - mean) / sqrt(var + eps), biased variance, no affine. */
void tpo_layernorm(long rows, long cols, double eps, const double* x, double* y);
/* The same with the affine part, y = gamma * LN(x) + beta (gamma, beta [cols] or
 * NULL for 1 and 0); the row means and 1/sqrt(var + eps) into mean, rstd [rows]
 * (may be NULL). */
void tpo_layernorm_affine(long rows, long cols, double eps, const double* x, const double* gamma,
                          const double* beta, double* y, double* mean, double* rstd);
/* Its backward: dx [rows,cols] from dy; dgamma, dbeta [cols] (may be NULL). */
void tpo_layernorm_bwd(long rows, long cols, double eps, const double* x, const double* gamma,
                       const double* dy, double* dx, double* dgamma, double* dbeta);

/* Number of OpenMP threads the oracle will use. */
int tpo_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
