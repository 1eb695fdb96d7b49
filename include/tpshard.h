/*
 * tpshard.h -- C ABI of libtpshard.so: one rank's shard of a Megatron-style
 * tensor-parallel transformer layer, forward and backward, on an MI355X
 * (gfx950) GPU.
 *
 * The operations (page "Megatron-LM: what the tensor parallelism paper
 * actually says"):
 *   - FFN shard, section "How transformer layers actually decompose": the
 *     FFN computes GeLU(x W1) W2 with W1 = A [h, F] split by columns and
 *     W2 = B [F, h] split by rows.  Shard i owns the columns / rows
 *     C_i = [i*F/t, (i+1)*F/t) and produces a partial sum of the output;
 *     the t partials add up to the unsharded FFN output.
 *   - Attention shard, section "The attention heads split": shard i owns
 *     the H/t heads G_i = [i*H/t, (i+1)*H/t); the Q, K, V projections
 *     ([h, h] each) are split by the columns of those heads, each head
 *     runs softmax attention locally, and the output projection Wo [h, h]
 *     is split by the rows of those heads, giving a partial output.
 *   - The backward of both (chain rule).  The input-gradient partials of
 *     the t shards add up to the full input gradient; weight gradients
 *     land in disjoint blocks.
 * On one GPU the cross-shard sum (an all-reduce on a real TP group) is
 * done by tp_sum_partials, for verification.
 *
 * Conventions
 *   - Matrices are row-major and oriented [in, out] as in x*W.  Tokens are
 *     rows: T = batch*seq, token r = b*seq + j.
 *   - Weights are passed as the FULL matrices; the library reads only the
 *     shard's slice (A columns C_i with row stride F, B rows C_i, Wq/Wk/Wv
 *     columns of G_i, Wo rows of G_i).  Head g owns columns [g*d, (g+1)*d),
 *     d = h/H.
 *   - Column-parallel biases (b1, bq, bk, bv) are added inside the shard.
 *     Row-parallel biases (b2, bo) are NOT added by the shard functions
 *     (they would be counted t times); tp_sum_partials adds them once.
 *   - GeLU is the exact form u * Phi(u); attention scores are scaled by
 *     1/sqrt(d); the causal mask allows key m for query j iff m <= j.
 *   - Data types: dims.act = TP_BF16: X, weights, biases, activations,
 *     saved tensors and partial outputs are bfloat16; GEMMs and softmax
 *     accumulate in fp32; weight and bias gradients are fp32.
 *     dims.act = TP_FP16: the same with IEEE half (binary16) storage in place
 *     of bfloat16 (fp16 MFMAs, fp32 accumulation; values are rounded to
 *     nearest even and overflow to +-inf past 65504: the caller scales).
 *     dims.act = TP_FP32: everything is fp32 (fp32 FMA arithmetic).
 *   - Gradients are written (overwritten), never accumulated, into the
 *     shard's block of the full-size caller buffers; entries outside the
 *     block are not touched.
 *   - Ownership: the caller allocates every buffer (device memory),
 *     including `saved` (written by fwd, read by bwd; size from
 *     tp_*_saved_bytes) and `work` (scratch of the backward; size from
 *     tp_*_work_bytes).  The library allocates no device memory; its
 *     mutable global state is the measurement hook (tp_profile_enable) and,
 *     per device, one auxiliary stream with two events (below).
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     legacy default stream) and the call returns without synchronising.
 *     Execution faults surface at the caller's next synchronisation.  The
 *     backward entry points run independent launches (a weight gradient, a
 *     bias column sum) on the device's auxiliary stream (created on first
 *     use, default priority), forked from and joined back to `stream` with
 *     events, so everything a call enqueues precedes later work on `stream`,
 *     also when a launch fails part-way (the auxiliary stream is joined back
 *     on every return); host threads that call them concurrently are
 *     serialised while they enqueue.
 *   - Errors: every argument is validated on the host BEFORE any HIP call
 *     or enqueue; on failure nothing is written and a tp_status is
 *     returned.  A failed launch returns TP_EHIP.  No C++ exception
 *     crosses this boundary.
 *   - Alignment: every device pointer must be 16-byte aligned; hidden,
 *     F/t and (H/t)*d must be multiples of 8.  Supported head dims:
 *     32, 64, 96, 128 (bf16, fp16) and 8..128 in steps of 8 (fp32).
 *   - Size limit: the kernels address operands through 32-bit byte ranges, so
 *     every matrix a shard call touches must be smaller than 2 GiB: [T, h],
 *     [T, F/t] and [T, 3w] in dims.act, and the fp32 gradients [h, F] and
 *     [h, h].  Larger dims are refused with TP_EUNSUPPORTED before any HIP
 *     call (tp_check_dims reports it too).
 *   - Calls on different streams may run concurrently if their output
 *     buffers do not overlap.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_EINVAL = 1,        /* NULL required pointer, non-positive size, NULL dims, bad flag */
    TP_EDIVIDE = 2,       /* t does not divide H or F, or H does not divide h         */
    TP_ESHARD = 3,        /* shard index outside [0, t) or t < 1                      */
    TP_EALIGN = 4,        /* pointer not 16-byte aligned or size not a multiple of 8  */
    TP_EDTYPE = 5,        /* dims.act is not one of TP_FP32, TP_BF16, TP_FP16         */
    TP_EUNSUPPORTED = 6,  /* head dimension not supported, or a matrix of 2 GiB or more */
    TP_EHIP = 7,          /* a kernel launch failed                                   */
    TP_ESIZE = 8,         /* work buffer smaller than tp_*_work_bytes                 */
    TP_ESCRATCH = 9       /* needs more than the no-allocation entry point's scratch  */
} tp_status;

typedef enum { TP_FP32 = 0, TP_BF16 = 1, TP_FP16 = 2 } tp_dtype;

/* GeLU form of the FFN shard.  The pages name only "GeLU"; the default is the
 * exact u * Phi(u) (erf form).  TP_GELU_TANH selects the tanh approximation
 * 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) and its derivative. */
typedef enum { TP_GELU_ERF = 0, TP_GELU_TANH = 1 } tp_gelu;

typedef struct {
    int64_t batch, seq;      /* T = batch * seq tokens                         */
    int64_t hidden;          /* h                                              */
    int64_t heads;           /* H (full, unsharded)                            */
    int64_t ffn;             /* F (full, unsharded; 4h in the pages' models)   */
    int32_t causal;          /* 1: causal mask, 0: none                        */
    int32_t act;             /* tp_dtype of activations / weights / partials   */
    int32_t gelu;            /* tp_gelu (0, the erf form, when zero-filled)    */
} tp_dims;

/* Library version (major * 10000 + minor * 100 + patch). */
int tp_version(void);

/* Human-readable text of a tp_status (static storage, never NULL). */
const char* tp_status_string(int status);

/*
 * Validate dims / shard / degree only (no pointers, no HIP call).
 * Returns TP_OK or the tp_status the entry points would return.
 */
int tp_check_dims(const tp_dims* dims, int shard, int degree);

/*
 * Bytes of the `saved` buffer.  Layout (each region 256-byte aligned, in
 * this order, elements of dims.act unless noted):
 *   MLP:       Gp [T, F/t] = GeLU'(U) (all the backward needs of the
 *              pre-GeLU U, which is not kept),  Y [T, F/t] = GeLU(U)
 *   attention: QKV [T, 3w] (columns [0,w) = Q, [w,2w) = K, [2w,3w) = V of
 *              the shard's heads, w = (H/t)*d, head-local column c of
 *              local head g at g*d + c), O [T, w], LSE [batch, H/t, seq]
 *              fp32 (natural-log log-sum-exp of each query's scaled scores);
 *              16-bit path with w a multiple of neither 192 nor 256 only:
 *              then Wst [h, 3w] and bst [3w], the shard's Wq|Wk|Wv column
 *              slices and bq|bk|bv side by side (a staging copy the forward
 *              makes so that its QKV GEMM takes wide tiles; not read by the
 *              backward)
 * Returns 0 if the dims are invalid.
 */
size_t tp_mlp_saved_bytes(const tp_dims* dims, int shard, int degree);
size_t tp_attn_saved_bytes(const tp_dims* dims, int shard, int degree);

/* Bytes of the `work` buffer the backward needs (0 if the dims are invalid):
 * the backward's intermediates (dU; dO and dQKV), column-sum partials and, for
 * the FFN on the 16-bit path, one fp32 slab the size of its weight gradients,
 * which takes the second half's partial sums when the weight-gradient GEMM
 * splits K in two (the halves are then added in one fixed order: results do not
 * depend on timing). */
size_t tp_mlp_work_bytes(const tp_dims* dims, int shard, int degree);
size_t tp_attn_work_bytes(const tp_dims* dims, int shard, int degree);

/*
 * FFN shard forward ("How transformer layers actually decompose"):
 *   U = X A[:, C_i] + b1[C_i],  Y = GeLU(U),  Z_part = Y B[C_i, :].
 * X [T, h]; A [h, F]; b1 [F] or NULL (zero); B [F, h]; Z_part [T, h] out;
 * saved: see tp_mlp_saved_bytes (Gp = GeLU'(U) and Y, both from the fp32 U).
 */
int tp_mlp_shard_fwd(const tp_dims* dims, int shard, int degree,
                     const void* X, const void* A, const void* b1, const void* B,
                     void* Z_part, void* saved, void* stream);

/*
 * FFN shard backward, given G = dZ [T, h] (the same G reaches every shard):
 *   dY = G B[C_i, :]^T,  dU = dY * GeLU'(U) (the saved Gp),
 *   dB[C_i, :] = Y^T G,  dA[:, C_i] = X^T dU,  db1[C_i] = column sums of dU,
 *   dX_part = dU A[:, C_i]^T.
 * dA [h, F], db1 [F] (NULL: skipped), dB [F, h] are full-size fp32 buffers;
 * only the shard's block is written.  dX_part [T, h] in dims.act.
 * saved: as written by tp_mlp_shard_fwd with the same arguments.
 */
int tp_mlp_shard_bwd(const tp_dims* dims, int shard, int degree,
                     const void* X, const void* A, const void* B,
                     const void* saved, const void* dZ,
                     void* dX_part, float* dA, float* db1, float* dB,
                     void* work, size_t work_bytes, void* stream);

/*
 * FFN shard backward that allocates nothing, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation, kernels and results (bitwise) as
 * tp_mlp_shard_bwd, with no `work` argument.  Its scratch (dU, the column-sum
 * partials and the K-split slab, tp_mlp_work_bytes of them) is a static device
 * array of TP_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends; dims whose tp_mlp_work_bytes exceed it return
 * TP_ESCRATCH before any HIP call (the 8.3B-shape t = 8 shard needs 63.1 MB).  Every launch
 * runs on `stream` (no auxiliary stream, no events); no device or host memory is
 * allocated and no allocating library routine is called (the first call on a
 * device looks up the array's device address once).  All calls on one device
 * share that device's array and each call overwrites it before reading it (no
 * part of it needs to start at zero): calls that overlap in time on one device
 * (two streams, two threads) race on it and must be serialised by the caller.
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int tp_mlp_shard_bwd_noalloc(const tp_dims* dims, int shard, int degree,
                             const void* X, const void* A, const void* B,
                             const void* saved, const void* dZ,
                             void* dX_part, float* dA, float* db1, float* dB, void* stream);

/*
 * Attention shard forward ("The attention heads split"), for every batch
 * element and each local head g of G_i:
 *   Q/K/V = X W{q,k,v}[:, head cols] + b{q,k,v}[head cols],
 *   S = Q K^T / sqrt(d) (+ causal mask), P = row softmax(S), O = P V,
 *   Z_part = O Wo[rows of G_i, :].
 * X [T, h]; Wq, Wk, Wv, Wo [h, h]; bq, bk, bv [h] or NULL; Z_part [T, h] out.
 */
int tp_attn_shard_fwd(const tp_dims* dims, int shard, int degree,
                      const void* X, const void* Wq, const void* Wk, const void* Wv,
                      const void* bq, const void* bk, const void* bv, const void* Wo,
                      void* Z_part, void* saved, void* stream);

/*
 * Attention shard backward, given G = dZ [T, h]:
 *   dWo[rows of G_i] = O^T G, dO = G Wo[rows of G_i]^T,
 *   per head: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 *             dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d),
 *   dW{q,k,v}[:, head cols] = X^T d{Q,K,V}, db{q,k,v} = column sums,
 *   dX_part = dQ Wq[:, cols]^T + dK Wk[:, cols]^T + dV Wv[:, cols]^T.
 * dWq, dWk, dWv, dWo [h, h] and dbq, dbk, dbv [h] (each NULL: all three
 * bias gradients skipped) are full-size fp32 buffers; only the shard's
 * block is written.
 */
int tp_attn_shard_bwd(const tp_dims* dims, int shard, int degree,
                      const void* X, const void* Wq, const void* Wk, const void* Wv,
                      const void* Wo, const void* saved, const void* dZ,
                      void* dX_part, float* dWq, float* dWk, float* dWv,
                      float* dbq, float* dbk, float* dbv, float* dWo,
                      void* work, size_t work_bytes, void* stream);

/*
 * Measurement hook.  Steps of the path, in launch order:
 */
enum {
    TP_STEP_MLP_UP = 0,      /* U = X A_i + b1; GeLU'(U), GeLU(U)   (column-parallel GEMM) */
    TP_STEP_MLP_DOWN = 1,    /* Z_part = Y B_i                      (row-parallel GEMM)    */
    TP_STEP_QKV = 2,         /* QKV = X W{q,k,v}_i + b               (column-parallel GEMM) */
    TP_STEP_ATTN_CORE = 3,   /* softmax attention forward -> O, LSE                          */
    TP_STEP_ATTN_OUT = 4,    /* Z_part = O Wo_i                     (row-parallel GEMM)    */
    TP_STEP_MLP_DU = 5,      /* dU = (dZ B_i^T) * GeLU'(U)  (GeLU'(U) saved by the forward) */
    TP_STEP_MLP_DW = 6,      /* dB_i = Y^T dZ and dA_i = X^T dU (one launch)                */
    TP_STEP_MLP_DB1 = 7,     /* db1_i = column sums of dU                                   */
    TP_STEP_MLP_DX = 8,      /* dX_part = dU A_i^T                                          */
    TP_STEP_ATTN_DO = 9,     /* dO = dZ Wo_i^T                                              */
    TP_STEP_ATTN_CORE_BWD = 10, /* softmax attention backward -> dQ, dK, dV                 */
    TP_STEP_ATTN_DW = 11,    /* dW{q,k,v}_i = X^T d{Q,K,V} and dWo_i = O^T dZ (one launch)  */
    TP_STEP_ATTN_DBIAS = 12, /* db{q,k,v}_i = column sums                                   */
    TP_STEP_ATTN_DX = 13,    /* dX_part = d{Q,K,V} W{q,k,v}_i^T                             */
    TP_STEP_ATTN_DWO = 14,   /* (not recorded: dWo_i is part of the TP_STEP_ATTN_DW launch) */
    TP_NUM_STEPS = 15
};

/*
 * Activation-recompute variants of the backward entry points (page
 * "Megatron-LM: what the tensor parallelism paper actually says", section
 * "What actually limits throughput in production": activation checkpointing
 * recomputes the forward's activations in the backward instead of keeping
 * them).  They take no `saved` buffer: the forward steps whose outputs the
 * backward reads (MLP: GeLU'(U) and Y, one GEMM; attention: QKV and the attention
 * core, O and LSE) run again from X into the front of `work`, then the
 * backward runs exactly as tp_*_shard_bwd, so the results are bitwise those of
 * the saved-activation path.  The caller need not keep `saved` from the
 * forward.  work: tp_*_recompute_work_bytes bytes (the saved layout followed
 * by the backward's work), else TP_ESIZE.  The column-parallel biases are
 * needed again (b1; bq, bk, bv), NULL meaning zero as in the forward.
 */
size_t tp_mlp_recompute_work_bytes(const tp_dims* dims, int shard, int degree);
size_t tp_attn_recompute_work_bytes(const tp_dims* dims, int shard, int degree);
int tp_mlp_shard_bwd_recompute(const tp_dims* dims, int shard, int degree,
                               const void* X, const void* A, const void* b1, const void* B,
                               const void* dZ, void* dX_part, float* dA, float* db1, float* dB,
                               void* work, size_t work_bytes, void* stream);
int tp_attn_shard_bwd_recompute(const tp_dims* dims, int shard, int degree,
                                const void* X, const void* Wq, const void* Wk, const void* Wv,
                                const void* bq, const void* bk, const void* bv, const void* Wo,
                                const void* dZ, void* dX_part,
                                float* dWq, float* dWk, float* dWv,
                                float* dbq, float* dbk, float* dbv, float* dWo,
                                void* work, size_t work_bytes, void* stream);

/*
 * While enabled, every launch of step s is bracketed by
 * hipEventRecord(events[2*(s*npairs + k)], stream) and
 * hipEventRecord(events[2*(s*npairs + k) + 1], stream), where k counts that
 * step's launches modulo npairs.  `events` is a host array of
 * 2*TP_NUM_STEPS*npairs hipEvent_t handles created by the caller and must stay
 * valid until the hook is disabled (events == NULL or npairs == 0).
 * tp_profile_count(s) returns how many launches of step s were recorded, and
 * tp_profile_kernels(s) how many GPU kernels those launches issued in total
 * (a step is one kernel when the two are equal).  Both reset when the hook is
 * enabled or disabled; -1 for a step out of range.
 * For measurement only: the hook is process-wide and not thread-safe.
 */
int tp_profile_enable(void* const* events, int npairs);
int tp_profile_count(int step);
int tp_profile_kernels(int step);

/*
 * Test hook (coverage of every GEMM tile shape against the oracle; no effect on
 * what is computed, only on how it is tiled).  The 16-bit GEMMs pick one of
 * tp_test_gemm_tile_count() tile shapes (and, for the fp32 weight gradients, a
 * K split of 1 or 2) by a cost model.  tp_test_force_gemm_tile(tile, ksplit)
 * makes every later GEMM for which tile `tile` is valid use it (a tile must
 * not straddle a Q|K|V segment; two tiles serve only the fp32 weight
 * gradients), with a K split of 2 where allowed if ksplit == 2; tile == -1
 * restores the cost model.  TP_EINVAL for tile outside [-1, count) or ksplit
 * outside [0, 2].  Process-wide and not thread-safe: for tests only.
 */
int tp_test_force_gemm_tile(int tile, int ksplit);
int tp_test_gemm_tile_count(void);

/*
 * Verification-only local sum that stands in for the all-reduce on one GPU
 * ("To get the correct final output, you sum the partial results"):
 *   out[r, c] = sum_p parts[p][r, c] + (bias ? bias[c] : 0), fp32 out.
 * parts: host array of `nparts` device pointers, each [rows, cols] of
 * `dtype`; bias [cols] of `dtype` or NULL.
 */
int tp_sum_partials(int dtype, int64_t rows, int64_t cols,
                    const void* const* parts, int nparts, const void* bias,
                    float* out, void* stream);

/*
 * The pre-LN residual stream around the shards (page "Megatron-LM: what the
 * tensor parallelism paper actually says", section "The layernorm placement
 * the paper flags as critical": LayerNorm is applied to the residual stream
 * before each sublayer, whose output is added back to the stream).  With
 * h1 = x + sum_i Attn_i(LN1(x)) + bo and out = h1 + sum_i MLP_i(LN2(h1)) + b2,
 * the layer on one GPU is: tp_residual_layernorm (LN1 of x) -> attention shards
 * -> tp_residual_layernorm (h1 and LN2 of it) -> MLP shards ->
 * tp_residual_layernorm (out); backward: MLP shards -> tp_layernorm_bwd (dh1,
 * db2, dbo is its dx_sum) -> attention shards -> tp_layernorm_bwd (dx).
 *
 * tp_residual_layernorm, one workgroup per row:
 *   h[r,c] = residual[r,c] + bias[c] + sum_k parts[k][r,c]   (fp32; into out if
 *            out != NULL; residual, bias may be NULL for 0, nparts may be 0)
 *   y[r,c] = gamma[c] * (h[r,c] - mean_r) * rstd_r + beta[c]  (if y != NULL)
 *   mean_r = (1/cols) sum_c h[r,c], rstd_r = 1/sqrt((1/cols) sum_c (h[r,c] -
 *   mean_r)^2 + eps) (biased variance), stored in mean[r], rstd[r] if non-NULL.
 * parts: host array of `nparts` (<= 16) device pointers to [rows, cols] of
 * `dtype`; bias [cols] of `dtype`; y [rows, cols] of `dtype`; residual, out
 * [rows, cols], gamma, beta [cols] (NULL: 1, 0), mean, rstd [rows]: fp32.  All
 * rows contiguous (row stride cols).  out may alias residual.  At least one of
 * out, y.  cols a multiple of 8 (else TP_EALIGN) and <= 8192 (else
 * TP_EUNSUPPORTED); eps > 0.
 */
int tp_residual_layernorm(int dtype, int64_t rows, int64_t cols,
                          const void* const* parts, int nparts, const void* bias,
                          const float* residual, float* out,
                          const float* gamma, const float* beta, double eps,
                          void* y, float* mean, float* rstd, void* stream);

/*
 * Backward of the LayerNorm y = gamma * (x - mean) * rstd + beta for the
 * gradient g = sum_k dparts[k] of y (the input-gradient partials of the next
 * sublayer's shards), plus a residual gradient:
 *   xhat = (x - mean_r) * rstd_r,  gg = g * gamma
 *   dx[r,c] = dres[r,c] + rstd_r * (gg - (1/cols) sum_c gg - xhat * (1/cols) sum_c gg*xhat)
 * dx (fp32) and, if dx_act != NULL, a copy in `dtype` (the next backward's
 * upstream gradient).  Column sums over rows into the non-NULL ones of:
 * dgamma = sum_r g*xhat, dbeta = sum_r g, dres_sum = sum_r dres,
 * dx_sum = sum_r dx ([cols] fp32).  x fp32 [rows, cols] (the LayerNorm input),
 * mean, rstd as written by tp_residual_layernorm, dres NULL for 0.  work: at
 * least tp_layernorm_bwd_work_bytes(rows, cols) bytes of device memory
 * (else TP_ESIZE).  Same layout and size rules as tp_residual_layernorm;
 * nparts >= 1.  Deterministic (fixed summation orders).
 */
size_t tp_layernorm_bwd_work_bytes(int64_t rows, int64_t cols);
int tp_layernorm_bwd(int dtype, int64_t rows, int64_t cols,
                     const float* x, const float* gamma, const float* mean, const float* rstd,
                     const void* const* dparts, int nparts, const float* dres,
                     float* dx, void* dx_act, float* dgamma, float* dbeta,
                     float* dres_sum, float* dx_sum, void* work, size_t work_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TPSHARD_H */
