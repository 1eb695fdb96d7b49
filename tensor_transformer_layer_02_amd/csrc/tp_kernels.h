// Host-side launch descriptors of the gfx950 kernels (shared by the C-ABI
// implementation and the kernel translation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// Counts every kernel launch the library makes (read by the measurement hook
// to tell single-launch steps apart).
void count_launch();

// Storage formats of activations, weights and partials (the values of tp_dtype).
enum Fmt : int { FMT_F32 = 0, FMT_BF16 = 1, FMT_F16 = 2 };

enum Epi : int {
    EPI_STORE = 0,      // C = acc (act dtype, or fp32 when out_f32)
    EPI_BIAS = 1,       // C = acc + bias[n]
    EPI_BIAS_GELU = 2,  // U = acc + bias[n]; C = Gp = GeLU'(U); C2 = Y = GeLU(U)
    EPI_GELU_BWD = 3,   // C = acc * aux[m, n] (aux: Gp of EPI_BIAS_GELU)
    // C = acc (16-bit), and per row m and head h (columns h rd_dh .. +rd_dh-1):
    // rd[(b rd_heads + h) rd_seq + j] = sum over the head's columns of C[m, n] aux[m, n],
    // m = b rd_seq + j, from the rounded C (the attention backward's D = rowsum(dO * O))
    EPI_STORE_ROWDOT = 4,
};

// C[M, N] (+epilogue) = sum_k A(m, k) B(k, n).
//   A(m, k) = A[m*lda + k]   if a_kcontig, else A[k*lda + m]
//   B(k, n) = Bp[n*ldb + k]  if b_kcontig, else Bp[k*ldb + n]
// B may be split into up to 3 segments of length bseg, along N (b_kseg = 0)
// or along K (b_kseg = 1); the index inside a segment is local to it.
// C (and bias) may be split into up to 3 segments of length cseg along N.
struct GemmDesc {
    int M = 0, N = 0, K = 0;
    const void* A = nullptr;
    int64_t lda = 0;
    bool a_kcontig = true;
    const void* B[3] = {nullptr, nullptr, nullptr};
    int64_t ldb = 0;
    bool b_kcontig = false;
    bool b_kseg = false;
    int bseg = 1 << 30;
    void* C[3] = {nullptr, nullptr, nullptr};
    int64_t ldc = 0;
    int cseg = 1 << 30;
    bool out_f32 = false;         // C stored as fp32 (weight gradients)
    void* C2 = nullptr;           // Y of EPI_BIAS_GELU
    int64_t ldc2 = 0;
    const void* bias[3] = {nullptr, nullptr, nullptr};
    const void* aux = nullptr;    // Gp of EPI_GELU_BWD
    int64_t ldaux = 0;
    int epi = EPI_STORE;
    bool gelu_tanh = false;       // EPI_BIAS_GELU / EPI_GELU_BWD: the tanh form of GeLU
    int cus = 0;                  // CUs the tile choice may count on (0: all 256); a launch that
                                  // shares the GPU with another stream's work plans for its share
    bool fp16 = false;            // 16-bit operands / outputs are IEEE half (else bfloat16)
    float* rd = nullptr;          // EPI_STORE_ROWDOT: the row dots and their layout
    int rd_seq = 0, rd_heads = 0, rd_dh = 0;
};

// bf16 operands, fp32 MFMA accumulation.  Returns hipSuccess or the launch error.
hipError_t gemm_bf16(const GemmDesc& d, hipStream_t s);
// One launch for n (1 or 2) independent problems of the same layout and
// epilogue.  fp32-output (weight-gradient) problems may be split in two along
// K when `part` (16-byte aligned) holds at least sum(M N) floats (*ksplit_out
// reports the split): the first half writes the outputs, the second its
// partial sums to `part`, and a kernel on the same stream then adds them in.
hipError_t gemm_bf16_batch(const GemmDesc* d, int n, float* part, int64_t part_floats, int* ksplit_out,
                           hipStream_t s);
// Test hook: every later 16-bit GEMM for which tile `tile` (0 .. gemm_tile_count()-1)
// is valid uses it, with a K split of `ksplit` (2: fp32-output GEMMs split in two;
// else no split); tile < 0 restores the cost model.  Process-wide, not thread-safe.
void gemm_force_tile(int tile, int ksplit);
int gemm_tile_count();
// Whether gemm_bf16 can run d with EPI_STORE_ROWDOT: plain 16-bit output of
// K-contiguous operands, one round of 64 x 192 tiles (ceil(M/64) ceil(N/192) <= the
// CUs), heads that divide 192 and N, aux 16-byte aligned with ldaux a multiple of 8.
bool gemm_rowdot_ok(const GemmDesc& d);

// dst[k] += src[k] for n (<= ZMAX) row-major fp32 blocks (rows[k] x cols[k],
// row strides ld[k] and lds[k]) in one launch.
constexpr int ZMAX = 6;
struct AddRegions {
    float* dst[ZMAX];
    const float* src[ZMAX];
    int64_t cols[ZMAX], ld[ZMAX], lds[ZMAX], start[ZMAX];
    int64_t total;
    int n;
};
hipError_t add_f32_2d(float* const* dst, const float* const* src, const int64_t* rows, const int64_t* cols,
                      const int64_t* ld, const int64_t* lds, int n, hipStream_t s);
// 16-bit gather of three column blocks side by side: dst[r][z w + c] =
// src[z][r lds + c] for r < rows, c < w (z = 0, 1, 2), and, when bdst is set,
// bdst[z w + c] = bsrc[z][c] (0 where bsrc[z] is null).  w and lds multiples of 8,
// pointers 16-byte aligned.
hipError_t gather3(const void* const* src, int64_t lds, int64_t rows, int64_t w, void* dst,
                   const void* const* bsrc, void* bdst, hipStream_t s);
// fp32 operands and outputs, fp32 FMA arithmetic.
hipError_t gemm_f32(const GemmDesc& d, hipStream_t s);

struct AttnDesc {
    int batch = 0, seq = 0, heads = 0;  // heads of this shard (H/t)
    int dh = 0;                         // head dim
    int causal = 1;
    const void* qkv = nullptr;          // [T, 3w]
    int64_t ld_qkv = 0;                 // 3w
    void* O = nullptr;                  // [T, w]
    int64_t ld_o = 0;                   // w
    float* lse = nullptr;               // [batch, heads, seq]
    // backward
    const void* dO = nullptr;           // [T, w]
    float* Dq = nullptr;                // [batch, heads, seq]
    void* dqkv = nullptr;               // [T, 3w]
    bool fp16 = false;                  // IEEE half storage (else bfloat16)
};

// The backward is three launches: D = rowsum(dO * O) first, then the dK/dV
// and dQ passes, which are independent of each other (both read D).
// ATTN_BWD_DKDV_DQ runs the last two as one launch (16-bit storage only).
enum AttnBwdPart { ATTN_BWD_ROWDOT = 0, ATTN_BWD_DKDV = 1, ATTN_BWD_DQ = 2, ATTN_BWD_DKDV_DQ = 3 };
hipError_t attn_fwd_bf16(const AttnDesc& a, hipStream_t s);
hipError_t attn_bwd_bf16(const AttnDesc& a, int part, hipStream_t s);
hipError_t attn_fwd_f32(const AttnDesc& a, hipStream_t s);
hipError_t attn_bwd_f32(const AttnDesc& a, int part, hipStream_t s);

// out[c] = sum_r X[r*ld + c] over rows, fp32, into up to 3 column segments of length seg.
// Deterministic two-pass reduction; `work` holds colsum_work_floats(cols) floats.
int64_t colsum_work_floats(int64_t cols);
hipError_t colsum(int fmt, const void* X, int64_t rows, int64_t cols, int64_t ld,
                  float* const out[3], int seg, float* work, hipStream_t s);

// out = sum_p parts[p] + bias (fp32 out).
hipError_t sum_partials(int fmt, int64_t rows, int64_t cols, const void* const* parts,
                        int nparts, const void* bias, float* out, hipStream_t s);

// ---- static scratch of the no-allocation FFN backward (noalloc.hip) ----
constexpr int64_t NOALLOC_SCRATCH_BYTES = (int64_t)64 << 20;
// Device address of the current device's scratch array (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

// ---- pre-LN residual stream (layernorm.hip) ----
constexpr int LN_MAXP = 16;  // partials per call
// h = residual + bias + sum_k parts[k] -> out (fp32, if non-null); then, if y is
// non-null, y = gamma * (h - mean) / sqrt(var + eps) + beta (biased var; gamma,
// beta null for 1, 0) in the activation dtype, row means / rstd into mean, rstd.
// Rows are contiguous ([rows, cols], cols <= 8192, a multiple of 4).
struct LnFwdDesc {
    int64_t rows = 0;
    int cols = 0;
    int fmt = FMT_F32;               // format of parts, bias and y
    const void* parts[LN_MAXP] = {};
    int nparts = 0;
    const void* bias = nullptr;
    const float* residual = nullptr;
    float* out = nullptr;
    const float* gamma = nullptr;
    const float* beta = nullptr;
    float eps = 1e-5f;
    void* y = nullptr;
    float* mean = nullptr;
    float* rstd = nullptr;
};
hipError_t residual_layernorm(const LnFwdDesc& d, hipStream_t s);

// LayerNorm backward for g = sum_k dparts[k] (the gradient of y):
// dx = dres + rstd * (g*gamma - mean_c(g*gamma) - xhat * mean_c(g*gamma*xhat)) (fp32,
// and in the activation dtype into dx_act if non-null); the column sums
// dgamma = sum_r g*xhat, dbeta = sum_r g, dres_sum = sum_r dres, dx_sum = sum_r dx
// into the non-null ones.  work: 4 * (ln_bwd_bands(rows) + LN_BWD_GROUPS) * cols floats.
struct LnBwdDesc {
    int64_t rows = 0;
    int cols = 0;
    int fmt = FMT_F32;               // format of dparts and dx_act
    const float* x = nullptr;
    const float* gamma = nullptr;
    const float* mean = nullptr;
    const float* rstd = nullptr;
    const void* dparts[LN_MAXP] = {};
    int nparts = 0;
    const float* dres = nullptr;
    float* dx = nullptr;
    void* dx_act = nullptr;
    float* dgamma = nullptr;
    float* dbeta = nullptr;
    float* dres_sum = nullptr;
    float* dx_sum = nullptr;
    float* work = nullptr;
};
int ln_bwd_bands(int64_t rows);
constexpr int LN_BWD_GROUPS = 32;
hipError_t layernorm_bwd(const LnBwdDesc& d, hipStream_t s);

}  // namespace tp
