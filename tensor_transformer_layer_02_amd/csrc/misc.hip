// Small memory-bound kernels of the shard: bias-gradient column sums and the
// verification-only sum of shard partials that stands in for the all-reduce
// on one GPU (page "Megatron-LM: what the tensor parallelism paper actually
// says", section "How transformer layers actually decompose": the partial
// results are summed to get the output).
#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int COLSUM_SPLITS = 32;   // row bands; partial sums land in work[band][col]
constexpr int CS_COLS = 64;         // columns per workgroup (8 groups of 8)

// Partial column sums of a [rows, cols] matrix over one band of rows.  Thread
// (row lane rl, column group cg) reads 8 consecutive columns per row with a
// 16-byte load (16-bit formats) or two (fp32); a wave covers 8 rows x 64 columns.
template <typename T>
__global__ void __launch_bounds__(256) colsum_partial_kernel(const T* __restrict__ X, int64_t rows, int64_t cols,
                                                             int64_t ld, float* __restrict__ work) {
    __shared__ float red[32][CS_COLS + 1];
    const int cg = threadIdx.x % 8, rl = threadIdx.x / 8;
    const int64_t c0 = (int64_t)blockIdx.x * CS_COLS + cg * 8;
    const int64_t band = (rows + COLSUM_SPLITS - 1) / COLSUM_SPLITS;
    const int64_t r0 = blockIdx.y * band, r1 = min(rows, r0 + band);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c0 < cols) {
        for (int64_t r = r0 + rl; r < r1; r += 32) {
            const T* src = X + r * ld + c0;
            if constexpr (sizeof(T) == 2) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] += Store16<T>::lo(v[q]);
                    acc[2 * q + 1] += Store16<T>::hi(v[q]);
                }
            } else {
                const f32x4 a = *reinterpret_cast<const f32x4*>(src);
                const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[q] += a[q];
                    acc[4 + q] += b[q];
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) red[rl][cg * 8 + q] = acc[q];
    __syncthreads();
    if (threadIdx.x < CS_COLS) {
        float sum = 0.f;
        for (int i = 0; i < 32; ++i) sum += red[i][threadIdx.x];
        const int64_t c = (int64_t)blockIdx.x * CS_COLS + threadIdx.x;
        if (c < cols) work[(int64_t)blockIdx.y * cols + c] = sum;
    }
}

struct Out3 {
    float* p[3];
};

__global__ void __launch_bounds__(256) colsum_final_kernel(const float* __restrict__ work, int64_t cols,
                                                           Out3 out, int seg) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.f;
    for (int i = 0; i < COLSUM_SPLITS; ++i) acc += work[(int64_t)i * cols + c];
    const int sg = (int)(c / seg);
    out.p[sg][c - (int64_t)sg * seg] = acc;
}

// Zero up to ZMAX row-major fp32 blocks in one launch; thread item i covers 4
// floats of one row (f32x4 store when aligned).
// dst[k] += src[k] over n row-major fp32 blocks (rows[k] x cols[k]; row strides
// ld[k] and lds[k]), four columns per item where both rows are 16-byte aligned.
__global__ void __launch_bounds__(256) add_f32_2d_kernel(const AddRegions z) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < z.total; i += (int64_t)gridDim.x * 256) {
        int k = 0;
        while (k + 1 < z.n && i >= z.start[k + 1]) ++k;
        const int64_t j = i - z.start[k];
        const int64_t c4 = (z.cols[k] + 3) / 4;
        const int64_t r = j / c4, c = (j % c4) * 4;
        float* q = z.dst[k] + r * z.ld[k] + c;
        const float* a = z.src[k] + r * z.lds[k] + c;
        if (c + 4 <= z.cols[k] && ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(a)) & 15) == 0) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(q), y = *reinterpret_cast<const f32x4*>(a);
            *reinterpret_cast<f32x4*>(q) = f32x4{x[0] + y[0], x[1] + y[1], x[2] + y[2], x[3] + y[3]};
        } else {
            for (int64_t e = 0; c + e < z.cols[k] && e < 4; ++e) q[e] += a[e];
        }
    }
}

constexpr int MAXP = 16;
struct Parts {
    const void* p[MAXP];
};

template <typename T>
__global__ void __launch_bounds__(256) sum_partials_kernel(int64_t rows, int64_t cols, Parts parts, int n,
                                                           const T* __restrict__ bias, int accumulate,
                                                           float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * cols) return;
    float acc = accumulate ? out[i] : (bias ? to_f<T>(bias[i % cols]) : 0.f);
    for (int k = 0; k < n; ++k) acc += to_f<T>(static_cast<const T*>(parts.p[k])[i]);
    out[i] = acc;
}

}  // namespace

int64_t colsum_work_floats(int64_t cols) { return (int64_t)COLSUM_SPLITS * cols; }

hipError_t colsum(int fmt, const void* X, int64_t rows, int64_t cols, int64_t ld, float* const out[3],
                  int seg, float* work, hipStream_t s) {
    if (cols <= 0) return hipSuccess;
    dim3 g1((unsigned)((cols + CS_COLS - 1) / CS_COLS), COLSUM_SPLITS);
    if (fmt == FMT_BF16)
        hipLaunchKernelGGL(colsum_partial_kernel<bf16_t>, g1, dim3(256), 0, s, static_cast<const bf16_t*>(X), rows,
                           cols, ld, work);
    else if (fmt == FMT_F16)
        hipLaunchKernelGGL(colsum_partial_kernel<f16_t>, g1, dim3(256), 0, s, static_cast<const f16_t*>(X), rows,
                           cols, ld, work);
    else
        hipLaunchKernelGGL(colsum_partial_kernel<float>, g1, dim3(256), 0, s, static_cast<const float*>(X), rows,
                           cols, ld, work);
    count_launch();
    Out3 o;
    for (int i = 0; i < 3; ++i) o.p[i] = out[i] ? out[i] : out[0];
    hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(work), cols, o, seg);
    count_launch();
    return hipGetLastError();
}

struct Gather3 {
    const u32x4* src[3];
    const u32x4* bsrc[3];
    int64_t lds8, rows, w8;  // row stride and width in 8-element (16-byte) units
    u32x4* dst;
    u32x4* bdst;
};

// One 16-byte item per thread and step: rows first, then the bias row.
__global__ void __launch_bounds__(256) gather3_kernel(const Gather3 g) {
    const int64_t per_row = 3 * g.w8, n = g.rows * per_row + (g.bdst ? per_row : 0);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / per_row, c = i % per_row;
        const int z = (int)(c / g.w8);
        const int64_t cc = c - z * g.w8;
        if (r < g.rows) {
            g.dst[r * per_row + c] = g.src[z][r * g.lds8 + cc];
        } else {
            g.bdst[c] = g.bsrc[z] ? g.bsrc[z][cc] : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

hipError_t gather3(const void* const* src, int64_t lds, int64_t rows, int64_t w, void* dst,
                   const void* const* bsrc, void* bdst, hipStream_t s) {
    if (rows <= 0 || w <= 0 || w % 8 || lds % 8) return hipErrorInvalidValue;
    Gather3 g;
    for (int z = 0; z < 3; ++z) {
        g.src[z] = static_cast<const u32x4*>(src[z]);
        g.bsrc[z] = bsrc ? static_cast<const u32x4*>(bsrc[z]) : nullptr;
    }
    g.lds8 = lds / 8;
    g.rows = rows;
    g.w8 = w / 8;
    g.dst = static_cast<u32x4*>(dst);
    g.bdst = static_cast<u32x4*>(bdst);
    const int64_t n = (rows + 1) * 3 * g.w8, blocks = (n + 255) / 256;
    hipLaunchKernelGGL(gather3_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, g);
    count_launch();
    return hipGetLastError();
}

hipError_t add_f32_2d(float* const* dst, const float* const* src, const int64_t* rows, const int64_t* cols,
                      const int64_t* ld, const int64_t* lds, int n, hipStream_t s) {
    if (n < 0 || n > ZMAX) return hipErrorInvalidValue;
    AddRegions z;
    z.n = 0;
    z.total = 0;
    for (int k = 0; k < n; ++k) {
        if (rows[k] <= 0 || cols[k] <= 0) continue;
        z.dst[z.n] = dst[k];
        z.src[z.n] = src[k];
        z.cols[z.n] = cols[k];
        z.ld[z.n] = ld[k];
        z.lds[z.n] = lds[k];
        z.start[z.n] = z.total;
        z.total += rows[k] * ((cols[k] + 3) / 4);
        ++z.n;
    }
    if (z.total == 0) return hipSuccess;
    const int64_t blocks = (z.total + 255) / 256;
    hipLaunchKernelGGL(add_f32_2d_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, z);
    count_launch();
    return hipGetLastError();
}

hipError_t sum_partials(int fmt, int64_t rows, int64_t cols, const void* const* parts, int nparts,
                        const void* bias, float* out, hipStream_t s) {
    const int64_t n = rows * cols;
    if (n <= 0) return hipSuccess;
    dim3 grid((unsigned)((n + 255) / 256));
    for (int k0 = 0; k0 < nparts || k0 == 0; k0 += MAXP) {
        Parts P;
        const int cnt = nparts - k0 < MAXP ? nparts - k0 : MAXP;
        for (int i = 0; i < MAXP; ++i) P.p[i] = i < cnt ? parts[k0 + i] : nullptr;
        if (fmt == FMT_BF16)
            hipLaunchKernelGGL(sum_partials_kernel<bf16_t>, grid, dim3(256), 0, s, rows, cols, P, cnt,
                               static_cast<const bf16_t*>(bias), k0 > 0 ? 1 : 0, out);
        else if (fmt == FMT_F16)
            hipLaunchKernelGGL(sum_partials_kernel<f16_t>, grid, dim3(256), 0, s, rows, cols, P, cnt,
                               static_cast<const f16_t*>(bias), k0 > 0 ? 1 : 0, out);
        else
            hipLaunchKernelGGL(sum_partials_kernel<float>, grid, dim3(256), 0, s, rows, cols, P, cnt,
                               static_cast<const float*>(bias), k0 > 0 ? 1 : 0, out);
        count_launch();
        if (nparts == 0) break;
    }
    return hipGetLastError();
}

}  // namespace tp
