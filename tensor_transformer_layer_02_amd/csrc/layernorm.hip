// The pre-LN residual stream around the shards (page "Megatron-LM: what the
// tensor parallelism paper actually says", section "The layernorm placement
// the paper flags as critical": LayerNorm is applied to the residual stream
// before each sublayer, and the sublayer output is added back to it).
//
// Forward, one kernel per residual step:
//   h = residual + bias + sum_k part_k        (the sum that stands in for the
//                                              all-reduce, the row-parallel bias
//                                              added once, the residual add)
//   y = gamma * (h - mean) * rstd + beta      (the next sublayer's LayerNorm;
//                                              rstd = 1/sqrt(var + eps), biased var)
// Backward, fed by the input-gradient partials of the sublayer's shards:
//   g = sum_k dpart_k,  gg = g * gamma
//   dx = dres + rstd * (gg - mean_c(gg) - xhat * mean_c(gg * xhat))
//   dgamma = sum_r g * xhat, dbeta = sum_r g, and the column sums of dres and
//   dx (the row-parallel bias gradients of the two sublayers).
//
// A 256-thread workgroup owns a row (forward) or a band of rows (backward);
// thread t holds the 4-column chunks t, t + 256, ... of a row in registers
// (NCH chunks, a template parameter, so cols <= 1024 * NCH).  Row sums use a
// fixed butterfly inside each wave and the four wave sums in order, and the
// column sums of the backward go through per-band partials added in two
// levels of fixed order, so every result is deterministic.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int LNT = 256;
constexpr int LN_GROUPS = LN_BWD_GROUPS;  // first-level groups of bands in the column sums

struct LnParts {
    const void* p[LN_MAXP];
};

template <typename T>
__device__ __forceinline__ f32x4 ld4(const T* p);
template <>
__device__ __forceinline__ f32x4 ld4<float>(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 ld4<bf16_t>(const bf16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xffff0000u)};
}

template <>
__device__ __forceinline__ f32x4 ld4<f16_t>(const f16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    using S = Store16<f16_t>;
    return f32x4{S::lo(w[0]), S::hi(w[0]), S::lo(w[1]), S::hi(w[1])};
}

// The four values of a ld4-sized load kept as loaded.
template <typename T>
__device__ __forceinline__ f32x4 raw_to_f4(const f32x4& w) {
    return w;
}
template <typename T>
__device__ __forceinline__ f32x4 raw_to_f4(const u32x2& w) {
    using S = Store16<T>;
    return f32x4{S::lo(w[0]), S::hi(w[0]), S::lo(w[1]), S::hi(w[1])};
}

template <typename T>
__device__ __forceinline__ void st4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void st4<float>(float* p, const f32x4& v) {
    *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void st4<bf16_t>(bf16_t* p, const f32x4& v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
}

template <>
__device__ __forceinline__ void st4<f16_t>(f16_t* p, const f32x4& v) {
    using S = Store16<f16_t>;
    *reinterpret_cast<u32x2*>(p) = u32x2{S::pack2(v[0], v[1]), S::pack2(v[2], v[3])};
}

// Sum of v over the workgroup, the same value in every thread.  red: 4 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    const float s = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return s;
}

// The same for two values at once (one pair of barriers).  red: 8 floats of LDS.
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[wave] = a;
        red[4 + wave] = b;
    }
    __syncthreads();
    a = (red[0] + red[1]) + (red[2] + red[3]);
    b = (red[4] + red[5]) + (red[6] + red[7]);
    __syncthreads();
}

// acc[k] += the nparts partial rows at row offset `base`, chunk k of this thread, added in
// partial order (acc[k] unchanged where the chunk lies past cols).  The partials go in groups
// of QG, each group's loads (every chunk) issued before any is added, so a thread has up to
// QG NCH loads in flight instead of one; past nparts a group re-reads the last partial (its
// values are not added), a thread whose chunk lies past cols re-reads the row's last chunk, and
// chunks past cols for the whole workgroup are skipped.
template <typename T, int NCH>
__device__ __forceinline__ void add_parts(f32x4 (&acc)[NCH], const LnParts& P, int nparts, int64_t base, int cols,
                                          int tid) {
    // The loads stay as loaded (8 bytes for 16-bit partials) until they are added.
    using Raw = typename std::conditional<sizeof(T) == 2, u32x2, f32x4>::type;
    constexpr int QG = NCH >= 4 ? 1 : NCH == 3 ? 8 : 4;  // registers: QG * NCH loads in flight
    for (int q0 = 0; q0 < nparts; q0 += QG) {
        Raw v[QG][NCH];
#pragma unroll
        for (int j = 0; j < QG; ++j) {
            const T* src = static_cast<const T*>(P.p[min(q0 + j, nparts - 1)]) + base;
#pragma unroll
            for (int k = 0; k < NCH; ++k)
                if (4 * LNT * k < cols) v[j][k] = *reinterpret_cast<const Raw*>(src + min(4 * (tid + LNT * k), cols - 4));
        }
#pragma unroll
        for (int j = 0; j < QG; ++j) {
            if (q0 + j >= nparts) break;
#pragma unroll
            for (int k = 0; k < NCH; ++k)
                if (4 * (tid + LNT * k) < cols) acc[k] += raw_to_f4<T>(v[j][k]);
        }
    }
}

template <typename T, int NCH>
__global__ void __launch_bounds__(LNT) residual_ln_kernel(int64_t rows, int cols, const LnParts parts, int nparts,
                                                          const T* __restrict__ bias,
                                                          const float* __restrict__ residual, float* __restrict__ out,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ beta, float eps, T* __restrict__ y,
                                                          float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t base = r * cols;
    // (one workgroup per row, many resident per CU: the partials' loads one after the other
    // keep the registers, and so the occupancy that hides their latency, low)
    f32x4 v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int c = 4 * (tid + LNT * k);
        v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c >= cols) continue;
        if (residual) v[k] = ld4<float>(residual + base + c);
        if (bias) v[k] += ld4<T>(bias + c);
        for (int q = 0; q < nparts; ++q) v[k] += ld4<T>(static_cast<const T*>(parts.p[q]) + base + c);
        if (out) st4<float>(out + base + c, v[k]);
    }
    if (!y) return;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);  // zero past cols
    const float mean = block_sum(s, red) / (float)cols;
    float s2 = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        if (4 * (tid + LNT * k) >= cols) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) s2 += (v[k][e] - mean) * (v[k][e] - mean);
    }
    const float rstd = 1.0f / sqrtf(block_sum(s2, red) / (float)cols + eps);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int c = 4 * (tid + LNT * k);
        if (c >= cols) continue;
        const f32x4 g = gamma ? ld4<float>(gamma + c) : f32x4{1.f, 1.f, 1.f, 1.f};
        const f32x4 b = beta ? ld4<float>(beta + c) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(g[e], (v[k][e] - mean) * rstd, b[e]);
        st4<T>(y + base + c, o);
    }
    if (tid == 0) {
        if (mean_out) mean_out[r] = mean;
        if (rstd_out) rstd_out[r] = rstd;
    }
}

// Band b of rows: per-row dx, and per-thread column sums of g * xhat, g, dres
// and dx over the band into work[q][b][cols] for the requested q (bit q of need).
template <typename T, int NCH>
__global__ void __launch_bounds__(LNT) ln_bwd_kernel(int64_t rows, int cols, int64_t band,
                                                     const float* __restrict__ x, const float* __restrict__ gamma,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const LnParts dparts, int nparts, const float* __restrict__ dres,
                                                     float* __restrict__ dx, T* __restrict__ dx_act,
                                                     float* __restrict__ work, int need) {
    // Up to 3 chunks per thread the band's column sums live in LDS (slot (q NCH + k) LNT + tid:
    // each thread owns its slots, 16 bytes apart), so that the registers they free hold a row's
    // loads in flight; wider rows keep them in registers.
    constexpr bool LACC = NCH <= 3;
    constexpr int NR = LACC ? 1 : NCH;
    __shared__ float red[8];
    __shared__ f32x4 lacc[LACC ? 4 * NCH * LNT : 1];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * band, r1 = min(rows, r0 + band);
    f32x4 sg[NR], sb[NR], sr[NR], sx[NR], gm[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (LACC) {
#pragma unroll
            for (int q = 0; q < 4; ++q) lacc[(q * NCH + k) * LNT + tid] = z;
        } else {
            sg[k] = sb[k] = sr[k] = sx[k] = z;
        }
        const int c = 4 * (tid + LNT * k);
        gm[k] = (gamma && c < cols) ? ld4<float>(gamma + c) : f32x4{1.f, 1.f, 1.f, 1.f};
    }
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t base = r * cols;
        const float mu = mean[r], rs = rstd[r];
        f32x4 g[NCH], xh[NCH], xv[NCH];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {  // x of the row first, then the partials
            g[k] = xh[k] = xv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (4 * LNT * k < cols) xv[k] = ld4<float>(x + base + min(4 * (tid + LNT * k), cols - 4));
        }
        add_parts<T, NCH>(g, dparts, nparts, base, cols, tid);
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = 4 * (tid + LNT * k);
            if (c >= cols) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xh[k][e] = (xv[k][e] - mu) * rs;
                const float gg = g[k][e] * gm[k][e];
                s1 += gg;
                s2 += gg * xh[k][e];
            }
        }
        block_sum2(s1, s2, red);
        const float m1 = s1 / (float)cols, m2 = s2 / (float)cols;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = 4 * (tid + LNT * k);
            if (c >= cols) continue;
            const f32x4 dr = dres ? ld4<float>(dres + base + c) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 o, gx;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] = dr[e] + rs * (g[k][e] * gm[k][e] - m1 - xh[k][e] * m2);
                gx[e] = g[k][e] * xh[k][e];
            }
            if constexpr (LACC) {
                f32x4* a = lacc + k * LNT + tid;
                a[0] += gx;
                a[NCH * LNT] += g[k];
                a[2 * NCH * LNT] += dr;
                a[3 * NCH * LNT] += o;
            } else {
                sg[k] += gx;
                sb[k] += g[k];
                sr[k] += dr;
                sx[k] += o;
            }
            st4<float>(dx + base + c, o);
            if (dx_act) st4<T>(dx_act + base + c, o);
        }
    }
    const int64_t nb = gridDim.x;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int c = 4 * (tid + LNT * k);
        if (c >= cols) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (!((need >> q) & 1)) continue;
            f32x4 v;
            if constexpr (LACC) v = lacc[(q * NCH + k) * LNT + tid];
            else v = q == 0 ? sg[k] : q == 1 ? sb[k] : q == 2 ? sr[k] : sx[k];
            st4<float>(work + (q * nb + blockIdx.x) * cols + c, v);
        }
    }
}

struct Out4 {
    float* p[4];
};

// Column sums of the band partials in two levels, each in a fixed order:
// part2[q][s][c] = sum over the bands of group s (nb / LN_GROUPS consecutive bands) ...
__global__ void __launch_bounds__(LNT) ln_bwd_colsum1_kernel(int cols, int nb, const float* __restrict__ work,
                                                             float* __restrict__ part2, int need) {
    const int c = blockIdx.x * LNT + threadIdx.x;
    const int q = blockIdx.y, g = blockIdx.z;
    if (c >= cols || !((need >> q) & 1)) return;
    const int per = (nb + LN_GROUPS - 1) / LN_GROUPS;
    const int b0 = g * per, b1 = min(nb, b0 + per);
    float s = 0.f;
    for (int b = b0; b < b1; ++b) s += work[((int64_t)q * nb + b) * cols + c];
    part2[((int64_t)q * LN_GROUPS + g) * cols + c] = s;
}

// ... and out[q][c] = sum over the groups s (in order) of part2[q][s][c].
__global__ void __launch_bounds__(LNT) ln_bwd_colsum2_kernel(int cols, const float* __restrict__ part2, Out4 o) {
    const int c = blockIdx.x * LNT + threadIdx.x;
    const int q = blockIdx.y;
    if (c >= cols || !o.p[q]) return;
    float s = 0.f;
    for (int g = 0; g < LN_GROUPS; ++g) s += part2[((int64_t)q * LN_GROUPS + g) * cols + c];
    o.p[q][c] = s;
}

template <typename T, int NCH>
hipError_t launch_fwd(const LnFwdDesc& d, hipStream_t s) {
    LnParts P;
    for (int i = 0; i < LN_MAXP; ++i) P.p[i] = i < d.nparts ? d.parts[i] : nullptr;
    hipLaunchKernelGGL((residual_ln_kernel<T, NCH>), dim3((unsigned)d.rows), dim3(LNT), 0, s, d.rows, d.cols, P,
                       d.nparts, static_cast<const T*>(d.bias), d.residual, d.out, d.gamma, d.beta, d.eps,
                       static_cast<T*>(d.y), d.mean, d.rstd);
    count_launch();
    return hipGetLastError();
}

template <typename T, int NCH>
hipError_t launch_bwd(const LnBwdDesc& d, hipStream_t s) {
    LnParts P;
    for (int i = 0; i < LN_MAXP; ++i) P.p[i] = i < d.nparts ? d.dparts[i] : nullptr;
    const int nb = ln_bwd_bands(d.rows);
    const int64_t band = (d.rows + nb - 1) / nb;
    Out4 o{{d.dgamma, d.dbeta, d.dres_sum, d.dx_sum}};
    const int need = (o.p[0] ? 1 : 0) | (o.p[1] ? 2 : 0) | (o.p[2] ? 4 : 0) | (o.p[3] ? 8 : 0);
    hipLaunchKernelGGL((ln_bwd_kernel<T, NCH>), dim3((unsigned)nb), dim3(LNT), 0, s, d.rows, d.cols, band, d.x,
                       d.gamma, d.mean, d.rstd, P, d.nparts, d.dres, d.dx, static_cast<T*>(d.dx_act), d.work, need);
    count_launch();
    if (need) {
        float* part2 = d.work + (int64_t)4 * nb * d.cols;
        const unsigned cb = (unsigned)((d.cols + LNT - 1) / LNT);
        hipLaunchKernelGGL(ln_bwd_colsum1_kernel, dim3(cb, 4, LN_GROUPS), dim3(LNT), 0, s, d.cols, nb, d.work, part2,
                           need);
        count_launch();
        hipLaunchKernelGGL(ln_bwd_colsum2_kernel, dim3(cb, 4), dim3(LNT), 0, s, d.cols, part2, o);
        count_launch();
    }
    return hipGetLastError();
}

// Chunks per thread for a row of `cols` columns (4 columns per chunk).
int nch_for(int cols) {
    const int per = (cols / 4 + LNT - 1) / LNT;
    return per <= 1 ? 1 : per <= 2 ? 2 : per <= 3 ? 3 : per <= 4 ? 4 : 8;
}

}  // namespace

// 768 bands: one round of workgroups on 256 CUs at three per CU (the backward
// kernel's registers allow three 4-wave workgroups).
int ln_bwd_bands(int64_t rows) { return (int)(rows < 768 ? rows : 768); }

template <int NCH>
hipError_t fwd_fmt(const LnFwdDesc& d, hipStream_t s) {
    if (d.fmt == FMT_BF16) return launch_fwd<bf16_t, NCH>(d, s);
    if (d.fmt == FMT_F16) return launch_fwd<f16_t, NCH>(d, s);
    return launch_fwd<float, NCH>(d, s);
}

template <int NCH>
hipError_t bwd_fmt(const LnBwdDesc& d, hipStream_t s) {
    if (d.fmt == FMT_BF16) return launch_bwd<bf16_t, NCH>(d, s);
    if (d.fmt == FMT_F16) return launch_bwd<f16_t, NCH>(d, s);
    return launch_bwd<float, NCH>(d, s);
}

hipError_t residual_layernorm(const LnFwdDesc& d, hipStream_t s) {
    if (d.rows <= 0) return hipSuccess;
    switch (nch_for(d.cols)) {
        case 1: return fwd_fmt<1>(d, s);
        case 2: return fwd_fmt<2>(d, s);
        case 3: return fwd_fmt<3>(d, s);
        case 4: return fwd_fmt<4>(d, s);
        default: return fwd_fmt<8>(d, s);
    }
}

hipError_t layernorm_bwd(const LnBwdDesc& d, hipStream_t s) {
    if (d.rows <= 0) return hipSuccess;
    switch (nch_for(d.cols)) {
        case 1: return bwd_fmt<1>(d, s);
        case 2: return bwd_fmt<2>(d, s);
        case 3: return bwd_fmt<3>(d, s);
        case 4: return bwd_fmt<4>(d, s);
        default: return bwd_fmt<8>(d, s);
    }
}

}  // namespace tp
