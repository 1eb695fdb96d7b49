// fp32 path of the layer shard (dims.act = TP_FP32): the same GEMMs and
// attention as the bf16 path, in plain fp32 FMA arithmetic (no reduced
// precision anywhere).  It serves small fp32 workloads, where latency rather
// than matrix-core throughput decides the time, so the kernels favour
// simplicity: a 64x64 register-blocked GEMM and one-thread-per-row attention.
#include <cfloat>
#include <cmath>

#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

struct GemmArgsF {
    int M, N, K;
    const float* A;
    int64_t sam, sak;  // A(m, k) = A[m*sam + k*sak]
    const float* B[3];
    int64_t sbk, sbn;  // B(k, n) = Bseg[kl*sbk + nl*sbn]
    int bseg, b_kseg;
    float* C[3];
    int64_t ldc;
    int cseg;
    float* C2;
    int64_t ldc2;
    const float* bias[3];
    const float* aux;
    int64_t ldaux;
    int gelu_tanh;
};

__device__ __forceinline__ float ldA(const GemmArgsF& p, int m, int k) {
    return (m < p.M && k < p.K) ? p.A[(int64_t)m * p.sam + (int64_t)k * p.sak] : 0.f;
}

__device__ __forceinline__ float ldB(const GemmArgsF& p, int k, int n) {
    if (k >= p.K || n >= p.N) return 0.f;
    int kl = k, nl = n, sg;
    if (p.b_kseg) { sg = k / p.bseg; kl = k - sg * p.bseg; }
    else { sg = n / p.bseg; nl = n - sg * p.bseg; }
    return p.B[sg][(int64_t)kl * p.sbk + (int64_t)nl * p.sbn];
}

template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const GemmArgsF p) {
    constexpr int TM = 64, TN = 64, TK = 16;
    __shared__ float As[TK][TM + 4];
    __shared__ float Bs[TK][TN + 4];
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += TK) {
        for (int e = tid; e < TM * TK; e += 256) {
            const int mm = e / TK, kk = e % TK;
            As[kk][mm] = ldA(p, m0 + mm, k0 + kk);
        }
        for (int e = tid; e < TN * TK; e += 256) {
            const int kk = e / TN, nn = e % TN;
            Bs[kk][nn] = ldB(p, k0 + kk, n0 + nn);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= p.N) continue;
            const int sg = n / p.cseg, nl = n - sg * p.cseg;
            float v = acc[i][j];
            float* c = p.C[sg] + (int64_t)m * p.ldc + nl;
            if constexpr (EPI == EPI_STORE) {
                *c = v;
            } else if constexpr (EPI == EPI_BIAS) {
                *c = v + (p.bias[sg] ? p.bias[sg][nl] : 0.f);
            } else if constexpr (EPI == EPI_BIAS_GELU) {
                const float u = v + (p.bias[sg] ? p.bias[sg][nl] : 0.f);
                float d;
                p.C2[(int64_t)m * p.ldc2 + nl] = gelu_and_prime(u, p.gelu_tanh != 0, d);
                *c = d;  // Gp = GeLU'(U), what the backward needs of U
            } else {
                *c = v * p.aux[(int64_t)m * p.ldaux + nl];  // dU = dY * Gp
            }
        }
    }
}

// ------------------------------------------------------------- attention

struct AttnArgsF {
    int batch, seq, heads, causal, dh, w;
    const float* qkv;
    int64_t ld_qkv;
    float* O;
    int64_t ld_o;
    float* lse;
    const float* dO;
    float* Dq;
    float* dqkv;
    float scale;
};

constexpr int RB = 64;  // rows per workgroup / per LDS block

template <int DMAX>
__global__ void __launch_bounds__(RB) attn_fwd_f32_kernel(const AttnArgsF a) {
    __shared__ float Ks[RB][DMAX];
    __shared__ float Vs[RB][DMAX];
    const int s = a.seq, d = a.dh;
    const int b = blockIdx.y / a.heads, g = blockIdx.y % a.heads;
    const int q = blockIdx.x * RB + threadIdx.x;
    const float* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * d;
    const float* Kg = Qg + a.w;
    const float* Vg = Qg + 2 * a.w;
    float qv[DMAX], o[DMAX];
#pragma unroll
    for (int c = 0; c < DMAX; ++c) {
        qv[c] = (c < d && q < s) ? Qg[(int64_t)q * a.ld_qkv + c] : 0.f;
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int last_key = a.causal ? min(s - 1, (int)(blockIdx.x * RB + RB - 1)) : s - 1;
    for (int k0 = 0; k0 <= last_key; k0 += RB) {
        for (int e = threadIdx.x; e < RB * d; e += RB) {
            const int r = e / d, c = e % d, key = k0 + r;
            Ks[r][c] = key < s ? Kg[(int64_t)key * a.ld_qkv + c] : 0.f;
            Vs[r][c] = key < s ? Vg[(int64_t)key * a.ld_qkv + c] : 0.f;
        }
        __syncthreads();
        for (int r = 0; r < RB; ++r) {
            const int key = k0 + r;
            if (key >= s || (a.causal && key > q)) continue;
            float sc = 0.f;
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) sc = fmaf(qv[c], Ks[r][c], sc);
            sc *= a.scale;
            const float mn = fmaxf(m, sc);
            const float alpha = expf(m - mn), pv = expf(sc - mn);
            l = l * alpha + pv;
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) o[c] = o[c] * alpha + pv * Vs[r][c];
            m = mn;
        }
        __syncthreads();
    }
    if (q < s) {
        const float inv = 1.f / l;
        float* orow = a.O + ((int64_t)b * s + q) * a.ld_o + g * d;
#pragma unroll
        for (int c = 0; c < DMAX; ++c)
            if (c < d) orow[c] = o[c] * inv;
        a.lse[((int64_t)b * a.heads + g) * s + q] = m + logf(l);
    }
}

// D[b, g, j] = dO_j . O_j
__global__ void attn_rowdot_f32_kernel(const AttnArgsF a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t T = (int64_t)a.batch * a.seq;
    if (idx >= T * a.heads) return;
    const int64_t r = idx / a.heads;
    const int g = (int)(idx % a.heads);
    const float* o = a.O + r * a.ld_o + g * a.dh;
    const float* dd = a.dO + r * a.ld_o + g * a.dh;
    float acc = 0.f;
    for (int c = 0; c < a.dh; ++c) acc = fmaf(o[c], dd[c], acc);
    const int b = (int)(r / a.seq), j = (int)(r % a.seq);
    a.Dq[((int64_t)b * a.heads + g) * a.seq + j] = acc;
}

// One thread per key: dV = sum_j P_jm dO_j, dK = sum_j dS_jm Q_j / sqrt(d).
template <int DMAX>
__global__ void __launch_bounds__(RB) attn_bwd_dkdv_f32_kernel(const AttnArgsF a) {
    __shared__ float Qs[RB][DMAX];
    __shared__ float dOs[RB][DMAX];
    __shared__ float ls[RB], Ds[RB];
    const int s = a.seq, d = a.dh;
    const int b = blockIdx.y / a.heads, g = blockIdx.y % a.heads;
    const int key = blockIdx.x * RB + threadIdx.x;
    const float* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * d;
    const float* Kg = Qg + a.w;
    const float* Vg = Qg + 2 * a.w;
    const float* dOg = a.dO + (int64_t)b * s * a.ld_o + g * d;
    const int64_t hrow = ((int64_t)b * a.heads + g) * s;
    float kv[DMAX], vv[DMAX], dk[DMAX], dv[DMAX];
#pragma unroll
    for (int c = 0; c < DMAX; ++c) {
        const bool ok = c < d && key < s;
        kv[c] = ok ? Kg[(int64_t)key * a.ld_qkv + c] : 0.f;
        vv[c] = ok ? Vg[(int64_t)key * a.ld_qkv + c] : 0.f;
        dk[c] = dv[c] = 0.f;
    }
    const int q_first = a.causal ? (int)(blockIdx.x * RB) : 0;
    for (int q0 = (q_first / RB) * RB; q0 < s; q0 += RB) {
        for (int e = threadIdx.x; e < RB * d; e += RB) {
            const int r = e / d, c = e % d, q = q0 + r;
            Qs[r][c] = q < s ? Qg[(int64_t)q * a.ld_qkv + c] : 0.f;
            dOs[r][c] = q < s ? dOg[(int64_t)q * a.ld_o + c] : 0.f;
        }
        if (threadIdx.x < RB) {
            const int q = q0 + threadIdx.x;
            ls[threadIdx.x] = q < s ? a.lse[hrow + q] : 0.f;
            Ds[threadIdx.x] = q < s ? a.Dq[hrow + q] : 0.f;
        }
        __syncthreads();
        for (int r = 0; r < RB; ++r) {
            const int q = q0 + r;
            if (q >= s || key >= s || (a.causal && key > q)) continue;
            float sc = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) {
                    sc = fmaf(Qs[r][c], kv[c], sc);
                    dp = fmaf(dOs[r][c], vv[c], dp);
                }
            const float pv = expf(sc * a.scale - ls[r]);
            const float dsv = pv * (dp - Ds[r]);
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) {
                    dv[c] = fmaf(pv, dOs[r][c], dv[c]);
                    dk[c] = fmaf(dsv, Qs[r][c], dk[c]);
                }
        }
        __syncthreads();
    }
    if (key < s) {
        float* dKr = a.dqkv + ((int64_t)b * s + key) * a.ld_qkv + a.w + g * d;
        float* dVr = dKr + a.w;
#pragma unroll
        for (int c = 0; c < DMAX; ++c)
            if (c < d) {
                dKr[c] = dk[c] * a.scale;
                dVr[c] = dv[c];
            }
    }
}

// One thread per query: dQ = sum_m dS_jm K_m / sqrt(d).
template <int DMAX>
__global__ void __launch_bounds__(RB) attn_bwd_dq_f32_kernel(const AttnArgsF a) {
    __shared__ float Ks[RB][DMAX];
    __shared__ float Vs[RB][DMAX];
    const int s = a.seq, d = a.dh;
    const int b = blockIdx.y / a.heads, g = blockIdx.y % a.heads;
    const int q = blockIdx.x * RB + threadIdx.x;
    const float* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * d;
    const float* Kg = Qg + a.w;
    const float* Vg = Qg + 2 * a.w;
    const float* dOg = a.dO + (int64_t)b * s * a.ld_o + g * d;
    const int64_t hrow = ((int64_t)b * a.heads + g) * s;
    float qv[DMAX], ov[DMAX], dq[DMAX];
#pragma unroll
    for (int c = 0; c < DMAX; ++c) {
        const bool ok = c < d && q < s;
        qv[c] = ok ? Qg[(int64_t)q * a.ld_qkv + c] : 0.f;
        ov[c] = ok ? dOg[(int64_t)q * a.ld_o + c] : 0.f;
        dq[c] = 0.f;
    }
    const float lq = q < s ? a.lse[hrow + q] : 0.f;
    const float Dv = q < s ? a.Dq[hrow + q] : 0.f;
    const int last_key = a.causal ? min(s - 1, (int)(blockIdx.x * RB + RB - 1)) : s - 1;
    for (int k0 = 0; k0 <= last_key; k0 += RB) {
        for (int e = threadIdx.x; e < RB * d; e += RB) {
            const int r = e / d, c = e % d, key = k0 + r;
            Ks[r][c] = key < s ? Kg[(int64_t)key * a.ld_qkv + c] : 0.f;
            Vs[r][c] = key < s ? Vg[(int64_t)key * a.ld_qkv + c] : 0.f;
        }
        __syncthreads();
        for (int r = 0; r < RB; ++r) {
            const int key = k0 + r;
            if (q >= s || key >= s || (a.causal && key > q)) continue;
            float sc = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) {
                    sc = fmaf(qv[c], Ks[r][c], sc);
                    dp = fmaf(ov[c], Vs[r][c], dp);
                }
            const float pv = expf(sc * a.scale - lq);
            const float dsv = pv * (dp - Dv);
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) dq[c] = fmaf(dsv, Ks[r][c], dq[c]);
        }
        __syncthreads();
    }
    if (q < s) {
        float* dQr = a.dqkv + ((int64_t)b * s + q) * a.ld_qkv + g * d;
#pragma unroll
        for (int c = 0; c < DMAX; ++c)
            if (c < d) dQr[c] = dq[c] * a.scale;
    }
}

AttnArgsF make_args(const AttnDesc& d) {
    AttnArgsF a;
    a.batch = d.batch; a.seq = d.seq; a.heads = d.heads; a.causal = d.causal; a.dh = d.dh;
    a.w = d.heads * d.dh;
    a.qkv = static_cast<const float*>(d.qkv); a.ld_qkv = d.ld_qkv;
    a.O = static_cast<float*>(d.O); a.ld_o = d.ld_o;
    a.lse = d.lse;
    a.dO = static_cast<const float*>(d.dO);
    a.Dq = d.Dq;
    a.dqkv = static_cast<float*>(d.dqkv);
    a.scale = 1.0f / sqrtf((float)d.dh);
    return a;
}

template <int DMAX>
hipError_t fwd_f32(const AttnArgsF& a, hipStream_t s) {
    dim3 grid((a.seq + RB - 1) / RB, a.batch * a.heads);
    hipLaunchKernelGGL(attn_fwd_f32_kernel<DMAX>, grid, dim3(RB), 0, s, a);
    count_launch();
    return hipGetLastError();
}

template <int DMAX>
hipError_t bwd_f32(const AttnArgsF& a, int part, hipStream_t s) {
    const int64_t n = (int64_t)a.batch * a.seq * a.heads;
    dim3 grid((a.seq + RB - 1) / RB, a.batch * a.heads);
    if (part == ATTN_BWD_ROWDOT)
        hipLaunchKernelGGL(attn_rowdot_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    else if (part == ATTN_BWD_DKDV)
        hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<DMAX>, grid, dim3(RB), 0, s, a);
    else if (part == ATTN_BWD_DQ)
        hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<DMAX>, grid, dim3(RB), 0, s, a);
    else
        return hipErrorInvalidValue;
    count_launch();
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_f32(const GemmDesc& d, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return hipSuccess;
    GemmArgsF p;
    p.M = d.M; p.N = d.N; p.K = d.K;
    p.A = static_cast<const float*>(d.A);
    if (d.a_kcontig) { p.sam = d.lda; p.sak = 1; } else { p.sam = 1; p.sak = d.lda; }
    for (int i = 0; i < 3; ++i) {
        p.B[i] = static_cast<const float*>(d.B[i] ? d.B[i] : d.B[0]);
        p.C[i] = static_cast<float*>(d.C[i] ? d.C[i] : d.C[0]);
        p.bias[i] = static_cast<const float*>(d.bias[i]);
    }
    if (d.b_kcontig) { p.sbk = 1; p.sbn = d.ldb; } else { p.sbk = d.ldb; p.sbn = 1; }
    p.bseg = d.bseg; p.b_kseg = d.b_kseg ? 1 : 0;
    p.ldc = d.ldc; p.cseg = d.cseg;
    p.C2 = static_cast<float*>(d.C2); p.ldc2 = d.ldc2;
    p.aux = static_cast<const float*>(d.aux); p.ldaux = d.ldaux;
    p.gelu_tanh = d.gelu_tanh ? 1 : 0;
    dim3 grid((d.N + 63) / 64, (d.M + 63) / 64);
    switch (d.epi) {
        case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, dim3(256), 0, s, p); break;
        case EPI_BIAS: hipLaunchKernelGGL(gemm_f32_kernel<EPI_BIAS>, grid, dim3(256), 0, s, p); break;
        case EPI_BIAS_GELU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_BIAS_GELU>, grid, dim3(256), 0, s, p); break;
        case EPI_GELU_BWD: hipLaunchKernelGGL(gemm_f32_kernel<EPI_GELU_BWD>, grid, dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    count_launch();
    return hipGetLastError();
}

hipError_t attn_fwd_f32(const AttnDesc& d, hipStream_t s) {
    const AttnArgsF a = make_args(d);
    if (d.dh <= 32) return fwd_f32<32>(a, s);
    if (d.dh <= 64) return fwd_f32<64>(a, s);
    if (d.dh <= 128) return fwd_f32<128>(a, s);
    return hipErrorInvalidValue;
}

hipError_t attn_bwd_f32(const AttnDesc& d, int part, hipStream_t s) {
    const AttnArgsF a = make_args(d);
    if (d.dh <= 32) return bwd_f32<32>(a, part, s);
    if (d.dh <= 64) return bwd_f32<64>(a, part, s);
    if (d.dh <= 128) return bwd_f32<128>(a, part, s);
    return hipErrorInvalidValue;
}

}  // namespace tp
