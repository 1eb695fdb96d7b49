// Fused per-head softmax attention on gfx950 matrix cores, bf16 in / fp32 math.
//
// Each shard runs full attention for its own heads with no communication
// (page "Megatron-LM: what the tensor parallelism paper actually says",
// section "The attention heads split").  Scores are Q K^T / sqrt(d) with an
// optional causal mask (key m allowed for query j iff m <= j).
//
// Forward: a workgroup owns 64 queries of one (sequence, head); each wave64
// owns 16 of them.  Keys and values stream through LDS in blocks of 64.  The
// score tile is formed transposed, S^T = K Q^T, so that each lane holds ONE
// query (lane % 16) and 16 of its keys: the running max and sum of the online
// softmax are lane-local plus a 4-lane butterfly.  O^T = V^T P^T keeps the same
// lane<->query mapping, so rescaling O by the softmax correction is
// lane-local too.  The kernel writes O token-major and the per-query
// log-sum-exp (natural log) for the backward.
//
// Backward: P is recomputed from Q, K and the saved log-sum-exp.
//   D_j = dO_j . O_j            (row sums, equal to sum_m P_jm dP_jm)
//   dV = P^T dO, dK = dS^T Q / sqrt(d)     one workgroup per 64 keys
//   dQ = dS K / sqrt(d)                    one workgroup per 64 queries
// with dP = dO V^T and dS = P * (dP - D).  Splitting dQ into its own pass
// keeps every output written by exactly one workgroup (no atomics; the result
// is deterministic) at the price of recomputing S and dP once more.
#include <cfloat>
#include <cmath>

#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int NT = 256;
constexpr int BQ = 64;   // queries per workgroup
constexpr int BKV = 64;  // keys per LDS block
constexpr int LDT = BKV + 8;  // row stride of transposed ([d][64]) LDS tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;

struct AttnArgs {
    int batch, seq, heads, causal;
    const bf16_t* qkv;
    int64_t ld_qkv;
    int w;  // heads * dh: column offset of K (w) and V (2w) inside qkv
    bf16_t* O;
    int64_t ld_o;
    float* lse;
    const bf16_t* dO;
    float* Dq;
    bf16_t* dqkv;
    float scale;       // 1/sqrt(d)
    float scale_log2;  // log2(e)/sqrt(d)
};

__device__ __forceinline__ u32x4 ld16(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const bf16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

__device__ __forceinline__ uint32_t half_of(const u32x4& v, int i) {
    const uint32_t w = v[i >> 1];
    return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// Stage 64 rows x D columns of a row-major bf16 matrix (rows >= nvalid read
// as zero) into LDS: STRAIGHT as [64][D + 8], TRANSP as [D][64 + 8].
template <int D, bool STRAIGHT, bool TRANSP>
__device__ __forceinline__ void stage_rows(const bf16_t* __restrict__ src, int64_t ld, int row0, int nvalid,
                                           bf16_t* straight, bf16_t* transp, int tid) {
    constexpr int LDK = D + 8;
    constexpr int CH = D / 8;
    for (int u = tid; u < 16 * CH; u += NT) {
        const int dc = (u % CH) * 8, rq = (u / CH) * 4;
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = row0 + rq + j;
            v[j] = (r < nvalid) ? ld16(src + (int64_t)r * ld + dc) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (STRAIGHT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(straight + (rq + j) * LDK + dc) = v[j];
        }
        if constexpr (TRANSP) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x2 t;
                t[0] = half_of(v[0], i) | (half_of(v[1], i) << 16);
                t[1] = half_of(v[2], i) | (half_of(v[3], i) << 16);
                *reinterpret_cast<u32x2*>(transp + (dc + i) * LDT + rq) = t;
            }
        }
    }
}

// A-operand fragment from a transposed [d][64] LDS tile: row (lane % 16) of
// subtile ds, the 8 keys (or queries) {32j + 4g .. +3, 32j + 16 + 4g .. +3},
// g = lane / 16 -- the same 8 indices a lane holds in a 16x16 result pair.
__device__ __forceinline__ u32x4 frag_t(const bf16_t* t, int ds, int j, int lane) {
    const bf16_t* p = t + (ds * 16 + (lane & 15)) * LDT + 32 * j + (lane >> 4) * 4;
    const u32x2 lo = ld8(p), hi = ld8(p + 16);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Pack the result-layout values of 16x16 subtiles 2j and 2j+1 into one
// 8-element bf16 operand fragment (matching frag_t's index order).
__device__ __forceinline__ u32x4 pack_pair(const f32x4& a, const f32x4& b) {
    return u32x4{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
}

template <int D>
__global__ void __launch_bounds__(NT) attn_fwd_kernel(const AttnArgs a) {
    constexpr int KS = D / 32, DS = D / 16, LDK = D + 8;
    __shared__ __attribute__((aligned(16))) bf16_t Ks[BKV * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[D * LDT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
    const int s = a.seq;
    const int nqb = (s + BQ - 1) / BQ;
    const int qb = a.causal ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;  // longest rows first
    const int b = blockIdx.y / a.heads, g = blockIdx.y % a.heads;
    const int q0 = qb * BQ;
    const int qw = q0 + wave * 16 + (lane & 15);

    const bf16_t* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * D;
    const bf16_t* Kg = Qg + a.w;
    const bf16_t* Vg = Qg + 2 * a.w;

    u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = (qw < s) ? ld16(Qg + (int64_t)qw * a.ld_qkv + ks * 32 + grp * 8) : u32x4{0u, 0u, 0u, 0u};

    f32x4 oacc[DS];
#pragma unroll
    for (int i = 0; i < DS; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow = -INFINITY, lsum = 0.f;

    const int nkb_all = (s + BKV - 1) / BKV;
    const int nkb = a.causal ? min(nkb_all, (q0 + BQ - 1) / BKV + 1) : nkb_all;
    for (int kb = 0; kb < nkb; ++kb) {
        const int k0 = kb * BKV;
        stage_rows<D, true, false>(Kg, a.ld_qkv, k0, s, Ks, nullptr, tid);
        stage_rows<D, false, true>(Vg, a.ld_qkv, k0, s, nullptr, Vt, tid);
        __syncthreads();

        f32x4 sacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 af = ld16(Ks + (kt * 16 + (lane & 15)) * LDK + ks * 32 + grp * 8);
                sacc[kt] = mfma16x16x32(af, qf[ks], sacc[kt]);
            }
        }
        // lane: query qw, keys k0 + kt*16 + 4*grp + r
        float bmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + kt * 16 + grp * 4 + r;
                float x = sacc[kt][r] * a.scale_log2;
                if (key >= s || (a.causal && key > qw)) x = -INFINITY;
                sacc[kt][r] = x;
                bmax = fmaxf(bmax, x);
            }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        const float mnew = fmaxf(mrow, bmax);
        const float msub = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2f(mrow - msub);
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pv = exp2f(sacc[kt][r] - msub);
                sacc[kt][r] = pv;
                psum += pv;
            }
        lsum = lsum * alpha + psum;
        mrow = mnew;
#pragma unroll
        for (int i = 0; i < DS; ++i) oacc[i] *= alpha;

        const u32x4 pf0 = pack_pair(sacc[0], sacc[1]);
        const u32x4 pf1 = pack_pair(sacc[2], sacc[3]);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            oacc[ds] = mfma16x16x32(frag_t(Vt, ds, 0, lane), pf0, oacc[ds]);
            oacc[ds] = mfma16x16x32(frag_t(Vt, ds, 1, lane), pf1, oacc[ds]);
        }
        __syncthreads();
    }

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (qw < s) {
        const float inv = 1.f / lsum;
        bf16_t* orow = a.O + ((int64_t)b * s + qw) * a.ld_o + g * D + grp * 4;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x2 t;
            t[0] = pack_bf2(oacc[ds][0] * inv, oacc[ds][1] * inv);
            t[1] = pack_bf2(oacc[ds][2] * inv, oacc[ds][3] * inv);
            *reinterpret_cast<u32x2*>(orow + ds * 16) = t;
        }
        if (grp == 0) a.lse[((int64_t)b * a.heads + g) * s + qw] = (mrow + log2f(lsum)) * LN2;
    }
}

// D[b, g, j] = dO_j . O_j per head (fp32).
template <int D>
__global__ void __launch_bounds__(NT) attn_rowdot_kernel(const AttnArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;  // (token, head)
    const int64_t T = (int64_t)a.batch * a.seq;
    if (idx >= T * a.heads) return;
    const int64_t r = idx / a.heads;
    const int g = (int)(idx % a.heads);
    const bf16_t* o = a.O + r * a.ld_o + g * D;
    const bf16_t* d = a.dO + r * a.ld_o + g * D;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 8) {
        const u32x4 ov = ld16(o + c), dv = ld16(d + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += bf2f((bf16_t)half_of(ov, i)) * bf2f((bf16_t)half_of(dv, i));
    }
    const int b = (int)(r / a.seq), j = (int)(r % a.seq);
    a.Dq[((int64_t)b * a.heads + g) * a.seq + j] = acc;
}

template <int D>
__global__ void __launch_bounds__(NT) attn_bwd_dkdv_kernel(const AttnArgs a) {
    constexpr int KS = D / 32, DS = D / 16, LDK = D + 8;
    __shared__ __attribute__((aligned(16))) bf16_t Qs[BQ * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t dOs[BQ * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Qt[D * LDT];
    __shared__ __attribute__((aligned(16))) bf16_t dOt[D * LDT];
    __shared__ float lse2s[BQ];
    __shared__ float Dqs[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
    const int s = a.seq;
    const int kb = blockIdx.x;
    const int b = blockIdx.y / a.heads, g = blockIdx.y % a.heads;
    const int k0 = kb * BKV;
    const int kw = k0 + wave * 16 + (lane & 15);  // this lane's key

    const bf16_t* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * D;
    const bf16_t* Kg = Qg + a.w;
    const bf16_t* Vg = Qg + 2 * a.w;
    const bf16_t* dOg = a.dO + (int64_t)b * s * a.ld_o + g * D;
    const float* lseg = a.lse + ((int64_t)b * a.heads + g) * s;
    const float* Dg = a.Dq + ((int64_t)b * a.heads + g) * s;

    u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bool ok = kw < s;
        kf[ks] = ok ? ld16(Kg + (int64_t)kw * a.ld_qkv + ks * 32 + grp * 8) : u32x4{0u, 0u, 0u, 0u};
        vf[ks] = ok ? ld16(Vg + (int64_t)kw * a.ld_qkv + ks * 32 + grp * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 dk[DS], dv[DS];
#pragma unroll
    for (int i = 0; i < DS; ++i) dk[i] = dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nqb = (s + BQ - 1) / BQ;
    const int qb0 = a.causal ? (k0 / BQ) : 0;
    for (int qb = qb0; qb < nqb; ++qb) {
        const int q0 = qb * BQ;
        stage_rows<D, true, true>(Qg, a.ld_qkv, q0, s, Qs, Qt, tid);
        stage_rows<D, true, true>(dOg, a.ld_o, q0, s, dOs, dOt, tid);
        if (tid < BQ) {
            const int q = q0 + tid;
            lse2s[tid] = q < s ? lseg[q] * LOG2E : 0.f;
            Dqs[tid] = q < s ? Dg[q] : 0.f;
        }
        __syncthreads();

        // S = Q K^T and dP = dO V^T: rows = queries (4 subtiles), column = this lane's key.
        f32x4 sacc[4], pacc[4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            sacc[qt] = pacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = (qt * 16 + (lane & 15)) * LDK + ks * 32 + grp * 8;
                sacc[qt] = mfma16x16x32(ld16(Qs + off), kf[ks], sacc[qt]);
                pacc[qt] = mfma16x16x32(ld16(dOs + off), vf[ks], pacc[qt]);
            }
        }
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ql = qt * 16 + grp * 4 + r, q = q0 + ql;
                const bool ok = q < s && kw < s && (!a.causal || kw <= q);
                const float pv = ok ? exp2f(sacc[qt][r] * a.scale_log2 - lse2s[ql]) : 0.f;
                sacc[qt][r] = pv;
                pacc[qt][r] = pv * (pacc[qt][r] - Dqs[ql]);
            }
        const u32x4 pf0 = pack_pair(sacc[0], sacc[1]), pf1 = pack_pair(sacc[2], sacc[3]);
        const u32x4 sf0 = pack_pair(pacc[0], pacc[1]), sf1 = pack_pair(pacc[2], pacc[3]);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            dv[ds] = mfma16x16x32(pf0, frag_t(dOt, ds, 0, lane), dv[ds]);
            dv[ds] = mfma16x16x32(pf1, frag_t(dOt, ds, 1, lane), dv[ds]);
            dk[ds] = mfma16x16x32(sf0, frag_t(Qt, ds, 0, lane), dk[ds]);
            dk[ds] = mfma16x16x32(sf1, frag_t(Qt, ds, 1, lane), dk[ds]);
        }
        __syncthreads();
    }

    // result layout: keys k0 + wave*16 + 4*grp + r, column ds*16 + lane % 16
    bf16_t* dKg = a.dqkv + (int64_t)b * s * a.ld_qkv + a.w + g * D;
    bf16_t* dVg = dKg + a.w;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int key = k0 + wave * 16 + grp * 4 + r;
        if (key >= s) continue;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            const int c = ds * 16 + (lane & 15);
            dKg[(int64_t)key * a.ld_qkv + c] = f2bf(dk[ds][r] * a.scale);
            dVg[(int64_t)key * a.ld_qkv + c] = f2bf(dv[ds][r]);
        }
    }
}

template <int D>
__global__ void __launch_bounds__(NT) attn_bwd_dq_kernel(const AttnArgs a) {
    constexpr int KS = D / 32, DS = D / 16, LDK = D + 8;
    __shared__ __attribute__((aligned(16))) bf16_t Ks[BKV * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Vs[BKV * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Kt[D * LDT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
    const int s = a.seq;
    const int nqb = (s + BQ - 1) / BQ;
    const int qb = a.causal ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int b = blockIdx.y / a.heads, g = blockIdx.y % a.heads;
    const int q0 = qb * BQ;
    const int qw = q0 + wave * 16 + (lane & 15);  // this lane's query

    const bf16_t* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * D;
    const bf16_t* Kg = Qg + a.w;
    const bf16_t* Vg = Qg + 2 * a.w;
    const bf16_t* dOg = a.dO + (int64_t)b * s * a.ld_o + g * D;

    u32x4 qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bool ok = qw < s;
        qf[ks] = ok ? ld16(Qg + (int64_t)qw * a.ld_qkv + ks * 32 + grp * 8) : u32x4{0u, 0u, 0u, 0u};
        of[ks] = ok ? ld16(dOg + (int64_t)qw * a.ld_o + ks * 32 + grp * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t hrow = ((int64_t)b * a.heads + g) * s;
    const float lse2 = qw < s ? a.lse[hrow + qw] * LOG2E : 0.f;
    const float Dv = qw < s ? a.Dq[hrow + qw] : 0.f;

    f32x4 dq[DS];
#pragma unroll
    for (int i = 0; i < DS; ++i) dq[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkb_all = (s + BKV - 1) / BKV;
    const int nkb = a.causal ? min(nkb_all, (q0 + BQ - 1) / BKV + 1) : nkb_all;
    for (int kb = 0; kb < nkb; ++kb) {
        const int k0 = kb * BKV;
        stage_rows<D, true, true>(Kg, a.ld_qkv, k0, s, Ks, Kt, tid);
        stage_rows<D, true, false>(Vg, a.ld_qkv, k0, s, Vs, nullptr, tid);
        __syncthreads();

        // S^T = K Q^T and dP^T = V dO^T: rows = keys (4 subtiles), column = this lane's query.
        f32x4 sacc[4], pacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sacc[kt] = pacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = (kt * 16 + (lane & 15)) * LDK + ks * 32 + grp * 8;
                sacc[kt] = mfma16x16x32(ld16(Ks + off), qf[ks], sacc[kt]);
                pacc[kt] = mfma16x16x32(ld16(Vs + off), of[ks], pacc[kt]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + kt * 16 + grp * 4 + r;
                const bool ok = qw < s && key < s && (!a.causal || key <= qw);
                const float pv = ok ? exp2f(sacc[kt][r] * a.scale_log2 - lse2) : 0.f;
                pacc[kt][r] = pv * (pacc[kt][r] - Dv);
            }
        const u32x4 sf0 = pack_pair(pacc[0], pacc[1]), sf1 = pack_pair(pacc[2], pacc[3]);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            dq[ds] = mfma16x16x32(sf0, frag_t(Kt, ds, 0, lane), dq[ds]);
            dq[ds] = mfma16x16x32(sf1, frag_t(Kt, ds, 1, lane), dq[ds]);
        }
        __syncthreads();
    }

    bf16_t* dQg = a.dqkv + (int64_t)b * s * a.ld_qkv + g * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int q = q0 + wave * 16 + grp * 4 + r;
        if (q >= s) continue;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            dQg[(int64_t)q * a.ld_qkv + ds * 16 + (lane & 15)] = f2bf(dq[ds][r] * a.scale);
    }
}

AttnArgs make_args(const AttnDesc& d) {
    AttnArgs a;
    a.batch = d.batch; a.seq = d.seq; a.heads = d.heads; a.causal = d.causal;
    a.qkv = static_cast<const bf16_t*>(d.qkv); a.ld_qkv = d.ld_qkv;
    a.w = d.heads * d.dh;
    a.O = static_cast<bf16_t*>(d.O); a.ld_o = d.ld_o;
    a.lse = d.lse;
    a.dO = static_cast<const bf16_t*>(d.dO);
    a.Dq = d.Dq;
    a.dqkv = static_cast<bf16_t*>(d.dqkv);
    a.scale = 1.0f / sqrtf((float)d.dh);
    a.scale_log2 = LOG2E / sqrtf((float)d.dh);
    return a;
}

template <int D>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
    dim3 grid((a.seq + BQ - 1) / BQ, a.batch * a.heads);
    hipLaunchKernelGGL(attn_fwd_kernel<D>, grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, hipStream_t s) {
    const int64_t T = (int64_t)a.batch * a.seq;
    hipLaunchKernelGGL(attn_rowdot_kernel<D>, dim3((unsigned)((T * a.heads + NT - 1) / NT)), dim3(NT), 0, s, a);
    dim3 grid((a.seq + BQ - 1) / BQ, a.batch * a.heads);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, grid, dim3(NT), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd_bf16(const AttnDesc& d, hipStream_t s) {
    const AttnArgs a = make_args(d);
    switch (d.dh) {
        case 32: return fwd_d<32>(a, s);
        case 64: return fwd_d<64>(a, s);
        case 96: return fwd_d<96>(a, s);
        case 128: return fwd_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t attn_bwd_bf16(const AttnDesc& d, hipStream_t s) {
    const AttnArgs a = make_args(d);
    switch (d.dh) {
        case 32: return bwd_d<32>(a, s);
        case 64: return bwd_d<64>(a, s);
        case 96: return bwd_d<96>(a, s);
        case 128: return bwd_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tp
