// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.
//
// Every projection of the layer shard is one of these GEMMs (page "Megatron-LM:
// what the tensor parallelism paper actually says", sections "How transformer
// layers actually decompose" and "The attention heads split"): the
// column-parallel X*A_i and X*W{q,k,v} with a fused bias (+GeLU) epilogue, the
// row-parallel Y*B_i and O*Wo_i producing partial sums, and their backward
// products (input gradients with a fused GeLU' epilogue, fp32 weight gradients).
//
// Design: a 256-thread workgroup (4 wave64s in a 2x2 grid) computes a BM x BN
// tile; K advances in BK = 64 steps through two LDS buffers, the next step's
// global loads in flight while the current step's MFMAs run.  LDS always holds
// both operands K-contiguous ([rows][BK], padded by 8 elements so the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks).  An operand that
// is contiguous along M or N in memory (the transposed operands of the weight
// gradients) is transposed in registers on its way into LDS: each thread loads
// KR rows of 8 consecutive elements and writes 8 rows of KR elements.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int NT = 256;

struct GemmArgs {
    int M, N, K;
    const bf16_t* A;
    int64_t lda;
    const bf16_t* B[3];
    int64_t ldb;
    int bseg;
    void* C[3];
    int64_t ldc;
    int cseg;
    bf16_t* C2;
    int64_t ldc2;
    const bf16_t* bias[3];
    const bf16_t* aux;
    int64_t ldaux;
};

// Loads a ROWS x BK tile of a K-contiguous operand (element (row, k) at
// base[row*ld + k]) and stores it to LDS as [ROWS][LDK].
template <int ROWS, int BK>
struct KContigTile {
    static constexpr int CPR = BK / 8;                 // 16-byte chunks per row
    static constexpr int PER = ROWS * CPR / NT;        // chunks per thread
    static_assert(PER >= 1 && ROWS * CPR % NT == 0, "tile too small for the workgroup");
    u32x4 v[PER];

    __device__ __forceinline__ void load(const bf16_t* __restrict__ base, int64_t ld, int rows_valid,
                                         int k0, int kvalid, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + NT * i;
            const int r = c / CPR, kc = (c % CPR) * 8;
            if (r < rows_valid && k0 + kc < kvalid)
                v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * ld + k0 + kc);
            else
                v[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    template <int LDK>
    __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + NT * i;
            const int r = c / CPR, kc = (c % CPR) * 8;
            *reinterpret_cast<u32x4*>(lds + r * LDK + kc) = v[i];
        }
    }
};

// Loads a BK x COLS tile of an operand contiguous along M/N (element (k, col)
// at base[k*ld + col]) and stores it transposed to LDS as [COLS][LDK].
template <int COLS, int BK>
struct MNContigTile {
    static constexpr int CCH = COLS / 8;               // 8-wide column chunks
    static constexpr int KR = BK * CCH / NT;           // k rows per thread
    static_assert(KR == 2 || KR == 4 || KR == 8, "unsupported tile shape");
    u32x4 v[KR];

    __device__ __forceinline__ void load(const bf16_t* __restrict__ base, int64_t ld, int cols_valid,
                                         int k0, int kvalid, int tid) {
        const int cc = (tid % CCH) * 8, kq = (tid / CCH) * KR;
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            const int k = k0 + kq + j;
            if (k < kvalid && cc < cols_valid)
                v[j] = *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + cc);
            else
                v[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // halfword i (0..7) of row j
    __device__ __forceinline__ uint32_t half(int j, int i) const {
        const uint32_t w = v[j][i >> 1];
        return (i & 1) ? (w >> 16) : (w & 0xffffu);
    }
    template <int LDK>
    __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
        const int cc = (tid % CCH) * 8, kq = (tid / CCH) * KR;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bf16_t* dst = lds + (cc + i) * LDK + kq;
            if constexpr (KR == 2) {
                *reinterpret_cast<uint32_t*>(dst) = half(0, i) | (half(1, i) << 16);
            } else if constexpr (KR == 4) {
                u32x2 w;
                w[0] = half(0, i) | (half(1, i) << 16);
                w[1] = half(2, i) | (half(3, i) << 16);
                *reinterpret_cast<u32x2*>(dst) = w;
            } else {
                u32x4 w;
#pragma unroll
                for (int p = 0; p < 4; ++p) w[p] = half(2 * p, i) | (half(2 * p + 1, i) << 16);
                *reinterpret_cast<u32x4*>(dst) = w;
            }
        }
    }
};

template <int BM, int BN, int BK, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32>
__global__ void __launch_bounds__(NT) gemm_bf16_kernel(const GemmArgs p) {
    constexpr int LDK = BK + 8;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;

    // Segment of B along N (the whole tile lies in one segment).
    int bsg = 0, nb0 = n0;
    if constexpr (!BKSEG) {
        bsg = n0 / p.bseg;
        nb0 = n0 - bsg * p.bseg;
    }
    const int mvalid = p.M - m0, nvalid = p.N - n0;

    using ATile = typename std::conditional<AK, KContigTile<BM, BK>, MNContigTile<BM, BK>>::type;
    using BTile = typename std::conditional<BKC, KContigTile<BN, BK>, MNContigTile<BN, BK>>::type;
    ATile at;
    BTile bt;

    const bf16_t* Abase = AK ? p.A + (int64_t)m0 * p.lda : p.A + m0;

    auto load = [&](int kt) {
        const int k0 = kt * BK;
        at.load(Abase, p.lda, mvalid, k0, p.K, tid);
        if constexpr (BKSEG) {
            // B segmented along K: tile kt lies in segment k0 / bseg.
            const int sg = k0 / p.bseg, kl = k0 - sg * p.bseg;
            const bf16_t* Bb = p.B[sg] + (int64_t)n0 * p.ldb;
            bt.load(Bb, p.ldb, nvalid, kl, kl + (p.K - k0), tid);
        } else if constexpr (BKC) {
            bt.load(p.B[bsg] + (int64_t)nb0 * p.ldb, p.ldb, nvalid, k0, p.K, tid);
        } else {
            bt.load(p.B[bsg] + nb0, p.ldb, nvalid, k0, p.K, tid);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (p.K + BK - 1) / BK;
    load(0);
    at.template store<LDK>(As[0], tid);
    bt.template store<LDK>(Bs[0], tid);
    __syncthreads();

    const int frow = lane & 15, fk = (lane >> 4) * 8;
    for (int kt = 0; kt < ntiles; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < ntiles) load(kt + 1);
        const bf16_t* as = As[cur];
        const bf16_t* bs = Bs[cur];
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            u32x4 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(as + (wm * WTM + i * 16 + frow) * LDK + ks * 32 + fk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const u32x4*>(bs + (wn * WTN + j * 16 + frow) * LDK + ks * 32 + fk);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < ntiles) {
            at.template store<LDK>(As[cur ^ 1], tid);
            bt.template store<LDK>(Bs[cur ^ 1], tid);
        }
        __syncthreads();
    }

    // Epilogue.  Lane layout of a 16x16 MFMA result: column = lane % 16,
    // rows 4*(lane/16) + r for r = 0..3.
    const int csg = n0 / p.cseg;
    const int cofs = csg * p.cseg;
    const bf16_t* bias = p.bias[csg];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 16 + (lane & 15);
            if (n >= p.N) continue;
            const int nl = n - cofs;
            float bv = 0.f;
            if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) bv = bias ? bf2f(bias[nl]) : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WTM + i * 16 + (lane >> 4) * 4 + r;
                if (m >= p.M) continue;
                float v = acc[i][j][r];
                if constexpr (OUTF32) {
                    reinterpret_cast<float*>(p.C[csg])[(int64_t)m * p.ldc + nl] = v;
                } else if constexpr (EPI == EPI_STORE) {
                    reinterpret_cast<bf16_t*>(p.C[csg])[(int64_t)m * p.ldc + nl] = f2bf(v);
                } else if constexpr (EPI == EPI_BIAS) {
                    reinterpret_cast<bf16_t*>(p.C[csg])[(int64_t)m * p.ldc + nl] = f2bf(v + bv);
                } else if constexpr (EPI == EPI_BIAS_GELU) {
                    const float u = v + bv;
                    reinterpret_cast<bf16_t*>(p.C[csg])[(int64_t)m * p.ldc + nl] = f2bf(u);
                    p.C2[(int64_t)m * p.ldc2 + nl] = f2bf(gelu_f(u));
                } else {  // EPI_GELU_BWD
                    const float u = bf2f(p.aux[(int64_t)m * p.ldaux + nl]);
                    reinterpret_cast<bf16_t*>(p.C[csg])[(int64_t)m * p.ldc + nl] = f2bf(v * gelu_prime_f(u));
                }
            }
        }
    }
}

template <int BM, int BN, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
    dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 64, AK, BKC, BKSEG, EPI, OUTF32>), grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <int BM, int BN>
hipError_t dispatch(const GemmDesc& d, const GemmArgs& a, hipStream_t s) {
    const bool ak = d.a_kcontig, bk = d.b_kcontig;
    if (ak && !bk && !d.b_kseg && !d.out_f32) {
        if (d.epi == EPI_BIAS_GELU) return launch<BM, BN, true, false, false, EPI_BIAS_GELU, false>(a, s);
        if (d.epi == EPI_BIAS) return launch<BM, BN, true, false, false, EPI_BIAS, false>(a, s);
        if (d.epi == EPI_STORE) return launch<BM, BN, true, false, false, EPI_STORE, false>(a, s);
    } else if (ak && bk && !d.out_f32) {
        if (d.b_kseg && d.epi == EPI_STORE) return launch<BM, BN, true, true, true, EPI_STORE, false>(a, s);
        if (!d.b_kseg && d.epi == EPI_GELU_BWD) return launch<BM, BN, true, true, false, EPI_GELU_BWD, false>(a, s);
        if (!d.b_kseg && d.epi == EPI_STORE) return launch<BM, BN, true, true, false, EPI_STORE, false>(a, s);
    } else if (!ak && !bk && !d.b_kseg && d.out_f32 && d.epi == EPI_STORE) {
        return launch<BM, BN, false, false, false, EPI_STORE, true>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm_bf16(const GemmDesc& d, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return hipSuccess;
    GemmArgs a;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.A = static_cast<const bf16_t*>(d.A); a.lda = d.lda;
    for (int i = 0; i < 3; ++i) {
        a.B[i] = static_cast<const bf16_t*>(d.B[i] ? d.B[i] : d.B[0]);
        a.C[i] = d.C[i] ? d.C[i] : d.C[0];
        a.bias[i] = static_cast<const bf16_t*>(d.bias[i]);
    }
    a.ldb = d.ldb; a.bseg = d.bseg; a.ldc = d.ldc; a.cseg = d.cseg;
    a.C2 = static_cast<bf16_t*>(d.C2); a.ldc2 = d.ldc2;
    a.aux = static_cast<const bf16_t*>(d.aux); a.ldaux = d.ldaux;

    // Tile choice: 128x128 when that still gives about a wave of workgroups
    // per CU and every N-segment holds whole tiles; 64x64 otherwise.
    const bool nseg_ok128 = (d.b_kseg || d.bseg >= (1 << 30) || d.bseg % 128 == 0) &&
                            (d.cseg >= (1 << 30) || d.cseg % 128 == 0);
    const int64_t tiles128 = (int64_t)((d.M + 127) / 128) * ((d.N + 127) / 128);
    if (nseg_ok128 && tiles128 >= 240) return dispatch<128, 128>(d, a, s);
    return dispatch<64, 64>(d, a, s);
}

}  // namespace tp
