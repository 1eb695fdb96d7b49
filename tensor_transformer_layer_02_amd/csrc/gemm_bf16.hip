// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// Every projection of the layer shard is one of these GEMMs (page "Megatron-LM:
// what the tensor parallelism paper actually says", sections "How transformer
// layers actually decompose" and "The attention heads split"): the
// column-parallel X*A_i and X*W{q,k,v} with a fused bias (+GeLU) epilogue, the
// row-parallel Y*B_i and O*Wo_i producing partial sums, and their backward
// products (input gradients with a fused GeLU' epilogue, fp32 weight gradients).
//
// Design (gfx950):
//  * 32x32x16 MFMAs: with one wave per SIMD they sustain ~86% of the bf16 peak,
//    the 16x16x32 form only ~55% (measured on MI355X), and a 256 x 256 tile
//    needs one wave per SIMD for its 256 accumulator registers.
//  * A 256-thread workgroup (4 wave64s, 2x2) computes a BM x BN tile; K advances
//    in steps of 32 through a ring of four LDS stages, three of them in flight
//    while one is consumed (one barrier per step).  The loads in flight per CU
//    must cover the global-memory latency at the MFMA rate: 96 KB for a
//    256 x 256 tile.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    over the 8 XCDs) owns a compact block of tiles that share A rows and B
//    columns in its L2.
//  * Operands go global -> LDS with buffer_load_dwordx4 ... lds: no VGPR
//    staging, and the buffer range check returns zeros for rows/columns past
//    the matrix edge and for the K tail (a lane whose source is out of range is
//    given an out-of-range offset).
//  * An operand that is contiguous along K is stored [rows][32] (64 B rows);
//    one that is contiguous along M or N (the transposed operands of the
//    weight gradients, and the weights of x*W) is stored [32][cols] as it
//    lies in memory.  Both layouts XOR-swizzle their 16-byte chunks by row so
//    that the MFMA fragment reads hit distinct LDS banks; the swizzle is
//    applied by choosing which global chunk each lane fetches.
//  * K-contiguous fragments are read with ds_read_b128; M/N-contiguous ones
//    with two ds_read_b64_tr_b16, which transpose 4x16 blocks across each
//    16-lane group so that every lane receives 4 consecutive K values of its
//    row.  No register transposes are needed.
//  * The epilogue stages each half of the fp32 tile through LDS so that every
//    thread owns 8 consecutive columns of a row: bias, GeLU, GeLU' (reading U)
//    and the stores all move 16 bytes per lane.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int NT = 256;
constexpr int BK = 32;      // K elements per pipeline stage
constexpr int STAGES = 4;   // LDS ring: three stages in flight while one is consumed
constexpr uint32_t OOB = 0x80000000u;  // voffset past any buffer: the load returns zeros

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short v4i16;

struct GemmArgs {
    int M, N, K;
    const bf16_t* A;
    int64_t lda;
    uint32_t a_bytes;   // readable extent of A from its base (buffer range)
    const bf16_t* B[3];
    int64_t ldb;
    uint32_t b_bytes[3];
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Swizzle of a [rows][32] K-contiguous tile (4 chunks of 16 B per 64-byte row):
// the fragment read of 16 consecutive rows at one logical chunk is conflict-free.
__device__ __forceinline__ int swz_k(int row) { return (row >> 2) & 3; }

// Swizzle of a [32][cols] M/N-contiguous tile, by k-row.  One transposed
// fragment read touches rows 8g + r (+4), g, r in 0..3; the XOR spreads those
// 16 rows over all banks (rows of a multiple of 256 B) or, with the row
// parity, over both halves of the banks (rows of an odd multiple of 128 B).
template <int COLS>
__device__ __forceinline__ int swz_mn(int k) {
    if constexpr ((COLS * 2) % 256 == 0)
        return 2 * ((k & 3) | (((k >> 3) & 1) << 2));   // 0..14, within 16-chunk groups
    else
        return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));  // 0..6, within 8-chunk groups
}

// One stage of a K-contiguous operand, [ROWS][32]: instruction q fills LDS
// bytes [q*1024, (q+1)*1024) = rows 16q..16q+15.
template <int ROWS>
struct KOperand {
    static constexpr int NI = ROWS / 64;  // instructions per wave
    static_assert(ROWS % 64 == 0, "rows must be a multiple of 64");
    int row[NI];
    int koff[NI];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int q = wave + 4 * i;
            row[i] = 16 * q + (lane >> 2);
            koff[i] = ((lane & 3) ^ swz_k(row[i])) * 8;
        }
    }
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t ld, int rows_valid, int k0,
                                          int kvalid, char* dst, int wave) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = k0 + koff[i];
            const bool ok = row[i] < rows_valid && k < kvalid;
            const uint32_t off = ok ? (uint32_t)(((int64_t)row[i] * ld + k) * 2) : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave + 4 * i) * 1024), 16, off, 0, 0, 0);
        }
    }
};

// One stage of an M/N-contiguous operand, [32][COLS] (k rows).
template <int COLS>
struct MNOperand {
    static constexpr int ROWB = COLS * 2;
    static constexpr int NI = COLS / 64;  // instructions per wave
    static_assert(COLS % 64 == 0, "cols must be a multiple of 64");
    int krow[NI];
    int col[NI];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int off = (wave + 4 * i) * 1024 + lane * 16;
            krow[i] = off / ROWB;
            const int p = (off % ROWB) / 16;
            col[i] = (p ^ swz_mn<COLS>(krow[i])) * 8;
        }
    }
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t ld, int cols_valid, int k0,
                                          int kvalid, char* dst, int wave) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = k0 + krow[i];
            const bool ok = col[i] < cols_valid && k < kvalid;
            const uint32_t off = ok ? (uint32_t)(((int64_t)k * ld + col[i]) * 2) : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave + 4 * i) * 1024), 16, off, 0, 0, 0);
        }
    }
};

// Fragment (32 rows x 8 k) of a K-contiguous tile for the 32x32x16 MFMA:
// lane l holds row rb + l%32, k = 16*kk + 8*(l/32) + 0..7.
__device__ __forceinline__ u32x4 frag_k(const char* t, int rb, int kk, int lane) {
    const int r = rb + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const u32x4*>(t + r * 64 + ((c ^ swz_k(r)) * 16));
}

// Same fragment from an M/N-contiguous [32][COLS] tile via two transposed
// reads.  ds_read_b64_tr_b16 works on 16-lane groups: lane j of a group
// supplies row j/4, columns 4*(j%4)..+3 of a 4x16 block and lane i receives
// column i, i.e. 4 consecutive k of one row.  Group G = l/16 covers rows
// cb + 16*(G%2) .. +15 and k-octet G/2.
template <int COLS>
__device__ __forceinline__ u32x4 frag_mn(const char* t, int cb, int kk, int lane) {
    const int j = lane & 15, G = lane >> 4;
    const int col = cb + 16 * (G & 1) + 4 * (j & 3);
    const int c = col >> 3;
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = 16 * kk + 8 * (G >> 1) + 4 * h + (j >> 2);
        const char* p = t + k * (COLS * 2) + ((c ^ swz_mn<COLS>(k)) * 16) + (col & 7) * 2;
        const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        out[2 * h] = w[0];
        out[2 * h + 1] = w[1];
    }
    return out;
}

// Workgroup barrier WITHOUT the release/acquire fences of __syncthreads():
// the fence would make the compiler wait for every in-flight global->LDS load
// (they count as LDS writes) and drain the prefetch pipeline at each step.
// Callers wait (vmcnt) for exactly the loads they need first; the scheduling
// barriers keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt vmcnt(N): vmcnt in bits [3:0] and [15:14]; expcnt/lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs; the
// first step makes the ids each XCD receives contiguous, the second walks the
// tiles in groups of GM tile-rows so that an XCD's tiles share A rows and B
// columns in its L2.
__device__ __forceinline__ void tile_of(int b, int mt, int nt, int& mtile, int& ntile) {
    constexpr int GM = 8;
    const int nwg = mt * nt;
    const int per = (nwg + 7) / 8, r = nwg % 8, x = b % 8, q = b / 8;
    const int id = (r == 0 || x < r) ? x * per + q : r * per + (x - r) * (per - 1) + q;
    const int gsize = GM * nt;
    const int first_m = (id / gsize) * GM;
    const int gm = min(mt - first_m, GM);
    const int in = id % gsize;
    mtile = first_m + in % gm;
    ntile = in / gm;
}

template <int BM, int BN, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32>
__global__ void __launch_bounds__(NT, 1) gemm_bf16_kernel(const GemmArgs p) {
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int RING = STAGES * STAGE;
    constexpr int EROWS = BM / 2, ELD = BN + 8;          // epilogue staging: half a tile of fp32
    constexpr int EBYTES = EROWS * ELD * 4;
    constexpr int SMEM = RING > EBYTES ? RING : EBYTES;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be made of 32x32 blocks");
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int mt = (p.M + BM - 1) / BM, nt = (p.N + BN - 1) / BN;
    int mtile, ntile;
    tile_of(blockIdx.x, mt, nt, mtile, ntile);
    const int n0 = ntile * BN, m0 = mtile * BM;
    const int mvalid = p.M - m0, nvalid = p.N - n0;

    const int64_t aoff = AK ? (int64_t)m0 * p.lda : m0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + aoff, p.a_bytes - (uint32_t)(aoff * 2));
    int bsg = 0, nb0 = n0;
    if constexpr (!BKSEG) {
        bsg = n0 / p.bseg;
        nb0 = n0 - bsg * p.bseg;
    }
    const int64_t boff = BKC ? (int64_t)nb0 * p.ldb : nb0;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B[bsg] + boff, p.b_bytes[bsg] - (uint32_t)(boff * 2));

    typename std::conditional<AK, KOperand<BM>, MNOperand<BM>>::type la;
    typename std::conditional<BKC, KOperand<BN>, MNOperand<BN>>::type lb;
    la.init(wave, lane);
    lb.init(wave, lane);
    constexpr int NL = decltype(la)::NI + decltype(lb)::NI;  // loads per thread per stage

    auto issue = [&](int kt) {
        char* base = smem + (kt % STAGES) * STAGE;
        const int k0 = kt * BK;
        la.issue(ra, p.lda, mvalid, k0, p.K, base, wave);
        if constexpr (BKSEG) {
            const int sg = k0 / p.bseg, kl = k0 - sg * p.bseg;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(p.B[sg] + boff, p.b_bytes[sg] - (uint32_t)(boff * 2));
            lb.issue(r, p.ldb, nvalid, kl, kl + (p.K - k0), base + A_BYTES, wave);
        } else {
            lb.issue(rb, p.ldb, nvalid, k0, p.K, base + A_BYTES, wave);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (p.K + BK - 1) / BK;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s);

    for (int kt = 0; kt < nk; ++kt) {
        // stages kt+1 .. kt+STAGES-2 may stay in flight; stage kt must have landed
        const int ahead = nk - 1 - kt;
        if (ahead >= 2) wait_vm<2 * NL>();
        else if (ahead == 1) wait_vm<NL>();
        else wait_vm<0>();
        stage_barrier();  // stage kt visible to all; every wave is done with stage kt-1
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);

        const char* as = smem + (kt % STAGES) * STAGE;
        const char* bs = as + A_BYTES;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            u32x4 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if constexpr (AK) af[i] = frag_k(as, wm * WTM + i * 32, kk, lane);
                else af[i] = frag_mn<BM>(as, wm * WTM + i * 32, kk, lane);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (BKC) bfr[j] = frag_k(bs, wn * WTN + j * 32, kk, lane);
                else bfr[j] = frag_mn<BN>(bs, wn * WTN + j * 32, kk, lane);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
        }
    }

    // Epilogue: each half of the tile (rows owned by wave-row wm) goes through
    // LDS as fp32 so that every thread then handles 8 consecutive columns of a
    // row: 16-byte loads of bias / U and 16-byte stores of the outputs.
    const int csg = n0 / p.cseg;
    const int cofs = csg * p.cseg;
    float* stage = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();
        if (wm == half) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        stage[(i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * ELD + wn * WTN + j * 32 +
                              (lane & 31)] = acc[i][j][r];
        }
        __syncthreads();
        constexpr int GPR = BN / 8;                 // 8-column groups per row
        constexpr int ITEMS = EROWS * GPR / NT;
        static_assert(ITEMS >= 1 && (EROWS * GPR) % NT == 0, "epilogue split");
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int e = tid + it * NT;
            const int lr = e / GPR, cg = e % GPR;
            const int m = m0 + half * EROWS + lr, n = n0 + cg * 8;
            if (m >= p.M || n >= p.N) continue;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(stage + lr * ELD + cg * 8);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(stage + lr * ELD + cg * 8 + 4);
            float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int nl = n - cofs;
            if constexpr (OUTF32) {
                float* c = reinterpret_cast<float*>(p.C[csg]) + (int64_t)m * p.ldc + nl;
                *reinterpret_cast<f32x4*>(c) = lo;
                *reinterpret_cast<f32x4*>(c + 4) = hi;
            } else {
                if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
                    const bf16_t* bias = p.bias[csg];
                    if (bias) {
                        const u32x4 bw = *reinterpret_cast<const u32x4*>(bias + nl);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            v[2 * q] += __uint_as_float(bw[q] << 16);
                            v[2 * q + 1] += __uint_as_float(bw[q] & 0xffff0000u);
                        }
                    }
                }
                if constexpr (EPI == EPI_GELU_BWD) {
                    const u32x4 uw = *reinterpret_cast<const u32x4*>(p.aux + (int64_t)m * p.ldaux + nl);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[2 * q] *= gelu_prime_f(__uint_as_float(uw[q] << 16));
                        v[2 * q + 1] *= gelu_prime_f(__uint_as_float(uw[q] & 0xffff0000u));
                    }
                }
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_bf2(v[2 * q], v[2 * q + 1]);
                *reinterpret_cast<u32x4*>(reinterpret_cast<bf16_t*>(p.C[csg]) + (int64_t)m * p.ldc + nl) = o;
                if constexpr (EPI == EPI_BIAS_GELU) {
                    u32x4 y;
#pragma unroll
                    for (int q = 0; q < 4; ++q) y[q] = pack_bf2(gelu_f(v[2 * q]), gelu_f(v[2 * q + 1]));
                    *reinterpret_cast<u32x4*>(p.C2 + (int64_t)m * p.ldc2 + nl) = y;
                }
            }
        }
    }
}

template <int BM, int BN, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
    const int tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BKC, BKSEG, EPI, OUTF32>), dim3(tiles), dim3(NT), 0, s, a);
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

// Bytes readable from `base` for a row-major operand with `rows` rows of
// `cols` elements and row stride `ld` (elements).
uint32_t extent(int64_t rows, int64_t cols, int64_t ld) {
    const int64_t e = ((rows - 1) * ld + cols) * 2;
    return (uint32_t)(e > 0x7fffffff ? 0x7fffffff : e);
}

}  // namespace

hipError_t gemm_bf16(const GemmDesc& d, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return hipSuccess;
    GemmArgs a;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.A = static_cast<const bf16_t*>(d.A); a.lda = d.lda;
    a.a_bytes = d.a_kcontig ? extent(d.M, d.K, d.lda) : extent(d.K, d.M, d.lda);
    // N-extent of one B segment
    const int nseg = (!d.b_kseg && d.bseg < (1 << 30)) ? d.bseg : d.N;
    const int kseg = (d.b_kseg && d.bseg < (1 << 30)) ? d.bseg : d.K;
    for (int i = 0; i < 3; ++i) {
        a.B[i] = static_cast<const bf16_t*>(d.B[i] ? d.B[i] : d.B[0]);
        a.b_bytes[i] = d.b_kcontig ? extent(nseg, kseg, d.ldb) : extent(kseg, nseg, d.ldb);
        a.C[i] = d.C[i] ? d.C[i] : d.C[0];
        a.bias[i] = static_cast<const bf16_t*>(d.bias[i]);
    }
    a.ldb = d.ldb; a.bseg = d.bseg; a.ldc = d.ldc; a.cseg = d.cseg;
    a.C2 = static_cast<bf16_t*>(d.C2); a.ldc2 = d.ldc2;
    a.aux = static_cast<const bf16_t*>(d.aux); a.ldaux = d.ldaux;

    // Tile choice: the tile shape with the least estimated time on 256 CUs:
    // (number of waves of workgroups) x (work per CU per wave) / (measured-ish
    // efficiency of the shape).  Every N-segment must be made of whole tiles.
    struct Cand {
        int bm, bn, occ;  // occ: workgroups resident per CU
        double eff;
    };
    static const Cand cands[] = {{256, 256, 1, 1.0}, {256, 192, 1, 0.97}, {256, 128, 1, 0.9},
                                 {128, 128, 2, 0.8}, {64, 192, 2, 0.6},  {64, 64, 4, 0.4}};
    auto seg_ok = [&](int bn) {
        return (d.b_kseg || d.bseg >= (1 << 30) || d.bseg % bn == 0) && (d.cseg >= (1 << 30) || d.cseg % bn == 0);
    };
    int best = -1;
    double best_cost = 1e300;
    for (int c = 0; c < (int)(sizeof(cands) / sizeof(cands[0])); ++c) {
        if (!seg_ok(cands[c].bn)) continue;
        const int64_t t = (int64_t)((d.M + cands[c].bm - 1) / cands[c].bm) * ((d.N + cands[c].bn - 1) / cands[c].bn);
        const int64_t slots = 256 * cands[c].occ;
        const double waves = (double)((t + slots - 1) / slots);
        const double cost = waves * cands[c].bm * cands[c].bn * cands[c].occ / cands[c].eff;
        if (cost < best_cost) { best_cost = cost; best = c; }
    }
    switch (best) {
        case 0: return dispatch<256, 256>(d, a, s);
        case 1: return dispatch<256, 192>(d, a, s);
        case 2: return dispatch<256, 128>(d, a, s);
        case 3: return dispatch<128, 128>(d, a, s);
        case 4: return dispatch<64, 192>(d, a, s);
        default: return dispatch<64, 64>(d, a, s);
    }
}

}  // namespace tp
