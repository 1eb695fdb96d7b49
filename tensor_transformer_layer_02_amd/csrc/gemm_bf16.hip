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
constexpr int STAGES = 3;   // LDS slots: one being read, one written, one free to write
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

// Up to two independent problems of the same layout and epilogue in one
// launch (their tiles are concatenated), each optionally split in K.
struct GemmBatch {
    GemmArgs g[2];
    int n;         // problems
    int tiles0;    // tiles of problem 0
    int tiles;     // tiles of all problems
    int ksplit;    // 1, or 2 (fp32 outputs only: partial tiles are added atomically)
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
// bytes [q*1024, (q+1)*1024) = rows 16q..16q+15.  The per-lane source offset
// (relative to the stage's k0, which moves the buffer base) is fixed.
template <int ROWS>
struct KOperand {
    static constexpr int NI = ROWS / 64;  // instructions per wave
    static_assert(ROWS % 64 == 0, "rows must be a multiple of 64");
    uint32_t off[NI];
    int koff[NI];
    __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int rows_valid) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int q = wave + 4 * i;
            const int row = 16 * q + (lane >> 2);
            koff[i] = ((lane & 3) ^ swz_k(row)) * 8;
            off[i] = row < rows_valid ? (uint32_t)(((int64_t)row * ld + koff[i]) * 2) : OOB;
        }
    }
    // base of the stage: element (0, k0) of the tile
    __device__ __forceinline__ static int64_t stage_elems(int k0, int64_t /*ld*/) { return k0; }
    // Load this thread's chunks of the stage into registers (zeros past the edges).
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int krem, u32x4 (&v)[NI]) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t o = (krem >= BK || koff[i] < krem) ? off[i] : OOB;  // K tail reads zeros
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        }
    }
    __device__ __forceinline__ void store(char* dst, int wave, int lane, const u32x4 (&v)[NI]) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(dst + (wave + 4 * i) * 1024 + lane * 16) = v[i];
    }
};

// One stage of an M/N-contiguous operand, [32][COLS] (k rows).
template <int COLS>
struct MNOperand {
    static constexpr int ROWB = COLS * 2;
    static constexpr int NI = COLS / 64;  // instructions per wave
    static_assert(COLS % 64 == 0, "cols must be a multiple of 64");
    uint32_t off[NI];
    int krow[NI];
    __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int cols_valid) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int o = (wave + 4 * i) * 1024 + lane * 16;
            krow[i] = o / ROWB;
            const int p = (o % ROWB) / 16;
            const int col = (p ^ swz_mn<COLS>(krow[i])) * 8;
            off[i] = col < cols_valid ? (uint32_t)(((int64_t)krow[i] * ld + col) * 2) : OOB;
        }
    }
    __device__ __forceinline__ static int64_t stage_elems(int k0, int64_t ld) { return (int64_t)k0 * ld; }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int krem, u32x4 (&v)[NI]) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t o = (krem >= BK || krow[i] < krem) ? off[i] : OOB;
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        }
    }
    __device__ __forceinline__ void store(char* dst, int wave, int lane, const u32x4 (&v)[NI]) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(dst + (wave + 4 * i) * 1024 + lane * 16) = v[i];
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

// s_waitcnt vmcnt(N) lgkmcnt(0): this thread's loads older than its last N
// have landed in LDS and its own LDS reads have returned.  (vmcnt sits in
// bits [3:0] and [15:14], lgkmcnt in [11:8]; expcnt is left at its maximum.)
// s_waitcnt lgkmcnt(0) only (this thread's LDS writes/reads have completed).
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
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

// Fragments of one k-step (two k16 halves) for one wave.
template <int FM, int FN>
struct Frags {
    u32x4 a[2][FM];
    u32x4 b[2][FN];
};

// MFMAs number FROM..TO-1 of a k-step (index = kk*FM*FN + i*FN + j).
template <int FROM, int TO, int FM, int FN>
__device__ __forceinline__ void run_mfmas(f32x16 (&acc)[FM][FN], const Frags<FM, FN>& F) {
#pragma unroll
    for (int idx = FROM; idx < TO; ++idx) {
        const int kk = idx / (FM * FN), i = (idx % (FM * FN)) / FN, j = idx % FN;
        acc[i][j] = mfma32x32x16(F.a[kk][i], F.b[kk][j], acc[i][j]);
    }
}

// Main loop of one workgroup tile: operand loaders, the LDS ring and the
// accumulators.  (Written as a struct rather than lambdas inside the kernel:
// closure types in a kernel template defeat the host-side stub emission of
// later instantiations with this compiler.)
template <int BM, int BN, bool AK, bool BKC, bool BKSEG>
struct GemmCore {
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int WTM = BM / 2, WTN = BN / 2;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be made of 32x32 blocks");
    using LA = typename std::conditional<AK, KOperand<BM>, MNOperand<BM>>::type;
    using LB = typename std::conditional<BKC, KOperand<BN>, MNOperand<BN>>::type;
    using FR = Frags<FM, FN>;
    static constexpr int NMF = 2 * FM * FN;     // MFMAs per k-step
    static constexpr int HEAD = NMF < 4 ? NMF : 4;  // MFMAs kept in flight across the barrier

    const GemmArgs& p;
    char* smem;
    int lane, wave, wm, wn, nk;
    const bf16_t* abase;
    uint32_t abytes;
    int bsg;
    int64_t boff;
    LA la;
    LB lb;
    u32x4 ra[LA::NI], rb[LB::NI];  // one k-step of operand data on its way to LDS
    f32x16 acc[FM][FN];

    int kbase;  // first k-step of this workgroup's K range

    __device__ __forceinline__ GemmCore(const GemmArgs& args, char* sm, int m0, int n0, int kb, int kn)
        : p(args), smem(sm) {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = tid >> 6;
        wm = wave >> 1;
        wn = wave & 1;
        const int64_t aoff = AK ? (int64_t)m0 * p.lda : m0;
        abase = p.A + aoff;
        abytes = p.a_bytes - (uint32_t)(aoff * 2);
        bsg = 0;
        int nb0 = n0;
        if constexpr (!BKSEG) {
            bsg = n0 / p.bseg;
            nb0 = n0 - bsg * p.bseg;
        }
        boff = BKC ? (int64_t)nb0 * p.ldb : nb0;
        la.init(wave, lane, p.lda, p.M - m0);
        lb.init(wave, lane, p.ldb, p.N - n0);
        kbase = kb;
        nk = kn;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    __device__ __forceinline__ static int64_t kadv(bool kcontig, int k, int64_t ld) {
        return kcontig ? (int64_t)k : (int64_t)k * ld;
    }

    // Global loads of k-step kt into registers.  The k advance moves the
    // buffer base (scalar arithmetic); the lane offsets stay fixed.
    __device__ __forceinline__ void load_stage(int kt) {
        const int k0 = (kbase + kt) * BK;
        const int krem = p.K - k0;
        const int64_t ea = kadv(AK, k0, p.lda);
        la.load(make_rsrc(abase + ea, abytes - (uint32_t)(ea * 2)), krem, ra);
        int sg = bsg, kl = k0;
        if constexpr (BKSEG) {
            sg = k0 / p.bseg;
            kl = k0 - sg * p.bseg;
        }
        const int64_t eb = boff + kadv(BKC, kl, p.ldb);
        lb.load(make_rsrc(p.B[sg] + eb, p.b_bytes[sg] - (uint32_t)(eb * 2)), krem, rb);
    }

    // Registers of k-step kt -> LDS slot kt % STAGES (swizzled layouts).
    __device__ __forceinline__ void store_stage(int kt) {
        char* base = smem + (kt % STAGES) * STAGE;
        la.store(base, wave, lane, ra);
        lb.store(base + A_BYTES, wave, lane, rb);
    }

    __device__ __forceinline__ void read_frags(int slot, FR& F) const {
        const char* as = smem + slot * STAGE;
        const char* bs = as + A_BYTES;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if constexpr (AK) F.a[kk][i] = frag_k(as, wm * WTM + i * 32, kk, lane);
                else F.a[kk][i] = frag_mn<BM>(as, wm * WTM + i * 32, kk, lane);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (BKC) F.b[kk][j] = frag_k(bs, wn * WTN + j * 32, kk, lane);
                else F.b[kk][j] = frag_mn<BN>(bs, wn * WTN + j * 32, kk, lane);
            }
        }
    }

    // One k-step, software-pipelined: the MFMAs of step kt run from registers
    // (Fc) while step kt+2's data goes registers -> LDS, step kt+3's global
    // loads are issued, and step kt+1's fragments are read into Fn.
    // Slot safety: slot (kt+2)%3 held step kt-1, whose fragments every wave
    // read before the barrier of step kt-1; slot (kt+1)%3 was written before
    // this step's barrier.
    __device__ __forceinline__ void step(int kt, FR& Fc, FR& Fn) {
        run_mfmas<0, HEAD>(acc, Fc);
        if (kt + 2 < nk) {
            wait_vm_lgkm<0>();
            store_stage(kt + 2);
        }
        if (kt + 3 < nk) load_stage(kt + 3);
        if (kt + 1 < nk) {
            wait_lgkm();
            stage_barrier();
            read_frags((kt + 1) % STAGES, Fn);
        }
        run_mfmas<HEAD, NMF>(acc, Fc);
    }

    __device__ __forceinline__ void run() {
        if (nk <= 0) return;
        load_stage(0);
        wait_vm_lgkm<0>();
        store_stage(0);
        if (nk > 1) {
            load_stage(1);
            wait_vm_lgkm<0>();
            store_stage(1);
        }
        if (nk > 2) load_stage(2);
        wait_lgkm();
        stage_barrier();
        FR F0, F1;
        read_frags(0, F0);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step(kt, F0, F1);
            step(kt + 1, F1, F0);
        }
        if (kt < nk) step(kt, F0, F1);
        wait_vm_lgkm<0>();
    }
};

template <int BM, int BN, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32>
__global__ void __launch_bounds__(NT, 1) gemm_bf16_kernel(const GemmBatch batch) {
    using Core = GemmCore<BM, BN, AK, BKC, BKSEG>;
    constexpr int RING = STAGES * Core::STAGE;
    constexpr int EROWS = BM / 2, ELD = BN + 8;          // epilogue staging: half a tile of fp32
    constexpr int EBYTES = EROWS * ELD * 4;
    constexpr int SMEM = RING > EBYTES ? RING : EBYTES;
    constexpr int WTM = Core::WTM, WTN = Core::WTN, FM = Core::FM, FN = Core::FN;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // workgroup -> (K split, problem, tile)
    const int split = (int)blockIdx.x / batch.tiles;
    int t = (int)blockIdx.x - split * batch.tiles;
    const int prob = (batch.n > 1 && t >= batch.tiles0) ? 1 : 0;
    if (prob) t -= batch.tiles0;
    const GemmArgs& p = batch.g[prob];
    const int mt = (p.M + BM - 1) / BM, nt = (p.N + BN - 1) / BN;
    int mtile, ntile;
    tile_of(t, mt, nt, mtile, ntile);
    const int n0 = ntile * BN, m0 = mtile * BM;
    const int nk_all = (p.K + BK - 1) / BK;
    const int kchunk = (nk_all + batch.ksplit - 1) / batch.ksplit;
    const int kb = split * kchunk;
    const int kn = min(kchunk, nk_all - kb);

    Core core(p, smem, m0, n0, kb, kn);
    core.run();
    auto& acc = core.acc;

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
                if (batch.ksplit > 1) {
                    continue;  // added below, lane-contiguous
                } else {
                    *reinterpret_cast<f32x4*>(c) = lo;
                    *reinterpret_cast<f32x4*>(c + 4) = hi;
                }
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
        if constexpr (OUTF32) {
            if (batch.ksplit > 1) {
                // The two K halves add into a zeroed block (0 + a + b == 0 + b + a
                // exactly, so the result does not depend on their order); consecutive
                // lanes take consecutive columns so each atomic covers whole lines.
                constexpr int AITEMS = EROWS * BN / NT;
#pragma unroll 4
                for (int it = 0; it < AITEMS; ++it) {
                    const int e = tid + it * NT;
                    const int lr = e / BN, c = e % BN;
                    const int m = m0 + half * EROWS + lr, n = n0 + c;
                    if (m < p.M && n < p.N)
                        atomicAdd(reinterpret_cast<float*>(p.C[csg]) + (int64_t)m * p.ldc + (n - cofs), stage[lr * ELD + c]);
                }
            }
        }
    }
}

template <int BM, int BN, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32>
hipError_t launch(GemmBatch b, hipStream_t s) {
    b.tiles0 = ((b.g[0].N + BN - 1) / BN) * ((b.g[0].M + BM - 1) / BM);
    b.tiles = b.tiles0;
    if (b.n > 1) b.tiles += ((b.g[1].N + BN - 1) / BN) * ((b.g[1].M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BKC, BKSEG, EPI, OUTF32>), dim3(b.tiles * b.ksplit), dim3(NT),
                       0, s, b);
    return hipGetLastError();
}

template <int BM, int BN>
hipError_t dispatch(const GemmDesc& d, const GemmBatch& a, hipStream_t s) {
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

// The 192 x 192 tile serves only the fp32-output weight-gradient GEMMs.
template <>
hipError_t dispatch<192, 192>(const GemmDesc& d, const GemmBatch& a, hipStream_t s) {
    if (!d.a_kcontig && !d.b_kcontig && !d.b_kseg && d.out_f32 && d.epi == EPI_STORE)
        return launch<192, 192, false, false, false, EPI_STORE, true>(a, s);
    return hipErrorInvalidValue;
}

// Bytes readable from `base` for a row-major operand with `rows` rows of
// `cols` elements and row stride `ld` (elements).
uint32_t extent(int64_t rows, int64_t cols, int64_t ld) {
    const int64_t e = ((rows - 1) * ld + cols) * 2;
    return (uint32_t)(e > 0x7fffffff ? 0x7fffffff : e);
}

}  // namespace

namespace {

GemmArgs make_args(const GemmDesc& d) {
    GemmArgs a;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.A = static_cast<const bf16_t*>(d.A); a.lda = d.lda;
    a.a_bytes = d.a_kcontig ? extent(d.M, d.K, d.lda) : extent(d.K, d.M, d.lda);
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
    return a;
}

struct Cand {
    int bm, bn, occ;  // occ: workgroups resident per CU
    double eff;       // relative efficiency of the shape
    bool f32_tn_only;
};
const Cand kCands[] = {{256, 256, 1, 1.0, false}, {256, 192, 1, 0.97, false}, {192, 192, 1, 0.93, true},
                       {256, 128, 1, 0.9, false},  {128, 128, 2, 0.8, false},  {64, 192, 2, 0.6, false},
                       {64, 64, 4, 0.4, false}};

hipError_t dispatch_idx(int c, const GemmDesc& d, const GemmBatch& b, hipStream_t s) {
    switch (c) {
        case 0: return dispatch<256, 256>(d, b, s);
        case 1: return dispatch<256, 192>(d, b, s);
        case 2: return dispatch<192, 192>(d, b, s);
        case 3: return dispatch<256, 128>(d, b, s);
        case 4: return dispatch<128, 128>(d, b, s);
        case 5: return dispatch<64, 192>(d, b, s);
        default: return dispatch<64, 64>(d, b, s);
    }
}

}  // namespace

// Tile shape (and K split) with the least estimated time on 256 CUs:
// waves of workgroups x work per CU per wave / efficiency of the shape.  Every
// N-segment must hold whole tiles; the 192 x 192 tile and the K split serve
// only the fp32 weight-gradient GEMMs (split outputs must be zeroed first).
hipError_t gemm_bf16_batch(const GemmDesc* d, int n, bool allow_split, int* ksplit_out, hipStream_t s) {
    if (n < 1 || n > 2) return hipErrorInvalidValue;
    GemmBatch b;
    b.n = 0;
    for (int i = 0; i < n; ++i)
        if (d[i].M > 0 && d[i].N > 0 && d[i].K > 0) b.g[b.n++] = make_args(d[i]);
    if (ksplit_out) *ksplit_out = 1;
    if (b.n == 0) return hipSuccess;
    const bool tn32 = !d[0].a_kcontig && !d[0].b_kcontig && !d[0].b_kseg && d[0].out_f32;
    int best = -1, best_split = 1;
    double best_cost = 1e300;
    for (int c = 0; c < (int)(sizeof(kCands) / sizeof(kCands[0])); ++c) {
        const Cand& k = kCands[c];
        if (k.f32_tn_only && !tn32) continue;
        bool ok = true;
        int64_t t = 0;
        for (int i = 0; i < n; ++i) {
            const GemmDesc& g = d[i];
            ok = ok && (g.b_kseg || g.bseg >= (1 << 30) || g.bseg % k.bn == 0) &&
                 (g.cseg >= (1 << 30) || g.cseg % k.bn == 0);
            t += (int64_t)((g.M + k.bm - 1) / k.bm) * ((g.N + k.bn - 1) / k.bn);
        }
        if (!ok) continue;
        for (int split = 1; split <= ((allow_split && tn32) ? 2 : 1); ++split) {
            const int64_t items = t * split;
            const int64_t slots = 256 * k.occ;
            const double waves = (double)((items + slots - 1) / slots);
            // per-wave time scales with the K range each workgroup covers
            const double cost = waves * k.bm * k.bn * k.occ / k.eff / split * (split > 1 ? 1.04 : 1.0);
            if (cost < best_cost) { best_cost = cost; best = c; best_split = split; }
        }
    }
    if (best < 0) return hipErrorInvalidValue;
    b.ksplit = best_split;
    if (ksplit_out) *ksplit_out = best_split;
    if (best_split > 1) {  // the K halves add into zeroed output blocks
        for (int i = 0; i < n; ++i) {
            const GemmDesc& g = d[i];
            if (g.M <= 0 || g.N <= 0 || g.K <= 0) continue;
            const int seg = g.cseg < (1 << 30) ? g.cseg : g.N;
            for (int z = 0; z * seg < g.N && z < 3; ++z) {
                const int cols = g.N - z * seg < seg ? g.N - z * seg : seg;
                hipError_t e = zero_f32_2d(static_cast<float*>(g.C[z] ? g.C[z] : g.C[0]), g.M, cols, g.ldc, s);
                if (e != hipSuccess) return e;
            }
        }
    }
    return dispatch_idx(best, d[0], b, s);
}

hipError_t gemm_bf16(const GemmDesc& d, hipStream_t s) { return gemm_bf16_batch(&d, 1, false, nullptr, s); }

}  // namespace tp
