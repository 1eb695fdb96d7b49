// 16-bit GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, or _f16 for
// IEEE half storage), fp32 accumulation.  The storage format is a template
// parameter (ST: bf16_t or f16_t) that only selects the MFMA and the
// conversions of the epilogue; loads, LDS layout and tiling are shared.
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
//  * A workgroup of 4 wave64s (2x2) computes a BM x BN tile; the 256 x 192
//    tile also comes with 8 (4x2, two waves per SIMD, which hide each
//    other's latencies: 3-16% faster on the same tile, and picked by the
//    cost model for most of the layer's GEMMs), and the 192 x 192 fp32
//    weight-gradient tile with 8 waves in two K groups (each group runs two
//    of the four k16 sub-steps of every step on the shared LDS stage; the
//    second group's sums are added into the first's at the end, in a fixed
//    order).  K
//    advances in steps of 64 (full 128-byte lines of a K-contiguous row) through
//    two LDS slots, one barrier per step; the pipeline is described at
//    GemmCore.  Operands travel global -> registers -> LDS: buffer loads are
//    issued one or two steps before their data is stored, and every LDS read,
//    LDS write and global load is paired with an MFMA by scheduling hints, in
//    a branch-free steady state.  The K-group tile instead loads straight into
//    LDS (buffer loads with the LDS flag) through three slots, two steps
//    ahead: no registers hold operands in transit and no LDS stores are
//    issued, which is what bounds the register-staged loop (timing copies
//    without the MFMAs run the MLP weight-gradient pair in 109 of its 150 us,
//    without the LDS stores in 83).
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    over the 8 XCDs) owns a compact block of tiles that share A rows and B
//    columns in its L2.
//  * The buffer range check returns zeros for rows/columns past the matrix
//    edge and for the K tail (a lane whose source is out of range is given an
//    out-of-range offset), so edge tiles need no special path.
//  * An operand that is contiguous along K is stored [rows][64] (128 B rows);
//    one that is contiguous along M or N (the transposed operands of the
//    weight gradients, and the weights of x*W) is stored [64][cols] as it
//    lies in memory.  Both layouts XOR-swizzle their 16-byte chunks by row so
//    that the MFMA fragment reads hit distinct LDS banks; the swizzle is
//    applied by choosing which global chunk each lane fetches.
//  * K-contiguous fragments are read with ds_read_b128; M/N-contiguous ones
//    with two ds_read_b64_tr_b16, which transpose 4x16 blocks across each
//    16-lane group so that every lane receives 4 consecutive K values of its
//    row.  No register transposes are needed.
//  * The MFMAs accumulate C^T blocks, so a lane holds 4 consecutive columns
//    of one row.  bf16 outputs get their bias and GeLU in registers and go
//    through LDS once as a bf16 image (8-byte writes, no bank conflicts), from
//    which every thread stores 16 bytes of a row; fp32 outputs and the GeLU'
//    epilogue (which reads U) stage half a tile at a time as fp32.
//  * Two independent problems of one layout (the two weight gradients of a
//    sublayer) share a launch; fp32 outputs may split K in two.  The first
//    split writes the output, the second its partial sums to a slab of the
//    caller's work buffer with plain stores, and a reduction kernel adds the
//    slab into the output (one fixed order: deterministic, and no atomics).
#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int BK = 64;      // K elements per pipeline stage (128-byte rows)
constexpr int STAGES = 2;   // LDS slots
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
    int gelu_tanh;
    float* rd;  // EPI_STORE_ROWDOT
    int rd_seq, rd_heads, rd_dh;
};

// Up to two independent problems of the same layout and epilogue in one
// launch (their tiles are concatenated), each optionally split in K.
struct GemmBatch {
    GemmArgs g[2];
    int n;         // problems
    int tiles0;    // tiles of problem 0
    int tiles;     // tiles of all problems
    int ksplit;    // 1, or 2 (fp32 outputs only)
    float* part;   // K split: split s > 0 writes slab s - 1, problem i at poff[i] (dense [M][N])
    int64_t pslab;
    int64_t poff[2];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Swizzle of a [rows][64] K-contiguous tile (8 chunks of 16 B per 128-byte
// row): rows 2r and 2r+1 sit in the two halves of the banks, and the XOR
// spreads 8 row pairs over the 8 chunk positions, so the fragment read of 16
// consecutive rows at one logical chunk is conflict-free.
__device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }

// Swizzle of a [64][cols] M/N-contiguous tile, by k-row.  A half-wave of a
// transposed fragment read touches 4 consecutive k-rows x 4 consecutive
// chunks (64 B per row); the XOR moves the 4 rows to 4 different 4-chunk
// bank groups (rows of a multiple of 256 B: by k & 3; rows of an odd
// multiple of 128 B, where consecutive rows already alternate halves: by
// bit 1 of k), so every half-wave hits each bank once.
template <int COLS>
__device__ __forceinline__ int swz_mn(int k) {
    if constexpr ((COLS * 2) % 256 == 0)
        return (k & 3) << 2;
    else
        return ((k >> 1) & 1) << 2;
}

// One stage of a K-contiguous operand, [ROWS][64], loaded by NWV waves:
// instruction q fills LDS bytes [q*1024, (q+1)*1024) = rows 8q..8q+7, eight
// lanes per 128-byte row.  The per-lane source offset (relative to the stage's
// k0, which moves the buffer base) is fixed; so is the lane's k chunk, since
// q = wave + NWV*i keeps the swizzle of its rows independent of i.
template <int ROWS, int NWV>
struct KOperand {
    static constexpr int NI = ROWS / (8 * NWV);  // instructions per wave
    static_assert(ROWS % (8 * NWV) == 0, "rows must be a multiple of 8 per wave");
    uint32_t off[NI];
    int koff;
    __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int rows_valid) {
        koff = ((lane & 7) ^ swz_k(8 * wave + (lane >> 3))) * 8;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = 8 * (wave + NWV * i) + (lane >> 3);
            off[i] = row < rows_valid ? (uint32_t)(((int64_t)row * ld + koff) * 2) : OOB;
        }
    }
    // Load this thread's chunks of the stage into registers (zeros past the edges).
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int krem, u32x4 (&v)[NI]) const {
        const bool kin = krem >= BK || koff < krem;  // K tail reads zeros
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t o = kin ? off[i] : OOB;
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        }
    }
    __device__ __forceinline__ void store(char* dst, int wave, int lane, const u32x4 (&v)[NI]) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(dst + (wave + NWV * i) * 1024 + lane * 16) = v[i];
    }
    // The same chunks straight into the LDS stage `dst` (buffer loads with the
    // LDS flag: lane l's 16 bytes land at the instruction's base + 16 l, the
    // bytes store() would write), no registers involved.
    __device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t rs, int krem, char* dst, int wave) const {
        const bool kin = krem >= BK || koff < krem;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave + NWV * i) * 1024), 16,
                                                     kin ? off[i] : OOB, 0, 0, 0);
    }
};

// One stage of an M/N-contiguous operand, [64][COLS] (k rows), loaded by NWV waves.
template <int COLS, int NWV>
struct MNOperand {
    static constexpr int ROWB = COLS * 2;
    static constexpr int NI = COLS / (8 * NWV);  // instructions per wave
    static_assert(COLS % (8 * NWV) == 0, "cols must be a multiple of 8 per wave");
    uint32_t off[NI];
    int o0;  // LDS byte offset of this lane's first chunk; chunk i is at o0 + 1024 NWV i
    __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int cols_valid) {
        o0 = wave * 1024 + lane * 16;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int o = o0 + 1024 * NWV * i;
            const int krow = o / ROWB;
            const int p = (o % ROWB) / 16;
            const int col = (p ^ swz_mn<COLS>(krow)) * 8;
            off[i] = col < cols_valid ? (uint32_t)(((int64_t)krow * ld + col) * 2) : OOB;
        }
    }
    // The chunk's k row is recomputed rather than kept: registers are scarce.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int krem, u32x4 (&v)[NI]) const {
        const int klim = krem >= BK ? BK : krem;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t o = (o0 + 1024 * NWV * i) / ROWB < klim ? off[i] : OOB;
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        }
    }
    __device__ __forceinline__ void store(char* dst, int wave, int lane, const u32x4 (&v)[NI]) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(dst + (wave + NWV * i) * 1024 + lane * 16) = v[i];
    }
    __device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t rs, int krem, char* dst, int wave) const {
        const int klim = krem >= BK ? BK : krem;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave + NWV * i) * 1024), 16,
                                                     (o0 + 1024 * NWV * i) / ROWB < klim ? off[i] : OOB, 0, 0, 0);
    }
};

// Fragment (32 rows x 8 k) of a K-contiguous tile for the 32x32x16 MFMA:
// lane l holds row rb + l%32, k = 16*kk + 8*(l/32) + 0..7.
__device__ __forceinline__ u32x4 frag_k(const char* t, int rb, int kk, int lane) {
    const int r = rb + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const u32x4*>(t + r * (BK * 2) + ((c ^ swz_k(r)) * 16));
}

// Same fragment from an M/N-contiguous [64][COLS] tile via two transposed
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

// Workgroup -> tile, in two steps.  Workgroups are dealt round-robin to the 8
// XCDs; xcd_id makes the ids each XCD receives contiguous over all the tiles of
// a launch (so with two problems each XCD works on one of them, or on the end of
// one and the start of the other), and tile_of walks a problem's tiles in groups
// of GM tile-rows so that an XCD's tiles share A rows and B columns in its L2.
__device__ __forceinline__ int xcd_id(int b, int nwg) {
    const int per = (nwg + 7) / 8, r = nwg % 8, x = b % 8, q = b / 8;
    return (r == 0 || x < r) ? x * per + q : r * per + (x - r) * (per - 1) + q;
}

__device__ __forceinline__ void tile_of(int id, int mt, int nt, int& mtile, int& ntile) {
    constexpr int GM = 8;
    const int gsize = GM * nt;
    const int first_m = (id / gsize) * GM;
    const int gm = min(mt - first_m, GM);
    const int in = id % gsize;
    mtile = first_m + in % gm;
    ntile = in / gm;
}

// Fragments of one k16 sub-step for one wave.
template <int FM, int FN>
struct Half {
    u32x4 a[FM];
    u32x4 b[FN];
};

// MFMAs number FROM..TO-1 of a sub-step (index = i*FN + j).  The B fragment
// goes in as the first operand, so block (i, j) accumulates C^T: lane l holds
// row l%32 of the block and the 4 consecutive columns 8q + 4*(l/32) .. +3 in
// values 4q .. 4q+3 (q = 0..3), which the epilogue writes 8 or 16 bytes at a time.
template <typename ST, int FROM, int TO, int FM, int FN>
__device__ __forceinline__ void run_mfmas(f32x16 (&acc)[FM][FN], const Half<FM, FN>& F) {
#pragma unroll
    for (int idx = FROM; idx < TO; ++idx) {
        const int i = idx / FN, j = idx % FN;
        acc[i][j] = Store16<ST>::mfma(F.b[j], F.a[i], acc[i][j]);
    }
}

// Scheduling hint for one scheduling region: pair each MFMA with one memory
// instruction, taking first NR LDS reads, then NW LDS writes, then NL global
// loads.
template <int NMFMA, int NR, int NW, int NL>
__device__ __forceinline__ void interleave() {
    constexpr int NOPS = NR + NW + NL;
    constexpr int N = NMFMA > NOPS ? NMFMA : NOPS;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // DS read
        else if (i < NR + NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        else if (i < NOPS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
        if (i < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    }
}

// Workgroups per CU a tile shape is built for (registers: 512 / occupancy per lane).
template <int BM, int BN, int NWV>
constexpr int tile_occupancy() {
    return NWV == 8 ? 1 : BM * BN <= 64 * 64 ? 4 : BM * BN <= 128 * 192 ? 2 : 1;
}

// Main loop of one workgroup tile: operand loaders, the LDS ring and the
// accumulators.  (Written as a struct rather than lambdas inside the kernel:
// closure types in a kernel template defeat the host-side stub emission of
// later instantiations with this compiler.)
//
// Pipeline.  A k-step (64 of K) is four k16 sub-steps of FM*FN MFMAs each,
// with one barrier per step, before the last sub-step.  Step kt lives in LDS
// slot kt&1; fragments alternate between two register sets Fa/Fb; operand
// data travels global -> registers (two sets per operand, by step parity) ->
// LDS:
//   sub-step 0: read k16 #1 of step kt; store A of step kt+1 to slot (kt+1)&1;
//               load A of step kt+1+NSET into the registers just stored;
//   sub-step 1: read #2; the same for B;
//   sub-step 2: read #3; wait for this wave's LDS operations; barrier;
//   sub-step 3: read #0 of step kt+1 (slot (kt+1)&1).
// A store to a slot comes after the barrier that follows every read of its
// previous contents (step kt-1, read up to sub-step 2 of step kt-1), and
// before the barrier that precedes every read of the new contents.  Global
// loads are issued NSET steps before their data is stored.  Steps past the end
// of the K range load from an empty buffer range (zeros, no memory access);
// their stores and fragment reads are never consumed, so the steady state has
// no branches for the scheduler to work around.
template <int BM, int BN, bool AK, bool BKC, bool BKSEG, int NWV, int KG = 1, typename ST = bf16_t>
struct GemmCore {
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // waves in (NWV/KG)/2 rows x 2 columns; KG groups of them split each K step
    static constexpr int WTM = BM / (NWV / KG / 2), WTN = BN / 2;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be made of 32x32 blocks");
    using LA = typename std::conditional<AK, KOperand<BM, NWV>, MNOperand<BM, NWV>>::type;
    using LB = typename std::conditional<BKC, KOperand<BN, NWV>, MNOperand<BN, NWV>>::type;
    using HF = Half<FM, FN>;
    static constexpr int NM = FM * FN;           // MFMAs per sub-step
    static constexpr int PRE = NM < 2 ? NM : 2;  // last-sub-step MFMAs issued before the barrier
    static constexpr int NRD = (AK ? 1 : 2) * FM + (BKC ? 1 : 2) * FN;  // LDS reads per sub-step
    static_assert(BK == 64, "four k16 sub-steps per step");
    // Register sets per operand for data on its way to LDS: two let the
    // global loads run two steps ahead; the 256 x 256 tile has no room for
    // the second set (except with two plain K-contiguous operands) and loads
    // one step ahead.
    // LDS slots: two for the register-staged pipeline; the K-group tiles load
    // straight into LDS through three, two steps ahead.
    static constexpr int RINGS = KG == 2 ? 3 : STAGES;
    static constexpr int NLD = LA::NI + LB::NI;  // direct loads per thread and step
    static constexpr int NSET = (KG == 2 || (BM == 256 && BN == 256 && (NWV == 8 || !(AK && BKC && !BKSEG)))) ? 1 : 2;
    // The 8-wave 256 x 192 tile: A goes straight into LDS through three slots
    // (two steps ahead), B through two register sets into two slots (three A
    // slots plus two B slots = 144 KB; three whole stages would not fit).
    // Only this one-per-CU tile: the same pipeline on the 4-wave tiles that
    // run two or four per CU gave intermittently wrong blocks on the GPU.
    static constexpr bool ADIRECT = KG == 1 && NSET == 2 && NWV == 8 && BM == 256 && BN == 192;
    static constexpr int LDS_BYTES = ADIRECT ? 3 * A_BYTES + 2 * B_BYTES : RINGS * STAGE;

    char* smem;
    int lane, wave, wm, wn, nk, kk0;
    int kbase;  // first k-step of this workgroup's K range
    int kend;   // end of this workgroup's K range (elements)
    const bf16_t* abase;
    uint32_t abytes;
    int64_t lda, ldb, boff;
    int bseg;
    uint64_t bsel[3];   // B base address selection (see load_b)
    uint32_t bbsel[3];
    LA la;
    LB lb;
    u32x4 ra[NSET][LA::NI], rb[NSET][LB::NI];  // operand data on its way to LDS
    f32x16 acc[FM][FN];

    __device__ __forceinline__ GemmCore(const GemmArgs& p, char* sm, int m0, int n0, int kb, int kn) : smem(sm) {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = tid >> 6;
        wm = (wave % (NWV / KG)) >> 1;
        wn = wave & 1;
        kk0 = KG == 2 ? 2 * (wave / (NWV / KG)) : 0;  // first k16 sub-step of this wave's group
        lda = p.lda;
        ldb = p.ldb;
        bseg = p.bseg;
        const int64_t aoff = AK ? (int64_t)m0 * lda : m0;
        abase = p.A + aoff;
        abytes = p.a_bytes - (uint32_t)(aoff * 2);
        int nb0 = n0;
        bsel[1] = bsel[2] = 0;
        bbsel[1] = bbsel[2] = 0;
        if constexpr (BKSEG) {
            // segment q's base and extent = entry 0 + entry q (wrapping arithmetic)
            bsel[0] = reinterpret_cast<uint64_t>(p.B[0]);
            bbsel[0] = p.b_bytes[0];
#pragma unroll
            for (int q = 1; q < 3; ++q) {
                bsel[q] = reinterpret_cast<uint64_t>(p.B[q]) - bsel[0];
                bbsel[q] = p.b_bytes[q] - bbsel[0];
            }
        } else {
            const int sg = n0 / bseg;
            nb0 = n0 - sg * bseg;
            bsel[0] = reinterpret_cast<uint64_t>(p.B[sg]);
            bbsel[0] = p.b_bytes[sg];
        }
        boff = BKC ? (int64_t)nb0 * ldb : nb0;
        la.init(wave, lane, lda, p.M - m0);
        lb.init(wave, lane, ldb, p.N - n0);
        kbase = kb;
        nk = kn;
        kend = min(p.K, (kb + kn) * BK);
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
    // buffer base (scalar arithmetic); the lane offsets stay fixed.  Past the
    // K range every lane takes the out-of-range offset; the base then stays
    // at k = 0 (no branch: a conditional 64-bit multiply would become one and
    // split the scheduling region).
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_a(int kt, int& krem) const {
        const int k0 = (kbase + kt) * BK;
        krem = kend - k0;
        const int kc = krem > 0 ? k0 : 0;
        const int64_t e = kadv(AK, kc, lda);
        return make_rsrc(abase + e, abytes - (uint32_t)(e * 2));
    }
    __device__ __forceinline__ void load_a(int kt, u32x4 (&v)[LA::NI]) const {
        int krem;
        const __amdgpu_buffer_rsrc_t rs = rsrc_a(kt, krem);
        la.load(rs, krem, v);
    }
    __device__ __forceinline__ void load_b(int kt, u32x4 (&v)[LB::NI]) const {
        int krem;
        const __amdgpu_buffer_rsrc_t rs = rsrc_b(kt, krem);
        lb.load(rs, krem, v);
    }
    // Direct global -> LDS loads of step kt into the stage at `dst` (the K-group tiles).
    __device__ __forceinline__ void load_lds(int kt, char* dst) const {
        int krem;
        const __amdgpu_buffer_rsrc_t ra_ = rsrc_a(kt, krem);
        la.load_lds(ra_, krem, dst, wave);
        const __amdgpu_buffer_rsrc_t rb_ = rsrc_b(kt, krem);
        lb.load_lds(rb_, krem, dst + A_BYTES, wave);
    }
    __device__ __forceinline__ void load_lds_a(int kt, char* dst) const {
        int krem;
        const __amdgpu_buffer_rsrc_t rs = rsrc_a(kt, krem);
        la.load_lds(rs, krem, dst, wave);
    }
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(int kt, int& krem) const {
        const int k0 = (kbase + kt) * BK;
        krem = kend - k0;
        const int kc = krem > 0 ? k0 : 0;
        int sg = 0, kl = kc;
        if constexpr (BKSEG) {
            sg = kc / bseg;
            kl = kc - sg * bseg;
        }
        const int64_t e = boff + kadv(BKC, kl, ldb);
        // Segment base by arithmetic: a select between two loads of members
        // is folded into one indexed load, which keeps the object in scratch.
        const uint64_t s1 = sg == 1, s2 = sg == 2;
        const bf16_t* b = reinterpret_cast<const bf16_t*>(bsel[0] + s1 * bsel[1] + s2 * bsel[2]);
        const uint32_t nb = bbsel[0] + (uint32_t)s1 * bbsel[1] + (uint32_t)s2 * bbsel[2];
        return make_rsrc(b + e, nb - (uint32_t)(e * 2));
    }

    // Registers -> LDS slot (swizzled layouts).
    __device__ __forceinline__ void store_a(int slot, const u32x4 (&v)[LA::NI]) const {
        la.store(smem + slot * STAGE, wave, lane, v);
    }
    __device__ __forceinline__ void store_b(int slot, const u32x4 (&v)[LB::NI]) const {
        lb.store(smem + slot * STAGE + A_BYTES, wave, lane, v);
    }

    __device__ __forceinline__ void read_sub(int slot, int kk, HF& F) const { read_at(smem + slot * STAGE, kk, F); }
    __device__ __forceinline__ void read_at(const char* as, int kk, HF& F) const { read_ab(as, as + A_BYTES, kk, F); }
    __device__ __forceinline__ void read_ab(const char* as, const char* bs, int kk, HF& F) const {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if constexpr (AK) F.a[i] = frag_k(as, wm * WTM + i * 32, kk, lane);
            else F.a[i] = frag_mn<BM>(as, wm * WTM + i * 32, kk, lane);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (BKC) F.b[j] = frag_k(bs, wn * WTN + j * 32, kk, lane);
            else F.b[j] = frag_mn<BN>(bs, wn * WTN + j * 32, kk, lane);
        }
    }

    // Step kt, kt & 1 == P; on entry Fa holds k16 #0 of step kt (possibly in flight).
    template <int P>
    __device__ __forceinline__ void step(int kt, HF& Fa, HF& Fb) {
        constexpr int R = (P ^ 1) % NSET;  // registers holding step kt+1
        run_mfmas<ST, 0, NM>(acc, Fa);
        read_sub(P, 1, Fb);
        store_a(P ^ 1, ra[R]);
        load_a(kt + 1 + NSET, ra[R]);
        interleave<NM, NRD, LA::NI, LA::NI>();
        run_mfmas<ST, 0, NM>(acc, Fb);
        read_sub(P, 2, Fa);
        store_b(P ^ 1, rb[R]);
        load_b(kt + 1 + NSET, rb[R]);
        interleave<NM, NRD, LB::NI, LB::NI>();
        run_mfmas<ST, 0, NM>(acc, Fa);
        read_sub(P, 3, Fb);
        interleave<NM, NRD, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm();
        run_mfmas<ST, 0, PRE>(acc, Fb);
        stage_barrier();
        run_mfmas<ST, PRE, NM>(acc, Fb);
        read_sub(P ^ 1, 0, Fa);
        interleave<NM - PRE, NRD, 0, 0>();
    }

    // KG == 2: the group's two sub-steps kk0, kk0+1 of step kt, whose stage is
    // `cur`; on entry Fa holds kk0.  The direct loads of step kt+2 go to `dst`,
    // the slot last read in step kt-1 (before the previous barrier).  Before
    // this step's barrier each thread waits for its loads of step kt+1 (all but
    // the NLD just issued), so the barrier publishes `nxt`.  The three slots
    // come in as distinct restrict pointers: the compiler then knows that the
    // reads of `nxt` after the barrier do not touch the slot still being
    // loaded, and does not wait for those loads (without that it waits for
    // every load in flight before the first LDS read after each barrier).
    __device__ __forceinline__ void step2(int kt, HF& Fa, HF& Fb, const char* __restrict__ cur,
                                          const char* __restrict__ nxt, char* __restrict__ dst) {
        run_mfmas<ST, 0, NM>(acc, Fa);
        read_at(cur, kk0 + 1, Fb);
        load_lds(kt + 2, dst);
        interleave<NM, NRD, 0, NLD>();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm<NLD>();
        run_mfmas<ST, 0, PRE>(acc, Fb);
        stage_barrier();
        run_mfmas<ST, PRE, NM>(acc, Fb);
        read_at(nxt, kk0, Fa);
        interleave<NM - PRE, NRD, 0, 0>();
    }

    // ADIRECT step kt: A stages at ca (this step), na (next), da (free: the
    // loads of A for step kt+2 go there, in sub-step 0); B stages at cb, nb.
    // Sub-step 1 stores B of step kt+1 (registers `rbv`, loaded two steps
    // earlier) to nb and loads B of step kt+3 into the same registers.  Loads
    // are issued in the order A(kt+2), B(kt+3) per step, so before the barrier
    // vmcnt(LA::NI + 2 LB::NI) leaves only B(kt+2), A(kt+2), B(kt+3) in flight:
    // A(kt+1) has landed, and with this thread's LDS stores done the barrier
    // publishes na and nb.  The slots are restrict pointers so that the
    // compiler does not wait for the loads into da before reading na.
    __device__ __forceinline__ void stepa(int kt, HF& Fa, HF& Fb, const char* __restrict__ ca,
                                          const char* __restrict__ na, char* __restrict__ da,
                                          const char* __restrict__ cb, char* __restrict__ nb,
                                          u32x4 (&rbv)[LB::NI]) {
        run_mfmas<ST, 0, NM>(acc, Fa);
        read_ab(ca, cb, 1, Fb);
        load_lds_a(kt + 2, da);
        interleave<NM, NRD, 0, LA::NI>();
        run_mfmas<ST, 0, NM>(acc, Fb);
        read_ab(ca, cb, 2, Fa);
        lb.store(nb, wave, lane, rbv);
        load_b(kt + 3, rbv);
        interleave<NM, NRD, LB::NI, LB::NI>();
        run_mfmas<ST, 0, NM>(acc, Fa);
        read_ab(ca, cb, 3, Fb);
        interleave<NM, NRD, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm<LA::NI + 2 * LB::NI>();
        run_mfmas<ST, 0, PRE>(acc, Fb);
        stage_barrier();
        run_mfmas<ST, PRE, NM>(acc, Fb);
        read_ab(na, nb, 0, Fa);
        interleave<NM - PRE, NRD, 0, 0>();
    }

    __device__ __forceinline__ void run() {
        if (nk <= 0) return;
        if constexpr (ADIRECT) {
            char* const a0 = smem;
            char* const a1 = smem + A_BYTES;
            char* const a2 = smem + 2 * A_BYTES;
            char* const b0 = smem + 3 * A_BYTES;
            char* const b1 = b0 + B_BYTES;
            // B of step j travels in register set j % 2
            load_lds_a(0, a0);
            load_b(0, rb[0]);
            lb.store(b0, wave, lane, rb[0]);
            load_b(1, rb[1]);
            __builtin_amdgcn_sched_barrier(0);
            load_lds_a(1, a1);
            __builtin_amdgcn_sched_barrier(0);
            load_b(2, rb[0]);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm_lgkm<LA::NI + 2 * LB::NI>();
            stage_barrier();
            HF Fa, Fb;
            read_ab(a0, b0, 0, Fa);
            // Whole rounds of six steps (the slot pattern repeats every six),
            // then the remaining 0..5 steps.  No exit from inside the loop: an
            // early exit makes the compiler wait for every load in flight at
            // the top of each round.
            int kt = 0;
            for (; kt + 6 <= nk; kt += 6) {
                stepa(kt, Fa, Fb, a0, a1, a2, b0, b1, rb[1]);
                stepa(kt + 1, Fa, Fb, a1, a2, a0, b1, b0, rb[0]);
                stepa(kt + 2, Fa, Fb, a2, a0, a1, b0, b1, rb[1]);
                stepa(kt + 3, Fa, Fb, a0, a1, a2, b1, b0, rb[0]);
                stepa(kt + 4, Fa, Fb, a1, a2, a0, b0, b1, rb[1]);
                stepa(kt + 5, Fa, Fb, a2, a0, a1, b1, b0, rb[0]);
            }
            const int rem = nk - kt;
            if (rem > 0) {
                stepa(kt, Fa, Fb, a0, a1, a2, b0, b1, rb[1]);
                if (rem > 1) {
                    stepa(kt + 1, Fa, Fb, a1, a2, a0, b1, b0, rb[0]);
                    if (rem > 2) {
                        stepa(kt + 2, Fa, Fb, a2, a0, a1, b0, b1, rb[1]);
                        if (rem > 3) {
                            stepa(kt + 3, Fa, Fb, a0, a1, a2, b1, b0, rb[0]);
                            if (rem > 4) stepa(kt + 4, Fa, Fb, a1, a2, a0, b0, b1, rb[1]);
                        }
                    }
                }
            }
            wait_vm_lgkm<0>();
            return;
        }
        if constexpr (KG == 2) {
            char* const s0 = smem;
            char* const s1 = smem + STAGE;
            char* const s2 = smem + 2 * STAGE;
            load_lds(0, s0);
            load_lds(1, s1);
            wait_vm_lgkm<NLD>();
            stage_barrier();
            HF Fa, Fb;
            read_at(s0, kk0, Fa);
            // Up to two more steps than the K range: their loads are out of
            // range, so they read zeros and add nothing.
            for (int kt = 0; kt < nk; kt += 3) {
                step2(kt, Fa, Fb, s0, s1, s2);
                step2(kt + 1, Fa, Fb, s1, s2, s0);
                step2(kt + 2, Fa, Fb, s2, s0, s1);
            }
            wait_vm_lgkm<0>();
            return;
        }
        load_a(0, ra[0]);
        load_b(0, rb[0]);
        if constexpr (NSET == 2) {
            load_a(1, ra[1]);
            load_b(1, rb[1]);
        }
        store_a(0, ra[0]);
        store_b(0, rb[0]);
        load_a(NSET, ra[0]);
        load_b(NSET, rb[0]);
        wait_lgkm();
        stage_barrier();
        HF Fa, Fb;
        read_sub(0, 0, Fa);
        // An odd step count gets one more step: its operands were loaded past
        // the K range, so they are zeros and add nothing.
        for (int kt = 0; kt < nk; kt += 2) {
            step<0>(kt, Fa, Fb);
            step<1>(kt + 1, Fa, Fb);
        }
        wait_vm_lgkm<0>();
    }
};

// bf16 epilogue, first half: the tile's values plus bias as bf16 into a
// [BM][SP bytes] LDS image.  Each lane writes 8 bytes (4
// columns of one row) per store; a row pitch of SP = 2*BN + 8 bytes (an odd
// number of 8-byte pairs) puts the 32 rows of a half-wave on distinct banks.
template <typename ST, int FM, int FN, int WTM, int WTN, int SP>
__device__ __forceinline__ void stage_bf16(char* st, const f32x16 (&acc)[FM][FN], const bf16_t* bias, int ncols,
                                           int wm, int wn, int lane) {
    // The wave's bias words, all loaded before the first is used (a lane past the valid
    // columns reads the first word instead and takes zeros).
    u32x2 bws[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) bws[j][q] = u32x2{0u, 0u};
    if (bias) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
                const u32x2 w = *reinterpret_cast<const u32x2*>(bias + (nl < ncols ? nl : 0));
                bws[j][q] = nl < ncols ? w : u32x2{0u, 0u};
            }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);  // first of the 4 columns
            const u32x2 bw = bws[j][q];
            const float b4[4] = {Store16<ST>::lo(bw[0]), Store16<ST>::hi(bw[0]), Store16<ST>::lo(bw[1]),
                                 Store16<ST>::hi(bw[1])};
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] + b4[e];
                const u32x2 o = {Store16<ST>::pack2(v[0], v[1]), Store16<ST>::pack2(v[2], v[3])};
                *reinterpret_cast<u32x2*>(st + (wm * WTM + i * 32 + (lane & 31)) * SP + nl * 2) = o;
            }
        }
}

// The GeLU epilogue, one 32-row fragment row i of every wave at a time: Gp =
// GeLU'(u) and Y = GeLU(u) of u = value + bias as bf16 into two [NWR * 32][SP
// bytes] images (wave row wm at image rows 32 wm ..), so that the stores of one
// chunk are in flight while the next chunk's exponentials and reciprocals run.
template <typename ST, int FM, int FN, int WTN, int SP>
__device__ __forceinline__ void stage_gelu_chunk(char* gimg, char* yimg, const f32x16 (&acc)[FM][FN],
                                                 const bf16_t* bias, int ncols, int wm, int wn, int lane,
                                                 bool tanh_form, int i) {
    const int r = wm * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);  // first of the 4 columns
            u32x2 bw = u32x2{0u, 0u};
            if (bias) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(bias + (nl < ncols ? nl : 0));
                bw = nl < ncols ? w : u32x2{0u, 0u};
            }
            const float b4[4] = {Store16<ST>::lo(bw[0]), Store16<ST>::hi(bw[0]), Store16<ST>::lo(bw[1]),
                                 Store16<ST>::hi(bw[1])};
            float g[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = gelu_and_prime(acc[i][j][4 * q + e] + b4[e], tanh_form, g[e]);
            *reinterpret_cast<u32x2*>(gimg + r * SP + nl * 2) = u32x2{Store16<ST>::pack2(g[0], g[1]),
                                                                     Store16<ST>::pack2(g[2], g[3])};
            *reinterpret_cast<u32x2*>(yimg + r * SP + nl * 2) = u32x2{Store16<ST>::pack2(y[0], y[1]),
                                                                     Store16<ST>::pack2(y[2], y[3])};
        }
}

// bf16 epilogue, second half: the LDS image to C rows m0.. (8 columns, 16
// bytes, per thread and item; rows past M and columns past ncols skipped).
// The stores are marked non-temporal: the next kernel reads C anyway, and lines
// the L2 does not hold dirty need no write-back when the kernel ends (measured:
// the gap to the next launch 4.0 -> 2.5 us, the bf16-output GEMMs 1-2 us
// faster).
// With RSTRIDE, the image holds one 32-row block per wave row (a chunk of the
// tile): image row lr is tile row (lr / 32) * RSTRIDE + roff + lr % 32.
template <int BM, int BN, int SP, int NTH, int RSTRIDE = 0>
__device__ __forceinline__ void store_bf16(const char* st, bf16_t* C, int64_t ldc, int rows, int ncols, int tid,
                                           int roff = 0) {
    constexpr int GPR = BN / 8;  // 8-column groups per row
    constexpr int ITEMS = BM * GPR / NTH;
    static_assert((BM * GPR) % NTH == 0, "epilogue split");
    // Items go in groups of G: the group's LDS reads (always inside the image) are
    // issued together, then the stores of its items inside the valid extent, so the
    // reads do not wait for one another behind the bounds test of each item.
    constexpr int G = ITEMS < 8 ? ITEMS : 8;
#pragma unroll
    for (int g0 = 0; g0 < ITEMS; g0 += G) {
        u32x4 v[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int e = tid + (g0 + k) * NTH;
            const int lr = e / GPR, cg = e % GPR;
            if (g0 + k < ITEMS) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(st + lr * SP + cg * 16);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(st + lr * SP + cg * 16 + 8);
                v[k] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int e = tid + (g0 + k) * NTH;
            const int lr = e / GPR, cg = e % GPR;
            const int tr = RSTRIDE ? (lr >> 5) * RSTRIDE + roff + (lr & 31) : lr;
            if (g0 + k < ITEMS && tr < rows && cg * 8 < ncols)
                __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(C + (int64_t)tr * ldc + cg * 8));
        }
    }
}

template <int BM, int BN, int NWV, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32, int KG = 1,
          typename ST = bf16_t>
__global__ void __launch_bounds__(64 * NWV, (tile_occupancy<BM, BN, NWV>())) gemm_bf16_kernel(const GemmBatch batch) {
    using Core = GemmCore<BM, BN, AK, BKC, BKSEG, NWV, KG, ST>;
    constexpr int NT = 64 * NWV / KG;  // epilogue threads (the first K group)
    constexpr int HR = NWV / KG / 4;   // wave rows per half tile
    constexpr int RING = Core::LDS_BYTES;
    // fp32 epilogues (weight gradients, GeLU') stage half a tile at a time as
    // fp32; the bf16 ones stage the whole tile as bf16.
    constexpr bool F32STAGE = OUTF32 || EPI == EPI_GELU_BWD;
    constexpr int EROWS = BM / 2, ELD = BN + 4;  // fp32 staging: row pitch BN + 4 floats
    constexpr int SP = BN * 2 + 8;               // bf16 staging: row pitch in bytes
    constexpr int EBYTES = F32STAGE ? EROWS * ELD * 4 : BM * SP;
    // EPI_STORE_ROWDOT: the tile of aux (O) comes straight into LDS behind the ring at the
    // start, and the row dots' per-chunk partial sums go behind the output image
    constexpr bool ROWDOT = EPI == EPI_STORE_ROWDOT;
    constexpr int ABYTES = ROWDOT ? BM * BN * 2 : 0;
    constexpr int RED_OFF = (EBYTES + 255) / 256 * 256;
    static_assert(!ROWDOT || (RED_OFF + BM * (BN / 8) * 4 <= RING && (BM * BN * 2) % (NWV * 1024) == 0),
                  "row-dot areas");
    constexpr int SMEM = (RING > EBYTES ? RING : EBYTES) + ABYTES;
    constexpr int WTM = Core::WTM, WTN = Core::WTN, FM = Core::FM, FN = Core::FN;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = (wave % (NWV / KG)) >> 1, wn = wave & 1;
    const bool epi_wave = wave < NWV / KG;  // the waves that hold the final sums
    // workgroup -> (K split, problem, tile)
    const int split = (int)blockIdx.x / batch.tiles;
    int t = xcd_id((int)blockIdx.x - split * batch.tiles, batch.tiles);
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

    if constexpr (ROWDOT) {  // the aux tile [BM][BN] (rows past M read as zeros), oldest loads in flight
        const int64_t aoff = (int64_t)m0 * p.ldaux + n0;
        const int64_t ext = ((int64_t)(p.M - m0 - 1) * p.ldaux + (p.N - n0)) * 2;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.aux + aoff, (uint32_t)(ext > 0x7fffffff ? 0x7fffffff : ext));
#pragma unroll
        for (int i = 0; i < ABYTES / (NWV * 1024); ++i) {
            const int q = wave + NWV * i, off = q * 1024 + 16 * lane;
            const int r = off / (BN * 2), cb = off % (BN * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(smem + SMEM - ABYTES + q * 1024), 16,
                                                     m0 + r < p.M ? (uint32_t)(r * p.ldaux * 2 + cb) : OOB, 0, 0, 0);
        }
    }
    Core core(p, smem, m0, n0, kb, kn);
    core.run();
    auto& acc = core.acc;
    if constexpr (KG == 2) {
        // the second K group adds its partial sums into the first's, one 32-column
        // block of the wave tile at a time (fixed order: deterministic)
        static_assert(OUTF32 || EPI == EPI_STORE || EPI == EPI_STORE_ROWDOT, "the K-group split serves plain stores");
        float* mg = reinterpret_cast<float*>(smem);
        const int wl = wave % 4, g = wave / 4;
#pragma unroll
        for (int j = 0; j < Core::FN; ++j) {
            __syncthreads();
            // value r of block i, lane l of wave wl at [((i * 4 + r / 4) * 4 + wl) * 256 + 4 l + r % 4]:
            // 16 bytes per lane and access, all reads of a block issued before the adds
            if (g == 1) {
#pragma unroll
                for (int i = 0; i < Core::FM; ++i)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        *reinterpret_cast<f32x4*>(mg + ((i * 4 + r4) * 4 + wl) * 256 + 4 * lane) =
                            f32x4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
            }
            __syncthreads();
            if (g == 0) {
#pragma unroll
                for (int i = 0; i < Core::FM; ++i) {
                    f32x4 t[4];
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        t[r4] = *reinterpret_cast<const f32x4*>(mg + ((i * 4 + r4) * 4 + wl) * 256 + 4 * lane);
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += t[r / 4][r % 4];
                }
            }
        }
    }

    const int csg = n0 / p.cseg;
    const int cofs = csg * p.cseg;
    const int rows = p.M - m0, ncols = p.N - n0;  // valid extent of the tile
    static_assert(F32STAGE || KG == 1 || EPI == EPI_STORE || EPI == EPI_STORE_ROWDOT,
                  "bf16 epilogues with K groups: plain stores only");
    if constexpr (!F32STAGE) {
        // Bias on the accumulators; the output image goes through LDS once.  With
        // GeLU, Gp = GeLU'(U) (saved for the backward, which needs only that of U)
        // and Y = GeLU(U) go through two images, one fragment row at a time.
        const bf16_t* bias = nullptr;
        if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) bias = p.bias[csg] ? p.bias[csg] + (n0 - cofs) : nullptr;
        bf16_t* C = reinterpret_cast<bf16_t*>(p.C[csg]) + (int64_t)m0 * p.ldc + (n0 - cofs);
        __syncthreads();  // every wave is done with the operand ring
        if constexpr (EPI == EPI_BIAS_GELU) {
            constexpr int CR = BM / FM;  // image rows per chunk
            static_assert(2 * CR * SP <= SMEM, "two chunk images must fit the LDS of the tile");
            bf16_t* const C2 = p.C2 + (int64_t)m0 * p.ldc2 + (n0 - cofs);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if (i > 0) {  // every thread has read the previous chunk's images (its stores may be in flight)
                    wait_lgkm();
                    stage_barrier();
                }
                stage_gelu_chunk<ST, FM, FN, WTN, SP>(smem, smem + CR * SP, acc, bias, ncols, wm, wn, lane,
                                                      p.gelu_tanh != 0, i);
                wait_lgkm();
                stage_barrier();
                store_bf16<CR, BN, SP, NT, WTM>(smem, C, p.ldc, rows, ncols, tid, i * 32);
                store_bf16<CR, BN, SP, NT, WTM>(smem + CR * SP, C2, p.ldc2, rows, ncols, tid, i * 32);
            }
        } else {
            // with K groups only the first group holds the sums; every thread stores
            if (epi_wave) stage_bf16<ST, FM, FN, WTM, WTN, SP>(smem, acc, bias, ncols, wm, wn, lane);
            __syncthreads();
            store_bf16<BM, BN, SP, 64 * NWV>(smem, C, p.ldc, rows, ncols, tid);
            if constexpr (ROWDOT) {
                // each 8-column chunk of the rounded image times the aux tile, then per row
                // and head the chunks' sums in chunk order (deterministic)
                constexpr int GPR = BN / 8, NTA = 64 * NWV;
                static_assert((BM * GPR) % NTA == 0, "row-dot split");
                float* red = reinterpret_cast<float*>(smem + RED_OFF);
                const char* at = smem + SMEM - ABYTES;
                __builtin_amdgcn_s_waitcnt(0);  // this thread's aux loads (long done: oldest in flight)
                __syncthreads();                // ... and every thread's
#pragma unroll
                for (int k = 0; k < BM * GPR / NTA; ++k) {
                    const int e = tid + k * NTA, lr = e / GPR, cg = e % GPR;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(smem + lr * SP + cg * 16);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(smem + lr * SP + cg * 16 + 8);
                    const u32x4 av = *reinterpret_cast<const u32x4*>(at + lr * (BN * 2) + cg * 16);
                    const uint32_t cv[4] = {lo[0], lo[1], hi[0], hi[1]};
                    float sum = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        sum += Store16<ST>::lo(av[q]) * Store16<ST>::lo(cv[q]);
                        sum += Store16<ST>::hi(av[q]) * Store16<ST>::hi(cv[q]);
                    }
                    red[e] = sum;  // e = lr GPR + cg
                }
                __syncthreads();
                const int cph = p.rd_dh / 8, hpt = BN / p.rd_dh;  // chunks per head, heads per tile
                if (tid < BM * hpt) {
                    const int r = tid / hpt, hh = tid % hpt, m = m0 + r;
                    if (m < p.M && n0 + (hh + 1) * p.rd_dh <= p.N) {
                        float d = 0.f;
                        for (int c = 0; c < cph; ++c) d += red[r * GPR + hh * cph + c];
                        const int b = m / p.rd_seq, j = m % p.rd_seq, g = n0 / p.rd_dh + hh;
                        p.rd[((int64_t)b * p.rd_heads + g) * p.rd_seq + j] = d;
                    }
                }
            }
        }
    } else {
        // fp32 staging, half a tile (the rows of wave rows wm / HR == half) at a time,
        // 16 bytes per lane and store; every thread then handles 8 consecutive
        // columns of a row (16-byte loads of U and stores of the outputs).  The
        // outputs are stored non-temporal, as the bf16 ones: whole 32-byte runs per
        // thread that no later step of the launch reads, so they need not sit dirty
        // in L2 to be written back when the launch ends.
        float* stage = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            __syncthreads();
            if (epi_wave && wm / HR == half) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<f32x4*>(stage + ((wm % HR) * WTM + i * 32 + (lane & 31)) * ELD +
                                                      wn * WTN + j * 32 + 8 * q +
                                                      4 * (lane >> 5)) =
                                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            }
            __syncthreads();
            constexpr int GPR = BN / 8;                 // 8-column groups per row
            constexpr int ITEMS = EROWS * GPR / NT;
            static_assert(ITEMS >= 1 && (EROWS * GPR) % NT == 0, "epilogue split");
            // Items in groups of G: the group's U loads (GeLU') and LDS reads are all
            // issued before its first use, so their latencies overlap instead of
            // adding up item by item.
            constexpr int G = ITEMS < 4 ? ITEMS : 4;
            // A K split's first part goes to the output, part s > 0 to its slab (dense
            // [M][N]).  fp32 output tiles may straddle N-segments: each 8-column item
            // (segments are multiples of 8 columns wide) finds its own.
            float* const slab = batch.part + (int64_t)(split > 0 ? split - 1 : 0) * batch.pslab + batch.poff[prob];
            if (epi_wave) {
#pragma unroll
                for (int g0 = 0; g0 < ITEMS; g0 += G) {
                    f32x4 lo[G], hi[G];
                    u32x4 uw[G];
                    bool ok[G];
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        const int e = tid + (g0 + k) * NT;
                        const int lr = e / GPR, cg = e % GPR;
                        const int m = m0 + half * EROWS + lr, n = n0 + cg * 8;
                        ok[k] = g0 + k < ITEMS && m < p.M && n < p.N;
                        if constexpr (!OUTF32)
                            uw[k] = ok[k] ? *reinterpret_cast<const u32x4*>(p.aux + (int64_t)m * p.ldaux + (n - cofs))
                                          : u32x4{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        const int e = tid + (g0 + k) * NT;
                        const int lr = e / GPR, cg = e % GPR;
                        if (g0 + k < ITEMS) {
                            lo[k] = *reinterpret_cast<const f32x4*>(stage + lr * ELD + cg * 8);
                            hi[k] = *reinterpret_cast<const f32x4*>(stage + lr * ELD + cg * 8 + 4);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        if (!ok[k]) continue;
                        const int e = tid + (g0 + k) * NT;
                        const int lr = e / GPR, cg = e % GPR;
                        const int m = m0 + half * EROWS + lr, nl = n0 + cg * 8 - cofs;
                        if constexpr (OUTF32) {
                            float* c;
                            if (split == 0) {
                                int seg = csg, off = n0 + cg * 8 - cofs;
                                while (off >= p.cseg && seg < 2) {
                                    off -= p.cseg;
                                    ++seg;
                                }
                                c = reinterpret_cast<float*>(p.C[seg]) + (int64_t)m * p.ldc + off;
                            } else {
                                c = slab + (int64_t)m * p.N + (n0 + cg * 8);
                            }
                            __builtin_nontemporal_store(lo[k], reinterpret_cast<f32x4*>(c));
                            __builtin_nontemporal_store(hi[k], reinterpret_cast<f32x4*>(c + 4));
                        } else {  // EPI_GELU_BWD: dU = dY * Gp, Gp = GeLU'(U) saved by the forward
                            float v[8] = {lo[k][0], lo[k][1], lo[k][2], lo[k][3], hi[k][0], hi[k][1], hi[k][2], hi[k][3]};
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                v[2 * q] *= Store16<ST>::lo(uw[k][q]);
                                v[2 * q + 1] *= Store16<ST>::hi(uw[k][q]);
                            }
                            u32x4 o;
#pragma unroll
                            for (int q = 0; q < 4; ++q) o[q] = Store16<ST>::pack2(v[2 * q], v[2 * q + 1]);
                            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(reinterpret_cast<bf16_t*>(p.C[csg]) + (int64_t)m * p.ldc + nl));
                        }
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int NWV, bool AK, bool BKC, bool BKSEG, int EPI, bool OUTF32, int KG, typename ST>
hipError_t launch(GemmBatch b, hipStream_t s) {
    b.tiles0 = ((b.g[0].N + BN - 1) / BN) * ((b.g[0].M + BM - 1) / BM);
    b.tiles = b.tiles0;
    if (b.n > 1) b.tiles += ((b.g[1].N + BN - 1) / BN) * ((b.g[1].M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, NWV, AK, BKC, BKSEG, EPI, OUTF32, KG, ST>), dim3(b.tiles * b.ksplit),
                       dim3(64 * NWV),
                       0, s, b);
    count_launch();
    return hipGetLastError();
}

template <int BM, int BN, int NWV, typename ST>
hipError_t dispatch_general(const GemmDesc& d, const GemmBatch& a, hipStream_t s);

// The 192 x 192 tile with 4 waves serves only the fp32-output weight-gradient GEMMs.
template <int BM, int BN, int NWV, typename ST>
hipError_t dispatch(const GemmDesc& d, const GemmBatch& a, hipStream_t s) {
    const bool ak = d.a_kcontig, bk = d.b_kcontig;
    if constexpr (BM == 192 && BN == 192 && NWV == 4) {
        if (!ak && !bk && !d.b_kseg && d.out_f32 && d.epi == EPI_STORE)
            return launch<192, 192, 4, false, false, false, EPI_STORE, true, 1, ST>(a, s);
        return hipErrorInvalidValue;
    } else {
        return dispatch_general<BM, BN, NWV, ST>(d, a, s);
    }
}

template <int BM, int BN, int NWV, typename ST>
hipError_t dispatch_general(const GemmDesc& d, const GemmBatch& a, hipStream_t s) {
    const bool ak = d.a_kcontig, bk = d.b_kcontig;
    if (ak && !bk && !d.b_kseg && !d.out_f32) {
        if (d.epi == EPI_BIAS_GELU) return launch<BM, BN, NWV, true, false, false, EPI_BIAS_GELU, false, 1, ST>(a, s);
        if (d.epi == EPI_BIAS) return launch<BM, BN, NWV, true, false, false, EPI_BIAS, false, 1, ST>(a, s);
        if (d.epi == EPI_STORE) return launch<BM, BN, NWV, true, false, false, EPI_STORE, false, 1, ST>(a, s);
    } else if (ak && bk && !d.out_f32) {
        if (d.b_kseg && d.epi == EPI_STORE) return launch<BM, BN, NWV, true, true, true, EPI_STORE, false, 1, ST>(a, s);
        if (!d.b_kseg && d.epi == EPI_GELU_BWD)
            return launch<BM, BN, NWV, true, true, false, EPI_GELU_BWD, false, 1, ST>(a, s);
        if (!d.b_kseg && d.epi == EPI_STORE) return launch<BM, BN, NWV, true, true, false, EPI_STORE, false, 1, ST>(a, s);
    } else if (!ak && !bk && !d.b_kseg && d.out_f32 && d.epi == EPI_STORE) {
        return launch<BM, BN, NWV, false, false, false, EPI_STORE, true, 1, ST>(a, s);
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
    a.gelu_tanh = d.gelu_tanh ? 1 : 0;
    a.rd = d.rd; a.rd_seq = d.rd_seq; a.rd_heads = d.rd_heads; a.rd_dh = d.rd_dh;
    return a;
}

struct Cand {
    int bm, bn, occ;  // occ: workgroups resident per CU
    double eff;       // throughput of the shape relative to 256 x 256 (measured on MI355X)
    bool f32_tn_only;
};
// Index 8 is the 256 x 192 tile with 8 waves (two per SIMD): 3-16% faster than
// with 4 waves on the same tile in a shape sweep.  Index 9 is the 192 x 192
// fp32 weight-gradient tile with 8 waves in two K groups: 4-6% faster than its
// 4-wave form on the MLP weight-gradient pair.  Index 10 is the 64 x 192 tile
// with 8 waves in two K groups, for plain 16-bit stores of K-contiguous
// operands where one round of its tiles fills the CUs (dO: N = w, K = h):
// against the 4-wave 64 x 192 tile, one workgroup per CU either way, it puts
// two waves on each SIMD (dO 29.7 against 33.8 us at the 8.3B shape).  Index
// 11 is the 256 x 128 tile with 8 waves (wave tiles 64 x 64), for N where it
// fills the CUs in one round and the 192-column tile does not (BERT's QKV: N =
// 960 gives 256 tiles of 128 columns against 160 of 192).
const Cand kCands[] = {{256, 256, 1, 1.0, false},  {256, 192, 1, 0.98, false}, {192, 192, 1, 0.93, true},
                       {256, 128, 1, 0.84, false}, {128, 128, 2, 0.835, false}, {64, 192, 2, 0.72, false},
                       {64, 64, 4, 0.4, false},    {128, 192, 2, 0.92, false}, {256, 192, 1, 1.10, false},
                       {192, 192, 1, 0.975, true}, {64, 192, 1, 0.80, false}, {256, 128, 1, 0.80, false}};
constexpr double K_OVERHEAD = 384.0;       // prologue + epilogue of a tile, in units of K
// The K split's reduction kernel in the same units (a CU's MACs at ~2.2 M per us):
// three fp32 passes over the outputs at ~5 TB/s, plus a launch (~3 us).
constexpr double RED_PER_ELEM = 5.3;
constexpr double RED_FIXED = 6.6e6;
constexpr double K_OVERHEAD_GELU = 1024.0;  // the same with a GeLU / GeLU' epilogue

// Operands and epilogues the 8-wave 256 x 128 tile (index 11) is built for.
bool tile11_ok(const GemmDesc& d) {
    return d.a_kcontig && !d.b_kcontig && !d.b_kseg && !d.out_f32 && (d.epi == EPI_BIAS || d.epi == EPI_STORE);
}

template <typename ST>
hipError_t dispatch_idx(int c, const GemmDesc& d, const GemmBatch& b, hipStream_t s) {
    switch (c) {
        case 0: return dispatch<256, 256, 4, ST>(d, b, s);
        case 1: return dispatch<256, 192, 4, ST>(d, b, s);
        case 2: return dispatch<192, 192, 4, ST>(d, b, s);
        case 3: return dispatch<256, 128, 4, ST>(d, b, s);
        case 4: return dispatch<128, 128, 4, ST>(d, b, s);
        case 5: return dispatch<64, 192, 4, ST>(d, b, s);
        case 6: return dispatch<64, 64, 4, ST>(d, b, s);
        case 7: return dispatch<128, 192, 4, ST>(d, b, s);
        case 8: return dispatch<256, 192, 8, ST>(d, b, s);
        case 9:  // fp32 weight gradients only
            if (!d.a_kcontig && !d.b_kcontig && !d.b_kseg && d.out_f32 && d.epi == EPI_STORE)
                return launch<192, 192, 8, false, false, false, EPI_STORE, true, 2, ST>(b, s);
            return hipErrorInvalidValue;
        case 10:  // K-contiguous operands, plain 16-bit stores (and their row dots) only
            if (d.a_kcontig && d.b_kcontig && !d.b_kseg && !d.out_f32 && d.epi == EPI_STORE)
                return launch<64, 192, 8, true, true, false, EPI_STORE, false, 2, ST>(b, s);
            if (d.a_kcontig && d.b_kcontig && !d.b_kseg && !d.out_f32 && d.epi == EPI_STORE_ROWDOT)
                return launch<64, 192, 8, true, true, false, EPI_STORE_ROWDOT, false, 2, ST>(b, s);
            return hipErrorInvalidValue;
        default:  // 11: K-contiguous A, B with N contiguous, 16-bit output with or without bias
            if (tile11_ok(d) && d.epi == EPI_BIAS)
                return launch<256, 128, 8, true, false, false, EPI_BIAS, false, 1, ST>(b, s);
            if (tile11_ok(d) && d.epi == EPI_STORE)
                return launch<256, 128, 8, true, false, false, EPI_STORE, false, 1, ST>(b, s);
            return hipErrorInvalidValue;
    }
}

// Test hook (gemm_force_tile): a tile index of kCands and a K split that replace
// the cost model's choice for every GEMM they are valid for; -1 / 0: the model.
int g_force_tile = -1;
int g_force_split = 0;

}  // namespace

void gemm_force_tile(int tile, int ksplit) {
    g_force_tile = tile;
    g_force_split = ksplit;
}

int gemm_tile_count() { return (int)(sizeof(kCands) / sizeof(kCands[0])); }

bool gemm_rowdot_ok(const GemmDesc& d) {
    const int cus = d.cus > 0 && d.cus < 256 ? d.cus : 256;
    const int64_t tiles = (int64_t)((d.M + 63) / 64) * ((d.N + 191) / 192);
    return d.M > 0 && d.N > 0 && d.K > 0 && d.a_kcontig && d.b_kcontig && !d.b_kseg && !d.out_f32 &&
           d.bseg >= (1 << 30) && d.cseg >= (1 << 30) && tiles <= cus && d.rd && d.aux && d.rd_dh > 0 &&
           d.rd_dh % 8 == 0 && 192 % d.rd_dh == 0 && d.N % d.rd_dh == 0 && d.rd_seq > 0 && d.rd_heads > 0 &&
           (int64_t)d.rd_heads * d.rd_dh >= d.N && d.M % d.rd_seq == 0 && d.ldaux % 8 == 0 && d.ldaux >= d.N &&
           (reinterpret_cast<uintptr_t>(d.aux) & 15u) == 0;
}

// Tile shape (and K split) with the least estimated time on 256 CUs (or the
// share `cus` of them the launch is given beside other work).  A CU
// gets ceil(items / 256) tiles and runs o = min(occupancy, that) of them at
// once; each costs BM * BN * (K per split + overhead / o) / efficiency, the
// overhead (prologue and epilogue, larger with GeLU math) being hidden by the
// other resident tiles; a K split adds its reduction kernel.  B's N-segments
// (and C's, for 16-bit outputs) must hold whole tiles; the 192 x 192 tile and
// the K split serve only the fp32 weight-gradient GEMMs.  The split needs a
// partial-sum slab of sum(M N) floats in `part` (part_floats of them available).
hipError_t gemm_bf16_batch(const GemmDesc* d, int n, float* part, int64_t part_floats, int* ksplit_out,
                           hipStream_t s) {
    if (n < 1 || n > 2) return hipErrorInvalidValue;
    GemmBatch b;
    b.n = 0;
    b.part = part;
    b.pslab = 0;
    const GemmDesc* live[2];
    for (int i = 0; i < n; ++i)
        if (d[i].M > 0 && d[i].N > 0 && d[i].K > 0) {
            b.poff[b.n] = b.pslab;
            b.pslab += (int64_t)d[i].M * d[i].N;
            live[b.n] = &d[i];
            b.g[b.n++] = make_args(d[i]);
        }
    if (ksplit_out) *ksplit_out = 1;
    if (b.n == 0) return hipSuccess;
    const bool allow_split = part && part_floats >= b.pslab && (reinterpret_cast<uintptr_t>(part) & 15u) == 0;
    const bool tn32 = !d[0].a_kcontig && !d[0].b_kcontig && !d[0].b_kseg && d[0].out_f32;
    const bool nt16 = d[0].a_kcontig && d[0].b_kcontig && !d[0].b_kseg && !d[0].out_f32 &&
                      (d[0].epi == EPI_STORE || d[0].epi == EPI_STORE_ROWDOT);
    const bool rowdot = d[0].epi == EPI_STORE_ROWDOT;  // only the 64 x 192 K-group tile has it
    if (rowdot && (n != 1 || !gemm_rowdot_ok(d[0]))) return hipErrorInvalidValue;
    int best = -1, best_split = 1;
    double best_cost = 1e300;
    int kmax = 0;
    for (int i = 0; i < n; ++i) kmax = d[i].K > kmax ? d[i].K : kmax;
    const double kov = (d[0].epi == EPI_BIAS_GELU || d[0].epi == EPI_GELU_BWD) ? K_OVERHEAD_GELU : K_OVERHEAD;
    const int ncand = (int)(sizeof(kCands) / sizeof(kCands[0]));
    const bool forced = g_force_tile >= 0 && g_force_tile < ncand;
    const int cus = d[0].cus > 0 && d[0].cus < 256 ? d[0].cus : 256;
    for (int c = 0; c < ncand; ++c) {
        const Cand& k = kCands[c];
        if (k.f32_tn_only && !tn32) continue;
        bool ok = true;
        int64_t t = 0;
        for (int i = 0; i < n; ++i) {
            const GemmDesc& g = d[i];
            // B's N-segments must hold whole tiles; so must C's, except for fp32 outputs
            // (their epilogue routes each 8-column item to its segment)
            ok = ok && (g.b_kseg || g.bseg >= (1 << 30) || g.bseg % k.bn == 0) &&
                 (g.cseg >= (1 << 30) || g.cseg % k.bn == 0 || g.out_f32);
            t += (int64_t)((g.M + k.bm - 1) / k.bm) * ((g.N + k.bn - 1) / k.bn);
        }
        if (!ok) continue;
        // the 8-wave K-group 64 x 192 tile: plain 16-bit stores of K-contiguous operands,
        // where its tiles fill the CUs in one round (small N, long K)
        if (c == 10 && (!nt16 || t > cus)) continue;
        if (c == 11 && (n != 1 || !tile11_ok(d[0]))) continue;
        if (rowdot && c != 10) continue;
        if (forced && c == g_force_tile) {  // test hook: this tile wherever it is valid
            best = c;
            best_split = (g_force_split == 2 && allow_split && tn32) ? 2 : 1;
            best_cost = -1.0;
            break;
        }
        for (int split = 1; split <= ((allow_split && tn32) ? 2 : 1); ++split) {
            const int64_t tpc = (t * split + cus - 1) / cus;  // tiles per CU
            const int64_t o = tpc < k.occ ? tpc : k.occ;
            const double kper = (double)((kmax + split - 1) / split);
            double cost = (double)((tpc + o - 1) / o) * o * k.bm * k.bn * (kper + kov / o) / k.eff;
            if (split > 1) cost += RED_PER_ELEM * (double)b.pslab + RED_FIXED;
            if (cost < best_cost) { best_cost = cost; best = c; best_split = split; }
        }
    }
    if (best < 0) return hipErrorInvalidValue;
    b.ksplit = best_split;
    if (ksplit_out) *ksplit_out = best_split;
    hipError_t e = d[0].fp16 ? dispatch_idx<f16_t>(best, d[0], b, s) : dispatch_idx<bf16_t>(best, d[0], b, s);
    if (e != hipSuccess || best_split == 1) return e;
    // The second K half's slab into the outputs (each N-segment its own block).
    float* dst[ZMAX];
    const float* src[ZMAX];
    int64_t rows[ZMAX], cols[ZMAX], ld[ZMAX], lds[ZMAX];
    int nr = 0;
    for (int i = 0; i < b.n; ++i) {
        const GemmDesc& g = *live[i];
        const int seg = g.cseg < (1 << 30) ? g.cseg : g.N;
        for (int z = 0; z * seg < g.N && z < 3; ++z) {
            dst[nr] = static_cast<float*>(g.C[z] ? g.C[z] : g.C[0]);
            src[nr] = part + b.poff[i] + (int64_t)z * seg;
            rows[nr] = g.M;
            cols[nr] = g.N - z * seg < seg ? g.N - z * seg : seg;
            ld[nr] = g.ldc;
            lds[nr] = g.N;
            ++nr;
        }
    }
    return add_f32_2d(dst, src, rows, cols, ld, lds, nr, s);
}

hipError_t gemm_bf16(const GemmDesc& d, hipStream_t s) { return gemm_bf16_batch(&d, 1, nullptr, 0, nullptr, s); }

}  // namespace tp
