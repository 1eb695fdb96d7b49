// Fused per-head softmax attention on gfx950 matrix cores, 16-bit in (bf16 or
// IEEE half, the template parameter ST) / fp32 math.
//
// Each shard runs full attention for its own heads with no communication
// (page "Megatron-LM: what the tensor parallelism paper actually says",
// section "The attention heads split").  Scores are Q K^T / sqrt(d) with an
// optional causal mask (key m allowed for query j iff m <= j).
//
// All products use v_mfma_f32_32x32x16_bf16 (_f16 for half storage).  For an operand tile the lane
// l holds row (or column) l % 32 and, per k16 chunk, the 8 k-slots
// 8*(l/32) .. +7; the 32x32 result gives lane l column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
//
// Forward: a workgroup owns two 64-query blocks of one (sequence, head), x
// and nb-1-x, so that under the causal mask every workgroup has about the
// same work; a wave takes 32 of the queries.  Scores are formed transposed, S^T = K Q^T, so that each lane holds
// ONE query and 16 keys of a 32-key block: the online-softmax max and sum are
// lane-local (plus one exchange between the lane pair l, l^32).  O^T = V^T P^T
// takes P^T straight from those registers: the k-slots of a k16 chunk are
// relabelled to the keys the lane already holds (slot s of chunk c is key
// 16c + 8*(s/4) + 4*(l/32) + s%4), and the V^T fragment is read with the
// same labelling by transposed LDS reads (ds_read_b64_tr_b16), which give a
// lane 4 consecutive rows of one column.  K and V stream through LDS in
// 64-key blocks, prefetched into registers one block ahead.
//
// Backward: P is recomputed from Q, K and the saved log-sum-exp.
//   D_j = dO_j . O_j            (row sums, equal to sum_m P_jm dP_jm)
//   dV = P^T dO, dK = dS^T Q / sqrt(d)     a workgroup per two 64-key blocks
//   dQ = dS K / sqrt(d)                    a workgroup per two 64-query blocks
// with dP = dO V^T and dS = P * (dP - D).  Splitting dQ into its own pass
// keeps every output written by exactly one workgroup (no atomics; the result
// is deterministic) at the price of recomputing S and dP once more.  The
// dK/dV pass forms S and dP with rows = queries and lane = key, so P^T and
// dS^T feed the next products from registers in the same way.
//
// LDS tiles are [rows][D] bf16 with the 16-byte chunks of each row permuted
// by an XOR of row bits, chosen so that both the 16-byte fragment reads (16
// rows, one chunk) and the transposed reads (8 rows x 4 chunks) hit every
// bank at most once per half-wave.
#include <cfloat>
#include <cmath>

#include "tp_common.h"
#include "tp_kernels.h"

namespace tp {

namespace {

constexpr int NT = 256;   // row sums
constexpr int NT8 = 512;  // 8 waves (forward, dK/dV, dQ): 4 row groups x 2 halves of the streamed rows
constexpr int BKV = 64;   // rows per streamed LDS block
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;

typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((address_space(3))) void lds_void;

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

__device__ __forceinline__ int bit(int r, int i) { return (r >> i) & 1; }

// 2^x on the hardware unit (no range fix-ups: inputs below -126 give 0 or a
// denormal, which only ever scales softmax terms that are negligible).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// True on every lane iff `p` holds on some lane of the wave.
__device__ __forceinline__ bool any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Chunk permutation of row r of a [rows][D] tile (16-byte chunks).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 64) return bit(r, 2) | (bit(r, 3) << 1) | (bit(r, 1) << 2);
    else if constexpr (D == 128) return bit(r, 2) | (bit(r, 3) << 1) | (bit(r, 0) << 2) | (bit(r, 1) << 3);
    else return (r >> 2) & 3;  // D = 32, 96
}

// Byte offset of element (r, col) in a swizzled [rows][D] tile.
template <int D>
__device__ __forceinline__ int toff(int r, int col) {
    return r * (D * 2) + ((((col >> 3) ^ swz<D>(r))) << 4) + (col & 7) * 2;
}

constexpr uint32_t OOB = 0x80000000u;  // buffer offset past any range: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}


// One 16-byte-per-lane buffer load into LDS (lane l writes dst + 16 l).  A
// plain function: with the builtin written inside the templates below, the
// compiler's host pass emitted launch stubs only for the first storage type.
__device__ __forceinline__ void load16_lds(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, off, 0, 0, 0);
}

// Direct global -> LDS loads of ROWS rows x D (row-major, stride ld) into a
// swizzled [ROWS][D] tile: instruction i of wave w fills tile bytes
// [(w + 8i) * 1024, +1024), lane l the 16 bytes at +16 l, so the lane holding
// row r, physical chunk pc fetches logical chunk pc ^ swz(r) of that row (the
// byte image toff() gives).  Rows at or past `nvalid` read as zeros.
template <int D, int ROWS>
struct TileDMA {
    static constexpr int BYTES = ROWS * D * 2;
    static constexpr int NI = BYTES / (8 * 1024);
    static_assert(BYTES % (8 * 1024) == 0, "the tile must split into 1 KB pieces over 8 waves");
    int row[NI];
    uint32_t off[NI];
    __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int q = (wave + 8 * i) * 1024 + 16 * lane;
            const int r = q / (2 * D), pc = (q % (2 * D)) / 16;
            row[i] = r;
            off[i] = (uint32_t)(r * ld * 2 + ((pc ^ swz<D>(r)) << 4));
        }
    }
    __device__ __forceinline__ void load(const bf16_t* src, int64_t ld, int row0, int nvalid, char* tile,
                                         int wave) const {
        const int rem = nvalid - row0;
        const uint32_t bytes = rem > 0 ? (uint32_t)((rem - 1) * ld * 2 + D * 2) : 0u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (int64_t)(rem > 0 ? row0 : 0) * ld, bytes);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            load16_lds(rs, tile + (wave + 8 * i) * 1024, row[i] < rem ? off[i] : OOB);
    }
};

// Direct global -> LDS loads of NTL (2 or 4) [64][D] tiles laid one after the
// other at dst (the swizzled image toff() gives).  Tile t holds 64 rows of a
// row-major source starting at row (t & (NTL/2) ? r1 : r0); with NTL = 4 odd
// tiles come from B (row stride ldb), even ones from A (stride lda); with NTL = 2
// both from A.  The tiles' 1 KB pieces are dealt over the 8 waves (piece q to
// wave q % 8), so every wave issues the same number of loads.  Rows at or past
// the sequence end read as zeros.
template <int D, int NTL>
__device__ __forceinline__ void load_tiles(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int r0,
                                           int r1, int s, char* dst, int wave, int lane) {
    constexpr int PPT = BKV * D * 2 / 1024;  // pieces per tile
    static_assert(NTL == 2 || NTL == 4, "two or four tiles");
    static_assert((NTL * PPT) % 8 == 0, "the tiles must split into 1 KB pieces over 8 waves");
#pragma unroll
    for (int i = 0; i < NTL * PPT / 8; ++i) {
        const int q = wave + 8 * i;  // wave-uniform
        const int t = q / PPT;
        const bool fromb = NTL == 4 && (t & 1);
        const bf16_t* sp = fromb ? B : A;
        const int64_t sl = fromb ? ldb : lda;
        const int rs0 = (t & (NTL / 2)) ? r1 : r0;
        const int off = (q % PPT) * 1024 + 16 * lane;
        const int r = off / (2 * D), pc = (off % (2 * D)) / 16;
        const int rem = s - rs0;
        const uint32_t bytes = rem > 0 ? (uint32_t)((rem - 1) * sl * 2 + D * 2) : 0u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sp + (int64_t)(rem > 0 ? rs0 : 0) * sl, bytes);
        load16_lds(rs, dst + q * 1024, r < rem ? (uint32_t)(r * sl * 2 + ((pc ^ swz<D>(r)) << 4)) : OOB);
    }
}

// Per-lane LDS byte offsets of the fragment reads of a [rows][D] tile.  The
// chunk swizzle depends only on the row modulo 16, so a row base that is a
// multiple of 16 (and the tile base) is a uniform addend.
//   rows[c]:  row l%32, d = 16c + 8*(l/32) .. +7 (16-byte read);
//   tr[h][db]: transposed read h of d block db: in each 16-lane group, lane j
//              addresses row 8h + 4*(G/2) + j/4 and d 32db + 16*(G%2) + 4*(j%4)
//              (G = l/16), and lane i receives column i, 4 consecutive rows.
template <int D>
struct FragAddr {
    static constexpr int ROWB = D * 2, KC = D / 16, DB = D / 32;
    // d = 128: rows are 256 bytes and a lane's offsets within a row stay below 256, so
    // every offset is rows[0] or tr[0][0] XOR a constant (chunk c: c << 5; d block db:
    // db << 6; read h = 1: eight rows further, 2048, and the swizzle's bit 1, 32); only
    // those two are held, leaving registers to the streams' accumulators.
    static constexpr bool XOR = D == 128;
    int rows[XOR ? 1 : KC];
    int tr[XOR ? 1 : 2][XOR ? 1 : DB];
    __device__ __forceinline__ void init(int lane) {
        const int lr = lane & 31, l5 = lane >> 5, G = lane >> 4, j = lane & 15;
#pragma unroll
        for (int c = 0; c < (XOR ? 1 : KC); ++c) rows[c] = toff<D>(lr, 16 * c + 8 * l5);
#pragma unroll
        for (int h = 0; h < (XOR ? 1 : 2); ++h)
#pragma unroll
            for (int db = 0; db < (XOR ? 1 : DB); ++db)
                tr[h][db] = toff<D>(8 * h + 4 * (G >> 1) + (j >> 2), 32 * db + 16 * (G & 1) + 4 * (j & 3));
    }
    __device__ __forceinline__ int row_off(int c) const {
        if constexpr (XOR) return rows[0] ^ (c << 5);
        else return rows[c];
    }
    __device__ __forceinline__ int tr_off(int h, int db) const {
        if constexpr (XOR) return tr[0][0] ^ (h ? 2048 + 32 : 0) ^ (db << 6);
        else return tr[h][db];
    }
    // Operand fragment of rows rb .. rb+31 (rb % 16 == 0), k = d chunk c:
    // lane l gets row rb + l%32, d = 16c + 8*(l/32) .. +7.
    __device__ __forceinline__ u32x4 frag_rows(const char* tile, int rb, int c) const {
        return *reinterpret_cast<const u32x4*>(tile + rb * ROWB + row_off(c));
    }
    // Operand fragment with rows = d (32db .. +31) and k = tile rows
    // rb + 16kc .. +15 (rb % 16 == 0) in the relabelled order: slot s of lane
    // l is tile row rb + 16kc + 8*(s/4) + 4*(l/32) + s%4.
    __device__ __forceinline__ u32x4 frag_tr(const char* tile, int rb, int db, int kc) const {
        const char* base = tile + (rb + 16 * kc) * ROWB;
        u32x4 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(base + tr_off(h, db)));
            const u32x2 w = __builtin_bit_cast(u32x2, t);
            out[2 * h] = w[0];
            out[2 * h + 1] = w[1];
        }
        return out;
    }
};

// bf16 operand fragment (k16 chunk kc of a 64-row block) from the fp32
// result registers of its 32-row half: slots s = values r = 8*(kc%2) + s.
template <typename ST>
__device__ __forceinline__ u32x4 pack_chunk(const f32x16& v, int half) {
    const int o = 8 * half;
    using S = Store16<ST>;
    return u32x4{S::pack2(v[o], v[o + 1]), S::pack2(v[o + 2], v[o + 3]), S::pack2(v[o + 4], v[o + 5]),
                 S::pack2(v[o + 6], v[o + 7])};
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// Row index (within a 32-row result block) of value r for lane l.
__device__ __forceinline__ int res_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Store a [D x 32] transposed fp32 accumulator (rows = d, lane column = one
// token row of `out`) as bf16, times `mul`: 4 consecutive d per 8-byte store.
template <int D, typename ST>
__device__ __forceinline__ void store_rowT(bf16_t* __restrict__ row, const f32x16 (&acc)[D / 32], float mul, int lane) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 t;
            t[0] = Store16<ST>::pack2(acc[db][4 * q] * mul, acc[db][4 * q + 1] * mul);
            t[1] = Store16<ST>::pack2(acc[db][4 * q + 2] * mul, acc[db][4 * q + 3] * mul);
            *reinterpret_cast<u32x2*>(row + 32 * db + 8 * q + 4 * (lane >> 5)) = t;
        }
}

// Workgroup -> (block pair x, sequence-head index bh) for a grid of (pairs,
// sequences x heads).  The hardware deals workgroups round-robin over the 8 XCDs
// by linear id; this numbering gives each XCD a contiguous range of (bh, x), so the
// pair workgroups of one (sequence, head) run on one XCD and share its L2 for that
// head's Q, K, V and dO (dealt over all XCDs, every L2 would hold every head).
__device__ __forceinline__ void xcd_map_n(int L, int n, int nx, int& x, int& bh) {
    const int per = (n + 7) / 8, r = n % 8, xc = L % 8, q = L / 8;
    const int id = (r == 0 || xc < r) ? xc * per + q : r * per + (xc - r) * (per - 1) + q;
    x = id % nx;
    bh = id / nx;
}
__device__ __forceinline__ void xcd_map(int& x, int& bh) {
    xcd_map_n((int)(blockIdx.x + blockIdx.y * gridDim.x), (int)(gridDim.x * gridDim.y), (int)gridDim.x, x, bh);
}

// Rows of a forward / dQ workgroup: the 64-row blocks x and nb-1-x of the
// sequence (nb blocks of 64 rows), so that under the causal mask a short and a
// long row range share every workgroup and all workgroups carry about the same
// work.  Row groups 0, 1 are the 32-row halves of block x, 2, 3 those of block
// nb-1-x (empty when the two coincide).  Wave w takes the key blocks of half
// kp = w / 4 of each streamed pair and row group (w + 2 kp) mod 4, so the two
// waves that share a SIMD (w and w + 4) hold rows of different blocks.
struct PairRows {
    int qg, kp;
    int qw0;  // first row of the wave's group (the sequence length when the group is empty)
    int nkb;  // 64-key blocks the workgroup streams
    __device__ __forceinline__ PairRows(int x, int s, int wave, int causal) {
        const int nb = (s + BKV - 1) / BKV, xl = nb - 1 - x;
        kp = wave >> 2;
        qg = (wave + 2 * kp) & 3;
        const int blk = qg < 2 ? x : xl;
        qw0 = (qg < 2 || xl != x) ? min(s, blk * BKV + 32 * (qg & 1)) : s;
        nkb = causal ? xl + 1 : nb;
    }
};

// One pair step of the forward for one wave: the online-softmax update of its 32
// queries (Q^T in qf) from the 64-key block at rows rb .. rb+63 of the pair tiles
// Kt, Vt (keys k0 ..).  The tiles are restrict pointers so that the compiler does
// not wait for the loads in flight into the other stage.
template <int D, typename ST>
__device__ __forceinline__ void fwd_pair(const AttnArgs& a, const FragAddr<D>& fa, const char* __restrict__ Kt,
                                         const char* __restrict__ Vt, const u32x4 (&qf)[D / 16],
                                         f32x16 (&oacc)[D / 32], float& mref, float& lsum, int rb, int k0,
                                         int qw0, int qw, int lane) {
    constexpr int KC = D / 16, DB = D / 32;
    constexpr float LAZY = 8.f;
    const int s = a.seq;
    f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
    for (int c = 0; c < KC; ++c)  // the two halves' chains interleaved
#pragma unroll
        for (int h = 0; h < 2; ++h) sacc[h] = Store16<ST>::mfma(fa.frag_rows(Kt, rb + 32 * h, c), qf[c], sacc[h]);
    // Keep two chunks' reads in flight: 4 LDS reads, then (2 MFMAs, 2 reads) per chunk.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int c = 0; c + 2 < KC; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // Masks only where the block reaches past the diagonal or the
    // sequence end; the scale 1/sqrt(d) (and log2 e) is folded into
    // the max and the exponent.
    if ((a.causal && k0 + BKV - 1 > qw0) || k0 + BKV > s) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 32 * h + res_row(r, lane);
                if (key >= s || (a.causal && key > qw)) sacc[h][r] = -INFINITY;
            }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, sacc[h][r]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32)) * a.scale_log2;
    if (any_lane(bmax > mref + LAZY)) {  // move the reference (to the block max where it grew)
        const float mnew = fmaxf(mref, bmax);
        const float alpha = ex2(mref - ((mnew == -INFINITY) ? 0.f : mnew));
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        mref = mnew;
    }
    const float msub = (mref == -INFINITY) ? 0.f : mref;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = ex2(fmaf(sacc[h][r], a.scale_log2, -msub));
            sacc[h][r] = pv;
            lsum += pv;
        }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        const u32x4 pf = pack_chunk<ST>(sacc[kc >> 1], kc & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = Store16<ST>::mfma(fa.frag_tr(Vt, rb, db, kc), pf, oacc[db]);
    }
}

// Forward.  The two waves of a row group (32 queries) take alternate 64-key
// blocks of each streamed pair; their online-softmax
// states (m, l, O^T) merge through LDS at the end.  The running max is a
// reference that moves only when some row's block max exceeds it by more
// than 2^8 (in the exponent's base 2): the softmax is the same for any
// reference, P stays <= 256, and O is rescaled rarely.
template <int D, typename ST>
__global__ void __launch_bounds__(NT8, 1) attn_fwd_kernel(const AttnArgs a) {
    constexpr int KC = D / 16, DB = D / 32, PT = 2 * BKV * D * 2;  // one [128][D] pair tile
    constexpr int TILE = BKV * D * 2;                              // one [64][D] tile
    constexpr int SLOT = 2 * PT;                                   // K pair, V pair
    constexpr int NMERGE = DB * 16 + 2;                            // m, l, O^T per lane
    // The Q tiles of both query blocks come into LDS once (each is read by the two
    // waves that share those queries) beside the two stages.
    constexpr int REG = 2 * SLOT + 2 * TILE;
    static_assert(REG <= 160 * 1024, "stages and Q tiles fit the LDS");
    constexpr int SMEM = REG > NMERGE * 4 * 64 * 4 ? REG : NMERGE * 4 * 64 * 4;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: derived conditions are scalar branches
    const int s = a.seq;
    int xb, bh;
    xcd_map(xb, bh);
    const PairRows pr(xb, s, wave, a.causal);
    const int qg = pr.qg, kp = pr.kp, qw0 = pr.qw0;
    const int b = bh / a.heads, g = bh % a.heads;
    const int qw = qw0 + (lane & 31);  // this lane's query

    const bf16_t* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * D;
    const bf16_t* Kg = Qg + a.w;
    const bf16_t* Vg = Qg + 2 * a.w;

    FragAddr<D> fa;
    fa.init(lane);
    TileDMA<D, 2 * BKV> gkv;  // K and V pair rows (both stride ld_qkv) straight into LDS
    gkv.init(a.ld_qkv, wave, lane);
    const int xq = xb, xlq = (s + BKV - 1) / BKV - 1 - xb;  // the workgroup's two query blocks
    char* const qt = smem + 2 * SLOT;                       // their Q tiles
    load_tiles<D, 2>(Qg, a.ld_qkv, Qg, a.ld_qkv, xq * BKV, xlq * BKV, s, qt, wave, lane);

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = zero16();
    float mref = -INFINITY, lsum = 0.f;

    const int nkb = pr.nkb;
    const int npair = (nkb + 1) / 2;
    gkv.load(Kg, a.ld_qkv, 0, s, smem, wave);
    gkv.load(Vg, a.ld_qkv, 0, s, smem + PT, wave);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads into LDS are done
    __syncthreads();
    u32x4 qf[KC];  // Q^T operand: column = query, k = d (rows past the sequence end are zeros)
    {
        const int blk = qg < 2 ? xq : xlq;
        const char* Qt = qt + (qg < 2 ? 0 : TILE);
        const int rb = (qw0 - blk * BKV) & 32;  // 0 or 32 (anything when the wave has no queries)
#pragma unroll
        for (int c = 0; c < KC; ++c) qf[c] = fa.frag_rows(Qt, rb, c);
    }

    for (int it = 0; it < npair; ++it) {
        char* const cur = smem + (it & 1) * SLOT;
        char* const nxt = smem + ((it + 1) & 1) * SLOT;
        if (it + 1 < npair) {  // slot (it+1)&1 was last read in iteration it-1, before its closing barrier
            gkv.load(Kg, a.ld_qkv, (it + 1) * 2 * BKV, s, nxt, wave);
            gkv.load(Vg, a.ld_qkv, (it + 1) * 2 * BKV, s, nxt + PT, wave);
        }
        const int kb = 2 * it + kp, k0 = kb * BKV, rb = BKV * kp;
        if (qw0 < s && kb < nkb && !(a.causal && k0 > qw0 + 31))  // some key of the block is visible to this wave
            fwd_pair<D, ST>(a, fa, cur, cur + PT, qf, oacc, mref, lsum, rb, k0, qw0, qw, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // merge the two halves: element e of row group qg, lane l at [(e*4 + qg)*64 + l]
    lsum += __shfl_xor(lsum, 32);
    float* mg = reinterpret_cast<float*>(smem);
    if (kp == 1) {
        mg[(0 * 4 + qg) * 64 + lane] = mref;
        mg[(1 * 4 + qg) * 64 + lane] = lsum;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) mg[((2 + 16 * db + r) * 4 + qg) * 64 + lane] = oacc[db][r];
    }
    __syncthreads();
    if (kp == 0) {
        const float m1 = mg[(0 * 4 + qg) * 64 + lane], l1 = mg[(1 * 4 + qg) * 64 + lane];
        const float mm = fmaxf(mref, m1);
        const float msub = (mm == -INFINITY) ? 0.f : mm;
        const float a0 = ex2(mref - msub), a1 = ex2(m1 - msub);
        const float l = lsum * a0 + l1 * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                oacc[db][r] = oacc[db][r] * a0 + mg[((2 + 16 * db + r) * 4 + qg) * 64 + lane] * a1;
        if (qw < s) {
            store_rowT<D, ST>(a.O + ((int64_t)b * s + qw) * a.ld_o + g * D, oacc, 1.f / l, lane);
            if (lane < 32) a.lse[((int64_t)b * a.heads + g) * s + qw] = (mm + log2f(l)) * LN2;
        }
    }
}

// D[b, g, j] = dO_j . O_j per head (fp32).  RD_LANES lanes per (token, head):
// lane part p reads chunks p, p + RD_LANES, ... of the head's row segment, so
// one load instruction covers 64-byte runs; the partial sums meet by two xor
// shuffles in a fixed order (deterministic).
constexpr int RD_LANES = 4;
template <int D, typename ST>
__global__ void __launch_bounds__(NT) attn_rowdot_kernel(const AttnArgs a) {
    constexpr int CPL = D / 8 / RD_LANES;  // 16-byte chunks per lane
    static_assert((D / 8) % RD_LANES == 0, "head dim must hold a multiple of 4 chunks");
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    const int64_t idx = gid / RD_LANES;  // (token, head)
    const int p = (int)(gid % RD_LANES);
    const int64_t T = (int64_t)a.batch * a.seq;
    const bool valid = idx < T * a.heads;
    const int64_t r = valid ? idx / a.heads : 0;
    const int g = valid ? (int)(idx % a.heads) : 0;
    float acc = 0.f;
    if (valid) {
        const bf16_t* o = a.O + r * a.ld_o + g * D;
        const bf16_t* d = a.dO + r * a.ld_o + g * D;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = 8 * (p + RD_LANES * k);
            const u32x4 ov = ld16(o + c), dv = ld16(d + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc += Store16<ST>::lo(ov[i]) * Store16<ST>::lo(dv[i]);
                acc += Store16<ST>::hi(ov[i]) * Store16<ST>::hi(dv[i]);
            }
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (valid && p == 0) {
        const int b = (int)(r / a.seq), j = (int)(r % a.seq);
        a.Dq[((int64_t)b * a.heads + g) * a.seq + j] = acc;
    }
}

// Sum of two partial dK, dV or dQ^T of the same rows through LDS: the wave with
// qh = 1 writes its values to slot kg and the wave with qh = 0 adds them (other
// values of qh only keep the barriers).  Every wave of the workgroup calls it.
// Up to d = 96 value r of d block db, lane l sits at
// [(((db*4 + r/4)*4 + kg)*64 + l)*4 + r%4] (16 bytes per lane and access, all
// reads of a block issued before its adds); at d = 128, where the registers
// for those reads would come from spills, at [((db*16 + r)*4 + kg)*64 + l].
template <int DB>
__device__ __forceinline__ void merge_halves(f32x16 (&acc)[DB], float* mg, int qh, int kg, int lane) {
    if constexpr (DB <= 3) {
        if (qh == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<f32x4*>(mg + (((db * 4 + r4) * 4 + kg) * 64 + lane) * 4) =
                        f32x4{acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]};
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                f32x4 t[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    t[r4] = *reinterpret_cast<const f32x4*>(mg + (((db * 4 + r4) * 4 + kg) * 64 + lane) * 4);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] += t[r / 4][r % 4];
            }
        }
    } else {
        if (qh == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mg[((16 * db + r) * 4 + kg) * 64 + lane] = acc[db][r];
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] += mg[((16 * db + r) * 4 + kg) * 64 + lane];
        }
    }
    __syncthreads();
}

// One wave's share of one streamed pair of 64-query blocks in the dK/dV pass:
// keys kw0 .. kw0+31 (K^T, V^T in kf, vf), queries 32 (half) of block j of
// the pair in LDS stage `cur` (Q and dO [128][D], then the log2-scaled LSE and
// D of the 128 queries).  The stage is a restrict pointer so that the
// compiler does not wait for the loads in flight into the other stage.
template <int D, typename ST>
__device__ __forceinline__ void dkdv_block(const AttnArgs& a, const FragAddr<D>& fa, const char* __restrict__ cur,
                                           const u32x4 (&kf)[D / 16], const u32x4 (&vf)[D / 16],
                                           f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], int q0, int j, int half,
                                           int kw0, int kw, int lane) {
    constexpr int KC = D / 16, DB = D / 32, TILE = BKV * D * 2;
    const int s = a.seq;
    const char* Qt = cur;
    const char* dOt = cur + 2 * TILE;
    const float* lse2 = reinterpret_cast<const float*>(cur + 4 * TILE) + BKV * j;
    const float* Dl = lse2 + 2 * BKV;
    const int rb = BKV * j;           // first row of block j in the tiles
    const int qh0 = q0 + 32 * half;   // this wave's 32 queries
    f32x16 sacc = zero16(), pacc = zero16();
    // The fragments of chunk c + 1 are read before the MFMAs of chunk c, so that an
    // LDS read is in flight behind every MFMA (same MFMA order per accumulator).
    u32x4 fq = fa.frag_rows(Qt, rb + 32 * half, 0), fo = fa.frag_rows(dOt, rb + 32 * half, 0);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        u32x4 nq = fq, no = fo;
        if (c + 1 < KC) {
            nq = fa.frag_rows(Qt, rb + 32 * half, c + 1);
            no = fa.frag_rows(dOt, rb + 32 * half, c + 1);
        }
        sacc = Store16<ST>::mfma(fq, kf[c], sacc);
        pacc = Store16<ST>::mfma(fo, vf[c], pacc);
        fq = nq;
        fo = no;
    }
    // rows = queries qh0 + res_row(r), column = this lane's key
    const bool edge = (a.causal && qh0 < kw0 + 31) || q0 + BKV > s || kw0 + 32 > s;  // wave-uniform
    f32x4 Dd[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int ql = 32 * half + 8 * r4 + 4 * (lane >> 5);
        const f32x4 L = *reinterpret_cast<const f32x4*>(lse2 + ql);
        Dd[r4] = *reinterpret_cast<const f32x4*>(Dl + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[4 * r4 + e] = ex2(fmaf(sacc[4 * r4 + e], a.scale_log2, -L[e]));
    }
    if (edge) {  // blocks that cross the diagonal or an end of the sequence only
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int q = q0 + 32 * half + res_row(r, lane);
            if (!(q < s && kw < s && (!a.causal || kw <= q))) sacc[r] = 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * (pacc[r] - Dd[r / 4][r % 4]);
    u32x4 to = fa.frag_tr(dOt, rb, 0, 2 * half), tq = fa.frag_tr(Qt, rb, 0, 2 * half);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const u32x4 pf = pack_chunk<ST>(sacc, hh), sf = pack_chunk<ST>(pacc, hh);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x4 no = to, nq = tq;  // the next (chunk, d block) pair's fragments
            const int nd = db + 1 < DB ? db + 1 : 0, nk = 2 * half + (db + 1 < DB ? hh : hh + 1);
            if (db + 1 < DB || hh == 0) {
                no = fa.frag_tr(dOt, rb, nd, nk);
                nq = fa.frag_tr(Qt, rb, nd, nk);
            }
            dv[db] = Store16<ST>::mfma(pf, to, dv[db]);
            dk[db] = Store16<ST>::mfma(sf, tq, dk[db]);
            to = no;
            tq = nq;
        }
    }
}

// The same at d = 128 (KVL): K^T and V^T fragments of the wave's key group from the
// phase's K/V tiles in LDS (kvt: K [64][D], then V), and the LSE and D of the
// wave's queries straight from memory (buffer ranges lrs / drs over this
// (sequence, head)'s rows; past the sequence end they read zeros), issued first
// so that their latency overlaps the S and dP products.
template <int D, typename ST>
__device__ __forceinline__ void dkdv_block_kvl(const AttnArgs& a, const char* __restrict__ cur,
                                               const char* __restrict__ kvt, __amdgpu_buffer_rsrc_t lrs,
                                               __amdgpu_buffer_rsrc_t drs, f32x16 (&dk)[D / 32],
                                               f32x16 (&dv)[D / 32], int q0, int j, int half, int kg2, int kw0,
                                               int kw, int lane, const FragAddr<D>& fa0) {
    constexpr int KC = D / 16, DB = D / 32, TILE = BKV * D * 2;
    static_assert(FragAddr<D>::XOR, "offsets derived from two registers");
    // The two base offsets pass through an empty asm statement, so that the compiler
    // derives the others here in each block instead of holding them (or their
    // spills) through the stream.
    FragAddr<D> fa = fa0;
    asm volatile("" : "+v"(fa.rows[0]), "+v"(fa.tr[0][0]));
    const int s = a.seq;
    const char* Qt = cur;
    const char* dOt = cur + 2 * TILE;
    const int rb = BKV * j;           // first row of block j in the tiles
    const int qh0 = q0 + 32 * half;   // this wave's 32 queries
    f32x4 L[4], Dd[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int q = qh0 + 8 * r4 + 4 * (lane >> 5);
        L[r4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(lrs, q * 4, 0, 0));
        Dd[r4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(drs, q * 4, 0, 0));
    }
    f32x16 sacc = zero16(), pacc = zero16();
    u32x4 fq = fa.frag_rows(Qt, rb + 32 * half, 0), fo = fa.frag_rows(dOt, rb + 32 * half, 0);
    u32x4 fk = fa.frag_rows(kvt, 32 * kg2, 0), fv = fa.frag_rows(kvt + TILE, 32 * kg2, 0);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        u32x4 nq = fq, no = fo, nk = fk, nv = fv;
        if (c + 1 < KC) {
            nq = fa.frag_rows(Qt, rb + 32 * half, c + 1);
            no = fa.frag_rows(dOt, rb + 32 * half, c + 1);
            nk = fa.frag_rows(kvt, 32 * kg2, c + 1);
            nv = fa.frag_rows(kvt + TILE, 32 * kg2, c + 1);
        }
        sacc = Store16<ST>::mfma(fq, fk, sacc);
        pacc = Store16<ST>::mfma(fo, fv, pacc);
        fq = nq;
        fo = no;
        fk = nk;
        fv = nv;
    }
    // rows = queries qh0 + res_row(r), column = this lane's key
    const bool edge = (a.causal && qh0 < kw0 + 31) || q0 + BKV > s || kw0 + 32 > s;  // wave-uniform
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sacc[4 * r4 + e] = ex2(fmaf(sacc[4 * r4 + e], a.scale_log2, -L[r4][e] * LOG2E));
    if (edge) {  // blocks that cross the diagonal or an end of the sequence only
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int q = q0 + 32 * half + res_row(r, lane);
            if (!(q < s && kw < s && (!a.causal || kw <= q))) sacc[r] = 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * (pacc[r] - Dd[r / 4][r % 4]);
    u32x4 to = fa.frag_tr(dOt, rb, 0, 2 * half), tq = fa.frag_tr(Qt, rb, 0, 2 * half);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const u32x4 pf = pack_chunk<ST>(sacc, hh), sf = pack_chunk<ST>(pacc, hh);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x4 no = to, nq = tq;  // the next (chunk, d block) pair's fragments
            const int nd = db + 1 < DB ? db + 1 : 0, nk = 2 * half + (db + 1 < DB ? hh : hh + 1);
            if (db + 1 < DB || hh == 0) {
                no = fa.frag_tr(dOt, rb, nd, nk);
                nq = fa.frag_tr(Qt, rb, nd, nk);
            }
            dv[db] = Store16<ST>::mfma(pf, to, dv[db]);
            dk[db] = Store16<ST>::mfma(sf, tq, dk[db]);
            to = no;
            tq = nq;
        }
    }
}

// dK, dV for the 64-key blocks x and nb-1-x.  Causal: one block after the
// other, each with all 8 waves: wave = (32-key group kg2 = wave & 1) x (query
// quarter qq = wave >> 1: block qq / 2 of each streamed pair of 64-query
// blocks, 32-query half qq % 2).  Block x sees nb - x query blocks and block
// nb-1-x sees x + 1, so every workgroup streams about (nb + 1) / 2 pairs
// whatever x is (a workgroup that ran both key blocks side by side over one
// query stream would take nb - x steps while the waves of the later block
// wait); the four quarters' dK, dV add through LDS in a fixed order,
// (q0 + q1) + (q2 + q3).  No mask (NOMASK, used up to d = 64): both key blocks
// see every query, so they run side by side over one stream (wave = 32-key
// group wave & 3 of the two blocks x 32-query half wave >> 2, both blocks of
// each pair), halves added q0 + q1; larger heads without a mask take the
// one-block-at-a-time form, whose registers fit.  Q and dO pairs go straight into LDS (two stages), the LSE and D
// of their queries through registers.  Deterministic either way.
// LDS of the dK/dV pass.
template <int D>
struct DkdvLds {
    static constexpr int TILE = BKV * D * 2, DB = D / 32;
    // KVL (d = 128): the K and V fragments of the phase's key block are read from LDS in every
    // block instead of being held in registers through the stream (which spilled), and the LSE
    // and D of the queries come from memory, so a stage is just the Q and dO pairs.
    static constexpr bool KVL = D == 128;
    static constexpr int SLOT = 4 * TILE + (KVL ? 0 : 4 * BKV * 4);  // Q pair, dO pair[, LSE pair, D pair]
    static constexpr int MERGE = 4 * DB * 16 * 64 * 4;   // one of dK / dV for four groups
    // PRE: the K and V tiles of both key blocks come into LDS once, at the start
    // (the fragments of a key group are then read from LDS by each of the four
    // waves that use them, instead of four times from memory), where they fit
    // beside the two stages (up to d = 96).
    static constexpr bool PRE = !KVL && 2 * SLOT + 4 * TILE <= 160 * 1024;
    static constexpr int REG = 2 * SLOT + (PRE ? 4 * TILE : KVL ? 2 * TILE : 0);
    static constexpr int SMEM = REG > MERGE ? REG : MERGE;
    static_assert(REG <= 160 * 1024, "the stages and K/V tiles fit the LDS");
};

template <int D, typename ST, bool NOMASK>
__device__ __forceinline__ void dkdv_body(const AttnArgs& a, char* __restrict__ smem, int x, int bh) {
    constexpr int KC = D / 16, DB = D / 32, TILE = DkdvLds<D>::TILE;
    constexpr int SLOT = DkdvLds<D>::SLOT, MERGE = DkdvLds<D>::MERGE;
    constexpr bool PRE = DkdvLds<D>::PRE, KVL = DkdvLds<D>::KVL;
    constexpr int PITCH = D * 2 + 16;  // row pitch of the bf16 dK / dV image (rows 4 apart on other banks)
    static_assert(2 * BKV * PITCH <= SLOT && MERGE <= SLOT, "epilogue areas fit one stage");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: derived conditions are scalar branches
    const int s = a.seq;
    const int nb = (s + BKV - 1) / BKV, xl = nb - 1 - x;
    const bool side = NOMASK && xl != x;  // both key blocks over one query stream
    const int kg2 = wave & 1, qq = side ? 2 * (wave >> 2) : wave >> 1;
    const int jb = qq >> 1, half = side ? wave >> 2 : qq & 1;
    const int b = bh / a.heads, g = bh % a.heads;

    const bf16_t* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * D;
    const bf16_t* Kg = Qg + a.w;
    const bf16_t* Vg = Qg + 2 * a.w;
    const bf16_t* dOg = a.dO + (int64_t)b * s * a.ld_o + g * D;
    const float* lseg = a.lse + ((int64_t)b * a.heads + g) * s;
    const float* Dg = a.Dq + ((int64_t)b * a.heads + g) * s;

    FragAddr<D> fa;
    fa.init(lane);
    TileDMA<D, 2 * BKV> gq, go;  // Q rows (stride ld_qkv), dO rows (stride ld_o)
    gq.init(a.ld_qkv, wave, lane);
    go.init(a.ld_o, wave, lane);
    char* const st0 = smem;
    char* const st1 = smem + SLOT;
    char* const kvt = smem + 2 * SLOT;  // PRE: [K | V] of key block x, then of key block nb-1-x;
                                        // KVL: [K | V] of the phase's key block
    if constexpr (PRE) load_tiles<D, 4>(Kg, a.ld_qkv, Vg, a.ld_qkv, x * BKV, xl * BKV, s, kvt, wave, lane);
    TileDMA<D, KVL ? BKV : 2 * BKV> gkv1;  // KVL: one 64-row K or V tile (unused otherwise)
    __amdgpu_buffer_rsrc_t lrs, drs;  // KVL: this (sequence, head)'s LSE and D rows
    if constexpr (KVL) {
        gkv1.init(a.ld_qkv, wave, lane);
        lrs = make_rsrc(lseg, (uint32_t)s * 4u);
        drs = make_rsrc(Dg, (uint32_t)s * 4u);
    }

    const int nphase = (xl != x && !side) ? 2 : 1;
    int sbase = 0;        // slot of the phase's first stage
    bool staged = false;  // that stage is already in LDS (loaded during the previous phase)
    for (int ph = 0; ph < nphase; ++ph) {
        const int kb = side ? ((wave & 2) ? xl : x) : (ph == 0 ? x : xl);
        const int kw0 = min(s, kb * BKV + 32 * kg2);  // first key of this wave's group (s: none)
        const int kw = kw0 + (lane & 31);              // this lane's key
        const int qs = a.causal ? kb : 0;     // the first query block that sees the key block
        const int npair = (nb - qs + 1) / 2;  // streamed pairs of query blocks
        float lsev = 0.f, dval = 0.f;         // threads < 128: one query's LSE and D
        if (!staged && npair > 0) {
            const int row0 = qs * BKV;
            gq.load(Qg, a.ld_qkv, row0, s, st0, wave);
            go.load(dOg, a.ld_o, row0, s, st0 + 2 * TILE, wave);
            if (!KVL && tid < 2 * BKV) {
                const int q = row0 + tid;
                lsev = q < s ? lseg[q] : 0.f;
                dval = q < s ? Dg[q] : 0.f;
            }
        }
        if constexpr (KVL) {  // the phase's K and V tiles (the previous phase's reads ended at its last barrier)
            gkv1.load(Kg, a.ld_qkv, kb * BKV, s, kvt, wave);
            gkv1.load(Vg, a.ld_qkv, kb * BKV, s, kvt + TILE, wave);
        }
        u32x4 kf[KC], vf[KC];  // K^T, V^T operands (not KVL): column = key, k = d
        if constexpr (!PRE && !KVL) {
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const bool ok = kw < s;
                const int64_t o = (int64_t)kw * a.ld_qkv + 16 * c + 8 * (lane >> 5);
                kf[c] = ok ? ld16(Kg + o) : u32x4{0u, 0u, 0u, 0u};
                vf[c] = ok ? ld16(Vg + o) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (!staged) {
            __builtin_amdgcn_s_waitcnt(0);  // this thread's loads are done
            if (!KVL && npair > 0 && tid < 2 * BKV) {
                reinterpret_cast<float*>(st0 + 4 * TILE)[tid] = lsev * LOG2E;
                reinterpret_cast<float*>(st0 + 4 * TILE + 2 * BKV * 4)[tid] = dval;
            }
            __syncthreads();
        }
        if constexpr (PRE) {  // rows past the sequence end are zeros in the tiles
            const char* Kt = kvt + (kb == x ? 0 : 2 * TILE);
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                kf[c] = fa.frag_rows(Kt, 32 * kg2, c);
                vf[c] = fa.frag_rows(Kt + TILE, 32 * kg2, c);
            }
        }
        f32x16 dk[DB], dv[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) dk[i] = dv[i] = zero16();

        const int qs_next = a.causal ? xl : 0;  // the next phase's first query block
        for (int it = 0; it < npair; ++it) {
            const int slot = (it + sbase) & 1;
            char* const cur = slot ? st1 : st0;
            char* const nxt = slot ? st0 : st1;
            const bool more = it + 1 < npair;
            const bool pre1 = PRE && !more && ph + 1 < nphase;  // the next phase's first stage
            if (more || pre1) {  // the other stage was last read in iteration it-1, before its closing barrier
                const int row1 = more ? (qs + 2 * (it + 1)) * BKV : qs_next * BKV;
                gq.load(Qg, a.ld_qkv, row1, s, nxt, wave);
                go.load(dOg, a.ld_o, row1, s, nxt + 2 * TILE, wave);
                if (!KVL && tid < 2 * BKV) {  // raw values: scaling them here would wait for every load in flight
                    const int q = row1 + tid;
                    lsev = q < s ? lseg[q] : 0.f;
                    dval = q < s ? Dg[q] : 0.f;
                }
            }
            if (NOMASK && side) {  // both query blocks of the pair, this wave's half of each
#pragma unroll 1
                for (int j = 0; j < 2; ++j) {  // rolled: two copies of the block would spill
                    const int q0 = (qs + 2 * it + j) * BKV;
                    if (kw0 < s && q0 < s) dkdv_block<D, ST>(a, fa, cur, kf, vf, dk, dv, q0, j, half, kw0, kw, lane);
                }
            } else {
                const int q0 = (qs + 2 * it + jb) * BKV;  // this wave's query block
                // skip when the key group or the query block is empty, or every query precedes every key
                if (kw0 < s && q0 < s && !(a.causal && q0 + 32 * half + 31 < kw0)) {
                    if constexpr (KVL)
                        dkdv_block_kvl<D, ST>(a, cur, kvt, lrs, drs, dk, dv, q0, jb, half, kg2, kw0, kw, lane, fa);
                    else
                        dkdv_block<D, ST>(a, fa, cur, kf, vf, dk, dv, q0, jb, half, kw0, kw, lane);
                }
            }
            if (!KVL && (more || pre1) && tid < 2 * BKV) {
                reinterpret_cast<float*>(nxt + 4 * TILE)[tid] = lsev * LOG2E;
                reinterpret_cast<float*>(nxt + 4 * TILE + 2 * BKV * 4)[tid] = dval;
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // the next phase's first stage (if loaded) sits in slot (npair + sbase) & 1; the
        // merges and the output image use the other slot
        const int nslot = (npair + sbase) & 1;
        staged = PRE && ph + 1 < nphase && npair > 0;
        sbase = staged ? nslot : 0;
        char* const ep = (staged && nslot == 0) ? st1 : st0;

        float* mg = reinterpret_cast<float*>(ep);
        if (NOMASK && side) {  // q0 + q1 per key group
            merge_halves<DB>(dk, mg, half, wave & 3, lane);
            merge_halves<DB>(dv, mg, half, wave & 3, lane);
        } else {  // (q0 + q1) + (q2 + q3): odd quarters into even ones, then quarter 2 into 0
            merge_halves<DB>(dk, mg, half, 2 * kg2 + jb, lane);
            merge_halves<DB>(dv, mg, half, 2 * kg2 + jb, lane);
            const int role2 = qq == 0 ? 0 : (qq == 2 ? 1 : 2);
            merge_halves<DB>(dk, mg, role2, kg2, lane);
            merge_halves<DB>(dv, mg, role2, kg2, lane);
        }

        // dk/dv: rows = keys kw0 + res_row(r), column = d 32db + lane%32
        bf16_t* dKg = a.dqkv + (int64_t)b * s * a.ld_qkv + a.w + g * D;
        bf16_t* dVg = dKg + a.w;
        if (!(PRE || KVL) || (NOMASK && side)) {  // each writer stores its values directly
            if ((side ? half == 0 : qq == 0) && kw0 < s) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kw0 + res_row(r, lane);
                    if (key >= s) continue;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int c = 32 * db + (lane & 31);
                        dKg[(int64_t)key * a.ld_qkv + c] = Store16<ST>::from_f(dk[db][r] * a.scale);
                        dVg[(int64_t)key * a.ld_qkv + c] = Store16<ST>::from_f(dv[db][r]);
                    }
                }
            }
        } else {  // the two writers' values as a bf16 [64][D] image per tensor, then 16-byte row stores
            if (qq == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * kg2 + res_row(r, lane);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int c = 32 * db + (lane & 31);
                        *reinterpret_cast<uint16_t*>(ep + row * PITCH + c * 2) = Store16<ST>::from_f(dk[db][r] * a.scale);
                        *reinterpret_cast<uint16_t*>(ep + (BKV + row) * PITCH + c * 2) = Store16<ST>::from_f(dv[db][r]);
                    }
                }
            }
            __syncthreads();
            constexpr int CH = D / 8;  // 16-byte chunks per row
#pragma unroll
            for (int e0 = 0; e0 < 2 * BKV * CH; e0 += NT8) {
                const int e = e0 + tid;
                const int tsel = e / (BKV * CH), rr = (e / CH) % BKV, cc = e % CH;
                const int key = kb * BKV + rr;
                if (e < 2 * BKV * CH && key < s) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(ep + (tsel * BKV + rr) * PITCH + cc * 16);
                    *reinterpret_cast<u32x4*>((tsel ? dVg : dKg) + (int64_t)key * a.ld_qkv + cc * 8) = v;
                }
            }
        }
        __syncthreads();  // the epilogue slot is a stage of the next phase
    }
}

// One wave's dQ^T update from 32 keys k0 .. k0+31 of a streamed K/V pair in LDS
// (rows rb .. rb+31 of the pair tiles) for its 32 queries (Q^T, dO^T in qf, of).
template <int D, typename ST>
__device__ __forceinline__ void dq_keys(const AttnArgs& a, const FragAddr<D>& fa, const char* __restrict__ Kt,
                                        const char* __restrict__ Vt,
                                        const u32x4 (&qf)[D / 16], const u32x4 (&of)[D / 16],
                                        f32x16 (&dq)[D / 32], int rb, int k0, int qw0, int qw, float lse2,
                                        float Dv, int lane) {
    constexpr int KC = D / 16, DB = D / 32;
    const int s = a.seq;
    f32x16 sacc = zero16(), pacc = zero16();  // S^T and dP^T: rows = keys, column = this lane's query
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        sacc = Store16<ST>::mfma(fa.frag_rows(Kt, rb, c), qf[c], sacc);
        pacc = Store16<ST>::mfma(fa.frag_rows(Vt, rb, c), of[c], pacc);
    }
    // Keep two chunks' reads in flight: 4 LDS reads, then (2 MFMAs, 2 reads) per chunk
    // (up to d = 96: at d = 128 the registers of the extra reads come from spills).
    if constexpr (D <= 96) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int c = 0; c + 2 < KC; ++c) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    const bool edge = (a.causal && k0 + 31 > qw0) || k0 + 32 > s || qw0 + 32 > s;  // wave-uniform
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = ex2(fmaf(sacc[r], a.scale_log2, -lse2));
    if (edge) {  // blocks that cross the diagonal or an end of the sequence only
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + res_row(r, lane);
            if (!(qw < s && key < s && (!a.causal || key <= qw))) sacc[r] = 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * (pacc[r] - Dv);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const u32x4 sf = pack_chunk<ST>(pacc, kc);
#pragma unroll
        for (int db = 0; db < DB; ++db) dq[db] = Store16<ST>::mfma(fa.frag_tr(Kt, rb, db, kc), sf, dq[db]);
    }
}

// The query rows of phase ph of a dQ workgroup for one wave: its 64-query block
// and its first query (s when the wave has none).  Causal (masked): block x,
// then nb-1-x, 32 queries per row group rg; no mask: the forward's pair layout.
__device__ __forceinline__ void dq_rows(bool masked, int ph, int x, int xl, int rg, const PairRows& pr, int s, int& blk,
                                        int& qw0) {
    blk = masked ? (ph == 0 ? x : xl) : (pr.qg < 2 ? x : xl);
    qw0 = masked ? min(s, blk * BKV + 32 * rg) : pr.qw0;
}

// dQ for the 64-query blocks x and nb-1-x.  Causal (MASKED): one block after the
// other, each with all 8 waves: wave = (32-query row group rg = wave & 1) x
// (key part kq = wave >> 1: 32-key half kq % 2 of key block kq / 2 of each
// streamed K/V pair).  Block x sees x + 1 key blocks and block nb-1-x sees
// nb - x, so every workgroup streams about (nb + 2) / 2 pairs of half the
// per-wave work whatever x is (side by side over one key stream it would take
// (nb - x) / 2 full steps while the waves of block x wait); the four parts'
// dQ^T add through LDS as (k0 + k1) + (k2 + k3).  No mask: both query blocks
// see every key, so they run side by side over one stream (the forward's
// layout: the two waves of a row group take alternate 64-key blocks of each
// pair), halves added k0 + k1.  Deterministic either way.
// LDS of the dQ pass.
template <int D>
struct DqLds {
    static constexpr int TILE = BKV * D * 2, PT = 2 * BKV * D * 2, DB = D / 32;
    static constexpr int SLOT = 2 * PT;  // K pair, V pair
    static constexpr int MERGE = DB * 16 * 4 * 64 * 4;
    // PRE: the Q and dO tiles of both query blocks come into LDS once, at the start
    // (each is read by the four waves that share those queries), where they fit
    // beside the two stages (up to d = 96).
    static constexpr bool PRE = 2 * SLOT + 4 * TILE <= 160 * 1024;
    static constexpr int REG = 2 * SLOT + (PRE ? 4 * TILE : 0);
    static constexpr int SMEM = REG > MERGE ? REG : MERGE;
};

template <int D, typename ST, bool MASKED>
__device__ __forceinline__ void dq_body(const AttnArgs& a, char* __restrict__ smem, int x, int bh) {
    constexpr int KC = D / 16, DB = D / 32, PT = DqLds<D>::PT, TILE = DqLds<D>::TILE;
    constexpr int SLOT = DqLds<D>::SLOT, MERGE = DqLds<D>::MERGE;
    constexpr bool PRE = DqLds<D>::PRE;
    static_assert(MERGE <= SLOT, "the merge area fits one stage");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: derived conditions are scalar branches
    const int s = a.seq;
    const int nb = (s + BKV - 1) / BKV, xl = nb - 1 - x;
    const int b = bh / a.heads, g = bh % a.heads;
    const PairRows pr(x, s, wave, a.causal);  // the side-by-side layout (no mask)
    const int rg = wave & 1, kq = wave >> 1;  // the one-after-the-other layout (causal)

    const bf16_t* Qg = a.qkv + (int64_t)b * s * a.ld_qkv + g * D;
    const bf16_t* Kg = Qg + a.w;
    const bf16_t* Vg = Qg + 2 * a.w;
    const bf16_t* dOg = a.dO + (int64_t)b * s * a.ld_o + g * D;
    const int64_t hrow = ((int64_t)b * a.heads + g) * s;

    FragAddr<D> fa;
    fa.init(lane);
    TileDMA<D, 2 * BKV> gkv;  // K and V pair rows (both stride ld_qkv) straight into LDS
    gkv.init(a.ld_qkv, wave, lane);
    char* const st0 = smem;
    char* const st1 = smem + SLOT;
    char* const qdt = smem + 2 * SLOT;  // PRE: [Q | dO] of query block x, then of query block nb-1-x
    if constexpr (PRE) load_tiles<D, 4>(Qg, a.ld_qkv, dOg, a.ld_o, x * BKV, xl * BKV, s, qdt, wave, lane);

    const int nphase = (MASKED && xl != x) ? 2 : 1;
    int blk, qw0;
    dq_rows(MASKED, 0, x, xl, rg, pr, s, blk, qw0);
    float lse_raw = 0.f, d_raw = 0.f;  // this lane's query: LSE and D, loaded a phase ahead
    {
        const int qw = qw0 + (lane & 31);
        if (qw < s) {
            lse_raw = a.lse[hrow + qw];
            d_raw = a.Dq[hrow + qw];
        }
    }
    int sbase = 0;        // slot of the phase's first stage
    bool staged = false;  // that stage is already in LDS (loaded during the previous phase)
    for (int ph = 0; ph < nphase; ++ph) {
        const int qb = MASKED ? (ph == 0 ? x : xl) : x;
        dq_rows(MASKED, ph, x, xl, rg, pr, s, blk, qw0);
        const int qw = qw0 + (lane & 31);  // this lane's query
        if (ph > 0 && !staged) {  // not loaded during the previous phase
            lse_raw = qw < s ? a.lse[hrow + qw] : 0.f;
            d_raw = qw < s ? a.Dq[hrow + qw] : 0.f;
        }
        const int nkb = MASKED ? (a.causal ? qb + 1 : nb) : pr.nkb;  // key blocks the phase streams
        const int npair = (nkb + 1) / 2;
        u32x4 qf[KC], of[KC];  // Q^T, dO^T operands: column = query, k = d
        if constexpr (!PRE) {
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const bool ok = qw < s;
                qf[c] = ok ? ld16(Qg + (int64_t)qw * a.ld_qkv + 16 * c + 8 * (lane >> 5)) : u32x4{0u, 0u, 0u, 0u};
                of[c] = ok ? ld16(dOg + (int64_t)qw * a.ld_o + 16 * c + 8 * (lane >> 5)) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (!staged) {
            gkv.load(Kg, a.ld_qkv, 0, s, st0, wave);
            gkv.load(Vg, a.ld_qkv, 0, s, st0 + PT, wave);
            __builtin_amdgcn_s_waitcnt(0);  // this thread's loads are done
            __syncthreads();
        }
        if constexpr (PRE) {  // rows past the sequence end are zeros in the tiles
            const char* Qt = qdt + (blk == x ? 0 : 2 * TILE);
            const int rb = qw0 - blk * BKV;  // 0 or 32 (anything when the wave has no queries)
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                qf[c] = fa.frag_rows(Qt, rb & 32, c);
                of[c] = fa.frag_rows(Qt + TILE, rb & 32, c);
            }
        }
        const float lse2 = lse_raw * LOG2E;
        const float Dv = d_raw;
        f32x16 dq[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) dq[i] = zero16();

        for (int it = 0; it < npair; ++it) {
            const int slot = (it + sbase) & 1;
            char* const Kt = slot ? st1 : st0;
            char* const Vt = Kt + PT;
            char* const nxt = slot ? st0 : st1;
            const bool more = it + 1 < npair;
            const bool pre1 = PRE && !more && ph + 1 < nphase;  // the next phase's first stage (keys 0 .. 127)
            if (more || pre1) {  // slot nxt was last read in iteration it-1, before its closing barrier
                const int row1 = more ? (it + 1) * 2 * BKV : 0;
                gkv.load(Kg, a.ld_qkv, row1, s, nxt, wave);
                gkv.load(Vg, a.ld_qkv, row1, s, nxt + PT, wave);
            }
            if (pre1) {  // the next phase's LSE and D of this lane's query
                int nblk, nq0;
                dq_rows(MASKED, ph + 1, x, xl, rg, pr, s, nblk, nq0);
                const int nq = nq0 + (lane & 31);
                lse_raw = nq < s ? a.lse[hrow + nq] : 0.f;
                d_raw = nq < s ? a.Dq[hrow + nq] : 0.f;
            }
            if constexpr (MASKED) {  // 32 keys: half kq % 2 of block 2 it + kq / 2
                const int kb = 2 * it + (kq >> 1), rb = BKV * (kq >> 1) + 32 * (kq & 1), k0 = 2 * it * BKV + rb;
                if (qw0 < s && kb < nkb && !(a.causal && k0 > qw0 + 31))
                    dq_keys<D, ST>(a, fa, Kt, Vt, qf, of, dq, rb, k0, qw0, qw, lse2, Dv, lane);
            } else {  // 64 keys: block 2 it + kp, both halves in order
                const int kb = 2 * it + pr.kp, k0 = kb * BKV, rb = BKV * pr.kp;
                if (qw0 < s && kb < nkb && !(a.causal && k0 > qw0 + 31)) {
                    dq_keys<D, ST>(a, fa, Kt, Vt, qf, of, dq, rb, k0, qw0, qw, lse2, Dv, lane);
                    dq_keys<D, ST>(a, fa, Kt, Vt, qf, of, dq, rb + 32, k0 + 32, qw0, qw, lse2, Dv, lane);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // the next phase's first stage (if loaded) sits in slot (npair + sbase) & 1; the
        // merges use the other slot
        const int nslot = (npair + sbase) & 1;
        staged = PRE && ph + 1 < nphase && npair > 0;
        sbase = staged ? nslot : 0;
        float* mg = reinterpret_cast<float*>((staged && nslot == 0) ? st1 : st0);
        bool writer;
        if constexpr (MASKED) {  // (k0 + k1) + (k2 + k3) per row group
            merge_halves<DB>(dq, mg, kq & 1, 2 * rg + (kq >> 1), lane);
            merge_halves<DB>(dq, mg, kq == 0 ? 0 : (kq == 2 ? 1 : 2), rg, lane);
            writer = kq == 0;
        } else {  // k0 + k1 per row group
            merge_halves<DB>(dq, mg, pr.kp, pr.qg, lane);
            writer = pr.kp == 0;
        }
        if (writer && qw < s) store_rowT<D, ST>(a.dqkv + ((int64_t)b * s + qw) * a.ld_qkv + g * D, dq, a.scale, lane);
        __syncthreads();  // the merge area is a stage of the next phase
    }
}

template <int D, typename ST, bool NOMASK>
__global__ void __launch_bounds__(NT8, 1) attn_bwd_dkdv_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[DkdvLds<D>::SMEM];
    int x, bh;
    xcd_map(x, bh);
    dkdv_body<D, ST, NOMASK>(a, smem, x, bh);
}

template <int D, typename ST, bool MASKED>
__global__ void __launch_bounds__(NT8, 1) attn_bwd_dq_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[DqLds<D>::SMEM];
    int x, bh;
    xcd_map(x, bh);
    dq_body<D, ST, MASKED>(a, smem, x, bh);
}

// The dK/dV and dQ passes (independent of each other) as one launch: grid rows
// 0 .. bh-1 are the dK/dV workgroups, the rest the dQ ones, numbered for the
// XCDs as two grids of their own.  The dK/dV workgroups come first in dispatch
// order; a dQ workgroup starts on a CU as soon as a dK/dV one leaves it, with no
// kernel boundary in between.
template <int D, typename ST, bool NOMASK, bool MASKED>
__global__ void __launch_bounds__(NT8, 1) attn_bwd_dkdv_dq_kernel(const AttnArgs a) {
    constexpr int SM = DkdvLds<D>::SMEM > DqLds<D>::SMEM ? DkdvLds<D>::SMEM : DqLds<D>::SMEM;
    __shared__ __attribute__((aligned(1024))) char smem[SM];
    const int nx = (int)gridDim.x, n = (int)(gridDim.x * gridDim.y) / 2;
    const int L = (int)(blockIdx.x + blockIdx.y * gridDim.x);
    int x, bh;
    if (L < n) {
        xcd_map_n(L, n, nx, x, bh);
        dkdv_body<D, ST, NOMASK>(a, smem, x, bh);
    } else {
        xcd_map_n(L - n, n, nx, x, bh);
        dq_body<D, ST, MASKED>(a, smem, x, bh);
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

template <int D, typename ST>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
    dim3 grid(((a.seq + BKV - 1) / BKV + 1) / 2, a.batch * a.heads);
    hipLaunchKernelGGL((attn_fwd_kernel<D, ST>), grid, dim3(NT8), 0, s, a);
    count_launch();
    return hipGetLastError();
}

template <int D, typename ST>
hipError_t bwd_d(const AttnArgs& a, int part, hipStream_t s) {
    const int64_t T = (int64_t)a.batch * a.seq;
    dim3 grid_pair(((a.seq + BKV - 1) / BKV + 1) / 2, a.batch * a.heads);
    if (part == ATTN_BWD_ROWDOT)
        hipLaunchKernelGGL((attn_rowdot_kernel<D, ST>), dim3((unsigned)((T * a.heads * RD_LANES + NT - 1) / NT)), dim3(NT), 0, s, a);
    else if (part == ATTN_BWD_DKDV)
    {
        // The side-by-side form for the unmasked case fits the registers only up to d = 64
        // (beyond, two query blocks per step spill); larger heads take the one-block-at-a-time form.
        if constexpr (D <= 64) {
            if (!a.causal) {
                hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, ST, true>), grid_pair, dim3(NT8), 0, s, a);
                count_launch();
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, ST, false>), grid_pair, dim3(NT8), 0, s, a);
    }
    else if (part == ATTN_BWD_DQ) {
        if (a.causal)
            hipLaunchKernelGGL((attn_bwd_dq_kernel<D, ST, true>), grid_pair, dim3(NT8), 0, s, a);
        else
            hipLaunchKernelGGL((attn_bwd_dq_kernel<D, ST, false>), grid_pair, dim3(NT8), 0, s, a);
    } else if (part == ATTN_BWD_DKDV_DQ) {
        const dim3 grid2(grid_pair.x, 2 * grid_pair.y);
        bool side = false;  // the side-by-side dK/dV form (unmasked, up to d = 64, as above)
        if constexpr (D <= 64) {
            if (!a.causal) {
                hipLaunchKernelGGL((attn_bwd_dkdv_dq_kernel<D, ST, true, false>), grid2, dim3(NT8), 0, s, a);
                side = true;
            }
        }
        if (!side) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dkdv_dq_kernel<D, ST, false, true>), grid2, dim3(NT8), 0, s, a);
            else
                hipLaunchKernelGGL((attn_bwd_dkdv_dq_kernel<D, ST, false, false>), grid2, dim3(NT8), 0, s, a);
        }
    }
    else
        return hipErrorInvalidValue;
    count_launch();
    return hipGetLastError();
}

template <typename ST>
hipError_t fwd_st(const AttnArgs& a, int dh, hipStream_t s) {
    switch (dh) {
        case 32: return fwd_d<32, ST>(a, s);
        case 64: return fwd_d<64, ST>(a, s);
        case 96: return fwd_d<96, ST>(a, s);
        case 128: return fwd_d<128, ST>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename ST>
hipError_t bwd_st(const AttnArgs& a, int dh, int part, hipStream_t s) {
    switch (dh) {
        case 32: return bwd_d<32, ST>(a, part, s);
        case 64: return bwd_d<64, ST>(a, part, s);
        case 96: return bwd_d<96, ST>(a, part, s);
        case 128: return bwd_d<128, ST>(a, part, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t attn_fwd_bf16(const AttnDesc& d, hipStream_t s) {
    const AttnArgs a = make_args(d);
    return d.fp16 ? fwd_st<f16_t>(a, d.dh, s) : fwd_st<bf16_t>(a, d.dh, s);
}

hipError_t attn_bwd_bf16(const AttnDesc& d, int part, hipStream_t s) {
    const AttnArgs a = make_args(d);
    return d.fp16 ? bwd_st<f16_t>(a, d.dh, part, s) : bwd_st<bf16_t>(a, d.dh, part, s);
}

}  // namespace tp
