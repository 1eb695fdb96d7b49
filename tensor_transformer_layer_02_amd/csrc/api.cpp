// C ABI of the tensor-parallel layer shard (declared in include/tpshard.h).
//
// Each entry point validates every argument on the host first (no HIP call
// before validation passes, nothing written on failure), then enqueues its
// kernels on the caller's stream:
//   tp_mlp_shard_fwd : [X*A_i + b1 -> U, GeLU'(U) -> Gp, GeLU(U) -> Y]  [Y*B_i -> Z_part]
//   tp_mlp_shard_bwd : [dZ*B_i^T (*) Gp -> dU]  [Y^T dZ -> dB_i]
//                      [X^T dU -> dA_i]  [colsum dU -> db1_i]  [dU*A_i^T -> dX_part]
//   tp_attn_shard_fwd: [X*[Wq|Wk|Wv]_i + b -> QKV]  [fused attention -> O, LSE]
//                      [O*Wo_i -> Z_part]
//   tp_attn_shard_bwd: [dZ*Wo_i^T -> dO]  [fused attention bwd -> dQKV]
//                      [X^T dQKV -> dW{q,k,v}_i, O^T dZ -> dWo_i] (one launch)
//                      [dQKV*[Wq|Wk|Wv]_i^T -> dX_part]; the last, and
//                      [colsum -> db{q,k,v}_i] before it, on the auxiliary stream
//                      beside the weight-gradient launch
// The MLP backward's column sum also runs on the auxiliary stream.
// The shard slices follow page "Megatron-LM: what the tensor parallelism paper
// actually says": FFN columns/rows C_i ("How transformer layers actually
// decompose"), head columns/rows G_i ("The attention heads split").
#include "../../include/tpshard.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "tp_kernels.h"

namespace {

constexpr int SEG_NONE = 1 << 30;

struct Shape {
    int64_t T, b, s, h, H, F, t, i, Fs, Hs, d, w;
    bool causal;
    bool h16;        // 16-bit storage (bfloat16 or IEEE half)
    bool fp16;       // dims.act == TP_FP16
    bool gelu_tanh;  // dims.gelu == TP_GELU_TANH
    int64_t e;  // bytes per element of dims.act
};

int derive(const tp_dims* dims, int shard, int degree, Shape* o) {
    if (!dims) return TP_EINVAL;
    if (dims->act != TP_FP32 && dims->act != TP_BF16 && dims->act != TP_FP16) return TP_EDTYPE;
    if (dims->batch <= 0 || dims->seq <= 0 || dims->hidden <= 0 || dims->heads <= 0 || dims->ffn <= 0)
        return TP_EINVAL;
    if (dims->causal != 0 && dims->causal != 1) return TP_EINVAL;
    if (dims->gelu != TP_GELU_ERF && dims->gelu != TP_GELU_TANH) return TP_EINVAL;
    if (degree < 1 || shard < 0 || shard >= degree) return TP_ESHARD;
    if (dims->hidden % dims->heads) return TP_EDIVIDE;
    if (dims->heads % degree || dims->ffn % degree) return TP_EDIVIDE;
    Shape s;
    s.b = dims->batch; s.s = dims->seq; s.T = s.b * s.s;
    s.h = dims->hidden; s.H = dims->heads; s.F = dims->ffn;
    s.t = degree; s.i = shard;
    s.Fs = s.F / degree; s.Hs = s.H / degree; s.d = s.h / s.H; s.w = s.Hs * s.d;
    s.causal = dims->causal != 0;
    s.gelu_tanh = dims->gelu == TP_GELU_TANH;
    s.h16 = dims->act != TP_FP32;
    s.fp16 = dims->act == TP_FP16;
    s.e = s.h16 ? 2 : 4;
    if (s.h % 8 || s.Fs % 8 || s.w % 8) return TP_EALIGN;
    if (s.h16) {
        if (s.d != 32 && s.d != 64 && s.d != 96 && s.d != 128) return TP_EUNSUPPORTED;
        if (s.w % 64) return TP_EUNSUPPORTED;  // K-segment of the fused QKV backward GEMM
    } else {
        if (s.d % 8 || s.d > 128) return TP_EUNSUPPORTED;
    }
    // Launch-grid limits (grid y <= 65535 with 64-row tiles; int indices).
    if (s.T > (int64_t)65535 * 64 || s.b * s.Hs > 65535) return TP_EUNSUPPORTED;
    if (s.h > INT_MAX / 4 || s.F > INT_MAX / 4) return TP_EUNSUPPORTED;
    // The kernels address their operands through buffer descriptors with 32-bit
    // byte ranges and offsets, so every matrix the shard reads or writes must stay
    // below 2 GiB: activations and partials [T, h], [T, F/t], [T, 3w], the weights
    // [h, F] and [h, h], and their fp32 gradients.
    const int64_t lim = (int64_t)1 << 31;
    const int64_t ext[] = {s.T * s.h * s.e, s.T * s.Fs * s.e, s.T * 3 * s.w * s.e,
                           s.h * s.F * 4, s.h * s.h * 4};
    for (int64_t x : ext)
        if (x >= lim) return TP_EUNSUPPORTED;
    if (o) *o = s;
    return TP_OK;
}

inline int fmt(const Shape& s) { return s.fp16 ? tp::FMT_F16 : s.h16 ? tp::FMT_BF16 : tp::FMT_F32; }

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename P>
inline P* at(P* base, int64_t elems, int64_t esize) {
    using C = typename std::conditional<std::is_const<P>::value, const char, char>::type;
    return reinterpret_cast<P*>(reinterpret_cast<C*>(base) + elems * esize);
}

struct MlpSaved {
    int64_t Gp, Y, total;
};
MlpSaved mlp_saved(const Shape& s) {
    const int64_t u = align256(s.T * s.Fs * s.e);
    return {0, u, 2 * u};
}

// Where a tile 192 or 256 columns wide does not fit a Q|K|V segment (w = H/t d
// a multiple of neither), the QKV GEMM would be held to narrow tiles (its B loader
// takes one segment per tile); the forward then first copies the three weight
// slices [h, w] (and biases) side by side into a staging region of `saved`, and
// the GEMM reads one contiguous [h, 3w] operand.
bool qkv_staged(const Shape& s) { return s.h16 && s.w % 192 != 0 && s.w % 256 != 0; }

struct AttnSaved {
    int64_t QKV, O, LSE, Wst, bst, total;
};
AttnSaved attn_saved(const Shape& s) {
    const int64_t q = align256(s.T * 3 * s.w * s.e);
    const int64_t o = align256(s.T * s.w * s.e);
    const int64_t l = align256(s.b * s.Hs * s.s * 4);
    const int64_t w = qkv_staged(s) ? align256(s.h * 3 * s.w * s.e) : 0;
    const int64_t b = qkv_staged(s) ? align256(3 * s.w * s.e) : 0;
    return {0, q, q + o, q + o + l, q + o + l + w, q + o + l + w + b};
}

// Work buffers.  `part` (fp32, 16-bit path only) takes the second K half's partial
// sums of the FFN weight-gradient launch when it is split in two: one float per
// weight gradient element of the launch.  (The attention one never splits: the
// auxiliary stream's launches fill the CUs its tiles leave.)
struct MlpWork {
    int64_t dU, cs, part, part_floats, total;
};
MlpWork mlp_work(const Shape& s) {
    const int64_t du = align256(s.T * s.Fs * s.e);
    const int64_t cs = align256(tp::colsum_work_floats(s.Fs) * 4);
    const int64_t pf = s.h16 ? 2 * s.Fs * s.h : 0;
    return {0, du, du + cs, pf, du + cs + align256(pf * 4)};
}

struct AttnWork {
    int64_t dO, dQKV, Dq, cs, total;
};
AttnWork attn_work(const Shape& s) {
    const int64_t dO = align256(s.T * s.w * s.e);
    const int64_t dq = align256(s.T * 3 * s.w * s.e);
    const int64_t D = align256(s.b * s.Hs * s.s * 4);
    const int64_t cs = align256(tp::colsum_work_floats(3 * s.w) * 4);
    return {0, dO, dO + dq, dO + dq + D, dO + dq + D + cs};
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_EHIP; }

// Measurement hook (tp_profile_enable): event pairs around each step's launches.
struct Prof {
    void* const* events = nullptr;
    int npairs = 0;
    int count[TP_NUM_STEPS] = {};
    int kernels[TP_NUM_STEPS] = {};
};
Prof g_prof;
long long g_launches = 0;  // every kernel launch of the library (tp::count_launch)

struct StepTimer {
    int step;
    hipStream_t st;
    hipEvent_t stop = nullptr;
    long long launches0 = 0;
    StepTimer(int s, hipStream_t stream) : step(s), st(stream) {
        if (!g_prof.events || g_prof.npairs <= 0) return;
        const int k = g_prof.count[s] % g_prof.npairs;
        const int base = 2 * (s * g_prof.npairs + k);
        hipEventRecord(static_cast<hipEvent_t>(g_prof.events[base]), st);
        stop = static_cast<hipEvent_t>(g_prof.events[base + 1]);
        g_prof.count[s]++;
        launches0 = g_launches;
    }
    ~StepTimer() {
        if (!stop) return;
        hipEventRecord(stop, st);
        g_prof.kernels[step] += (int)(g_launches - launches0);
    }
};

// The GEMM descriptor with the storage format of the call.
inline tp::GemmDesc fmt_of(const Shape& s, const tp::GemmDesc& g) {
    tp::GemmDesc d = g;
    d.fp16 = s.fp16;
    return d;
}

inline hipError_t gemm(const Shape& s, const tp::GemmDesc& g, hipStream_t st, int step) {
    StepTimer t(step, st);
    return s.h16 ? tp::gemm_bf16(fmt_of(s, g), st) : tp::gemm_f32(g, st);
}

// Per-device auxiliary stream for launches that are independent of the main
// chain of a backward call: to_aux(k) makes it wait for everything enqueued on
// the caller's stream so far, to_main(k) makes the caller's stream wait for
// everything enqueued on it (k: one of the call's events, each used once per
// call).  The lock is held from the first to the last of these in one call,
// so the shared events are never re-recorded by another host thread in
// between.  The events only order the two streams (nothing waits for them on
// the host), and every kernel launch already carries the acquire and release
// fences that make one kernel's writes visible to the next on the device, so
// they are created without the system-scope fence a recorded event otherwise
// adds (a cache write-back and invalidation at each fork and join).
constexpr int AUX_EVENTS = 6;
struct Aux {
    hipStream_t st = nullptr;
    hipEvent_t ev[AUX_EVENTS] = {};
    std::mutex mu;
};
constexpr int AUX_DEVICES = 64;
Aux g_aux[AUX_DEVICES];
std::mutex g_aux_init;

struct AuxScope {
    Aux* a = nullptr;
    std::unique_lock<std::mutex> lock;
    hipError_t err = hipSuccess;
    hipStream_t main_st = nullptr;
    bool forked = false;  // work is on the auxiliary stream that `main_st` does not yet wait for
    AuxScope() {
        int dev = 0;
        if ((err = hipGetDevice(&dev)) != hipSuccess) return;
        if (dev < 0 || dev >= AUX_DEVICES) { err = hipErrorInvalidDevice; return; }
        Aux& x = g_aux[dev];
        {
            std::lock_guard<std::mutex> g(g_aux_init);
            if (!x.st) {
                hipStream_t st = nullptr;
                hipEvent_t ev[AUX_EVENTS] = {};
                if ((err = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return;
                for (int k = 0; k < AUX_EVENTS && err == hipSuccess; ++k)
                    err = hipEventCreateWithFlags(&ev[k], hipEventDisableTiming | hipEventDisableSystemFence);
                if (err != hipSuccess) {
                    for (int k = 0; k < AUX_EVENTS; ++k)
                        if (ev[k]) hipEventDestroy(ev[k]);
                    hipStreamDestroy(st);
                    return;
                }
                for (int k = 0; k < AUX_EVENTS; ++k) x.ev[k] = ev[k];
                x.st = st;
            }
        }
        lock = std::unique_lock<std::mutex>(x.mu);
        a = &x;
    }
    hipError_t to_aux(hipStream_t main, int k) {
        main_st = main;
        forked = true;  // from here on the destructor joins, whatever the outcome
        hipError_t e = hipEventRecord(a->ev[k], main);
        return e != hipSuccess ? e : hipStreamWaitEvent(a->st, a->ev[k], 0);
    }
    hipError_t to_main(hipStream_t main, int k) {
        hipError_t e = hipEventRecord(a->ev[k], a->st);
        if (e == hipSuccess) e = hipStreamWaitEvent(main, a->ev[k], 0);
        if (e == hipSuccess) forked = false;
        return e;
    }
    // An early (error) return after a fork still orders the caller's stream after
    // everything enqueued on the auxiliary stream, which may read or write the
    // caller's buffers.  Best effort: there is no status left to report.
    ~AuxScope() {
        if (a && forked) {
            if (hipEventRecord(a->ev[AUX_EVENTS - 1], a->st) == hipSuccess)
                (void)hipStreamWaitEvent(main_st, a->ev[AUX_EVENTS - 1], 0);
        }
    }
};

// Two independent weight-gradient GEMMs of the same layout in one launch (16-bit
// path; may split K in two, the second half's partial sums going to `part`), or
// one after the other.
inline hipError_t gemm2(const Shape& s, const tp::GemmDesc* g, float* part, int64_t part_floats, hipStream_t st,
                        int step) {
    StepTimer t(step, st);
    if (s.h16) {
        const tp::GemmDesc d[2] = {fmt_of(s, g[0]), fmt_of(s, g[1])};
        return tp::gemm_bf16_batch(d, 2, part, part_floats, nullptr, st);
    }
    hipError_t e = tp::gemm_f32(g[0], st);
    return e != hipSuccess ? e : tp::gemm_f32(g[1], st);
}

// The forward steps whose outputs the backward needs, into `saved`:
// Gp = GeLU'(U) and Y = GeLU(U) of U = X A[:, C_i] + b1[C_i] (one GEMM with a fused
// epilogue).  U itself is not kept: the backward needs only GeLU'(U).
hipError_t mlp_fwd_saved(const Shape& s, const void* X, const void* A, const void* b1, void* saved,
                         hipStream_t st) {
    const MlpSaved L = mlp_saved(s);
    const int64_t c0 = s.i * s.Fs;
    tp::GemmDesc g1;
    g1.M = (int)s.T; g1.N = (int)s.Fs; g1.K = (int)s.h;
    g1.A = X; g1.lda = s.h; g1.a_kcontig = true;
    g1.B[0] = at(A, c0, s.e); g1.ldb = s.F; g1.b_kcontig = false;
    g1.C[0] = at(saved, L.Gp, 1); g1.ldc = s.Fs; g1.C2 = at(saved, L.Y, 1); g1.ldc2 = s.Fs;
    g1.bias[0] = b1 ? at(b1, c0, s.e) : nullptr;
    g1.epi = tp::EPI_BIAS_GELU;
    g1.gelu_tanh = s.gelu_tanh;
    return gemm(s, g1, st, TP_STEP_MLP_UP);
}

// QKV = X [Wq|Wk|Wv][:, cols of G_i] + [bq|bk|bv], then per-head attention: O and LSE.
hipError_t attn_fwd_saved(const Shape& s, const void* X, const void* Wq, const void* Wk, const void* Wv,
                          const void* bq, const void* bk, const void* bv, void* saved, hipStream_t st) {
    const AttnSaved L = attn_saved(s);
    void* QKV = at(saved, L.QKV, 1);
    const int64_t col0 = s.i * s.w;
    tp::GemmDesc g;
    g.M = (int)s.T; g.N = (int)(3 * s.w); g.K = (int)s.h;
    g.A = X; g.lda = s.h; g.a_kcontig = true;
    const void* W3[3] = {Wq, Wk, Wv};
    const void* b3[3] = {bq, bk, bv};
    const void* Ws[3];
    const void* bs[3];
    for (int z = 0; z < 3; ++z) {
        Ws[z] = at(W3[z], col0, s.e);
        bs[z] = b3[z] ? at(b3[z], col0, s.e) : nullptr;
    }
    g.b_kcontig = false;
    g.epi = tp::EPI_BIAS;
    hipError_t e;
    {
        StepTimer qt(TP_STEP_QKV, st);  // the staging copy counts with the GEMM
        if (qkv_staged(s)) {  // one [h, 3w] operand, one [3w] bias, one output block
            void* Wst = at(saved, L.Wst, 1);
            void* bst = at(saved, L.bst, 1);
            const bool any_bias = bs[0] || bs[1] || bs[2];
            e = tp::gather3(Ws, s.h, s.h, s.w, Wst, bs, any_bias ? bst : nullptr, st);
            if (e != hipSuccess) return e;
            g.B[0] = Wst; g.ldb = 3 * s.w;
            g.C[0] = QKV; g.ldc = 3 * s.w;
            g.bias[0] = any_bias ? bst : nullptr;
        } else {
            for (int z = 0; z < 3; ++z) {
                g.B[z] = Ws[z];
                g.C[z] = at(QKV, z * s.w, s.e);
                g.bias[z] = bs[z];
            }
            g.ldb = s.h; g.bseg = (int)s.w;
            g.ldc = 3 * s.w; g.cseg = (int)s.w;
        }
        e = s.h16 ? tp::gemm_bf16(fmt_of(s, g), st) : tp::gemm_f32(g, st);
    }
    if (e != hipSuccess) return e;
    tp::AttnDesc ad;
    ad.batch = (int)s.b; ad.seq = (int)s.s; ad.heads = (int)s.Hs; ad.dh = (int)s.d; ad.causal = s.causal;
    ad.qkv = QKV; ad.ld_qkv = 3 * s.w; ad.O = at(saved, L.O, 1); ad.ld_o = s.w;
    ad.lse = static_cast<float*>(at(saved, L.LSE, 1));
    StepTimer t(TP_STEP_ATTN_CORE, st);
    ad.fp16 = s.fp16;
    return s.h16 ? tp::attn_fwd_bf16(ad, st) : tp::attn_fwd_f32(ad, st);
}

// Pointer checks of the FFN backward (everything but the work buffer).
int mlp_bwd_check(const void* X, const void* A, const void* B, const void* saved, const void* dZ,
                  const void* dX_part, const float* dA, const float* db1, const float* dB) {
    if (!X || !A || !B || !saved || !dZ || !dX_part || !dA || !dB) return TP_EINVAL;
    if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(saved) || !aligned16(dZ) ||
        !aligned16(dX_part) || !aligned16(dA) || !aligned16(dB) || (db1 && !aligned16(db1)))
        return TP_EALIGN;
    return TP_OK;
}

// The FFN backward's launches: dU (GEMM with the GeLU' epilogue), db1 (column
// sums of dU), dB and dA (one GEMM launch), dX_part.  dU, the column-sum
// partials and the K-split partial sums go to `work` (laid out by mlp_work: the
// caller's buffer or the library's static one).
// With `aux`, the column sum runs on the auxiliary stream beside the GEMMs;
// without, every launch runs on `st` (same kernels, same results).
int mlp_bwd_run(const Shape& s, const void* X, const void* A, const void* B, const void* saved, const void* dZ,
                void* dX_part, float* dA, float* db1, float* dB, void* work, hipStream_t st, AuxScope* aux) {
    const MlpWork W = mlp_work(s);
    void* dU = at(work, W.dU, 1);
    float* cs = static_cast<float*>(at(work, W.cs, 1));
    const MlpSaved L = mlp_saved(s);
    const void* Gp = at(saved, L.Gp, 1);
    const void* Y = at(saved, L.Y, 1);
    const int64_t c0 = s.i * s.Fs;

    tp::GemmDesc g;  // dU = (dZ B[C_i, :]^T) * Gp, Gp = GeLU'(U)
    g.M = (int)s.T; g.N = (int)s.Fs; g.K = (int)s.h;
    g.A = dZ; g.lda = s.h; g.a_kcontig = true;
    g.B[0] = at(B, c0 * s.h, s.e); g.ldb = s.h; g.b_kcontig = true;
    g.C[0] = dU; g.ldc = s.Fs; g.aux = Gp; g.ldaux = s.Fs;
    g.epi = tp::EPI_GELU_BWD;
    g.gelu_tanh = s.gelu_tanh;
    if (gemm(s, g, st, TP_STEP_MLP_DU) != hipSuccess) return TP_EHIP;

    if (db1) {  // db1[C_i] = column sums of dU (beside the GEMMs below when there is an aux stream)
        float* outs[3] = {db1 + c0, nullptr, nullptr};
        hipStream_t cst = st;
        if (aux) {
            if (aux->to_aux(st, 0) != hipSuccess) return TP_EHIP;
            cst = aux->a->st;
        }
        StepTimer t(TP_STEP_MLP_DB1, cst);
        if (tp::colsum(fmt(s), dU, s.T, s.Fs, s.Fs, outs, SEG_NONE, cs, cst) != hipSuccess) return TP_EHIP;
    }

    tp::GemmDesc gw[2];  // one launch: dB[C_i, :] = Y^T dZ and dA[:, C_i] = X^T dU
    tp::GemmDesc& gb = gw[0];
    gb.M = (int)s.Fs; gb.N = (int)s.h; gb.K = (int)s.T;
    gb.A = Y; gb.lda = s.Fs; gb.a_kcontig = false;
    gb.B[0] = dZ; gb.ldb = s.h; gb.b_kcontig = false;
    gb.C[0] = dB + c0 * s.h; gb.ldc = s.h; gb.out_f32 = true;
    tp::GemmDesc& ga = gw[1];
    ga.M = (int)s.h; ga.N = (int)s.Fs; ga.K = (int)s.T;
    ga.A = X; ga.lda = s.h; ga.a_kcontig = false;
    ga.B[0] = dU; ga.ldb = s.Fs; ga.b_kcontig = false;
    ga.C[0] = dA + c0; ga.ldc = s.F; ga.out_f32 = true;
    if (gemm2(s, gw, static_cast<float*>(at(work, W.part, 1)), W.part_floats, st, TP_STEP_MLP_DW) != hipSuccess)
        return TP_EHIP;

    tp::GemmDesc gx;  // dX_part = dU A[:, C_i]^T
    gx.M = (int)s.T; gx.N = (int)s.h; gx.K = (int)s.Fs;
    gx.A = dU; gx.lda = s.Fs; gx.a_kcontig = true;
    gx.B[0] = at(A, c0, s.e); gx.ldb = s.F; gx.b_kcontig = true;
    gx.C[0] = dX_part; gx.ldc = s.h;
    if (gemm(s, gx, st, TP_STEP_MLP_DX) != hipSuccess) return TP_EHIP;
    if (aux && db1 && aux->to_main(st, 1) != hipSuccess) return TP_EHIP;
    return TP_OK;
}

}  // namespace

namespace tp {
void count_launch() { ++g_launches; }
}  // namespace tp

extern "C" {

int tp_version(void) { return 300; }

const char* tp_status_string(int status) {
    switch (status) {
        case TP_OK: return "ok";
        case TP_EINVAL: return "invalid argument (NULL pointer, non-positive size or bad flag)";
        case TP_EDIVIDE: return "degree must divide heads and ffn, and heads must divide hidden";
        case TP_ESHARD: return "shard index out of range [0, degree)";
        case TP_EALIGN: return "pointer not 16-byte aligned or size not a multiple of 8";
        case TP_EDTYPE: return "unknown dtype";
        case TP_EUNSUPPORTED: return "unsupported shape (head dimension or size limit)";
        case TP_EHIP: return "HIP kernel launch failed";
        case TP_ESIZE: return "work buffer smaller than required";
        case TP_ESCRATCH: return "problem needs more scratch than the no-allocation entry point's static buffer";
        default: return "unknown status";
    }
}

int tp_check_dims(const tp_dims* dims, int shard, int degree) { return derive(dims, shard, degree, nullptr); }

int tp_profile_enable(void* const* events, int npairs) {
    if (events && npairs > 0) {
        for (int i = 0; i < 2 * TP_NUM_STEPS * npairs; ++i)
            if (!events[i]) return TP_EINVAL;
        g_prof.events = events;
        g_prof.npairs = npairs;
    } else {
        g_prof.events = nullptr;
        g_prof.npairs = 0;
    }
    for (int i = 0; i < TP_NUM_STEPS; ++i) g_prof.count[i] = g_prof.kernels[i] = 0;
    return TP_OK;
}

int tp_test_force_gemm_tile(int tile, int ksplit) {
    if (tile < -1 || tile >= tp::gemm_tile_count() || ksplit < 0 || ksplit > 2) return TP_EINVAL;
    tp::gemm_force_tile(tile, ksplit);
    return TP_OK;
}

int tp_test_gemm_tile_count(void) { return tp::gemm_tile_count(); }

int tp_profile_count(int step) { return (step >= 0 && step < TP_NUM_STEPS) ? g_prof.count[step] : -1; }

int tp_profile_kernels(int step) { return (step >= 0 && step < TP_NUM_STEPS) ? g_prof.kernels[step] : -1; }

size_t tp_mlp_saved_bytes(const tp_dims* dims, int shard, int degree) {
    Shape s;
    return derive(dims, shard, degree, &s) == TP_OK ? (size_t)mlp_saved(s).total : 0;
}

size_t tp_attn_saved_bytes(const tp_dims* dims, int shard, int degree) {
    Shape s;
    return derive(dims, shard, degree, &s) == TP_OK ? (size_t)attn_saved(s).total : 0;
}

size_t tp_mlp_work_bytes(const tp_dims* dims, int shard, int degree) {
    Shape s;
    return derive(dims, shard, degree, &s) == TP_OK ? (size_t)mlp_work(s).total : 0;
}

size_t tp_attn_work_bytes(const tp_dims* dims, int shard, int degree) {
    Shape s;
    return derive(dims, shard, degree, &s) == TP_OK ? (size_t)attn_work(s).total : 0;
}

int tp_mlp_shard_fwd(const tp_dims* dims, int shard, int degree, const void* X, const void* A, const void* b1,
                     const void* B, void* Z_part, void* saved, void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if (!X || !A || !B || !Z_part || !saved) return TP_EINVAL;
    if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Z_part) || !aligned16(saved) ||
        (b1 && !aligned16(b1)))
        return TP_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mlp_fwd_saved(s, X, A, b1, saved, st) != hipSuccess) return TP_EHIP;
    const void* Y = at(saved, mlp_saved(s).Y, 1);
    const int64_t c0 = s.i * s.Fs;

    tp::GemmDesc g2;  // Z_part = Y B[C_i, :]
    g2.M = (int)s.T; g2.N = (int)s.h; g2.K = (int)s.Fs;
    g2.A = Y; g2.lda = s.Fs; g2.a_kcontig = true;
    g2.B[0] = at(B, c0 * s.h, s.e); g2.ldb = s.h; g2.b_kcontig = false;
    g2.C[0] = Z_part; g2.ldc = s.h;
    g2.epi = tp::EPI_STORE;
    return hip_status(gemm(s, g2, st, TP_STEP_MLP_DOWN));
}

int tp_mlp_shard_bwd(const tp_dims* dims, int shard, int degree, const void* X, const void* A, const void* B,
                     const void* saved, const void* dZ, void* dX_part, float* dA, float* db1, float* dB, void* work,
                     size_t work_bytes, void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if (!work) return TP_EINVAL;
    if ((rc = mlp_bwd_check(X, A, B, saved, dZ, dX_part, dA, db1, dB))) return rc;
    if (!aligned16(work)) return TP_EALIGN;
    const MlpWork W = mlp_work(s);
    if (work_bytes < (size_t)W.total) return TP_ESIZE;
    AuxScope aux;
    if (aux.err != hipSuccess) return TP_EHIP;
    return mlp_bwd_run(s, X, A, B, saved, dZ, dX_part, dA, db1, dB, work, static_cast<hipStream_t>(stream), &aux);
}

int tp_mlp_shard_bwd_noalloc(const tp_dims* dims, int shard, int degree, const void* X, const void* A,
                             const void* B, const void* saved, const void* dZ, void* dX_part, float* dA, float* db1,
                             float* dB, void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if ((rc = mlp_bwd_check(X, A, B, saved, dZ, dX_part, dA, db1, dB))) return rc;
    const MlpWork W = mlp_work(s);
    if (W.total > tp::NOALLOC_SCRATCH_BYTES) return TP_ESCRATCH;
    void* scratch = nullptr;  // the device address of this device's static array
    if (tp::noalloc_scratch(&scratch) != hipSuccess) return TP_EHIP;
    return mlp_bwd_run(s, X, A, B, saved, dZ, dX_part, dA, db1, dB, scratch, static_cast<hipStream_t>(stream),
                       nullptr);
}

int tp_attn_shard_fwd(const tp_dims* dims, int shard, int degree, const void* X, const void* Wq, const void* Wk,
                      const void* Wv, const void* bq, const void* bk, const void* bv, const void* Wo, void* Z_part,
                      void* saved, void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if (!X || !Wq || !Wk || !Wv || !Wo || !Z_part || !saved) return TP_EINVAL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wo) ||
        !aligned16(Z_part) || !aligned16(saved) || (bq && !aligned16(bq)) || (bk && !aligned16(bk)) ||
        (bv && !aligned16(bv)))
        return TP_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (attn_fwd_saved(s, X, Wq, Wk, Wv, bq, bk, bv, saved, st) != hipSuccess) return TP_EHIP;
    const void* O = at(saved, attn_saved(s).O, 1);
    const int64_t col0 = s.i * s.w;

    tp::GemmDesc go;  // Z_part = O Wo[rows of G_i, :]
    go.M = (int)s.T; go.N = (int)s.h; go.K = (int)s.w;
    go.A = O; go.lda = s.w; go.a_kcontig = true;
    go.B[0] = at(Wo, col0 * s.h, s.e); go.ldb = s.h; go.b_kcontig = false;
    go.C[0] = Z_part; go.ldc = s.h;
    return hip_status(gemm(s, go, st, TP_STEP_ATTN_OUT));
}

int tp_attn_shard_bwd(const tp_dims* dims, int shard, int degree, const void* X, const void* Wq, const void* Wk,
                      const void* Wv, const void* Wo, const void* saved, const void* dZ, void* dX_part, float* dWq,
                      float* dWk, float* dWv, float* dbq, float* dbk, float* dbv, float* dWo, void* work,
                      size_t work_bytes, void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if (!X || !Wq || !Wk || !Wv || !Wo || !saved || !dZ || !dX_part || !dWq || !dWk || !dWv || !dWo || !work)
        return TP_EINVAL;
    const bool bias_grads = dbq && dbk && dbv;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wo) ||
        !aligned16(saved) || !aligned16(dZ) || !aligned16(dX_part) || !aligned16(dWq) || !aligned16(dWk) ||
        !aligned16(dWv) || !aligned16(dWo) || !aligned16(work) ||
        (bias_grads && (!aligned16(dbq) || !aligned16(dbk) || !aligned16(dbv))))
        return TP_EALIGN;
    const AttnWork W = attn_work(s);
    if (work_bytes < (size_t)W.total) return TP_ESIZE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const AttnSaved L = attn_saved(s);
    const void* QKV = at(saved, L.QKV, 1);
    const void* O = at(saved, L.O, 1);
    const float* lse = static_cast<const float*>(at(saved, L.LSE, 1));
    void* dO = at(work, W.dO, 1);
    void* dQKV = at(work, W.dQKV, 1);
    float* Dq = static_cast<float*>(at(work, W.Dq, 1));
    float* cs = static_cast<float*>(at(work, W.cs, 1));
    const int64_t col0 = s.i * s.w;

    AuxScope aux;
    if (aux.err != hipSuccess) return TP_EHIP;

    tp::GemmDesc go;  // dWo[rows of G_i, :] = O^T dZ: shares one launch with dW{q,k,v} (below)
    go.M = (int)s.w; go.N = (int)s.h; go.K = (int)s.T;
    go.A = O; go.lda = s.w; go.a_kcontig = false;
    go.B[0] = dZ; go.ldb = s.h; go.b_kcontig = false;
    go.C[0] = dWo + col0 * s.h; go.ldc = s.h; go.out_f32 = true;

    tp::GemmDesc g;  // dO = dZ Wo[rows of G_i, :]^T
    g.M = (int)s.T; g.N = (int)s.w; g.K = (int)s.h;
    g.A = dZ; g.lda = s.h; g.a_kcontig = true;
    g.B[0] = at(Wo, col0 * s.h, s.e); g.ldb = s.h; g.b_kcontig = true;
    g.C[0] = dO; g.ldc = s.w;
    // D = rowsum(dO * O) per head from the dO GEMM's epilogue where its tile allows (16-bit path:
    // one round of 64 x 192 tiles, heads that divide 192), else by its own kernel below
    g.epi = tp::EPI_STORE_ROWDOT;
    g.aux = O; g.ldaux = s.w;
    g.rd = Dq; g.rd_seq = (int)s.s; g.rd_heads = (int)s.Hs; g.rd_dh = (int)s.d;
    const bool fused_rd = s.h16 && tp::gemm_rowdot_ok(g);
    if (!fused_rd) g.epi = tp::EPI_STORE;
    if (gemm(s, g, st, TP_STEP_ATTN_DO) != hipSuccess) return TP_EHIP;


    tp::AttnDesc ad;
    ad.batch = (int)s.b; ad.seq = (int)s.s; ad.heads = (int)s.Hs; ad.dh = (int)s.d; ad.causal = s.causal;
    ad.qkv = QKV; ad.ld_qkv = 3 * s.w; ad.O = const_cast<void*>(O); ad.ld_o = s.w;
    ad.lse = const_cast<float*>(lse); ad.dO = dO; ad.Dq = Dq; ad.dqkv = dQKV;
    ad.fp16 = s.fp16;
    auto core = [&](int part, hipStream_t q) {
        return s.h16 ? tp::attn_bwd_bf16(ad, part, q) : tp::attn_bwd_f32(ad, part, q);
    };
    {   // D = rowsum(dO * O) (unless the dO GEMM formed it), then the dK/dV and dQ passes: on the 16-bit path as one
        // launch, the dQ workgroups queued behind the dK/dV ones (on two streams side by
        // side they measured slower: their workgroups compete for the same CUs)
        StepTimer t(TP_STEP_ATTN_CORE_BWD, st);
        if (!fused_rd && core(tp::ATTN_BWD_ROWDOT, st) != hipSuccess) return TP_EHIP;
        if (s.h16 ? core(tp::ATTN_BWD_DKDV_DQ, st) != hipSuccess
                  : (core(tp::ATTN_BWD_DKDV, st) != hipSuccess || core(tp::ATTN_BWD_DQ, st) != hipSuccess))
            return TP_EHIP;
    }

    // One launch on the caller's stream: dW{q,k,v}[:, cols of G_i] = X^T dQKV and dWo (same
    // layout: transposed operands, fp32 output, K = T; dWo needs only forward outputs, but run
    // beside dO and the core it took CUs from the core's one-workgroup-per-CU grid).  Its tiles
    // (without a K split) hold part of the CUs for the whole launch; enqueued before the
    // auxiliary stream's launches, so that it takes its CUs first, while on the auxiliary stream
    // db{q,k,v}[cols of G_i] = column sums of dQKV and dX_part = dQKV [Wq|Wk|Wv][:, cols of G_i]^T
    // run on the rest.
    if (aux.to_aux(st, 0) != hipSuccess) return TP_EHIP;
    tp::GemmDesc gw[2];
    tp::GemmDesc& gq = gw[0];
    gq.M = (int)s.h; gq.N = (int)(3 * s.w); gq.K = (int)s.T;
    gq.A = X; gq.lda = s.h; gq.a_kcontig = false;
    gq.B[0] = dQKV; gq.ldb = 3 * s.w; gq.b_kcontig = false;
    float* dW3[3] = {dWq, dWk, dWv};
    for (int z = 0; z < 3; ++z) gq.C[z] = dW3[z] + col0;
    gq.ldc = s.h; gq.cseg = (int)s.w; gq.out_f32 = true;
    gq.cus = 128;  // tiles for half the CUs (the K-group tile at the 8.3B and BERT shapes)
    gw[1] = go;
    if (gemm2(s, gw, nullptr, 0, st, TP_STEP_ATTN_DW) != hipSuccess) return TP_EHIP;
    if (bias_grads) {
        float* outs[3] = {dbq + col0, dbk + col0, dbv + col0};
        StepTimer t(TP_STEP_ATTN_DBIAS, aux.a->st);
        if (tp::colsum(fmt(s), dQKV, s.T, 3 * s.w, 3 * s.w, outs, (int)s.w, cs, aux.a->st) != hipSuccess)
            return TP_EHIP;
    }
    tp::GemmDesc gx;
    gx.M = (int)s.T; gx.N = (int)s.h; gx.K = (int)(3 * s.w);
    gx.A = dQKV; gx.lda = 3 * s.w; gx.a_kcontig = true;
    const void* W3[3] = {Wq, Wk, Wv};
    for (int z = 0; z < 3; ++z) gx.B[z] = at(W3[z], col0, s.e);
    gx.ldb = s.h; gx.b_kcontig = true; gx.b_kseg = true; gx.bseg = (int)s.w;
    gx.C[0] = dX_part; gx.ldc = s.h;
    if (gemm(s, gx, aux.a->st, TP_STEP_ATTN_DX) != hipSuccess) return TP_EHIP;
    return aux.to_main(st, 1) != hipSuccess ? TP_EHIP : TP_OK;
}

int tp_sum_partials(int dtype, int64_t rows, int64_t cols, const void* const* parts, int nparts, const void* bias,
                    float* out, void* stream) {
    if (dtype != TP_FP32 && dtype != TP_BF16 && dtype != TP_FP16) return TP_EDTYPE;
    if (rows <= 0 || cols <= 0 || nparts < 1 || !parts || !out) return TP_EINVAL;
    for (int k = 0; k < nparts; ++k) {
        if (!parts[k]) return TP_EINVAL;
        if (!aligned16(parts[k])) return TP_EALIGN;
    }
    if (!aligned16(out) || (bias && !aligned16(bias))) return TP_EALIGN;
    return hip_status(tp::sum_partials(dtype, rows, cols, parts, nparts, bias, out,
                                       static_cast<hipStream_t>(stream)));
}

size_t tp_mlp_recompute_work_bytes(const tp_dims* dims, int shard, int degree) {
    Shape s;
    return derive(dims, shard, degree, &s) == TP_OK ? (size_t)(mlp_saved(s).total + mlp_work(s).total) : 0;
}

size_t tp_attn_recompute_work_bytes(const tp_dims* dims, int shard, int degree) {
    Shape s;
    return derive(dims, shard, degree, &s) == TP_OK ? (size_t)(attn_saved(s).total + attn_work(s).total) : 0;
}

int tp_mlp_shard_bwd_recompute(const tp_dims* dims, int shard, int degree, const void* X, const void* A,
                               const void* b1, const void* B, const void* dZ, void* dX_part, float* dA, float* db1,
                               float* dB, void* work, size_t work_bytes, void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if (!X || !A || !B || !dZ || !dX_part || !dA || !dB || !work) return TP_EINVAL;
    if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(dZ) || !aligned16(dX_part) ||
        !aligned16(dA) || !aligned16(dB) || !aligned16(work) || (db1 && !aligned16(db1)) || (b1 && !aligned16(b1)))
        return TP_EALIGN;
    const int64_t sv = mlp_saved(s).total;
    if (work_bytes < (size_t)(sv + mlp_work(s).total)) return TP_ESIZE;
    if (mlp_fwd_saved(s, X, A, b1, work, static_cast<hipStream_t>(stream)) != hipSuccess) return TP_EHIP;
    return tp_mlp_shard_bwd(dims, shard, degree, X, A, B, work, dZ, dX_part, dA, db1, dB, at(work, sv, 1),
                            work_bytes - (size_t)sv, stream);
}

int tp_attn_shard_bwd_recompute(const tp_dims* dims, int shard, int degree, const void* X, const void* Wq,
                                const void* Wk, const void* Wv, const void* bq, const void* bk, const void* bv,
                                const void* Wo, const void* dZ, void* dX_part, float* dWq, float* dWk, float* dWv,
                                float* dbq, float* dbk, float* dbv, float* dWo, void* work, size_t work_bytes,
                                void* stream) {
    Shape s;
    int rc = derive(dims, shard, degree, &s);
    if (rc) return rc;
    if (!X || !Wq || !Wk || !Wv || !Wo || !dZ || !dX_part || !dWq || !dWk || !dWv || !dWo || !work) return TP_EINVAL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wo) || !aligned16(dZ) ||
        !aligned16(dX_part) || !aligned16(dWq) || !aligned16(dWk) || !aligned16(dWv) || !aligned16(dWo) ||
        !aligned16(work) || (bq && !aligned16(bq)) || (bk && !aligned16(bk)) || (bv && !aligned16(bv)) ||
        (dbq && !aligned16(dbq)) || (dbk && !aligned16(dbk)) || (dbv && !aligned16(dbv)))
        return TP_EALIGN;
    const int64_t sv = attn_saved(s).total;
    if (work_bytes < (size_t)(sv + attn_work(s).total)) return TP_ESIZE;
    if (attn_fwd_saved(s, X, Wq, Wk, Wv, bq, bk, bv, work, static_cast<hipStream_t>(stream)) != hipSuccess)
        return TP_EHIP;
    return tp_attn_shard_bwd(dims, shard, degree, X, Wq, Wk, Wv, Wo, work, dZ, dX_part, dWq, dWk, dWv, dbq, dbk,
                             dbv, dWo, at(work, sv, 1), work_bytes - (size_t)sv, stream);
}

namespace {
constexpr int64_t LN_MAX_COLS = 8192;
bool ln_cols_ok(int64_t cols) { return cols % 8 == 0; }
}  // namespace

int tp_residual_layernorm(int dtype, int64_t rows, int64_t cols, const void* const* parts, int nparts,
                          const void* bias, const float* residual, float* out, const float* gamma,
                          const float* beta, double eps, void* y, float* mean, float* rstd, void* stream) {
    if (dtype != TP_FP32 && dtype != TP_BF16 && dtype != TP_FP16) return TP_EDTYPE;
    if (rows <= 0 || cols <= 0 || nparts < 0 || nparts > tp::LN_MAXP || (nparts > 0 && !parts) || (!out && !y) ||
        !(eps > 0.0))
        return TP_EINVAL;
    if (!ln_cols_ok(cols)) return TP_EALIGN;
    if (cols > LN_MAX_COLS || rows > 0x7fffffff) return TP_EUNSUPPORTED;
    tp::LnFwdDesc d;
    for (int k = 0; k < nparts; ++k) {
        if (!parts[k]) return TP_EINVAL;
        if (!aligned16(parts[k])) return TP_EALIGN;
        d.parts[k] = parts[k];
    }
    const void* ptrs[] = {bias, residual, out, gamma, beta, y, mean, rstd};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return TP_EALIGN;
    d.rows = rows; d.cols = (int)cols; d.fmt = dtype; d.nparts = nparts;
    d.bias = bias; d.residual = residual; d.out = out; d.gamma = gamma; d.beta = beta; d.eps = (float)eps;
    d.y = y; d.mean = mean; d.rstd = rstd;
    return hip_status(tp::residual_layernorm(d, static_cast<hipStream_t>(stream)));
}

size_t tp_layernorm_bwd_work_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)4 * ((size_t)tp::ln_bwd_bands(rows) + tp::LN_BWD_GROUPS) * (size_t)cols * sizeof(float);
}

int tp_layernorm_bwd(int dtype, int64_t rows, int64_t cols, const float* x, const float* gamma, const float* mean,
                     const float* rstd, const void* const* dparts, int nparts, const float* dres, float* dx,
                     void* dx_act, float* dgamma, float* dbeta, float* dres_sum, float* dx_sum, void* work,
                     size_t work_bytes, void* stream) {
    if (dtype != TP_FP32 && dtype != TP_BF16 && dtype != TP_FP16) return TP_EDTYPE;
    if (rows <= 0 || cols <= 0 || nparts < 1 || nparts > tp::LN_MAXP || !dparts || !x || !mean || !rstd || !dx ||
        !work)
        return TP_EINVAL;
    if (!ln_cols_ok(cols)) return TP_EALIGN;
    if (cols > LN_MAX_COLS || rows > 0x7fffffff) return TP_EUNSUPPORTED;
    tp::LnBwdDesc d;
    for (int k = 0; k < nparts; ++k) {
        if (!dparts[k]) return TP_EINVAL;
        if (!aligned16(dparts[k])) return TP_EALIGN;
        d.dparts[k] = dparts[k];
    }
    const void* ptrs[] = {x, gamma, mean, rstd, dres, dx, dx_act, dgamma, dbeta, dres_sum, dx_sum, work};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return TP_EALIGN;
    if (work_bytes < tp_layernorm_bwd_work_bytes(rows, cols)) return TP_ESIZE;
    d.rows = rows; d.cols = (int)cols; d.fmt = dtype; d.nparts = nparts;
    d.x = x; d.gamma = gamma; d.mean = mean; d.rstd = rstd; d.dres = dres; d.dx = dx; d.dx_act = dx_act;
    d.dgamma = dgamma; d.dbeta = dbeta; d.dres_sum = dres_sum; d.dx_sum = dx_sum;
    d.work = static_cast<float*>(work);
    return hip_status(tp::layernorm_bwd(d, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
