"""ctypes binding of libtpshard.so (include/tpshard.h).

Argument marshalling only: device memory and streams come from PyTorch
(tensors' data_ptr and torch.cuda.current_stream()), every step of the shard
runs in the library's HIP kernels.  The names match the C entry points.  If
the library is missing the binding raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtpshard.so")

TP_FP32, TP_BF16, TP_FP16 = 0, 1, 2
TP_GELU_ERF, TP_GELU_TANH = 0, 1
STATUS = {0: "TP_OK", 1: "TP_EINVAL", 2: "TP_EDIVIDE", 3: "TP_ESHARD", 4: "TP_EALIGN", 5: "TP_EDTYPE",
          6: "TP_EUNSUPPORTED", 7: "TP_EHIP", 8: "TP_ESIZE", 9: "TP_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # TP_NOALLOC_SCRATCH_BYTES

EXPORTS = ["tp_version", "tp_status_string", "tp_check_dims", "tp_mlp_saved_bytes", "tp_attn_saved_bytes",
           "tp_mlp_work_bytes", "tp_attn_work_bytes", "tp_mlp_shard_fwd", "tp_mlp_shard_bwd",
           "tp_attn_shard_fwd", "tp_attn_shard_bwd", "tp_sum_partials", "tp_profile_enable",
           "tp_profile_count", "tp_profile_kernels", "tp_residual_layernorm", "tp_layernorm_bwd_work_bytes",
           "tp_layernorm_bwd", "tp_mlp_recompute_work_bytes", "tp_attn_recompute_work_bytes",
           "tp_mlp_shard_bwd_recompute", "tp_attn_shard_bwd_recompute", "tp_test_force_gemm_tile",
           "tp_test_gemm_tile_count", "tp_mlp_shard_bwd_noalloc"]

# step ids of the measurement hook (TP_STEP_* in tpshard.h), in launch order
STEPS = ["MLP_UP", "MLP_DOWN", "QKV", "ATTN_CORE", "ATTN_OUT", "MLP_DU", "MLP_DW", "MLP_DB1", "MLP_DX",
         "ATTN_DO", "ATTN_CORE_BWD", "ATTN_DW", "ATTN_DBIAS", "ATTN_DX", "ATTN_DWO"]


class TpError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({text})")
        self.code = code


class tp_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("ffn", ctypes.c_int64), ("causal", ctypes.c_int32),
                ("act", ctypes.c_int32), ("gelu", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtpshard.so; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m "
                               "tensor_transformer_layer_02_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        D = ctypes.POINTER(tp_dims)
        fp = ctypes.c_void_p
        L.tp_version.restype = i32
        L.tp_status_string.restype = ctypes.c_char_p
        L.tp_status_string.argtypes = [i32]
        L.tp_check_dims.argtypes = [D, i32, i32]
        for n in ("tp_mlp_saved_bytes", "tp_attn_saved_bytes", "tp_mlp_work_bytes", "tp_attn_work_bytes",
                  "tp_mlp_recompute_work_bytes", "tp_attn_recompute_work_bytes"):
            getattr(L, n).restype = sz
            getattr(L, n).argtypes = [D, i32, i32]
        L.tp_mlp_shard_fwd.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.tp_mlp_shard_bwd.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, fp, fp, fp, vp, sz, vp]
        L.tp_mlp_shard_bwd_noalloc.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, fp, fp, fp, vp]
        L.tp_attn_shard_fwd.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.tp_attn_shard_bwd.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp,
                                        vp, sz, vp]
        L.tp_sum_partials.argtypes = [i32, i64, i64, ctypes.POINTER(vp), i32, vp, fp, vp]
        L.tp_mlp_shard_bwd_recompute.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, fp, fp, fp, vp, sz, vp]
        L.tp_attn_shard_bwd_recompute.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, fp, fp, fp,
                                                  fp, fp, fp, fp, vp, sz, vp]
        L.tp_profile_enable.argtypes = [ctypes.POINTER(vp), i32]
        L.tp_profile_count.argtypes = [i32]
        L.tp_profile_kernels.argtypes = [i32]
        PP = ctypes.POINTER(vp)
        L.tp_residual_layernorm.argtypes = [i32, i64, i64, PP, i32, vp, fp, fp, fp, fp, ctypes.c_double, vp, fp, fp,
                                            vp]
        L.tp_layernorm_bwd_work_bytes.restype = sz
        L.tp_layernorm_bwd_work_bytes.argtypes = [i64, i64]
        L.tp_layernorm_bwd.argtypes = [i32, i64, i64, fp, fp, fp, fp, PP, i32, fp, fp, vp, fp, fp, fp, fp, vp, sz,
                                       vp]
        _lib = L
    return _lib


def make_dims(batch, seq, hidden, heads, ffn, causal=True, act=TP_BF16, gelu=TP_GELU_ERF) -> tp_dims:
    return tp_dims(batch, seq, hidden, heads, ffn, int(bool(causal)), int(act), int(gelu))


def dims_of(cfg, act=None) -> tp_dims:
    if act is None:
        act = {"fp32": TP_FP32, "bf16": TP_BF16, "fp16": TP_FP16}[cfg.dtype]
    gelu = TP_GELU_TANH if getattr(cfg, "gelu", "erf") == "tanh" else TP_GELU_ERF
    return make_dims(cfg.batch, cfg.seq, cfg.hidden, cfg.heads, cfg.ffn, cfg.causal, act, gelu)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise TpError(name, rc, lib().tp_status_string(rc).decode())
    return rc


def tp_version() -> int:
    return lib().tp_version()


def tp_status_string(code: int) -> str:
    return lib().tp_status_string(code).decode()


def tp_check_dims(dims, shard, degree) -> int:
    return lib().tp_check_dims(ctypes.byref(dims), shard, degree)


def tp_mlp_saved_bytes(dims, shard, degree) -> int:
    return lib().tp_mlp_saved_bytes(ctypes.byref(dims), shard, degree)


def tp_attn_saved_bytes(dims, shard, degree) -> int:
    return lib().tp_attn_saved_bytes(ctypes.byref(dims), shard, degree)


def tp_mlp_work_bytes(dims, shard, degree) -> int:
    return lib().tp_mlp_work_bytes(ctypes.byref(dims), shard, degree)


def tp_attn_work_bytes(dims, shard, degree) -> int:
    return lib().tp_attn_work_bytes(ctypes.byref(dims), shard, degree)


def tp_mlp_shard_fwd(dims, shard, degree, X, A, b1, B, Z_part, saved, stream=None):
    return _call("tp_mlp_shard_fwd", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(A), _ptr(b1), _ptr(B),
                 _ptr(Z_part), _ptr(saved), _stream(stream))


def tp_mlp_shard_bwd(dims, shard, degree, X, A, B, saved, dZ, dX_part, dA, db1, dB, work, stream=None):
    nbytes = work.numel() * work.element_size() if hasattr(work, "numel") else 0
    return _call("tp_mlp_shard_bwd", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(A), _ptr(B), _ptr(saved),
                 _ptr(dZ), _ptr(dX_part), _ptr(dA), _ptr(db1), _ptr(dB), _ptr(work), nbytes, _stream(stream))


def tp_mlp_shard_bwd_noalloc(dims, shard, degree, X, A, B, saved, dZ, dX_part, dA, db1, dB, stream=None):
    return _call("tp_mlp_shard_bwd_noalloc", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(A), _ptr(B),
                 _ptr(saved), _ptr(dZ), _ptr(dX_part), _ptr(dA), _ptr(db1), _ptr(dB), _stream(stream))


def tp_attn_shard_fwd(dims, shard, degree, X, Wq, Wk, Wv, bq, bk, bv, Wo, Z_part, saved, stream=None):
    return _call("tp_attn_shard_fwd", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                 _ptr(bq), _ptr(bk), _ptr(bv), _ptr(Wo), _ptr(Z_part), _ptr(saved), _stream(stream))


def tp_attn_shard_bwd(dims, shard, degree, X, Wq, Wk, Wv, Wo, saved, dZ, dX_part, dWq, dWk, dWv, dbq, dbk, dbv,
                      dWo, work, stream=None):
    nbytes = work.numel() * work.element_size() if hasattr(work, "numel") else 0
    return _call("tp_attn_shard_bwd", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                 _ptr(Wo), _ptr(saved), _ptr(dZ), _ptr(dX_part), _ptr(dWq), _ptr(dWk), _ptr(dWv), _ptr(dbq),
                 _ptr(dbk), _ptr(dbv), _ptr(dWo), _ptr(work), nbytes, _stream(stream))


def tp_mlp_recompute_work_bytes(dims, shard, degree) -> int:
    return lib().tp_mlp_recompute_work_bytes(ctypes.byref(dims), shard, degree)


def tp_attn_recompute_work_bytes(dims, shard, degree) -> int:
    return lib().tp_attn_recompute_work_bytes(ctypes.byref(dims), shard, degree)


def tp_mlp_shard_bwd_recompute(dims, shard, degree, X, A, b1, B, dZ, dX_part, dA, db1, dB, work, stream=None):
    nbytes = work.numel() * work.element_size() if hasattr(work, "numel") else 0
    return _call("tp_mlp_shard_bwd_recompute", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(A), _ptr(b1),
                 _ptr(B), _ptr(dZ), _ptr(dX_part), _ptr(dA), _ptr(db1), _ptr(dB), _ptr(work), nbytes,
                 _stream(stream))


def tp_attn_shard_bwd_recompute(dims, shard, degree, X, Wq, Wk, Wv, bq, bk, bv, Wo, dZ, dX_part, dWq, dWk, dWv,
                                dbq, dbk, dbv, dWo, work, stream=None):
    nbytes = work.numel() * work.element_size() if hasattr(work, "numel") else 0
    return _call("tp_attn_shard_bwd_recompute", ctypes.byref(dims), shard, degree, _ptr(X), _ptr(Wq), _ptr(Wk),
                 _ptr(Wv), _ptr(bq), _ptr(bk), _ptr(bv), _ptr(Wo), _ptr(dZ), _ptr(dX_part), _ptr(dWq), _ptr(dWk),
                 _ptr(dWv), _ptr(dbq), _ptr(dbk), _ptr(dbv), _ptr(dWo), _ptr(work), nbytes, _stream(stream))


def tp_sum_partials(dtype, rows, cols, parts, bias, out, stream=None):
    arr = (ctypes.c_void_p * len(parts))(*[_ptr(p) for p in parts])
    return _call("tp_sum_partials", int(dtype), int(rows), int(cols), arr, len(parts), _ptr(bias), _ptr(out),
                 _stream(stream))


# ----------------------------------------------------------- buffer helpers

def saved_layout(dims, shard, degree):
    """Views of the documented `saved` regions (offsets per include/tpshard.h)."""
    T = dims.batch * dims.seq
    Fs = dims.ffn // degree
    Hs = dims.heads // degree
    d = dims.hidden // dims.heads
    w = Hs * d
    e = 4 if dims.act == TP_FP32 else 2
    a = lambda x: (x + 255) // 256 * 256
    mlp = {"Gp": (0, (T, Fs)), "Y": (a(T * Fs * e), (T, Fs))}  # Gp = GeLU'(U), Y = GeLU(U)
    attn = {"QKV": (0, (T, 3 * w)), "O": (a(T * 3 * w * e), (T, w)),
            "LSE": (a(T * 3 * w * e) + a(T * w * e), (dims.batch, Hs, dims.seq))}
    return mlp, attn


def view(buf: torch.Tensor, offset: int, shape, dtype) -> torch.Tensor:
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.tensor([], dtype=dtype).element_size()
    return buf[offset:offset + nbytes].view(dtype).view(*shape)


def tp_profile_enable(events, npairs) -> int:
    """events: ctypes array of 2*len(STEPS)*npairs hipEvent_t handles, or None to disable."""
    return _call("tp_profile_enable", events, int(npairs))


def tp_profile_count(step: int) -> int:
    return lib().tp_profile_count(int(step))


def tp_profile_kernels(step: int) -> int:
    return lib().tp_profile_kernels(int(step))


def _parr(ts):
    arr = (ctypes.c_void_p * max(1, len(ts)))(*[_ptr(t) for t in ts])
    return arr


def tp_residual_layernorm(dtype, rows, cols, parts, bias, residual, out, gamma, beta, eps, y, mean, rstd,
                          stream=None):
    return _call("tp_residual_layernorm", int(dtype), int(rows), int(cols), _parr(parts), len(parts), _ptr(bias),
                 _ptr(residual), _ptr(out), _ptr(gamma), _ptr(beta), float(eps), _ptr(y), _ptr(mean), _ptr(rstd),
                 _stream(stream))


def tp_layernorm_bwd_work_bytes(rows, cols) -> int:
    return lib().tp_layernorm_bwd_work_bytes(int(rows), int(cols))


def tp_layernorm_bwd(dtype, rows, cols, x, gamma, mean, rstd, dparts, dres, dx, dx_act, dgamma, dbeta, dres_sum,
                     dx_sum, work, stream=None):
    return _call("tp_layernorm_bwd", int(dtype), int(rows), int(cols), _ptr(x), _ptr(gamma), _ptr(mean),
                 _ptr(rstd), _parr(dparts), len(dparts), _ptr(dres), _ptr(dx), _ptr(dx_act), _ptr(dgamma),
                 _ptr(dbeta), _ptr(dres_sum), _ptr(dx_sum), _ptr(work), work.numel() * work.element_size(),
                 _stream(stream))


def tp_test_force_gemm_tile(tile: int, ksplit: int = 0) -> int:
    """Test hook: force GEMM tile `tile` (-1: the cost model) and K split `ksplit`."""
    return _call("tp_test_force_gemm_tile", int(tile), int(ksplit))


def tp_test_gemm_tile_count() -> int:
    return lib().tp_test_gemm_tile_count()
