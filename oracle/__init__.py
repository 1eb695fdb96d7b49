"""ctypes binding of the float64 CPU oracle (libtpo.so, built from tpo.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  It shares no code
with the HIP library.

All arrays are float64 numpy arrays, C-contiguous; shapes follow tpo.h.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpo.so")
SRC = os.path.join(_HERE, "tpo.c")

# x86-64-v3 (AVX2 + FMA) so the library built here also runs on the GPU host.
CFLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall"]


def build(force: bool = True) -> str:
    """Compile libtpo.so with gcc (plain C11 + OpenMP)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], cwd=_HERE)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_long), ("seq", ctypes.c_long), ("hidden", ctypes.c_long),
                ("heads", ctypes.c_long), ("ffn", ctypes.c_long), ("causal", ctypes.c_int),
                ("gelu", ctypes.c_int)]


_lib = None
_P = ctypes.POINTER(ctypes.c_double)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        for name in ("tpo_mlp_shard_fwd", "tpo_mlp_shard_bwd", "tpo_attn_shard_fwd",
                     "tpo_attn_shard_bwd", "tpo_mlp_full_fwd", "tpo_mlp_full_bwd",
                     "tpo_attn_full_fwd", "tpo_attn_full_bwd"):
            getattr(_lib, name).restype = ctypes.c_int
        _lib.tpo_num_threads.restype = ctypes.c_int
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], "oracle wants C-contiguous float64"
    return a.ctypes.data_as(_P)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _dims(d: dict) -> Dims:
    return Dims(d["batch"], d["seq"], d["hidden"], d["heads"], d["ffn"], int(d["causal"]), int(d.get("gelu", 0)))


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected the shapes (code {rc})")


def num_threads() -> int:
    return lib().tpo_num_threads()


def gelu(u):
    u = _f64(u)
    y = np.empty_like(u)
    lib().tpo_gelu(_p(u), _p(y), ctypes.c_long(u.size))
    return y


def gelu_prime(u):
    u = _f64(u)
    y = np.empty_like(u)
    lib().tpo_gelu_prime(_p(u), _p(y), ctypes.c_long(u.size))
    return y


def gelu_tanh(u):
    u = _f64(u)
    y = np.empty_like(u)
    lib().tpo_gelu_tanh(_p(u), _p(y), ctypes.c_long(u.size))
    return y


def gelu_tanh_prime(u):
    u = _f64(u)
    y = np.empty_like(u)
    lib().tpo_gelu_tanh_prime(_p(u), _p(y), ctypes.c_long(u.size))
    return y


def mlp_shard_fwd(d, shard, degree, X, A, b1, B):
    X, A, b1, B = map(_f64, (X, A, b1, B))
    T, h, Fs = d["batch"] * d["seq"], d["hidden"], d["ffn"] // degree
    Z = np.empty((T, h)); U = np.empty((T, Fs)); Y = np.empty((T, Fs))
    _check(lib().tpo_mlp_shard_fwd(ctypes.byref(_dims(d)), shard, degree, _p(X), _p(A), _p(b1),
                                   _p(B), _p(Z), _p(U), _p(Y)), "mlp_shard_fwd")
    return {"Z": Z, "U": U, "Y": Y}


def mlp_shard_bwd(d, shard, degree, X, A, b1, B, G, dA=None, db1=None, dB=None):
    """Weight/bias gradients are full-size arrays of which only the shard block is written;
    pass existing arrays to fill several shards' blocks into one."""
    X, A, b1, B, G = map(_f64, (X, A, b1, B, G))
    T, h, F = d["batch"] * d["seq"], d["hidden"], d["ffn"]
    dX = np.empty((T, h))
    dA = np.zeros((h, F)) if dA is None else dA
    db1 = np.zeros(F) if db1 is None else db1
    dB = np.zeros((F, h)) if dB is None else dB
    _check(lib().tpo_mlp_shard_bwd(ctypes.byref(_dims(d)), shard, degree, _p(X), _p(A), _p(b1),
                                   _p(B), _p(G), _p(dX), _p(dA), _p(db1), _p(dB)), "mlp_shard_bwd")
    return {"dX": dX, "dA": dA, "db1": db1, "dB": dB}


def attn_shard_fwd(d, shard, degree, X, Wq, Wk, Wv, bq, bk, bv, Wo):
    X, Wq, Wk, Wv, bq, bk, bv, Wo = map(_f64, (X, Wq, Wk, Wv, bq, bk, bv, Wo))
    T, h, H, s, b = d["batch"] * d["seq"], d["hidden"], d["heads"], d["seq"], d["batch"]
    Hs, dh = H // degree, h // H
    w = Hs * dh
    Z = np.empty((T, h))
    Q, K, V, O = (np.empty((T, w)) for _ in range(4))
    lse = np.empty((b, Hs, s))
    _check(lib().tpo_attn_shard_fwd(ctypes.byref(_dims(d)), shard, degree, _p(X), _p(Wq), _p(Wk),
                                    _p(Wv), _p(bq), _p(bk), _p(bv), _p(Wo), _p(Z), _p(Q), _p(K),
                                    _p(V), _p(O), _p(lse)), "attn_shard_fwd")
    return {"Z": Z, "Q": Q, "K": K, "V": V, "O": O, "lse": lse}


def attn_shard_bwd(d, shard, degree, X, Wq, Wk, Wv, bq, bk, bv, Wo, G, out=None):
    X, Wq, Wk, Wv, bq, bk, bv, Wo, G = map(_f64, (X, Wq, Wk, Wv, bq, bk, bv, Wo, G))
    T, h = d["batch"] * d["seq"], d["hidden"]
    o = out if out is not None else {}
    for k in ("dWq", "dWk", "dWv", "dWo"):
        o.setdefault(k, np.zeros((h, h)))
    for k in ("dbq", "dbk", "dbv"):
        o.setdefault(k, np.zeros(h))
    o["dX"] = np.empty((T, h))
    _check(lib().tpo_attn_shard_bwd(ctypes.byref(_dims(d)), shard, degree, _p(X), _p(Wq), _p(Wk),
                                    _p(Wv), _p(bq), _p(bk), _p(bv), _p(Wo), _p(G), _p(o["dX"]),
                                    _p(o["dWq"]), _p(o["dWk"]), _p(o["dWv"]), _p(o["dbq"]),
                                    _p(o["dbk"]), _p(o["dbv"]), _p(o["dWo"])), "attn_shard_bwd")
    return o


def attn_head_fwd(Q, K, V, causal):
    """One head: Q, K, V [s, d] -> P [s, s], O [s, d], lse [s]."""
    Q, K, V = map(_f64, (Q, K, V))
    s, dh = Q.shape
    P = np.empty((s, s)); O = np.empty((s, dh)); lse = np.empty(s)
    lib().tpo_attn_head_fwd(ctypes.c_long(s), ctypes.c_long(dh), ctypes.c_long(dh), int(causal),
                            _p(Q), _p(K), _p(V), _p(P), _p(O), _p(lse))
    return {"P": P, "O": O, "lse": lse}


def mlp_full_fwd(d, X, A, b1, B, b2):
    X, A, b1, B, b2 = map(_f64, (X, A, b1, B, b2))
    Z = np.empty((d["batch"] * d["seq"], d["hidden"]))
    _check(lib().tpo_mlp_full_fwd(ctypes.byref(_dims(d)), _p(X), _p(A), _p(b1), _p(B), _p(b2),
                                  _p(Z)), "mlp_full_fwd")
    return Z


def mlp_full_bwd(d, X, A, b1, B, G):
    X, A, b1, B, G = map(_f64, (X, A, b1, B, G))
    T, h, F = d["batch"] * d["seq"], d["hidden"], d["ffn"]
    o = {"dX": np.empty((T, h)), "dA": np.empty((h, F)), "db1": np.empty(F),
         "dB": np.empty((F, h)), "db2": np.empty(h)}
    _check(lib().tpo_mlp_full_bwd(ctypes.byref(_dims(d)), _p(X), _p(A), _p(b1), _p(B), _p(G),
                                  _p(o["dX"]), _p(o["dA"]), _p(o["db1"]), _p(o["dB"]),
                                  _p(o["db2"])), "mlp_full_bwd")
    return o


def attn_full_fwd(d, X, Wq, Wk, Wv, bq, bk, bv, Wo, bo):
    X, Wq, Wk, Wv, bq, bk, bv, Wo, bo = map(_f64, (X, Wq, Wk, Wv, bq, bk, bv, Wo, bo))
    Z = np.empty((d["batch"] * d["seq"], d["hidden"]))
    _check(lib().tpo_attn_full_fwd(ctypes.byref(_dims(d)), _p(X), _p(Wq), _p(Wk), _p(Wv), _p(bq),
                                   _p(bk), _p(bv), _p(Wo), _p(bo), _p(Z)), "attn_full_fwd")
    return Z


def attn_full_bwd(d, X, Wq, Wk, Wv, bq, bk, bv, Wo, G):
    X, Wq, Wk, Wv, bq, bk, bv, Wo, G = map(_f64, (X, Wq, Wk, Wv, bq, bk, bv, Wo, G))
    T, h = d["batch"] * d["seq"], d["hidden"]
    o = {k: np.empty((h, h)) for k in ("dWq", "dWk", "dWv", "dWo")}
    o.update({k: np.empty(h) for k in ("dbq", "dbk", "dbv", "dbo")})
    o["dX"] = np.empty((T, h))
    _check(lib().tpo_attn_full_bwd(ctypes.byref(_dims(d)), _p(X), _p(Wq), _p(Wk), _p(Wv), _p(bq),
                                   _p(bk), _p(bv), _p(Wo), _p(G), _p(o["dX"]), _p(o["dWq"]),
                                   _p(o["dWk"]), _p(o["dWv"]), _p(o["dbq"]), _p(o["dbk"]),
                                   _p(o["dbv"]), _p(o["dWo"]), _p(o["dbo"])), "attn_full_bwd")
    return o


def layernorm(x, eps=1e-5, gamma=None, beta=None, stats=False):
    """Row-wise LayerNorm y = gamma * (x - mean) / sqrt(var + eps) + beta (biased variance;
    gamma, beta None for 1 and 0).  With stats, also the row means and 1/sqrt(var + eps)."""
    x, gamma, beta = map(_f64, (x, gamma, beta))
    y = np.empty_like(x)
    mean = np.empty(x.shape[0]); rstd = np.empty(x.shape[0])
    lib().tpo_layernorm_affine(ctypes.c_long(x.shape[0]), ctypes.c_long(x.shape[1]), ctypes.c_double(eps),
                               _p(x), _p(gamma), _p(beta), _p(y), _p(mean), _p(rstd))
    return (y, mean, rstd) if stats else y


def layernorm_bwd(x, dy, eps=1e-5, gamma=None):
    """Backward of layernorm: dx, dgamma, dbeta for the upstream gradient dy."""
    x, dy, gamma = map(_f64, (x, dy, gamma))
    dx = np.empty_like(x); dg = np.empty(x.shape[1]); db = np.empty(x.shape[1])
    lib().tpo_layernorm_bwd(ctypes.c_long(x.shape[0]), ctypes.c_long(x.shape[1]), ctypes.c_double(eps),
                            _p(x), _p(gamma), _p(dy), _p(dx), _p(dg), _p(db))
    return dx, dg, db


def _ln_params(p, k):
    return p.get(f"ln{k}_g"), p.get(f"ln{k}_b")


def prelayer_fwd(d, degree, X, p, eps=1e-5, full=False):
    """Pre-LN layer from the shard partials (page "what the tensor parallelism paper actually
    says", section "The layernorm placement the paper flags as critical": LayerNorm on the
    residual stream before each sublayer):
        h1  = x + sum_i Attn_i(LN1(x)) + bo
        out = h1 + sum_i MLP_i(LN2(h1)) + b2
    LN k has the affine part p["lnk_g"], p["lnk_b"] when present (else gamma = 1, beta = 0).
    With full, a dict of out and the intermediates h1, ln1, ln2."""
    X = _f64(X)
    g1, be1 = _ln_params(p, 1)
    g2, be2 = _ln_params(p, 2)
    ln1 = layernorm(X, eps, g1, be1)
    att = sum(attn_shard_fwd(d, i, degree, ln1, p["Wq"], p["Wk"], p["Wv"], p["bq"], p["bk"],
                             p["bv"], p["Wo"])["Z"] for i in range(degree))
    h1 = X + att + _f64(p["bo"])[None, :]
    ln2 = layernorm(h1, eps, g2, be2)
    mlp = sum(mlp_shard_fwd(d, i, degree, ln2, p["A"], p["b1"], p["B"])["Z"] for i in range(degree))
    out = h1 + mlp + _f64(p["b2"])[None, :]
    return {"out": out, "h1": h1, "ln1": ln1, "ln2": ln2} if full else out


def prelayer_bwd(d, degree, X, p, G, eps=1e-5):
    """Chain rule back through prelayer_fwd for the upstream gradient G = dL/d out:
        dh1 = G + LN2_bwd(sum_i dX_i^mlp(G))           (dZ of every MLP shard is G)
        dx  = dh1 + LN1_bwd(sum_i dX_i^att(dh1))       (dZ of every attention shard is dh1)
    Returns dx and every parameter gradient (shard blocks filled into full-size arrays;
    b2 and bo, added once after the sum, get the column sums of G and dh1)."""
    X, G = _f64(X), _f64(G)
    g1, _ = _ln_params(p, 1)
    g2, _ = _ln_params(p, 2)
    f = prelayer_fwd(d, degree, X, p, eps, full=True)
    o = {}
    dx2 = np.zeros_like(X)
    for i in range(degree):
        r = mlp_shard_bwd(d, i, degree, f["ln2"], p["A"], p["b1"], p["B"], G,
                          o.get("dA"), o.get("db1"), o.get("dB"))
        o["dA"], o["db1"], o["dB"] = r["dA"], r["db1"], r["dB"]
        dx2 += r["dX"]
    o["db2"] = G.sum(axis=0)
    dln2, o["ln2_dg"], o["ln2_db"] = layernorm_bwd(f["h1"], dx2, eps, g2)
    dh1 = G + dln2
    dx1 = np.zeros_like(X)
    att = {}
    for i in range(degree):
        att = attn_shard_bwd(d, i, degree, f["ln1"], p["Wq"], p["Wk"], p["Wv"], p["bq"], p["bk"],
                             p["bv"], p["Wo"], dh1, out=att)
        dx1 += att["dX"]
    for k in ("dWq", "dWk", "dWv", "dWo", "dbq", "dbk", "dbv"):
        o[k] = att[k]
    o["dbo"] = dh1.sum(axis=0)
    dln1, o["ln1_dg"], o["ln1_db"] = layernorm_bwd(X, dx1, eps, g1)
    o["dX"] = dh1 + dln1
    o["dh1"] = dh1
    return o
