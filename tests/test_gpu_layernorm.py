"""GPU parity of the pre-LN residual stream around the shards (page "Megatron-LM: what the
tensor parallelism paper actually says", section "The layernorm placement the paper flags as
critical"): the fused residual-sum + LayerNorm kernel, the LayerNorm backward fed by shard
partials, and the whole pre-LN layer (all t shards on one GPU) against the float64 oracle.

Tolerance as for the shards (max |gpu - oracle| / max |oracle| per tensor): 1e-4 for fp32
workloads, 2e-2 for bf16, 3e-3 for fp16.  The LayerNorm statistics and the fp32
residual-stream outputs of a 16-bit call are held to 1e-4: they are fp32 sums of exactly
representable inputs.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, TORCH_DTYPE, check
from tensor_transformer_layer_02_amd import tpshard as tp
from tensor_transformer_layer_02_amd.configs import CONFIGS, LayerConfig
from tensor_transformer_layer_02_amd.inputs import as_f64, make_layer_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rand(gen, shape, std=1.0, dtype=torch.float32):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(dtype)


LN_CASES = [
    # rows, cols, nparts, bias, affine, dtype
    (37, 200, 3, True, True, "bf16"),
    (64, 3072, 8, True, False, "bf16"),
    (5, 8, 0, False, True, "fp32"),
    (129, 7168, 2, True, True, "fp32"),
    (16, 1024, 1, False, False, "bf16"),
    (37, 200, 3, True, True, "fp16"),
    (64, 3072, 8, True, False, "fp16"),
    (48, 2560, 8, True, True, "bf16"),   # three chunks per thread, the last one partly past cols
]


@pytest.mark.parametrize("case", LN_CASES, ids=[f"{c[0]}x{c[1]}p{c[2]}{c[5]}" for c in LN_CASES])
def test_residual_layernorm_matches_oracle(case):
    rows, cols, nparts, with_bias, affine, dt = case
    _say(f"[residual_layernorm] rows={rows} cols={cols} parts={nparts} {dt}")
    gen = torch.Generator().manual_seed(rows * 7 + cols)
    tdt = TORCH_DTYPE[dt]
    act = {"fp32": tp.TP_FP32, "bf16": tp.TP_BF16, "fp16": tp.TP_FP16}[dt]
    res = _rand(gen, (rows, cols), 2.0) + 0.5
    parts = [_rand(gen, (rows, cols), 1.0, tdt) for _ in range(nparts)]
    bias = _rand(gen, (cols,), 0.1, tdt) if with_bias else None
    gam = 1.0 + _rand(gen, (cols,), 0.3) if affine else None
    bet = _rand(gen, (cols,), 0.1) if affine else None
    dev = lambda t: None if t is None else t.cuda()
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    y = torch.empty((rows, cols), dtype=tdt, device="cuda")
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    tp.tp_residual_layernorm(act, rows, cols, [p.cuda() for p in parts], dev(bias), res.cuda(), out, dev(gam),
                             dev(bet), 1e-5, y, mean, rstd)
    torch.cuda.synchronize()
    h = as_f64(res) + sum(as_f64(p) for p in parts) + (as_f64(bias)[None, :] if with_bias else 0.0)
    ref, m, r = oracle.layernorm(h, 1e-5, None if gam is None else as_f64(gam),
                                 None if bet is None else as_f64(bet), stats=True)
    rep = []
    check("h", out, h, 1e-4 if dt != "fp32" else TOL["fp32"], rep)
    check("y", y, ref, TOL[dt], rep)
    check("mean", mean, m, 1e-4, rep)
    check("rstd", rstd, r, 1e-4, rep)
    _say("; ".join(f"{n}={e:.1e}" for n, e in rep))


BWD_CASES = [(37, 200, 3, "bf16"), (64, 3072, 8, "bf16"), (300, 520, 2, "fp32"), (9, 7168, 1, "fp32"),
             (64, 3072, 8, "fp16"), (48, 2560, 7, "bf16")]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"{c[0]}x{c[1]}p{c[2]}{c[3]}" for c in BWD_CASES])
def test_layernorm_bwd_matches_oracle(case):
    rows, cols, nparts, dt = case
    _say(f"[layernorm_bwd] rows={rows} cols={cols} parts={nparts} {dt}")
    gen = torch.Generator().manual_seed(rows * 11 + cols)
    tdt = TORCH_DTYPE[dt]
    act = {"fp32": tp.TP_FP32, "bf16": tp.TP_BF16, "fp16": tp.TP_FP16}[dt]
    x = _rand(gen, (rows, cols), 1.5) - 0.3
    gam = 1.0 + _rand(gen, (cols,), 0.3)
    dparts = [_rand(gen, (rows, cols), 1.0, tdt) for _ in range(nparts)]
    dres = _rand(gen, (rows, cols))
    xc = x.cuda()
    # row statistics from the forward kernel
    y = torch.empty((rows, cols), dtype=tdt, device="cuda")
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    tp.tp_residual_layernorm(act, rows, cols, [], None, xc, None, None, None, 1e-5, y, mean, rstd)
    f32 = dict(dtype=torch.float32, device="cuda")
    dx = torch.empty((rows, cols), **f32)
    dx_act = torch.empty((rows, cols), dtype=tdt, device="cuda")
    dg, db, rs, xs = (torch.empty(cols, **f32) for _ in range(4))
    work = torch.empty(tp.tp_layernorm_bwd_work_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    tp.tp_layernorm_bwd(act, rows, cols, xc, gam.cuda(), mean, rstd, [p.cuda() for p in dparts], dres.cuda(),
                        dx, dx_act, dg, db, rs, xs, work)
    torch.cuda.synchronize()
    g = sum(as_f64(p) for p in dparts)
    odx, odg, odb = oracle.layernorm_bwd(as_f64(x), g, 1e-5, as_f64(gam))
    full = odx + as_f64(dres)
    rep = []
    tol = TOL[dt] if dt == "fp32" else 1e-4  # fp32 math on exactly representable inputs
    check("dx", dx, full, tol, rep)
    check("dx_act", dx_act, full, TOL[dt], rep)
    check("dgamma", dg, odg, tol, rep)
    check("dbeta", db, odb, tol, rep)
    check("dres_sum", rs, as_f64(dres).sum(axis=0), tol, rep)
    check("dx_sum", xs, full.sum(axis=0), max(tol, 1e-4), rep)
    _say("; ".join(f"{n}={e:.1e}" for n, e in rep))


def test_layernorm_bwd_is_deterministic():
    rows, cols = 1000, 3072
    gen = torch.Generator().manual_seed(5)
    x = _rand(gen, (rows, cols)).cuda()
    dp = [_rand(gen, (rows, cols), 1.0, torch.bfloat16).cuda() for _ in range(4)]
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    tp.tp_residual_layernorm(tp.TP_BF16, rows, cols, [], None, x, None, None, None, 1e-5, y, mean, rstd)
    work = torch.empty(tp.tp_layernorm_bwd_work_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        dx = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
        dg = torch.empty(cols, dtype=torch.float32, device="cuda")
        tp.tp_layernorm_bwd(tp.TP_BF16, rows, cols, x, None, mean, rstd, dp, None, dx, None, dg, None, None, None,
                            work)
        outs.append((dx, dg))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_layernorm_entry_points_reject_bad_arguments():
    x = torch.zeros((4, 12), dtype=torch.float32, device="cuda")
    y = torch.empty((4, 12), dtype=torch.float32, device="cuda")
    with pytest.raises(tp.TpError) as e:   # 12 columns: not a multiple of 8
        tp.tp_residual_layernorm(tp.TP_FP32, 4, 12, [], None, x, None, None, None, 1e-5, y, None, None)
    assert e.value.code == 4
    x = torch.zeros((4, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(tp.TpError) as e:   # neither out nor y
        tp.tp_residual_layernorm(tp.TP_FP32, 4, 16, [], None, x, None, None, None, 1e-5, None, None, None)
    assert e.value.code == 1
    big = torch.zeros((1, 8200), dtype=torch.float32, device="cuda")
    with pytest.raises(tp.TpError) as e:   # wider than the kernel's 8192 columns
        tp.tp_residual_layernorm(tp.TP_FP32, 1, 8200, [], None, big, None, None, None, 1e-5, big, None, None)
    assert e.value.code == 6
    m = torch.zeros(4, dtype=torch.float32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tp.TpError) as e:   # work buffer too small
        tp.tp_layernorm_bwd(tp.TP_FP32, 4, 16, x, None, m, m, [x], None, x, None, None, None, None, None, small)
    assert e.value.code == 8


LAYER_CASES = [
    # name, batch, seq, hidden, heads, ffn, t, causal, dtype
    ("tiny_fp32", 2, 64, 128, 4, 512, 2, True, "fp32"),
    ("small_bf16_d96", 2, 130, 384, 4, 1536, 2, True, "bf16"),
    ("small_bf16_d64_t4", 3, 64, 256, 4, 1024, 4, False, "bf16"),
    ("small_fp16_d96", 2, 130, 384, 4, 1536, 2, True, "fp16"),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_preln_layer_matches_oracle(case):
    """All t shards of both sublayers plus the residual / LayerNorm kernels on one GPU: the
    layer output, the input gradient and every parameter gradient against the oracle's
    pre-LN composition (itself pinned to torch float64 autograd)."""
    from tensor_transformer_layer_02_amd.layer import PreLNLayer
    name, b, s, h, H, F, t, causal, dt = case
    cfg = LayerConfig(140 + LAYER_CASES.index(case), name, b, s, h, H, F, t, causal, dt, True)
    _say(f"[{name}] pre-LN layer T={cfg.tokens} h={h} F={F} H={H} t={t}")
    inp = make_layer_inputs(cfg, bias_std=0.02, ln_std=0.2)
    layer = PreLNLayer(cfg, inp)
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    p = {k: as_f64(v) for k, v in inp.items()}
    p["X"] = p["X32"]
    d = cfg.dims()
    fwd = oracle.prelayer_fwd(d, t, p["X32"], p, full=True)
    bwd = oracle.prelayer_bwd(d, t, p["X32"], p, p["G32"])
    tol = TOL[dt]
    rep = []
    check("h1", layer.a["h1"], fwd["h1"], tol, rep)
    check("out", layer.a["out"], fwd["out"], tol, rep)
    check("ln1", layer.a["ln1"], fwd["ln1"], tol, rep)
    check("ln2", layer.a["ln2"], fwd["ln2"], tol, rep)
    check("dh1", layer.a["dh1"], bwd["dh1"], tol, rep)
    check("dX", layer.a["dX"], bwd["dX"], tol, rep)
    for k in ("dA", "db1", "dB", "dWq", "dWv", "dWo", "dbq", "dbv", "db2", "dbo", "ln1_dg", "ln1_db", "ln2_dg",
              "ln2_db", "dWk"):
        check(k, layer.grads[k], bwd[k], tol, rep)
    # dbk is zero in exact arithmetic (a key bias shifts a query's scores by one constant)
    # against the scale of the attention's bias gradients (with one key per query dQ and dK are
    # exactly zero too, so dbq alone is no scale for the rounding noise)
    scale = max(float(layer.grads["dbq"].abs().max()), float(layer.grads["dbv"].abs().max()))
    assert float(layer.grads["dbk"].abs().max()) <= tol * scale
    _say(f"[{name}] " + "; ".join(f"{n}={e:.1e}" for n, e in rep))
