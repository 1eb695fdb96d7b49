"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same seeded inputs.

Tolerance (max |gpu - oracle| / max |oracle| per output tensor): 1e-4 for fp32 workloads,
2e-2 for bf16 and 3e-3 for fp16 (IEEE half) workloads with fp32 accumulation.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, check, oracle_inputs, oracle_shard, relerr
from tensor_transformer_layer_02_amd.configs import CONFIGS, LayerConfig
from tensor_transformer_layer_02_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_all_shards(cfg: LayerConfig, bias_std: float, report):
    from tensor_transformer_layer_02_amd.shard import ShardRun
    inp = make_inputs(cfg, bias_std=bias_std)
    p = oracle_inputs(inp)
    run = ShardRun(cfg, inp)
    tol = TOL[cfg.dtype]
    grads = {}
    oz = {}
    for i in range(cfg.degree):
        _say(f"[{cfg.name}] shard {i}/{cfg.degree} T={cfg.tokens} h={cfg.hidden} d={cfg.head_dim}")
        run.step(i, backward=True)
        torch.cuda.synchronize()
        o = oracle_shard(cfg.with_(backward=True), p, i, grads=grads)
        sv = run.saved(i)
        for k in ("U", "Y", "QKV", "O", "LSE"):
            check(f"shard{i}.{k}", sv[k], o[k], tol, report)
        for k in ("Z_mlp", "Z_attn", "dX_mlp", "dX_attn"):
            check(f"shard{i}.{k}", run.buf[i][k], o[k], tol, report)
        oz[i] = o
    for k in ("dA", "db1", "dB", "dWq", "dWv", "dWo", "dbq", "dbv"):
        check(k, run.grads[k], grads[k], tol, report)
    # the key-bias gradient is zero in exact arithmetic (softmax ignores a per-row shift)
    # against the scale of the attention's bias gradients (with one key per query dQ and dK are
    # exactly zero too, so dbq alone is no scale for the rounding noise)
    scale = max(float(run.grads["dbq"].abs().max()), float(run.grads["dbv"].abs().max()))
    assert float(run.grads["dbk"].abs().max()) <= tol * scale
    # sum of partials + row-parallel bias == unsharded sublayer
    import oracle
    d = cfg.dims()
    Zm = run.sum_partials("Z_mlp", "b2")
    Za = run.sum_partials("Z_attn", "bo")
    full_m = oracle.mlp_full_fwd(d, p["X"], p["A"], p["b1"], p["B"], p["b2"])
    full_a = oracle.attn_full_fwd(d, *[p[n] for n in ("X", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo")], p["bo"])
    check("sum(Z_mlp)+b2 vs unsharded", Zm, full_m, tol, report)
    check("sum(Z_attn)+bo vs unsharded", Za, full_a, tol, report)
    dXm = run.sum_partials("dX_mlp")
    dXa = run.sum_partials("dX_attn")
    fb_m = oracle.mlp_full_bwd(d, p["X"], p["A"], p["b1"], p["B"], p["dZ"])
    fb_a = oracle.attn_full_bwd(d, *[p[n] for n in ("X", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo")], p["dZ"])
    check("sum(dX_mlp) vs unsharded", dXm, fb_m["dX"], tol, report)
    check("sum(dX_attn) vs unsharded", dXa, fb_a["dX"], tol, report)
    return run


@pytest.mark.parametrize("bias_std", [0.0, 0.02])
def test_tiny_fp32_config_all_shards(bias_std):
    """Tiny GPT-2-style causal layer, fp32, t = 2: every output of both shards, and the
    sum of the 2 partials against the unsharded layer, to 1e-4."""
    report = []
    run_all_shards(CONFIGS["tiny"], bias_std, report)
    _say("; ".join(f"{n}={e:.1e}" for n, e in report))


SMALL_BF16 = [
    # name, batch, seq, hidden, heads, ffn, t, causal  (head dims 32 / 64 / 96 / 128, ragged T)
    ("tiny_bf16_d32", 2, 64, 128, 4, 512, 2, True),
    ("bert_like_d64_ragged", 3, 100, 256, 4, 1024, 2, False),
    ("gpt_like_d96_ragged", 2, 130, 384, 4, 1536, 2, True),
    ("d128_t4_ragged", 1, 257, 512, 4, 2048, 4, True),
]


@pytest.mark.parametrize("case", SMALL_BF16, ids=[c[0] for c in SMALL_BF16])
def test_small_bf16_all_shards(case):
    name, b, s, h, H, F, t, causal = case
    cfg = LayerConfig(100 + SMALL_BF16.index(case), name, b, s, h, H, F, t, causal, "bf16", True)
    report = []
    run_all_shards(cfg, 0.02, report)
    _say(f"[{name}] " + "; ".join(f"{n}={e:.1e}" for n, e in report))


@pytest.mark.parametrize("case", SMALL_BF16, ids=[c[0].replace("bf16", "") + "_fp16" for c in SMALL_BF16])
def test_small_fp16_all_shards(case):
    """The IEEE-half storage variant (tp_dims.act = TP_FP16) on the same shapes as the bf16
    cases: fp16 MFMAs with fp32 accumulation, every output against the oracle to 3e-3."""
    name, b, s, h, H, F, t, causal = case
    cfg = LayerConfig(170 + SMALL_BF16.index(case), name + "_fp16", b, s, h, H, F, t, causal, "fp16", True)
    report = []
    run_all_shards(cfg, 0.02, report)
    _say(f"[{cfg.name}] " + "; ".join(f"{n}={e:.1e}" for n, e in report))


@pytest.mark.parametrize("cfg", [
    CONFIGS["tiny"].with_(cid=130, name="tiny_tanh", gelu="tanh", backward=True),
    LayerConfig(131, "bf16_d96_tanh", 2, 130, 384, 4, 1536, 2, True, "bf16", True, gelu="tanh"),
    LayerConfig(134, "fp16_d64_tanh", 3, 100, 256, 4, 1024, 2, False, "fp16", True, gelu="tanh"),
], ids=["tiny_fp32_tanh", "bf16_d96_tanh", "fp16_d64_tanh"])
def test_tanh_gelu_variant_all_shards(cfg):
    """The tanh-form GeLU variant (tp_dims.gelu = TP_GELU_TANH) against the oracle's tanh form."""
    report = []
    run_all_shards(cfg, 0.02, report)
    _say(f"[{cfg.name}] " + "; ".join(f"{n}={e:.1e}" for n, e in report))


def test_fp32_ragged_noncausal():
    cfg = LayerConfig(120, "fp32_ragged", 3, 37, 64, 8, 256, 4, False, "fp32", True)
    report = []
    run_all_shards(cfg, 0.02, report)
    _say("; ".join(f"{n}={e:.1e}" for n, e in report))


EDGE = [
    # name, batch, seq, hidden, heads, ffn, t, causal, dtype
    ("bf16_seq1", 5, 1, 128, 4, 512, 2, True),              # one token per sequence: softmax over one key
    ("bf16_seq7_ragged", 3, 7, 256, 4, 1024, 2, True),      # T = 21: every tile ragged, one key block
    ("bf16_t1_unsharded", 1, 96, 256, 4, 1024, 1, True),    # degree 1: the shard is the whole sublayer
    ("bf16_one_head_per_shard", 2, 80, 256, 4, 512, 4, False),  # H/t = 1, F/t = 128
    ("bf16_seq65", 2, 65, 256, 2, 1024, 2, True),           # d = 128, one row past a 64-row block
    ("fp16_seq1", 5, 1, 128, 4, 512, 2, True),
    ("fp16_seq65", 2, 65, 256, 2, 1024, 2, False),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_degenerate_and_edge_shapes(case):
    """Degenerate cases of the method: a single token per sequence, degree 1, one head per shard,
    sequences one row past a block, all-ragged tiles; every output against the oracle."""
    name, b, s, h, H, F, t, causal = case
    cfg = LayerConfig(180 + EDGE.index(case), name, b, s, h, H, F, t, causal, name[:4], True)
    report = []
    run_all_shards(cfg, 0.02, report)
    _say(f"[{name}] " + "; ".join(f"{n}={e:.1e}" for n, e in report))


def test_repeat_is_bitwise_deterministic():
    """Running the same shard twice gives bitwise-identical outputs (no atomics, fixed order)."""
    from tensor_transformer_layer_02_amd.shard import ShardRun
    cfg = LayerConfig(130, "det", 2, 96, 384, 4, 1536, 2, True, "bf16", True)
    run = ShardRun(cfg, make_inputs(cfg, bias_std=0.02))
    run.step(1)
    first = {k: run.buf[1][k].clone() for k in ("Z_mlp", "Z_attn", "dX_mlp", "dX_attn")}
    g1 = {k: v.clone() for k, v in run.grads.items()}
    run.step(1)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, run.buf[1][k]), k
    for k, v in g1.items():
        assert torch.equal(v, run.grads[k]), k


def test_shard_leaves_other_blocks_untouched():
    """Gradients are written only into the shard's block of the full-size buffers."""
    from tensor_transformer_layer_02_amd.shard import ShardRun
    cfg = LayerConfig(131, "blocks", 1, 64, 256, 4, 1024, 4, True, "bf16", True)
    run = ShardRun(cfg, make_inputs(cfg), shards=[2])
    for v in run.grads.values():
        v.fill_(float("nan"))
    run.step(2)
    torch.cuda.synchronize()
    Fs, w, h = cfg.ffn_per_shard, cfg.attn_width, cfg.hidden
    c = slice(2 * Fs, 3 * Fs)
    hc = slice(2 * w, 3 * w)
    g = run.grads
    assert torch.isfinite(g["dA"][:, c]).all() and torch.isnan(g["dA"][:, :2 * Fs]).all()
    assert torch.isfinite(g["dB"][c, :]).all() and torch.isnan(g["dB"][3 * Fs:, :]).all()
    assert torch.isfinite(g["dWq"][:, hc]).all() and torch.isnan(g["dWq"][:, :2 * w]).all()
    assert torch.isfinite(g["dWo"][hc, :]).all() and torch.isnan(g["dWo"][:2 * w, :]).all()
    assert torch.isfinite(g["dbv"][hc]).all() and torch.isnan(g["dbv"][3 * w:]).all()


def test_concurrent_calls_on_two_streams_match_serial():
    """Two host threads, each driving one shard on its own stream (the backward passes share the
    device's auxiliary stream), give bitwise the same results as the shards run one after the
    other."""
    import threading
    from tensor_transformer_layer_02_amd.shard import ShardRun
    cfg = LayerConfig(132, "conc", 2, 96, 384, 4, 1536, 2, True, "bf16", True)
    inp = make_inputs(cfg, bias_std=0.02)
    ref = ShardRun(cfg, inp)
    ref.step(0)
    ref.step(1)
    torch.cuda.synchronize()
    run = ShardRun(cfg, inp)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def drive(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    run.step(i, stream=streams[i])
        except Exception as e:  # reported below; the assertion names the shard
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=drive, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for k in ("Z_mlp", "Z_attn", "dX_mlp", "dX_attn"):
            assert torch.equal(ref.buf[i][k], run.buf[i][k]), (i, k)
    for k, v in ref.grads.items():
        assert torch.equal(v, run.grads[k]), k
