"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same seeded inputs.

Tolerance (max |gpu - oracle| / max |oracle| per output tensor): 1e-4 for fp32 workloads,
2e-2 for bf16 and 3e-3 for fp16 (IEEE half) workloads with fp32 accumulation.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, check, check_lse, oracle_inputs, oracle_shard, relerr, run_all_shards
from tensor_transformer_layer_02_amd.configs import CONFIGS, LayerConfig
from tensor_transformer_layer_02_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


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


LARGE_LOGITS = [
    # name, batch, seq, hidden, heads, ffn, t, causal, std of Wq and Wk
    ("logits_d64_causal", 2, 200, 256, 4, 1024, 2, True, 0.07),
    ("logits_d64_noncausal", 2, 160, 256, 4, 1024, 2, False, 0.07),
    ("logits_d96_causal", 2, 190, 384, 4, 1536, 2, True, 0.06),
    ("logits_d96_noncausal", 2, 190, 384, 4, 1536, 2, False, 0.06),
    ("logits_d128_causal", 1, 300, 512, 4, 2048, 2, True, 0.045),
    ("logits_d128_noncausal", 2, 257, 512, 4, 2048, 2, False, 0.045),
]
LAZY_LOG2 = 8.0   # the forward moves its softmax reference when a block max exceeds it by 2^8


@pytest.mark.parametrize("case", LARGE_LOGITS, ids=[c[0] for c in LARGE_LOGITS])
def test_large_logit_softmax(case):
    """Scores that span tens (per-head softmax, page "Megatron-LM: what the tensor parallelism
    paper actually says", section "The attention heads split"): Wq and Wk scaled up and X
    ramped along each sequence, so that later keys score far above earlier ones.  The forward
    then has to move its running softmax reference (and rescale O) as keys stream in, and the
    two halves of a row group, which take alternate key blocks, merge states whose maxima
    differ widely.  Every output of every shard against the oracle at the usual bar."""
    name, b, s, h, H, F, t, causal, qk = case
    cfg = LayerConfig(200 + LARGE_LOGITS.index(case), name, b, s, h, H, F, t, causal, "bf16", True)
    # the inputs must exercise the rescale: in some row a later 64-key block's max score
    # exceeds the first block's by more than the lazy threshold (base-2 units)
    import oracle
    p = oracle_inputs(make_inputs(cfg, bias_std=0.02, qk_std=qk, x_ramp=1.0))
    af = oracle.attn_shard_fwd(cfg.dims(), 0, t, *[p[n] for n in ("X", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo")])
    d = cfg.head_dim
    Q, K = af["Q"][:s, :d], af["K"][:s, :d]
    S = Q @ K.T / np.sqrt(d) * 1.4426950408889634
    if causal:
        S = np.where(np.tril(np.ones((s, s), bool)), S, -np.inf)
    first = S[:, :64].max(axis=1)
    later = S[:, 64:].max(axis=1)
    assert np.nanmax(later - first) > LAZY_LOG2, "inputs do not reach the rescale"
    assert np.ptp(S[np.isfinite(S)]) > 30.0
    report = []
    run_all_shards(cfg, 0.02, report, qk_std=qk, x_ramp=1.0)
    _say(f"[{name}] " + "; ".join(f"{n}={e:.1e}" for n, e in report))
