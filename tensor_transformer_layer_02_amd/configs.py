"""Workload presets and algorithmic FLOP / byte counts for one tensor-parallel layer shard.

The layer shapes follow the Megatron-LM tensor-parallel description on the
"what the tensor parallelism paper actually says" page (sections "How
transformer layers actually decompose" and "The attention heads split"): an
FFN with hidden -> 4*hidden -> hidden matrices, and multi-head attention
whose heads are dealt out H/t per shard.  The 30B FFN shape (hidden 7168,
FFN 28672) is the one that page quotes in "The problem ZeRO doesn't solve";
the other shapes are GPT-2 8.3B-like, BERT 3.9B-like and a tiny GPT-2-like
layer.

Nothing here computes the method: these are sizes and counts used by the
benchmark and the tests.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerConfig:
    cid: int            # seed namespace: seed = 1000 * cid + tensor index
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    degree: int         # tensor-parallel degree t
    causal: bool
    dtype: str          # "fp32", "bf16" or "fp16"
    backward: bool      # whether the workload includes the backward pass
    note: str = ""
    gelu: str = "erf"   # GeLU form of the FFN: "erf" (exact, the default) or "tanh"

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def heads_per_shard(self) -> int:
        return self.heads // self.degree

    @property
    def ffn_per_shard(self) -> int:
        return self.ffn // self.degree

    @property
    def attn_width(self) -> int:
        """w = (H/t) * d: the shard's Q/K/V/O column count."""
        return self.heads_per_shard * self.head_dim

    def dims(self) -> dict:
        return dict(batch=self.batch, seq=self.seq, hidden=self.hidden,
                    heads=self.heads, ffn=self.ffn, causal=int(self.causal),
                    gelu=int(self.gelu == "tanh"))

    def with_(self, **kw) -> "LayerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return LayerConfig(**d)


CONFIGS = {
    "tiny": LayerConfig(1, "tiny", 2, 64, 128, 4, 512, 2, True, "fp32", False,
                        "tiny GPT-2-style causal layer, fp32, t=2"),
    "gpt8b_fwd": LayerConfig(2, "gpt8b_fwd", 8, 1024, 3072, 32, 12288, 8, True, "bf16", False,
                             "GPT-2 8.3B-shape layer, one t=8 shard, forward"),
    "gpt8b": LayerConfig(3, "gpt8b", 8, 1024, 3072, 32, 12288, 8, True, "bf16", True,
                         "GPT-2 8.3B-shape layer, one t=8 shard, forward+backward"),
    "bert4b": LayerConfig(4, "bert4b", 16, 512, 2560, 40, 10240, 8, False, "bf16", True,
                          "BERT 3.9B-shape bidirectional layer, one t=8 shard, forward+backward"),
    "g30b_t1": LayerConfig(5, "g30b_t1", 4, 2048, 7168, 56, 28672, 1, True, "bf16", True,
                           "30B-style layer, unsharded (t=1), forward+backward"),
    "g30b_t4": LayerConfig(6, "g30b_t4", 4, 2048, 7168, 56, 28672, 4, True, "bf16", True,
                           "30B-style layer, one t=4 shard, forward+backward"),
}

HEADLINE = "gpt8b"


def causal_pairs(seq: int, causal: bool) -> int:
    """(query, allowed key) pairs per (sequence, head)."""
    return seq * (seq + 1) // 2 if causal else seq * seq


def shard_flops(cfg: LayerConfig, backward: bool | None = None) -> dict:
    """Algorithmic FLOPs of one shard: 2*M*N*K per GEMM, 2*d per (query, allowed key)
    per attention matmul.  No recompute is counted."""
    if backward is None:
        backward = cfg.backward
    T, h, Fs, w, d = cfg.tokens, cfg.hidden, cfg.ffn_per_shard, cfg.attn_width, cfg.head_dim
    pairs = cfg.batch * cfg.heads_per_shard * causal_pairs(cfg.seq, cfg.causal)
    gemm = lambda m, n, k: 2 * m * n * k
    f = {
        "mlp_fwd": gemm(T, Fs, h) + gemm(T, h, Fs),
        "attn_fwd": gemm(T, 3 * w, h) + 2 * (2 * d * pairs) + gemm(T, h, w),
    }
    if backward:
        # dY, dB, dA, dX
        f["mlp_bwd"] = 4 * gemm(T, Fs, h)
        # dO, dWo, (dV, dP, dQ, dK), dWqkv, dX
        f["attn_bwd"] = 2 * gemm(T, w, h) + 4 * (2 * d * pairs) + 2 * gemm(T, 3 * w, h)
    f["total"] = sum(f.values())
    return f


def shard_min_bytes(cfg: LayerConfig, backward: bool | None = None) -> int:
    """Minimum HBM bytes of one shard pass: every tensor read or written once."""
    if backward is None:
        backward = cfg.backward
    e = 4 if cfg.dtype == "fp32" else 2
    T, h, Fs, w = cfg.tokens, cfg.hidden, cfg.ffn_per_shard, cfg.attn_width
    Hs, s, b = cfg.heads_per_shard, cfg.seq, cfg.batch
    weights = (2 * h * Fs + 4 * h * w) * e
    fwd = (T * h * e                    # X
           + weights
           + 2 * T * Fs * e             # U, Y saved
           + 4 * T * w * e              # Q, K, V, O saved
           + b * Hs * s * 4             # LSE
           + 2 * T * h * e)             # two partial outputs
    if not backward:
        return fwd
    bwd = (T * h * e                    # dZ
           + weights                    # weights read again
           + 2 * T * Fs * e + 4 * T * w * e + b * Hs * s * 4   # saved read back
           + (2 * h * Fs + 4 * h * w + Fs + 3 * w) * 4          # fp32 weight/bias grads
           + 2 * T * h * e)             # two dX partials
    return fwd + bwd
