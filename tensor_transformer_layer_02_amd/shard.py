"""Device buffers and call sequence for one layer shard, on top of the C ABI.

`ShardRun` owns the device copies of a workload's inputs and the output,
saved and work buffers of shard `shard` (allocated with torch: plumbing),
and calls the library entry points in the order forward (MLP, attention),
backward (MLP, attention).  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import torch

from . import tpshard as tp
from .configs import LayerConfig
from .inputs import storage_dtype


class ShardRun:
    def __init__(self, cfg: LayerConfig, inputs: dict, device="cuda", degree=None, shards=None,
                 recompute=False):
        self.cfg = cfg
        self.degree = cfg.degree if degree is None else degree
        self.dims = tp.dims_of(cfg)
        self.dt = storage_dtype(cfg)
        self.dev = torch.device(device)
        self.x = {k: v.to(self.dev).contiguous() for k, v in inputs.items()}
        T, h, F = cfg.tokens, cfg.hidden, cfg.ffn
        f32 = dict(dtype=torch.float32, device=self.dev)
        # full-size fp32 gradient buffers (each shard writes its own block)
        self.grads = {"dA": torch.zeros((h, F), **f32), "db1": torch.zeros(F, **f32),
                      "dB": torch.zeros((F, h), **f32), "dWq": torch.zeros((h, h), **f32),
                      "dWk": torch.zeros((h, h), **f32), "dWv": torch.zeros((h, h), **f32),
                      "dWo": torch.zeros((h, h), **f32), "dbq": torch.zeros(h, **f32),
                      "dbk": torch.zeros(h, **f32), "dbv": torch.zeros(h, **f32)}
        self.shards = list(range(self.degree)) if shards is None else list(shards)
        self.buf = {}
        for i in self.shards:
            d, t = self.dims, self.degree
            u8 = dict(dtype=torch.uint8, device=self.dev)
            self.buf[i] = {
                "mlp_saved": torch.empty(tp.tp_mlp_saved_bytes(d, i, t), **u8),
                "attn_saved": torch.empty(tp.tp_attn_saved_bytes(d, i, t), **u8),
                "mlp_work": torch.empty(tp.tp_mlp_work_bytes(d, i, t), **u8),
                "attn_work": torch.empty(tp.tp_attn_work_bytes(d, i, t), **u8),
                # the recompute backward's work: saved layout + backward work
                "mlp_rwork": torch.empty(tp.tp_mlp_recompute_work_bytes(d, i, t) if recompute else 0, **u8),
                "attn_rwork": torch.empty(tp.tp_attn_recompute_work_bytes(d, i, t) if recompute else 0, **u8),
                "Z_mlp": torch.empty((T, h), dtype=self.dt, device=self.dev),
                "Z_attn": torch.empty((T, h), dtype=self.dt, device=self.dev),
                "dX_mlp": torch.empty((T, h), dtype=self.dt, device=self.dev),
                "dX_attn": torch.empty((T, h), dtype=self.dt, device=self.dev),
            }

    def poison(self, i=None, grads=False):
        """Fill the outputs, saved and work buffers of shard i (all shards if None), and the
        gradient buffers if asked, with all-ones bytes: a NaN in bfloat16, IEEE half and
        float32 alike, so anything a kernel leaves unwritten shows up as non-finite."""
        for k in (self.shards if i is None else [i]):
            for v in self.buf[k].values():
                v.view(torch.uint8).fill_(255)
        if grads:
            for v in self.grads.values():
                v.view(torch.uint8).fill_(255)

    # ------------------------------------------------------------- passes
    def mlp_fwd(self, i, stream=None):
        x, b = self.x, self.buf[i]
        tp.tp_mlp_shard_fwd(self.dims, i, self.degree, x["X"], x["A"], x.get("b1"), x["B"], b["Z_mlp"],
                            b["mlp_saved"], stream)

    def attn_fwd(self, i, stream=None):
        x, b = self.x, self.buf[i]
        tp.tp_attn_shard_fwd(self.dims, i, self.degree, x["X"], x["Wq"], x["Wk"], x["Wv"], x.get("bq"),
                             x.get("bk"), x.get("bv"), x["Wo"], b["Z_attn"], b["attn_saved"], stream)

    def mlp_bwd(self, i, stream=None):
        x, b, g = self.x, self.buf[i], self.grads
        tp.tp_mlp_shard_bwd(self.dims, i, self.degree, x["X"], x["A"], x["B"], b["mlp_saved"], x["dZ"],
                            b["dX_mlp"], g["dA"], g["db1"], g["dB"], b["mlp_work"], stream)

    def attn_bwd(self, i, stream=None):
        x, b, g = self.x, self.buf[i], self.grads
        tp.tp_attn_shard_bwd(self.dims, i, self.degree, x["X"], x["Wq"], x["Wk"], x["Wv"], x["Wo"],
                             b["attn_saved"], x["dZ"], b["dX_attn"], g["dWq"], g["dWk"], g["dWv"], g["dbq"],
                             g["dbk"], g["dbv"], g["dWo"], b["attn_work"], stream)

    def mlp_bwd_recompute(self, i, stream=None):
        x, b, g = self.x, self.buf[i], self.grads
        tp.tp_mlp_shard_bwd_recompute(self.dims, i, self.degree, x["X"], x["A"], x.get("b1"), x["B"], x["dZ"],
                                      b["dX_mlp"], g["dA"], g["db1"], g["dB"], b["mlp_rwork"], stream)

    def attn_bwd_recompute(self, i, stream=None):
        x, b, g = self.x, self.buf[i], self.grads
        tp.tp_attn_shard_bwd_recompute(self.dims, i, self.degree, x["X"], x["Wq"], x["Wk"], x["Wv"], x.get("bq"),
                                       x.get("bk"), x.get("bv"), x["Wo"], x["dZ"], b["dX_attn"], g["dWq"],
                                       g["dWk"], g["dWv"], g["dbq"], g["dbk"], g["dbv"], g["dWo"],
                                       b["attn_rwork"], stream)

    def step(self, i, backward=True, stream=None, recompute=False):
        """One pass of the shard's hot path: forward of both sublayers, then backward (with
        recompute, the backward rebuilds the forward's activations instead of reading them)."""
        self.mlp_fwd(i, stream)
        self.attn_fwd(i, stream)
        if backward and recompute:
            self.mlp_bwd_recompute(i, stream)
            self.attn_bwd_recompute(i, stream)
        elif backward:
            self.mlp_bwd(i, stream)
            self.attn_bwd(i, stream)

    # ------------------------------------------------------ verification
    def sum_partials(self, key: str, bias_name: str | None = None) -> torch.Tensor:
        """Local stand-in for the all-reduce: fp32 sum of every shard's partial (+ bias once)."""
        T, h = self.cfg.tokens, self.cfg.hidden
        out = torch.empty((T, h), dtype=torch.float32, device=self.dev)
        parts = [self.buf[i][key] for i in self.shards]
        bias = self.x.get(bias_name) if bias_name else None
        tp.tp_sum_partials(self.dims.act, T, h, parts, bias, out)
        return out

    def saved(self, i) -> dict:
        mlp, attn = tp.saved_layout(self.dims, i, self.degree)
        out = {}
        for k, (off, shape) in mlp.items():
            out[k] = tp.view(self.buf[i]["mlp_saved"], off, shape, self.dt)
        for k, (off, shape) in attn.items():
            out[k] = tp.view(self.buf[i]["attn_saved"], off, shape, torch.float32 if k == "LSE" else self.dt)
        return out
