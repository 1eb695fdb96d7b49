"""The whole pre-LN transformer layer on one GPU, on top of the C ABI.

Page "Megatron-LM: what the tensor parallelism paper actually says", section
"The layernorm placement the paper flags as critical": LayerNorm acts on the
residual stream before each sublayer and the sublayer's output is added back:
    h1  = x + sum_i Attn_i(LN1(x)) + bo
    out = h1 + sum_i MLP_i(LN2(h1)) + b2
All t shards of both sublayers run here one after the other (on a real tensor-
parallel group each would sit on its own GPU and the sums would be all-reduces).
`PreLNLayer` owns the device buffers (torch allocations: plumbing) and calls the
library in order; no arithmetic of the layer happens in Python.  The residual
stream (x, h1, out and their gradients) is fp32; the LayerNorm outputs, shard
partials and the gradients fed to the shards are in the activation dtype.
"""
from __future__ import annotations

import torch

from . import tpshard as tp
from .configs import LayerConfig
from .inputs import storage_dtype

EPS = 1e-5


class PreLNLayer:
    def __init__(self, cfg: LayerConfig, inputs: dict, device="cuda"):
        self.cfg, self.t = cfg, cfg.degree
        self.dims = tp.dims_of(cfg)
        self.act = self.dims.act
        self.dt = storage_dtype(cfg)
        dev = self.dev = torch.device(device)
        self.x = {k: v.to(dev).contiguous() for k, v in inputs.items()}
        T, h, F = cfg.tokens, cfg.hidden, cfg.ffn
        f32 = dict(dtype=torch.float32, device=dev)
        act = dict(dtype=self.dt, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.a = {"ln1": torch.empty((T, h), **act), "ln2": torch.empty((T, h), **act),
                  "h1": torch.empty((T, h), **f32), "out": torch.empty((T, h), **f32),
                  "mean1": torch.empty(T, **f32), "rstd1": torch.empty(T, **f32),
                  "mean2": torch.empty(T, **f32), "rstd2": torch.empty(T, **f32),
                  "dh1": torch.empty((T, h), **f32), "dh1_act": torch.empty((T, h), **act),
                  "dX": torch.empty((T, h), **f32),
                  "ln_work": torch.empty(tp.tp_layernorm_bwd_work_bytes(T, h), **u8)}
        self.grads = {"dA": torch.zeros((h, F), **f32), "db1": torch.zeros(F, **f32),
                      "dB": torch.zeros((F, h), **f32), "dWq": torch.zeros((h, h), **f32),
                      "dWk": torch.zeros((h, h), **f32), "dWv": torch.zeros((h, h), **f32),
                      "dWo": torch.zeros((h, h), **f32), "dbq": torch.zeros(h, **f32),
                      "dbk": torch.zeros(h, **f32), "dbv": torch.zeros(h, **f32),
                      "db2": torch.zeros(h, **f32), "dbo": torch.zeros(h, **f32),
                      "ln1_dg": torch.zeros(h, **f32), "ln1_db": torch.zeros(h, **f32),
                      "ln2_dg": torch.zeros(h, **f32), "ln2_db": torch.zeros(h, **f32)}
        d, t = self.dims, self.t
        self.buf = [{"mlp_saved": torch.empty(tp.tp_mlp_saved_bytes(d, i, t), **u8),
                     "attn_saved": torch.empty(tp.tp_attn_saved_bytes(d, i, t), **u8),
                     "mlp_work": torch.empty(tp.tp_mlp_work_bytes(d, i, t), **u8),
                     "attn_work": torch.empty(tp.tp_attn_work_bytes(d, i, t), **u8),
                     "Z_attn": torch.empty((T, h), **act), "Z_mlp": torch.empty((T, h), **act),
                     "dX_attn": torch.empty((T, h), **act), "dX_mlp": torch.empty((T, h), **act)}
                    for i in range(t)]

    # ------------------------------------------------------------ phases
    def ln1(self, stream=None):
        x, a, T, h = self.x, self.a, self.cfg.tokens, self.cfg.hidden
        tp.tp_residual_layernorm(self.act, T, h, [], None, x["X32"], None, x["ln1_g"], x["ln1_b"], EPS,
                                 a["ln1"], a["mean1"], a["rstd1"], stream)

    def attn_fwd(self, stream=None):
        x, a = self.x, self.a
        for i, b in enumerate(self.buf):
            tp.tp_attn_shard_fwd(self.dims, i, self.t, a["ln1"], x["Wq"], x["Wk"], x["Wv"], x.get("bq"),
                                 x.get("bk"), x.get("bv"), x["Wo"], b["Z_attn"], b["attn_saved"], stream)

    def residual_ln2(self, stream=None):
        """h1 = x + sum_i Z_i + bo, and LN2(h1)."""
        x, a, T, h = self.x, self.a, self.cfg.tokens, self.cfg.hidden
        tp.tp_residual_layernorm(self.act, T, h, [b["Z_attn"] for b in self.buf], x.get("bo"), x["X32"], a["h1"],
                                 x["ln2_g"], x["ln2_b"], EPS, a["ln2"], a["mean2"], a["rstd2"], stream)

    def mlp_fwd(self, stream=None):
        x, a = self.x, self.a
        for i, b in enumerate(self.buf):
            tp.tp_mlp_shard_fwd(self.dims, i, self.t, a["ln2"], x["A"], x.get("b1"), x["B"], b["Z_mlp"],
                                b["mlp_saved"], stream)

    def residual_out(self, stream=None):
        """out = h1 + sum_i Z_i + b2."""
        x, a, T, h = self.x, self.a, self.cfg.tokens, self.cfg.hidden
        tp.tp_residual_layernorm(self.act, T, h, [b["Z_mlp"] for b in self.buf], x.get("b2"), a["h1"], a["out"],
                                 None, None, EPS, None, None, None, stream)

    def mlp_bwd(self, stream=None):
        x, a, g = self.x, self.a, self.grads
        for i, b in enumerate(self.buf):
            tp.tp_mlp_shard_bwd(self.dims, i, self.t, a["ln2"], x["A"], x["B"], b["mlp_saved"], x["dZ"],
                                b["dX_mlp"], g["dA"], g["db1"], g["dB"], b["mlp_work"], stream)

    def ln2_bwd(self, stream=None):
        """dh1 = G + LN2_bwd(sum_i dX_i); db2 = column sums of G, dbo = those of dh1."""
        x, a, g, T, h = self.x, self.a, self.grads, self.cfg.tokens, self.cfg.hidden
        tp.tp_layernorm_bwd(self.act, T, h, a["h1"], x["ln2_g"], a["mean2"], a["rstd2"],
                            [b["dX_mlp"] for b in self.buf], x["G32"], a["dh1"], a["dh1_act"], g["ln2_dg"],
                            g["ln2_db"], g["db2"], g["dbo"], a["ln_work"], stream)

    def attn_bwd(self, stream=None):
        x, a, g = self.x, self.a, self.grads
        for i, b in enumerate(self.buf):
            tp.tp_attn_shard_bwd(self.dims, i, self.t, a["ln1"], x["Wq"], x["Wk"], x["Wv"], x["Wo"],
                                 b["attn_saved"], a["dh1_act"], b["dX_attn"], g["dWq"], g["dWk"], g["dWv"],
                                 g["dbq"], g["dbk"], g["dbv"], g["dWo"], b["attn_work"], stream)

    def ln1_bwd(self, stream=None):
        """dx = dh1 + LN1_bwd(sum_i dX_i)."""
        x, a, g, T, h = self.x, self.a, self.grads, self.cfg.tokens, self.cfg.hidden
        tp.tp_layernorm_bwd(self.act, T, h, x["X32"], x["ln1_g"], a["mean1"], a["rstd1"],
                            [b["dX_attn"] for b in self.buf], a["dh1"], a["dX"], None, g["ln1_dg"], g["ln1_db"],
                            None, None, a["ln_work"], stream)

    FORWARD = ("ln1", "attn_fwd", "residual_ln2", "mlp_fwd", "residual_out")
    BACKWARD = ("mlp_bwd", "ln2_bwd", "attn_bwd", "ln1_bwd")

    def forward(self, stream=None):
        for ph in self.FORWARD:
            getattr(self, ph)(stream)
        return self.a["out"]

    def backward(self, stream=None):
        """Upstream gradient: x["dZ"] (activation dtype, fed to the MLP shards) and x["G32"]
        (the same values in fp32, on the residual path)."""
        for ph in self.BACKWARD:
            getattr(self, ph)(stream)
        return self.a["dX"]

    def ln_bytes(self) -> dict:
        """Algorithmic HBM bytes of each LayerNorm / residual phase (every tensor read or
        written once; the backward's band partials counted)."""
        T, h, t = self.cfg.tokens, self.cfg.hidden, self.t
        e = self.dt.itemsize
        nb = min(T, 768)
        # band partials: written, read, and their 32 group sums written and read
        part = lambda q: q * 2 * (nb + 32) * h * 4
        return {"ln1": T * h * (4 + e) + 8 * T,
                "residual_ln2": T * h * (4 + t * e + 4 + e) + h * e + 8 * T,
                "residual_out": T * h * (4 + t * e + 4) + h * e,
                "ln2_bwd": T * h * (4 + t * e + 4 + 4 + e) + 8 * T + part(4),
                "ln1_bwd": T * h * (4 + t * e + 4 + 4) + 8 * T + part(2)}
