"""Seeded synthetic inputs for a layer shard.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the layer's arithmetic.  Both the HIP path and the CPU
oracle take their inputs from here.

Recipe: a torch CPU ``Generator`` seeded with ``1000 * cid + k``, where k is
the tensor's index in TENSOR_ORDER; values are drawn as float32 ``randn`` and
scaled (activations and the upstream gradient N(0, 1), weights N(0, 0.02),
biases 0 unless ``bias_std`` is given), then rounded to the storage
format (bfloat16 or IEEE half) with round-to-nearest-even for 16-bit workloads.  The oracle receives the same
(rounded) values widened to float64.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import LayerConfig

TENSOR_ORDER = ["X", "A", "b1", "B", "b2", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo", "bo", "dZ"]

WEIGHT_STD = 0.02


def tensor_shapes(cfg: LayerConfig) -> dict:
    T, h, F = cfg.tokens, cfg.hidden, cfg.ffn
    return {
        "X": (T, h), "A": (h, F), "b1": (F,), "B": (F, h), "b2": (h,),
        "Wq": (h, h), "Wk": (h, h), "Wv": (h, h),
        "bq": (h,), "bk": (h,), "bv": (h,),
        "Wo": (h, h), "bo": (h,), "dZ": (T, h),
    }


def storage_dtype(cfg: LayerConfig) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[cfg.dtype]


def make_inputs(cfg: LayerConfig, bias_std: float = 0.0, names=None,
                seed_base: int | None = None, qk_std: float | None = None,
                x_ramp: float = 0.0) -> dict:
    """Return {name: CPU tensor in the storage dtype} for the requested tensors.

    Large-logit variant (tests of the softmax at large score magnitudes): ``qk_std``
    replaces the standard deviation of Wq and Wk, and ``x_ramp`` scales row j of each
    sequence of X by 1 + x_ramp * j / (seq - 1), so that later keys carry larger scores
    than earlier ones.  Both default to the plain recipe."""
    shapes = tensor_shapes(cfg)
    base = 1000 * cfg.cid if seed_base is None else seed_base
    dt = storage_dtype(cfg)
    out = {}
    for k, name in enumerate(TENSOR_ORDER):
        if names is not None and name not in names:
            continue
        shape = shapes[name]
        if name in ("X", "dZ"):
            std = 1.0
        elif name.startswith("b"):
            std = bias_std
        elif name in ("Wq", "Wk") and qk_std is not None:
            std = qk_std
        else:
            std = WEIGHT_STD
        if std == 0.0:
            t = torch.zeros(shape, dtype=torch.float32)
        else:
            g = torch.Generator().manual_seed(base + k)
            t = torch.randn(shape, generator=g, dtype=torch.float32)
            t.mul_(std)
            if name == "X" and x_ramp:
                pos = torch.arange(cfg.seq, dtype=torch.float32) / max(1, cfg.seq - 1)
                t.view(cfg.batch, cfg.seq, -1).mul_((1.0 + x_ramp * pos)[None, :, None])
        out[name] = t.to(dt)
    return out


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a stored tensor to a contiguous float64 numpy array."""
    return np.ascontiguousarray(t.to(torch.float64).numpy())


LAYER_EXTRA = ["X32", "ln1_g", "ln1_b", "ln2_g", "ln2_b"]


def make_layer_inputs(cfg: LayerConfig, bias_std: float = 0.0, ln_std: float = 0.0) -> dict:
    """Inputs of the whole pre-LN layer: the shard tensors of make_inputs, plus the fp32
    residual-stream input X32 ~ N(0, 1), LayerNorm gains 1 + N(0, ln_std) and shifts
    N(0, ln_std) (fp32), and the upstream gradient twice: dZ in the storage dtype (what
    the shards take) and G32, the same values widened to fp32 (what the residual path
    adds).  Seeds continue after TENSOR_ORDER (k = 14, 15, ...)."""
    out = make_inputs(cfg, bias_std)
    base = 1000 * cfg.cid
    T, h = cfg.tokens, cfg.hidden
    for j, name in enumerate(LAYER_EXTRA):
        g = torch.Generator().manual_seed(base + len(TENSOR_ORDER) + j)
        if name == "X32":
            out[name] = torch.randn((T, h), generator=g, dtype=torch.float32)
        elif ln_std == 0.0:
            out[name] = (torch.ones if name.endswith("_g") else torch.zeros)(h, dtype=torch.float32)
        else:
            t = torch.randn(h, generator=g, dtype=torch.float32) * ln_std
            out[name] = t + 1.0 if name.endswith("_g") else t
    out["G32"] = out["dZ"].to(torch.float32)
    return out
