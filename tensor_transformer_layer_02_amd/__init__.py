"""MI355X-native tensor-parallel transformer layer shard (Megatron-style), forward and backward.

The compute path is the C-ABI library ``libtpshard.so`` (hand-written HIP for
gfx950); ``tensor_transformer_layer_02_amd.tpshard`` is its thin ctypes binding.
Importing this package does not load the library, so the CPU-only parts
(configs, seeded inputs) work on machines without a GPU.
"""
from .configs import CONFIGS, HEADLINE, LayerConfig, shard_flops, shard_min_bytes  # noqa: F401

__all__ = ["CONFIGS", "HEADLINE", "LayerConfig", "shard_flops", "shard_min_bytes"]
