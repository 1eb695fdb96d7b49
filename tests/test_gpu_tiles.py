"""Every GEMM tile shape against the oracle on ragged shapes.

The GEMMs pick a tile shape (and, for the fp32 weight gradients, a K split) with a cost model;
at full size most of the shard runs on the 8-wave tiles, whose operand pipelines load global
memory straight into LDS and handle the K range in rounds of six steps plus a tail (in rounds
of three for the two K-group tiles: the 192 x 192 fp32 weight-gradient one and the 64 x 192
one for plain 16-bit stores, dO and the FFN's dX at these sizes).  At small
sizes the model picks other tiles, so these tests force each tile in turn (the library's test
hook tp_test_force_gemm_tile; every GEMM the tile is valid for uses it) and check every output
of every shard against the float64 oracle.  The shapes make M, N and K ragged for every tile,
and give K step counts (K / 64) with every remainder modulo 6 (the 8-wave pipeline's round):
hidden 832 (13 steps), 640 (10), 1728 (27); FFN shard 1088 (17), 896 (14), 1536 (24); tokens
63, 185, 257 (the weight gradients' K: 1, 3 and 5 steps).  The IEEE-half instantiations of every
tile run the t = 3 shape once more at the fp16 bar.
"""
from __future__ import annotations

import pytest

from gpu_helpers import _say, run_all_shards
from tensor_transformer_layer_02_amd.configs import LayerConfig

pytestmark = pytest.mark.gpu

CASES = [
    # name, batch, seq, hidden, heads, ffn, t, causal
    ("T63_h832_d64_t1", 1, 63, 832, 13, 1088, 1, True),
    ("T185_h640_d64_t1", 5, 37, 640, 10, 896, 1, False),
    ("T257_h1728_d96_t3", 1, 257, 1728, 18, 4608, 3, True),   # w = 576: the 192-wide tiles fit Q|K|V
]
NTILES = 12


@pytest.mark.parametrize("ksplit", [1, 2])
@pytest.mark.parametrize("tile", list(range(NTILES)))
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forced_tile_matches_oracle(case, tile, ksplit):
    from tensor_transformer_layer_02_amd import tpshard as tp
    assert tp.tp_test_gemm_tile_count() == NTILES
    name, b, s, h, H, F, t, causal = case
    cfg = LayerConfig(400 + CASES.index(case), name, b, s, h, H, F, t, causal, "bf16", True)
    _say(f"[tiles] {name} tile {tile} ksplit {ksplit}")
    report = []
    tp.tp_test_force_gemm_tile(tile, ksplit)
    try:
        run_all_shards(cfg, 0.02, report)
    finally:
        tp.tp_test_force_gemm_tile(-1, 0)
    _say(f"[tiles] {name} tile {tile} ksplit {ksplit}: worst {max(e for _, e in report):.1e}")


@pytest.mark.parametrize("tile", list(range(NTILES)))
def test_forced_tile_fp16_matches_oracle(tile):
    """The IEEE-half instantiations of every tile (fp16 MFMAs, fp32 accumulation) on the
    ragged t = 3 shape, every output of every shard against the oracle at the fp16 bar."""
    from tensor_transformer_layer_02_amd import tpshard as tp
    name, b, s, h, H, F, t, causal = CASES[2]
    cfg = LayerConfig(420, name + "_fp16", b, s, h, H, F, t, causal, "fp16", True)
    _say(f"[tiles fp16] {name} tile {tile}")
    report = []
    tp.tp_test_force_gemm_tile(tile, 0)
    try:
        run_all_shards(cfg, 0.02, report)
    finally:
        tp.tp_test_force_gemm_tile(-1, 0)
    _say(f"[tiles fp16] {name} tile {tile}: worst {max(e for _, e in report):.1e}")
