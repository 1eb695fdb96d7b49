"""Host-side checks of the attention kernels' LDS fragment addressing (no GPU).

csrc/attn_bf16.hip stores [rows][D] bf16 tiles with the 16-byte chunks of each row permuted
by an XOR of row bits (swz / toff), and each lane reads its MFMA fragments at fixed offsets
(FragAddr).  At d = 128 FragAddr holds only two of those offsets and derives the others by
XOR with constants (rows of 256 bytes, offsets within a row below 256).  These tests restate
the layout from its description and check, for every lane: the derived offsets equal the
direct ones; the fragment reads of a half-wave touch every LDS bank at most once per
128-byte phase for the row reads; and the swizzle is a permutation of each row's chunks.
"""
from __future__ import annotations

import pytest


def _bit(r, i):
    return (r >> i) & 1


def swz(d, r):
    if d == 64:
        return _bit(r, 2) | (_bit(r, 3) << 1) | (_bit(r, 1) << 2)
    if d == 128:
        return _bit(r, 2) | (_bit(r, 3) << 1) | (_bit(r, 0) << 2) | (_bit(r, 1) << 3)
    return (r >> 2) & 3  # d = 32, 96


def toff(d, r, col):
    return r * (d * 2) + (((col >> 3) ^ swz(d, r)) << 4) + (col & 7) * 2


def direct_offsets(d, lane):
    lr, l5, g, j = lane & 31, lane >> 5, lane >> 4, lane & 15
    rows = [toff(d, lr, 16 * c + 8 * l5) for c in range(d // 16)]
    tr = [[toff(d, 8 * h + 4 * (g >> 1) + (j >> 2), 32 * db + 16 * (g & 1) + 4 * (j & 3)) for db in range(d // 32)]
          for h in range(2)]
    return rows, tr


def test_d128_offsets_derive_from_two_registers():
    for lane in range(64):
        rows, tr = direct_offsets(128, lane)
        for c, off in enumerate(rows):
            assert off == rows[0] ^ (c << 5), (lane, c)
        for h in range(2):
            for db in range(4):
                assert tr[h][db] == tr[0][0] ^ ((2048 + 32) if h else 0) ^ (db << 6), (lane, h, db)


@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_swizzle_permutes_each_row(d):
    for r in range(64):
        chunks = sorted(((c ^ swz(d, r)) for c in range(d // 8)))
        assert chunks == list(range(d // 8))


@pytest.mark.parametrize("d", [64, 96, 128])
def test_row_fragment_reads_spread_over_banks(d):
    """A 16-byte read by 16 lanes (a quarter-wave phase) covers 64 dwords: 16 different rows at one
    logical chunk must land on distinct 16-byte bank groups (64 banks of 4 bytes = 16 groups)."""
    for c in range(d // 16):
        for q in range(4):
            lanes = range(16 * q, 16 * q + 16)
            groups = {((direct_offsets(d, l)[0][c]) // 16) % 16 for l in lanes}
            assert len(groups) == 16, (d, c, q)
