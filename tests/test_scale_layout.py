"""The TILED scale layout's index map, pinned by building the layout from
its description: 2 KiB atoms, one per (256-row band, group of 8 blocks),
atoms band by band, inside an atom 256 rows of 8 scale bytes one after the
other (padding rows and blocks included)."""
import numpy as np
import pytest

from fp4_block_scaled_x16_amd import api
from scale_layout import tiled_offsets, untile


def constructed(rows, kb):
    pos = {}
    off = 0
    bands, groups = -(-rows // 256), -(-kb // 8)
    for band in range(bands):
        for g in range(groups):
            for rr in range(256):
                for jj in range(8):
                    r, j = band * 256 + rr, g * 8 + jj
                    if r < rows and j < kb:
                        pos[(r, j)] = off
                    off += 1
    return pos, off


@pytest.mark.parametrize("rows,kb", [(1, 1), (256, 8), (300, 38), (513, 17), (40, 128)])
def test_offsets_match_construction(rows, kb):
    pos, size = constructed(rows, kb)
    off = tiled_offsets(rows, kb)
    assert size == api.tiled_scale_bytes(rows, kb)
    want = np.array([[pos[(r, j)] for j in range(kb)] for r in range(rows)])
    assert np.array_equal(off, want)
    assert len(np.unique(off)) == rows * kb and off.max() < size


def test_untile_roundtrip():
    rng = np.random.default_rng(0)
    rows, kb = 300, 38
    s = rng.integers(0, 256, (rows, kb), dtype=np.uint8)
    buf = np.zeros(api.tiled_scale_bytes(rows, kb), np.uint8)
    buf[tiled_offsets(rows, kb)] = s
    assert np.array_equal(untile(buf, rows, kb), s)
