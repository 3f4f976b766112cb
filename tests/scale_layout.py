"""Index map of the TILED block-scale layout (include/fp4.h, fp4_scale_layout).

Test helper: turns a TILED scale buffer back into the row-major [rows, KB]
scale matrix the oracle produces, so GPU output in either layout is compared
with the same oracle values.  The scale values themselves do not depend on
the layout.
"""
import numpy as np


def tiled_offsets(rows, kb):
    """Byte offset of the scale of (row r, block j), int64 [rows, kb]:
    ((r / 256) * KG + j / 8) * 2048 + (r % 256) * 8 + j % 8, KG = ceil(kb / 8)."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(kb, dtype=np.int64)[None, :]
    kg = -(-kb // 8)
    return (((r >> 8) * kg + (j >> 3)) << 11) + ((r & 255) << 3) + (j & 7)


def untile(buf, rows, kb):
    """Row-major [rows, kb] scale matrix from a TILED scale buffer."""
    return np.asarray(buf).reshape(-1)[tiled_offsets(rows, kb)]
