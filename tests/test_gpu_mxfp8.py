"""GPU parity of the MXFP8 quantizer and dequantizer (the Q/K projections of
the 2D-block FP4 page) against the oracle: codes, scales and counters
bit-exact rowwise and colwise, both scale layouts; values spanning E4M3's
subnormals, zero blocks and exact ties; dequantized values bit-exact in fp32
and bf16; a Q/K-projection-sized tensor of the 8B model (8192 tokens x 4096)
compared whole."""
import numpy as np
import pytest
import torch

from fp4_block_scaled_x16_amd import api, inputs
from oracle import formats as F
from oracle import quantize as Q
from scale_layout import untile

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def qk_like(shape, cfg_seed):
    v = F.bf16_bits_to_f32(inputs.normal(shape, cfg_seed=cfg_seed))
    v = v * np.exp2(np.arange(shape[0]) % 29 - 14.0).astype(np.float32)[:, None]
    v[1, :] = 0.0                                        # a zero row: zero blocks
    v[2, :32] = np.float32(2.0 ** -30)                   # far below 448 * 2^e: subnormals, ties
    v[2, 3] = 7.0
    return inputs.to_bf16_bits(v.astype(np.float32))


def check(x_bits, orient, layout):
    cnt = api.new_counters()
    q = api.quantize(dev(x_bits), "mxfp8", orient=orient, counters=cnt, scale_layout=layout)
    torch.cuda.synchronize()
    r = Q.quantize(x_bits, "mxfp8", orient=orient)
    assert np.array_equal(q.codes.cpu().numpy(), r["codes"]), "codes differ"
    s = q.scales.cpu().numpy()
    if layout == "tiled":
        s = untile(s, q.rows, q.cols // 32)
    assert np.array_equal(s, r["scales"]), "scales differ"
    assert api.counters_dict(cnt) == r["counters"]
    return q, r


@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("orient,R,C", [("row", 64, 96), ("row", 96, 544), ("row", 320, 1056),
                                        # colwise: the blocked axis is the rows; columns
                                        # beyond a multiple of the 256-column tile
                                        ("col", 64, 96), ("col", 96, 520), ("col", 320, 1032)])
def test_mxfp8_quantize(orient, layout, R, C):
    check(qk_like((R, C), R + C), orient, layout)


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("orient,layout,R,C", [("row", "tiled", 96, 256), ("row", "rowmajor", 96, 544),
                                               ("col", "tiled", 320, 1032), ("col", "rowmajor", 64, 96)])
def test_mxfp8_dequantize(out, orient, layout, R, C):
    """Dequantized values bit for bit (fp32, and bf16 rounded once) for
    rowwise and colwise codes in both scale layouts; the shapes leave the
    last grid stride of 16-byte stores partial."""
    x = qk_like((R, C), R + C + 5)
    q, r = check(x, orient, layout)
    d = api.dequantize(q, out)
    torch.cuda.synchronize()
    Rq, Cq = (R, C) if orient == "row" else (C, R)
    want = Q.dequantize(r["codes"], r["scales"], "mxfp8", "1d", 1.0, Rq, Cq,
                        out="f32" if out == torch.float32 else "bf16")
    got = d.cpu()
    assert tuple(got.shape) == (Rq, Cq)
    if out == torch.float32:
        assert np.array_equal(got.numpy().view(np.uint32), want.view(np.uint32))
    else:
        assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("orient", ["row", "col"])
def test_mxfp8_qk_projection_size(orient):
    """A Q (or K) projection output of the 8B model: 8192 tokens x 4096."""
    x = inputs.activations((8192, 4096), cfg_seed=61)
    check(x, orient, "tiled")
