"""Race guard: every tile / persistent kernel gives bit-identical results at
different launch geometries.

Each quantizer, amax, dequantize and RHT kernel runs the same work with its
default persistent grid and with at most 1, 3 and 37 workgroups (each then
walks many tiles or rows, so a missing barrier between a workgroup's tiles,
or LDS reused before every wave is done with it, shows as a difference);
the two-level DMA GEMM runs with 192- and 256-row tiles.  Outputs (codes,
scales, amax, s_dec, counters, fp32 values, D) must match bit for bit.
"""
import numpy as np
import pytest
import torch

from fp4_block_scaled_x16_amd import api, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
SIGNS = inputs.rht_sign_mask()
CAPS = (1, 3, 37)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


@pytest.fixture(autouse=True)
def default_geometry():
    api.selftest_set_geometry(0, 0)
    yield
    api.selftest_set_geometry(0, 0)


def snapshot(obj):
    """Host copies of every tensor in a result (Quantized, tuple or tensor)."""
    if isinstance(obj, torch.Tensor):
        return [obj.detach().cpu().clone()]
    if isinstance(obj, (tuple, list)):
        return [t for o in obj for t in snapshot(o)]
    out = []
    for k in ("codes", "scales", "codes_t", "amax", "s_dec"):
        v = getattr(obj, k, None)
        if v is not None:
            out.append(v.detach().cpu().clone())
    return out


def same_at_all_geometries(run):
    """run(counters) -> result; compared with the default geometry's result."""
    def once():
        cnt = api.new_counters()
        r = run(cnt)
        torch.cuda.synchronize()
        return snapshot(r) + [cnt.cpu()]
    want = once()
    for cap in CAPS:
        api.selftest_set_geometry(cap, 0)
        got = once()
        api.selftest_set_geometry(0, 0)
        assert len(got) == len(want)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                               b.view(torch.uint8) if b.dtype == torch.float32 else b), (cap, i)


X = inputs.activations((384, 640), cfg_seed=5)
G = inputs.gradients((384, 640), cfg_seed=5)


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3", "mxfp4"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("orient", ["row", "col"])
def test_quantize_1d(fmt, rnd, orient):
    x = dev(G if rnd == "sr" else X)
    same_at_all_geometries(lambda c: api.quantize(x, fmt, orient=orient, rnd=rnd, seed=3,
                                                  offset=1, counters=c, scale_layout="tiled"))


@pytest.mark.parametrize("orient", ["row", "col"])
def test_quantize_mxfp8(orient):
    x = dev(X)
    same_at_all_geometries(lambda c: api.quantize(x, "mxfp8", orient=orient, counters=c,
                                                  scale_layout="tiled"))


@pytest.mark.parametrize("rht_n", [16, 64])
def test_quantize_col_rht(rht_n):
    x = dev(X)
    same_at_all_geometries(lambda c: api.quantize(x, "nvfp4", orient="col", rht=True,
                                                  signs=inputs.rht_sign_bits(rht_n), rht_n=rht_n,
                                                  rnd="sr", seed=2, counters=c))


@pytest.mark.parametrize("fmt,rnd,rht", [("nvfp4", "rne", False), ("ue5m3", "sr", False),
                                         ("mxfp4", "sr", False), ("nvfp4", "rne", True),
                                         ("ue5m3", "sr", True)])
def test_quantize_dual(fmt, rnd, rht):
    x = dev(G if rnd == "sr" else X)
    kd = dict(rht_row=True, signs_row=SIGNS) if rht else {}
    same_at_all_geometries(lambda c: api.quantize_dual(x, fmt, rnd=rnd, seed=4, rht=rht,
                                                       signs=SIGNS if rht else 0, counters=c,
                                                       scale_layout="tiled", **kd))


@pytest.mark.parametrize("fmt,rnd", [("nvfp4", "rne"), ("ue5m3", "sr")])
def test_quantize_2d(fmt, rnd):
    x = dev(inputs.weights((384, 640), cfg_seed=6))
    same_at_all_geometries(lambda c: api.quantize(x, fmt, block="2d", emit_transpose=True,
                                                  rnd=rnd, seed=5, counters=c))


@pytest.mark.parametrize("cols,rnd", [(640, "rne"), (2048, "sr"), (4096, "rne"), (8192, "sr")])
def test_quantize_row_scope(cols, rnd):
    x = dev(inputs.gradients((300, cols), cfg_seed=7))
    same_at_all_geometries(lambda c: api.quantize(x, "nvfp4", rnd=rnd, seed=6, counters=c,
                                                  global_scope="row"))


@pytest.mark.parametrize("kw", [dict(), dict(rht=True, signs=SIGNS),
                                dict(rht=True, signs=inputs.rht_sign_bits(32), rht_n=32),
                                dict(rht=True, signs=SIGNS, orient="row")])
def test_amax(kw):
    x = dev(X)
    same_at_all_geometries(lambda c: api.amax(x, **kw))


@pytest.mark.parametrize("orient,rht_n", [("col", 16), ("col", 64), ("row", 4)])
def test_rht(orient, rht_n):
    x = dev(X)
    same_at_all_geometries(lambda c: api.rht16(x, inputs.rht_sign_bits(rht_n), rht_n=rht_n,
                                               orient=orient))


def test_dequantize():
    q = api.quantize(dev(X), "nvfp4", scale_layout="tiled")
    same_at_all_geometries(lambda c: api.dequantize(q))


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
def test_gemm_tile_heights(fmt):
    """The DMA GEMM with 192- and 256-row tiles: the same MFMA sequence per
    output element, so the same bits."""
    M, N, K = 520, 300, 1024
    qa = api.quantize(dev(inputs.activations((M, K), cfg_seed=8)), fmt, scale_layout="tiled")
    qb = api.quantize(dev(inputs.weights((N, K), cfg_seed=8)), fmt, scale_layout="tiled")
    outs = []
    for rows in (192, 256):
        api.selftest_set_geometry(0, rows)
        outs.append(api.gemm(qa.operand(), qb.operand(), M, N, K, device=DEV))
        torch.cuda.synchronize()
    api.selftest_set_geometry(0, 0)
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
