"""GPU parity of the quantization kernels against the CPU oracle.

Bar: bit-exact codes, scales, tensor amax, s_dec and event counters.
Small cases span several kernel tiles plus a ragged tail in each dimension
(rowwise: grid-stride over 1xBS blocks; colwise: 8BS x 64 tiles; 2D: 64 x 64
regions); the full-size cases run the workloads' real shapes in the launch
configuration the benchmark uses and compare sampled row/column slabs.
"""
import numpy as np
import pytest
import torch

from fp4_block_scaled_x16_amd import api, inputs
from oracle import formats as F
from oracle import quantize as Q
from oracle.rht import rht16_cols
from scale_layout import untile

pytestmark = pytest.mark.gpu
DEV = "cuda"
SIGNS = inputs.rht_sign_mask()


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def f32_bits(v):
    return np.float32(v).view(np.uint32)


def run_both(x_bits, fmt, block="1d", orient="row", rnd="rne", seed=1, offset=0, rht=False,
             target=448.0, stale=None, emit_transpose=False, scale_layout="rowmajor"):
    x = dev(x_bits)
    cnt = api.new_counters()
    amax_in = None if stale is None else torch.tensor([stale], dtype=torch.float32, device=DEV)
    q = api.quantize(x, fmt, block=block, orient=orient, rnd=rnd, seed=seed, offset=offset,
                     rht=rht, signs=SIGNS if rht else 0, target=target, amax_in=amax_in,
                     emit_transpose=emit_transpose, counters=cnt, scale_layout=scale_layout)
    torch.cuda.synchronize()
    r = Q.quantize(x_bits, fmt, block=block, orient=orient, rnd=rnd, seed=seed, offset=offset,
                   rht=rht, signs=SIGNS if rht else 0, target=target,
                   amax=None if stale is None else np.float32(stale),
                   emit_transpose=emit_transpose)
    return q, r, api.counters_dict(cnt)


def gpu_scales(q):
    """Row-major scale matrix of a quantized result, whatever its layout."""
    s = q.scales.cpu().numpy()
    if q.scale_layout == api.SCALES_TILED:
        return untile(s, q.rows, q.cols // api.BLOCK_LEN[q.fmt])
    return s


def assert_same(q, r, cnt):
    assert np.array_equal(q.codes.cpu().numpy(), r["codes"]), "codes differ"
    assert np.array_equal(gpu_scales(q), r["scales"]), "scales differ"
    if r.get("codes_t") is not None:
        assert np.array_equal(q.codes_t.cpu().numpy(), r["codes_t"]), "codes_t differ"
    if r["amax"] is not None:
        assert f32_bits(q.amax.item()) == f32_bits(r["amax"]), "amax differs"
    assert f32_bits(q.s_dec.item()) == f32_bits(r["s_dec"]), "s_dec differs"
    assert cnt == r["counters"], "counters differ"


GEN = {
    "act": lambda s, seed: inputs.activations(s, cfg_seed=seed),
    "grad": lambda s, seed: inputs.gradients(s, cfg_seed=seed),
    "wgt": lambda s, seed: inputs.weights(s, cfg_seed=seed),
}


# ------------------------------------------------------------- rowwise ----
@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3", "mxfp4"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("dist", ["act", "grad"])
def test_rowwise(fmt, rnd, dist):
    cols = 160 if fmt == "mxfp4" else 208
    x = GEN[dist]((1037, cols), 31)
    q, r, c = run_both(x, fmt, rnd=rnd, offset=3)
    assert_same(q, r, c)


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3", "mxfp4"])
@pytest.mark.parametrize("orient", ["row", "col"])
def test_tiled_scale_layout(fmt, orient):
    """TILED scales hold the same values as row-major ones: output code
    matrices of 300 / 264 rows (a partial 256-row band) and 38 / 19 blocks
    per row (a partial group of 8), SR on gradients."""
    shape = (300, 608) if orient == "row" else (608, 264)
    x = inputs.gradients(shape, cfg_seed=33)
    q, r, c = run_both(x, fmt, orient=orient, rnd="sr", offset=2, scale_layout="tiled")
    assert q.scales.dim() == 1 and q.scales.numel() == api.tiled_scale_bytes(
        q.rows, q.cols // api.BLOCK_LEN[q.fmt])
    assert_same(q, r, c)
    d = api.dequantize(q)
    torch.cuda.synchronize()
    want = Q.dequantize(r["codes"], r["scales"], fmt, "1d", r["s_dec"], q.rows, q.cols, out="f32")
    assert np.array_equal(d.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt,target", [("nvfp4", 448.0), ("ue5m3", 448.0), ("ue5m3", 2048.0)])
def test_rowwise_stale_amax(fmt, target):
    x = inputs.activations((300, 256), cfg_seed=32)
    stale = np.float32(np.abs(F.bf16_bits_to_f32(x)).max() / 6.0)
    q, r, c = run_both(x, fmt, target=target, stale=stale)
    assert_same(q, r, c)
    if fmt == "nvfp4":
        assert c["scale_saturated"] > 0 and c["elem_saturated"] > 0


# ------------------------------------------------------------- colwise ----
# the RHT is defined for the two-level formats only (MXFP4 + RHT is rejected)
@pytest.mark.parametrize("fmt,rht", [("nvfp4", False), ("nvfp4", True), ("ue5m3", False),
                                     ("ue5m3", True), ("mxfp4", False)])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_colwise(fmt, rnd, rht):
    rows = 320 if fmt == "mxfp4" else 304        # 2 or 1 full tiles plus a ragged tile
    x = inputs.gradients((rows, 200), cfg_seed=33) if rnd == "sr" else \
        inputs.activations((rows, 200), cfg_seed=33)
    q, r, c = run_both(x, fmt, orient="col", rnd=rnd, offset=1, rht=rht)
    assert_same(q, r, c)


# ------------------------------------------------------------------ 2D ----
@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
@pytest.mark.parametrize("emit", [False, True])
def test_2d(fmt, emit):
    w = inputs.weights((208, 144), cfg_seed=34)
    q, r, c = run_both(w, fmt, block="2d", emit_transpose=emit)
    assert_same(q, r, c)


def test_2d_outliers_and_stale():
    x = inputs.activations((192, 320), cfg_seed=35)
    stale = np.float32(np.abs(F.bf16_bits_to_f32(x)).max() / 4.0)
    q, r, c = run_both(x, "nvfp4", block="2d", emit_transpose=True, stale=stale)
    assert_same(q, r, c)


# ---------------------------------------------------------- degenerate ----
def _bits(a):
    return inputs.to_bf16_bits(np.asarray(a, np.float32))


@pytest.mark.parametrize("orient", ["row", "col"])
def test_zeros_and_signed_zeros(orient):
    x = np.zeros((64, 64), np.float32)
    x[3, 5] = -0.0
    q, r, c = run_both(_bits(x), "nvfp4", orient=orient)
    assert_same(q, r, c)
    assert q.s_dec.item() == 1.0 and q.amax.item() == 0.0


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
def test_scale_underflow_block(fmt):
    x = np.full((32, 64), 1e-10, np.float32)
    x[1, 3] = 1e30
    x[5, :16] = 2.0 ** -126          # bf16-normal tiny values
    x[6, :8] = 1e-38                 # bf16 subnormals
    q, r, c = run_both(_bits(x), fmt)
    assert_same(q, r, c)
    assert c["scale_underflow"] > 0


def _tiny_tiles(rows, cols, seed=5):
    """bf16 bits of a tensor of tiny values whose 16x16 tiles have the block
    amaxes in TINY_AMAX (each reached on the tile's diagonal, so every 1x16
    and 16x1 block of a tile has that amax), the tensor amax 2^-110."""
    rng = np.random.default_rng(seed)
    x = np.zeros((rows, cols), np.float32)
    k = 0
    for r0 in range(0, rows, 16):
        for c0 in range(0, cols, 16):
            a = TINY_AMAX[k % len(TINY_AMAX)]
            k += 1
            t = (a * rng.uniform(-1, 1, (16, 16))).astype(np.float32)
            t[np.arange(16), np.arange(16)] = a * rng.choice([-1.0, 1.0], 16)
            x[r0:r0 + 16, c0:c0 + 16] = t
    return _bits(x)


# Block amaxes around 2^-125, where the quantizers' amax_B / 6 switches
# from the multiply-and-correct form to a division, down to the smallest
# bf16 subnormal and zero; 2^-110 sets a tensor scale that brings them into
# the scale formats' normal and subnormal ranges.
TINY_AMAX = [2.0 ** -110, 2.0 ** -120, 2.0 ** -125 * 1.0078125, 2.0 ** -125,
             2.0 ** -125 * 0.99609375, 2.0 ** -126, 2.0 ** -129, 2.0 ** -133, 0.0]


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("kind", ["row", "col", "2d", "dual"])
def test_tiny_block_amaxes(kind, fmt, rnd):
    xb = _tiny_tiles(128, 96)
    assert np.abs(F.bf16_bits_to_f32(xb)).max() == np.float32(2.0 ** -110)
    if kind == "dual":
        cnt = api.new_counters()
        qr, qc = api.quantize_dual(dev(xb), fmt, rnd=rnd, seed=3, offset=0, offset_t=1,
                                   counters=cnt)
        torch.cuda.synchronize()
        rr = Q.quantize(xb, fmt, orient="row", rnd=rnd, seed=3, offset=0)
        rc = Q.quantize(xb, fmt, orient="col", rnd=rnd, seed=3, offset=1)
        for q, r in ((qr, rr), (qc, rc)):
            assert np.array_equal(q.codes.cpu().numpy(), r["codes"]), "codes differ"
            assert np.array_equal(gpu_scales(q), r["scales"]), "scales differ"
            assert f32_bits(q.s_dec.item()) == f32_bits(r["s_dec"]), "s_dec differs"
        assert api.counters_dict(cnt) == {k: rr["counters"][k] + rc["counters"][k]
                                          for k in rr["counters"]}
        return
    block, orient = ("2d", "row") if kind == "2d" else ("1d", kind)
    q, r, c = run_both(xb, fmt, block=block, orient=orient, rnd=rnd,
                       emit_transpose=kind == "2d")
    assert_same(q, r, c)
    # the mix reaches the subnormal scale codes, and (E4M3) the underflow to
    # code 0
    assert c["scale_subnormal"] > 0 and (fmt != "nvfp4" or c["scale_underflow"] > 0)


def test_hand_example():
    b0 = [6, -0.5, 1, 1.5, 2, 3, 4, -6, 0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5]
    x = _bits([b0 + [10.5] + [1.75] * 15])
    q, r, c = run_both(x, "nvfp4")
    assert_same(q, r, c)
    assert q.scales.cpu().numpy().tolist() == [[0x78, 0x7E]]


def test_mx_extremes():
    rng = np.random.default_rng(36)
    x = (rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-38, 38, (64, 1))).astype(np.float32)
    q, r, c = run_both(_bits(x), "mxfp4")
    assert_same(q, r, c)


def test_empty():
    q = api.quantize(dev(np.zeros((16, 64), np.uint16))[:0], "nvfp4")
    torch.cuda.synchronize()
    assert q.codes.shape == (0, 32) and q.amax.item() == 0.0 and q.s_dec.item() == 1.0


# --------------------------------------------------- amax, RHT, dequant ----
def test_amax_plain_and_rht():
    x = inputs.activations((4096, 392), cfg_seed=37)
    xd = dev(x)
    a = api.amax(xd)
    b = api.amax(xd, rht=True, signs=SIGNS)
    torch.cuda.synchronize()
    xf = F.bf16_bits_to_f32(x)
    assert f32_bits(a.item()) == f32_bits(Q.tensor_amax(xf))
    assert f32_bits(b.item()) == f32_bits(Q.tensor_amax(rht16_cols(xf, SIGNS)))


def test_amax_strided_view():
    x = inputs.activations((100, 256), cfg_seed=38)
    xd = dev(x)[:, 64:192]
    a = api.amax(xd)
    torch.cuda.synchronize()
    assert f32_bits(a.item()) == f32_bits(Q.tensor_amax(F.bf16_bits_to_f32(x)[:, 64:192]))


def test_rht16_values():
    x = inputs.gradients((1040, 136), cfg_seed=39)
    y = api.rht16(dev(x), SIGNS)
    torch.cuda.synchronize()
    want = rht16_cols(F.bf16_bits_to_f32(x), SIGNS)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt,block", [("nvfp4", "1d"), ("ue5m3", "1d"), ("mxfp4", "1d"),
                                       ("nvfp4", "2d"), ("ue5m3", "2d")])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dequantize(fmt, block, out):
    x = inputs.gradients((272, 320), cfg_seed=40)
    q = api.quantize(dev(x), fmt, block=block, rnd="rne")
    d = api.dequantize(q, out)
    torch.cuda.synchronize()
    r = Q.quantize(x, fmt, block=block)
    want = Q.dequantize(r["codes"], r["scales"], fmt, block, r["s_dec"], 272, 320,
                        out="f32" if out == torch.float32 else "bf16")
    got = d.cpu()
    got = got.numpy().view(np.uint32) if out == torch.float32 else got.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want.view(np.uint32) if out == torch.float32 else want)


# ------------------------------------------------- full-size workloads ----
def _slabs(n, k, rng):
    starts = np.concatenate([[0, n - k], rng.integers(0, n - k, 6)]) // 16 * 16
    return [(int(a), int(a) + k) for a in np.unique(starts)]


def _check_rows(q, x_bits, fmt, block="1d", rnd="rne", seed=1, offset=0, target=448.0,
                amax=None, orient="row", rht=False, rng=None):
    """Compare 32-row slabs of the output code matrix of a full-size run."""
    for a, b in _slabs(q.rows, 32, rng):
        xs = x_bits[a:b] if orient == "row" else x_bits[:, a:b]
        r = Q.quantize(xs, fmt, block=block, orient=orient, rnd=rnd, seed=seed, offset=offset,
                       rht=rht, signs=SIGNS if rht else 0, target=target, amax=amax,
                       index_base=a * q.cols, emit_transpose=(block == "2d"))
        assert np.array_equal(q.codes[a:b].cpu().numpy(), r["codes"]), (a, b)
        sc = q.scales[a // 16:b // 16] if block == "2d" else q.scales[a:b]
        assert np.array_equal(sc.cpu().numpy(), r["scales"]), (a, b)
        if block == "2d":
            # columns a..b of W: their W^T codes come from the same tiles
            rc = Q.quantize(x_bits[:, a:b], fmt, block="2d", amax=amax, emit_transpose=True)
            assert np.array_equal(q.codes_t[a:b].cpu().numpy(), rc["codes_t"]), (a, b)


def _stale_amax(name, shape):
    gen = {"X": inputs.activations, "W": inputs.weights, "dY": inputs.gradients}[name]
    stale = gen(shape, cfg_seed=inputs.STALE_SEED_OFFSET)
    return np.float32(Q.tensor_amax(F.bf16_bits_to_f32(stale)) / np.float32(1.5))


FMT = {2: "nvfp4", 3: "nvfp4", 4: "ue5m3", 5: "mxfp4"}


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
@pytest.mark.parametrize("name", ["X", "W", "dY"])
def test_workload_1d(cfg, name):
    """Every 1D quantization the workload's Fprop/Dgrad/Wgrad consume."""
    fmt = FMT[cfg]
    xb = inputs.linear_tensors(cfg, which=(name,))[name]
    rng = np.random.default_rng(cfg)
    xd = dev(xb)
    xf = F.bf16_bits_to_f32(xb)
    orients = ("row", "col")
    if name == "W" and fmt != "mxfp4":
        orients = ()                    # two-level weights use 2D blocks
    for orient in orients:
        rnd = "sr" if name == "dY" else "rne"
        offset = 0 if orient == "row" else 1
        rht = cfg == 3 and orient == "col"
        target, amax = 448.0, None
        if fmt == "ue5m3":
            target = 2048.0 if name == "dY" else 448.0
            amax = _stale_amax(name, xb.shape)
        amax_dev = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
        q = api.quantize(xd, fmt, orient=orient, rnd=rnd, seed=1, offset=offset, rht=rht,
                         signs=SIGNS if rht else 0, target=target, amax_in=amax_dev)
        # the same quantization with TILED scales: identical codes, same scale values
        qt = api.quantize(xd, fmt, orient=orient, rnd=rnd, seed=1, offset=offset, rht=rht,
                          signs=SIGNS if rht else 0, target=target, amax_in=amax_dev,
                          scale_layout="tiled")
        torch.cuda.synchronize()
        assert torch.equal(q.codes, qt.codes), (name, orient)
        assert np.array_equal(gpu_scales(qt), q.scales.cpu().numpy()), (name, orient)
        del qt
        want = None
        if fmt != "mxfp4":
            want = amax if amax is not None else Q.tensor_amax(rht16_cols(xf, SIGNS) if rht else xf)
            assert f32_bits(q.amax.item()) == f32_bits(want), (name, orient)
            assert f32_bits(q.s_dec.item()) == f32_bits(Q.global_scales(want, target)[1])
        _check_rows(q, xb, fmt, rnd=rnd, offset=offset, target=target, amax=want,
                    orient=orient, rht=rht, rng=rng)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_workload_2d_weights(cfg):
    fmt = FMT[cfg]
    xb = inputs.linear_tensors(cfg, which=("W",))["W"]
    rng = np.random.default_rng(cfg)
    amax = _stale_amax("W", xb.shape) if fmt == "ue5m3" else None
    amax_dev = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    cnt = api.new_counters()
    q = api.quantize(dev(xb), fmt, block="2d", emit_transpose=True, amax_in=amax_dev, counters=cnt)
    torch.cuda.synchronize()
    want = amax if amax is not None else Q.tensor_amax(F.bf16_bits_to_f32(xb))
    assert f32_bits(q.amax.item()) == f32_bits(want)
    _check_rows(q, xb, fmt, block="2d", amax=want, rng=rng)
    if cfg == 4:
        # the UE5M3 workload counts events: compare the whole tensor's counters
        assert api.counters_dict(cnt) == Q.quantize(xb, fmt, block="2d", amax=want)["counters"]


@pytest.mark.parametrize("T", [448.0, 2048.0])
def test_workload4_counters_slab(T):
    """UE5M3 with a stale amax: event counters of a 512-row slab of dY (SR)
    and of X, quantized as their own tensors with the full tensors' stale amax."""
    t = inputs.linear_tensors(4, which=("X", "dY"))
    for name, rnd in (("X", "rne"), ("dY", "sr")):
        xb = t[name][1024:1536]
        amax = _stale_amax(name, t[name].shape)
        q, r, c = run_both(xb, "ue5m3", rnd=rnd, target=T, stale=amax)
        assert_same(q, r, c)
        assert c["scale_saturated"] == 0          # UE5M3 range absorbs the stale amax


# ------------------------------------------------ RHT sizes N = 4 ... 128 --
@pytest.mark.parametrize("n", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("fmt,rnd", [("nvfp4", "rne"), ("nvfp4", "sr"), ("ue5m3", "rne")])
def test_colwise_rht_sizes(n, fmt, rnd):
    """Colwise quantization with the N-point RHT, the tensor amax taken in
    the rotated space by the library (N = 16 by its own kernel, the other
    sizes by the colwise kernel's amax mode): everything bit-exact."""
    rows = 384 if n == 128 else 320        # whole 128-row tiles, or 2 tiles + a 64-row tile
    x = inputs.gradients((rows, 200), cfg_seed=44) if rnd == "sr" else \
        inputs.activations((rows, 200), cfg_seed=44)
    signs = inputs.rht_sign_bits(n)
    cnt = api.new_counters()
    q = api.quantize(dev(x), fmt, orient="col", rnd=rnd, seed=2, offset=5, rht=True, signs=signs,
                     rht_n=n, counters=cnt)
    torch.cuda.synchronize()
    r = Q.quantize(x, fmt, orient="col", rnd=rnd, seed=2, offset=5, rht=True, signs=signs,
                   rht_n=n)
    assert_same(q, r, api.counters_dict(cnt))


@pytest.mark.parametrize("n,rnd", [(4, "rne"), (32, "sr"), (128, "sr")])
def test_dual_rht_sizes(n, rnd):
    x = inputs.gradients((384, 208), cfg_seed=45)
    signs = inputs.rht_sign_bits(n)
    cnt = api.new_counters()
    qr, qc = api.quantize_dual(dev(x), "nvfp4", rnd=rnd, seed=2, offset=0, offset_t=1, rht=True,
                               signs=signs, rht_n=n, counters=cnt, scale_layout="tiled")
    torch.cuda.synchronize()
    rr = Q.quantize(x, "nvfp4", orient="row", rnd=rnd, seed=2, offset=0)
    rc = Q.quantize(x, "nvfp4", orient="col", rnd=rnd, seed=2, offset=1, rht=True, signs=signs,
                    rht_n=n)
    for q, r in ((qr, rr), (qc, rc)):
        assert np.array_equal(q.codes.cpu().numpy(), r["codes"])
        assert np.array_equal(gpu_scales(q), r["scales"])
        assert f32_bits(q.amax.item()) == f32_bits(r["amax"])
        assert f32_bits(q.s_dec.item()) == f32_bits(r["s_dec"])
    assert api.counters_dict(cnt) == {k: rr["counters"][k] + rc["counters"][k]
                                      for k in rr["counters"]}


# ------------------------- truncation-free scales, stochastic rounding in 2D --
@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
@pytest.mark.parametrize("orient", ["row", "col"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_scale_round_up(fmt, orient, rnd):
    x = inputs.activations((304, 208), cfg_seed=46)      # outliers: nearest scales clip some
    cnt = api.new_counters()
    q = api.quantize(dev(x), fmt, orient=orient, rnd=rnd, seed=3, offset=2, counters=cnt,
                     scale_round="up", scale_layout="tiled")
    torch.cuda.synchronize()
    r = Q.quantize(x, fmt, orient=orient, rnd=rnd, seed=3, offset=2, scale_round="up")
    assert_same(q, r, api.counters_dict(cnt))
    assert r["counters"]["elem_saturated"] == 0


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
@pytest.mark.parametrize("scale_round", ["rne", "up"])
def test_2d_stochastic_rounding(fmt, scale_round):
    """16x16 blocks with SR (2D-block FP4 page): W and W^T codes are exact
    transposes, every output bit-exact with the oracle."""
    w = inputs.gradients((336, 208), cfg_seed=47)         # several 64 x 64 regions + a ragged one
    cnt = api.new_counters()
    q = api.quantize(dev(w), fmt, block="2d", rnd="sr", seed=5, offset=7, emit_transpose=True,
                     counters=cnt, scale_round=scale_round)
    torch.cuda.synchronize()
    r = Q.quantize(w, fmt, block="2d", rnd="sr", seed=5, offset=7, emit_transpose=True,
                   scale_round=scale_round)
    assert_same(q, r, api.counters_dict(cnt))


def test_dual_scale_round_up():
    x = inputs.gradients((256, 192), cfg_seed=48)
    cnt = api.new_counters()
    qr, qc = api.quantize_dual(dev(x), "nvfp4", rnd="sr", seed=4, offset=0, offset_t=1,
                               counters=cnt, scale_round="up")
    torch.cuda.synchronize()
    rr = Q.quantize(x, "nvfp4", orient="row", rnd="sr", seed=4, offset=0, scale_round="up")
    rc = Q.quantize(x, "nvfp4", orient="col", rnd="sr", seed=4, offset=1, scale_round="up")
    for q, r in ((qr, rr), (qc, rc)):
        assert np.array_equal(q.codes.cpu().numpy(), r["codes"])
        assert np.array_equal(q.scales.cpu().numpy(), r["scales"])
    assert api.counters_dict(cnt) == {k: rr["counters"][k] + rc["counters"][k]
                                      for k in rr["counters"]}


# -------------------------------------- whole tensors at full size ----
@pytest.mark.parametrize("cfg,name", [(2, "dY"), (4, "X"), (5, "X")])
def test_workload_whole_tensor(cfg, name):
    """One full-size rowwise quantization per format, compared whole: every
    code, every scale and the five event counters (NVFP4: the 1.2B dY with
    stochastic rounding; UE5M3: the 8B X with its stale amax; MXFP4: the 8B
    X), in the TILED scale layout the GEMMs read."""
    fmt = FMT[cfg]
    xb = inputs.linear_tensors(cfg, which=(name,))[name]
    rnd = "sr" if name == "dY" else "rne"
    amax = _stale_amax(name, xb.shape) if fmt == "ue5m3" else None
    amax_dev = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    cnt = api.new_counters()
    q = api.quantize(dev(xb), fmt, rnd=rnd, seed=1, offset=0, amax_in=amax_dev, counters=cnt,
                     scale_layout="tiled")
    torch.cuda.synchronize()
    r = Q.quantize(xb, fmt, rnd=rnd, seed=1, offset=0, amax=amax)
    assert np.array_equal(q.codes.cpu().numpy(), r["codes"])
    assert np.array_equal(gpu_scales(q), r["scales"])
    assert api.counters_dict(cnt) == r["counters"]
    if fmt != "mxfp4":
        assert f32_bits(q.s_dec.item()) == f32_bits(r["s_dec"])


def test_workload_dual_whole_tensor():
    """The dual quantizer on the whole 1.2B X (both code matrices, scales and
    the summed counters), as the benchmark step runs it."""
    xb = inputs.linear_tensors(2, which=("X",))["X"]
    cnt = api.new_counters()
    qr, qc = api.quantize_dual(dev(xb), "nvfp4", counters=cnt, scale_layout="tiled")
    torch.cuda.synchronize()
    rr = Q.quantize(xb, "nvfp4", orient="row")
    rc = Q.quantize(xb, "nvfp4", orient="col")
    for q, r in ((qr, rr), (qc, rc)):
        assert np.array_equal(q.codes.cpu().numpy(), r["codes"])
        assert np.array_equal(gpu_scales(q), r["scales"])
        assert f32_bits(q.amax.item()) == f32_bits(r["amax"])
    assert api.counters_dict(cnt) == {k: rr["counters"][k] + rc["counters"][k]
                                      for k in rr["counters"]}


# ------------------- RHT along the rows: the Fprop / Dgrad operands ----
from oracle.rht import rht_cols


def _rot(xf, signs, n, orient):
    """The oracle's rotation along the blocked axis of `orient`."""
    return rht_cols(xf, signs, n) if orient == "col" else rht_cols(xf.T, signs, n).T


@pytest.mark.parametrize("n", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("fmt,rnd", [("nvfp4", "rne"), ("nvfp4", "sr"), ("ue5m3", "rne")])
def test_rowwise_rht_sizes(n, fmt, rnd):
    """Rowwise quantization with every N-column group of each row rotated
    (the lanes of a group combine by shuffles for N > 16), the tensor amax
    taken in the rotated space by the library: bit-exact with the oracle."""
    x = inputs.gradients((40, 384), cfg_seed=62) if rnd == "sr" else \
        inputs.activations((40, 384), cfg_seed=62)
    signs = inputs.rht_sign_bits(n)
    cnt = api.new_counters()
    q = api.quantize(dev(x), fmt, orient="row", rnd=rnd, seed=2, offset=5, rht=True, signs=signs,
                     rht_n=n, counters=cnt, scale_layout="tiled")
    torch.cuda.synchronize()
    r = Q.quantize(x, fmt, orient="row", rnd=rnd, seed=2, offset=5, rht=True, signs=signs, rht_n=n)
    assert_same(q, r, api.counters_dict(cnt))


@pytest.mark.parametrize("n", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("orient", ["row", "col"])
def test_rht_alone_and_rotated_amax(n, orient):
    """fp4_rht16 and fp4_amax with every RHT size in both orientations:
    the rotated values bit for bit, and their amax, equal the oracle's."""
    x = inputs.activations((256, 384), cfg_seed=63)
    signs = inputs.rht_sign_bits(n)
    y = api.rht16(dev(x), signs, rht_n=n, orient=orient)
    a = api.amax(dev(x), rht=True, signs=signs, rht_n=n, orient=orient)
    torch.cuda.synchronize()
    want = _rot(F.bf16_bits_to_f32(x), signs, n, orient)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert f32_bits(a.item()) == f32_bits(Q.tensor_amax(want))


@pytest.mark.parametrize("n", [16, 64])
def test_rht_alone_rows_ragged(n):
    """The RHT along rows alone when the last wave of 16-element segments is
    partial (37 x 384: 888 segments, 13.875 waves of 64): every value bit
    for bit as the oracle's, and nothing written past the output (a guard
    row after it stays untouched)."""
    x = inputs.activations((37, 384), cfg_seed=64)
    signs = inputs.rht_sign_bits(n)
    guard = torch.full((38, 384), 7.0, dtype=torch.float32, device=DEV)
    y = api.rht16(dev(x), signs, rht_n=n, orient="row", out=guard[:37])
    torch.cuda.synchronize()
    want = _rot(F.bf16_bits_to_f32(x), signs, n, "row")
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert torch.equal(guard[37].cpu(), torch.full((384,), 7.0))


@pytest.mark.parametrize("n_row,n_col,rnd", [(16, 16, "rne"), (4, 64, "sr"), (16, 128, "sr")])
def test_dual_rht_both_sides(n_row, n_col, rnd):
    """The dual quantizer with the rowwise side rotated along the rows and
    the colwise side along the columns (a linear layer with the RHT on all
    three GEMMs' operands), both amaxes computed by the library."""
    x = inputs.gradients((384, 208), cfg_seed=64)
    sr, sc = inputs.rht_sign_bits(n_row), inputs.rht_sign_bits(n_col)
    cnt = api.new_counters()
    qr, qc = api.quantize_dual(dev(x), "nvfp4", rnd=rnd, seed=2, offset=0, offset_t=1, rht=True,
                               signs=sc, rht_n=n_col, rht_row=True, signs_row=sr,
                               rht_n_row=n_row, counters=cnt, scale_layout="tiled")
    torch.cuda.synchronize()
    rr = Q.quantize(x, "nvfp4", orient="row", rnd=rnd, seed=2, offset=0, rht=True, signs=sr,
                    rht_n=n_row)
    rc = Q.quantize(x, "nvfp4", orient="col", rnd=rnd, seed=2, offset=1, rht=True, signs=sc,
                    rht_n=n_col)
    for q, r in ((qr, rr), (qc, rc)):
        assert np.array_equal(q.codes.cpu().numpy(), r["codes"])
        assert np.array_equal(gpu_scales(q), r["scales"])
        assert f32_bits(q.amax.item()) == f32_bits(r["amax"])
        assert f32_bits(q.s_dec.item()) == f32_bits(r["s_dec"])
    assert api.counters_dict(cnt) == {k: rr["counters"][k] + rc["counters"][k]
                                      for k in rr["counters"]}


@pytest.mark.parametrize("kind", ["row", "col", "dual", "2d", "row_scope"])
@pytest.mark.parametrize("fmt,rnd", [("nvfp4", "rne"), ("ue5m3", "sr")])
def test_count_scales_only(kind, fmt, rnd):
    """count="scales": the same codes and scales as counting everything, the
    block-scale events equal to the oracle's, the element events untouched."""
    x = inputs.gradients((288, 320), cfg_seed=44)
    xd = dev(x)
    kw = dict(rnd=rnd, seed=3)
    names = ("scale_saturated", "scale_underflow", "scale_subnormal")
    if kind == "dual":
        oracle = [Q.quantize(x, fmt, orient="row", **kw),
                  Q.quantize(x, fmt, orient="col", offset=1, **kw)]
        run = lambda c, level: api.quantize_dual(xd, fmt, counters=c, count=level, offset=0, **kw)
    else:
        okw = dict(block="2d") if kind == "2d" else dict(scope="row") if kind == "row_scope" \
            else dict(orient=kind)
        gkw = dict(block="2d", emit_transpose=True) if kind == "2d" else \
            dict(global_scope="row") if kind == "row_scope" else dict(orient=kind)
        oracle = [Q.quantize(x, fmt, **okw, **kw)]
        run = lambda c, level: api.quantize(xd, fmt, counters=c, count=level, **gkw, **kw)
    c_all, c_sc = api.new_counters(), api.new_counters()
    c_sc.fill_(7)                          # element fields must stay as they were
    r_all, r_sc = run(c_all, "all"), run(c_sc, "scales")
    torch.cuda.synchronize()
    for a, b in zip(r_all if isinstance(r_all, tuple) else (r_all,),
                    r_sc if isinstance(r_sc, tuple) else (r_sc,)):
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    got = api.counters_dict(c_sc)
    for k in names:
        assert got[k] == 7 + sum(o["counters"][k] for o in oracle), k
    assert got["elem_saturated"] == 7 and got["elem_underflow"] == 7
    assert api.counters_dict(c_all) == {k: sum(o["counters"][k] for o in oracle)
                                        for k in api.COUNTER_NAMES}
