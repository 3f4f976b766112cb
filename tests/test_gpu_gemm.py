"""GPU parity of fp4_gemm against the CPU oracle.

Bar: |D_gpu - D_ref| <= 1e-5 * s_A * s_B * sum_k |a b| per element, where
D_ref is the oracle's fp64 GEMM of the oracle's own quantized operands.
Small cases cover several 256 x 256 output tiles, ragged M and N, K steps
with partial tails, every operand layout (1D, 2D weights, transposed 2D
weights), accumulation and K = 0.  Full-size cases run each workload's
Fprop / Dgrad / Wgrad at its real shape and check a grid of sampled entries,
for which the oracle quantizes only the rows the entries need.
"""
import numpy as np
import pytest
import torch

from fp4_block_scaled_x16_amd import api, inputs
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from bf16_check import bf16_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5
SIGNS = inputs.rht_sign_mask()


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def check(d_gpu, ref, bound):
    d = d_gpu.astype(np.float64)
    err = np.abs(d - ref.astype(np.float64))
    bad = err > TOL * bound
    assert not bad.any(), "max err/bound %.3g at %s" % (
        float((err / np.maximum(bound, 1e-300)).max()), np.argwhere(bad)[:5].tolist())


def oracle_operand(bits, fmt, layout, **kw):
    """Oracle values (float64, no tensor scale) of a GEMM operand and its s_dec.

    layout: "row" (1D, K along cols), "col" (1D of X^T), "2d" (W), "2dT" (W^T).
    """
    if layout in ("row", "col"):
        q = Q.quantize(bits, fmt, orient=layout, **kw)
        R, Cc = q["codes"].shape
        return Q.operand_values(q["codes"], q["scales"], fmt, "1d", R, 2 * Cc), q["s_dec"]
    q = Q.quantize(bits, fmt, block="2d", emit_transpose=True, **kw)
    R, C = bits.shape
    vals = Q.operand_values(q["codes"], q["scales"], fmt, "2d", R, C)
    return (vals if layout == "2d" else vals.T.copy()), q["s_dec"]


def gpu_operand(q, layout):
    return q.operand(transposed=(layout == "2dT"))


def gpu_quant(bits, fmt, layout, scales="rowmajor", **kw):
    if layout in ("row", "col"):
        return api.quantize(dev(bits), fmt, orient=layout, scale_layout=scales, **kw)
    return api.quantize(dev(bits), fmt, block="2d", emit_transpose=True, **kw)


CASES = [
    # fmt, A layout, B layout, M, N, K
    ("nvfp4", "row", "row", 600, 520, 208),
    ("nvfp4", "row", "2d", 300, 528, 400),
    ("nvfp4", "row", "2dT", 272, 336, 528),
    ("ue5m3", "row", "2d", 520, 272, 272),
    ("ue5m3", "row", "2dT", 256, 256, 256),
    ("ue5m3", "row", "row", 130, 70, 48),
    ("mxfp4", "row", "row", 600, 520, 224),
    ("mxfp4", "row", "row", 33, 17, 32),
    ("nvfp4", "col", "col", 512, 264, 304),
    # NVFP4 with K a multiple of 256: codes by DMA, ragged tiles with clamped
    # rows, every scale-loader variant (contiguous / strided for A and B)
    ("nvfp4", "row", "row", 300, 264, 512),
    ("nvfp4", "row", "2dT", 272, 336, 512),
    ("nvfp4", "2dT", "row", 336, 280, 768),
    ("nvfp4", "2dT", "2dT", 272, 304, 256),
    # ... tile height: shapes that fill at most one round of the CUs take
    # 192-row tiles (all of the above); this one has 192 256-row tiles but
    # 264 192-row tiles, so on a 256-CU device it takes 256-row tiles
    ("nvfp4", "row", "row", 2048, 6144, 256),
    # MXFP4 with K a multiple of 512: the LDS-DMA ring kernel (one turn of
    # the ring only, ragged tiles with clamped rows, several turns)
    ("mxfp4", "row", "row", 300, 264, 512),
    ("mxfp4", "col", "col", 520, 264, 1024),
    ("mxfp4", "row", "row", 256, 512, 2048),
]


TILED_CASES = [
    # fmt, A layout, B layout, M, N, K, A scales, B scales
    ("nvfp4", "row", "row", 600, 520, 208, "tiled", "tiled"),     # ragged, partial K step
    ("nvfp4", "row", "2d", 512, 512, 512, "tiled", "rowmajor"),   # tile-aligned loader
    ("ue5m3", "row", "row", 256, 512, 1024, "tiled", "tiled"),
    ("mxfp4", "row", "row", 600, 520, 224, "tiled", "tiled"),     # register-staged MXFP4
    ("mxfp4", "row", "col", 300, 264, 512, "tiled", "rowmajor"),  # DMA ring, mixed layouts
    ("mxfp4", "row", "row", 300, 264, 512, "tiled", "tiled"),     # K-256 kernel, 2 steps
    ("mxfp4", "col", "col", 520, 264, 1024, "tiled", "tiled"),    # ... one loop turn
    ("mxfp4", "row", "row", 256, 512, 2048, "tiled", "tiled"),    # ... several turns
]


@pytest.mark.parametrize("fmt,la,lb,M,N,K,sa_layout,sb_layout", TILED_CASES)
def test_gemm_tiled_scales(fmt, la, lb, M, N, K, sa_layout, sb_layout):
    a_shape = (M, K) if la == "row" else (K, M)
    a_bits = inputs.activations(a_shape, cfg_seed=53)
    b_bits = inputs.weights((N, K), cfg_seed=53) if lb in ("row", "2d") else \
        inputs.gradients((K, N), cfg_seed=53)
    qa = gpu_quant(a_bits, fmt, la, scales=sa_layout)
    qb = gpu_quant(b_bits, fmt, lb, scales=sb_layout)
    d = api.gemm(gpu_operand(qa, la), gpu_operand(qb, lb), M, N, K, device=DEV)
    torch.cuda.synchronize()
    av, sa = oracle_operand(a_bits, fmt, la)
    bv, sb = oracle_operand(b_bits, fmt, lb)
    if fmt == "mxfp4":
        sa = sb = 1.0
    check(d.cpu().numpy(), G.gemm_ref(av, bv, sa, sb), G.gemm_abs_bound(av, bv, sa, sb))


@pytest.mark.parametrize("fmt,la,lb,M,N,K", CASES)
def test_gemm_small(fmt, la, lb, M, N, K):
    # A operand [M, K]; B operand [N, K] (for 2dT, W is [K, N])
    a_shape = (M, K) if la == "row" else (K, M)
    a_bits = (inputs.weights(a_shape, cfg_seed=50) if la.startswith("2d")
              else inputs.activations(a_shape, cfg_seed=50))
    if lb == "row":
        b_bits = inputs.weights((N, K), cfg_seed=50)
    elif lb == "col":
        b_bits = inputs.gradients((K, N), cfg_seed=50)
    elif lb == "2d":
        b_bits = inputs.weights((N, K), cfg_seed=50)
    else:
        b_bits = inputs.weights((K, N), cfg_seed=50)
    qa = gpu_quant(a_bits, fmt, la)
    qb = gpu_quant(b_bits, fmt, lb)
    d = api.gemm(gpu_operand(qa, la), gpu_operand(qb, lb), M, N, K, device=DEV)
    torch.cuda.synchronize()
    av, sa = oracle_operand(a_bits, fmt, la)
    bv, sb = oracle_operand(b_bits, fmt, lb)
    if fmt == "mxfp4":
        sa = sb = 1.0
    assert av.shape == (M, K) and bv.shape == (N, K)
    check(d.cpu().numpy(), G.gemm_ref(av, bv, sa, sb), G.gemm_abs_bound(av, bv, sa, sb))


@pytest.mark.parametrize("fmt,K", [("nvfp4", 256), ("mxfp4", 256), ("mxfp4", 512)])
def test_gemm_accumulate_and_ldd(fmt, K):
    M, N = 280, 300
    a_bits = inputs.activations((M, K), cfg_seed=51)
    b_bits = inputs.weights((N, K), cfg_seed=51)
    qa, qb = gpu_quant(a_bits, fmt, "row"), gpu_quant(b_bits, fmt, "row")
    big = torch.randn((M, N + 24), dtype=torch.float32, device=DEV)
    init = big.clone()
    out = big[:, 8:8 + N]                       # ldd = N + 24, offset view
    api.gemm(qa.operand(), qb.operand(), M, N, K, out=out, accumulate=True)
    torch.cuda.synchronize()
    av, sa = oracle_operand(a_bits, fmt, "row")
    bv, sb = oracle_operand(b_bits, fmt, "row")
    if fmt == "mxfp4":
        sa = sb = 1.0
    ref = G.gemm_ref(av, bv, sa, sb).astype(np.float64) + init[:, 8:8 + N].cpu().numpy()
    bound = G.gemm_abs_bound(av, bv, sa, sb) + np.abs(init[:, 8:8 + N].cpu().numpy())
    got = big.cpu().numpy()
    check(got[:, 8:8 + N], ref, bound)
    # columns outside the view are untouched
    assert torch.equal(big[:, :8].cpu(), init[:, :8].cpu())
    assert torch.equal(big[:, 8 + N:].cpu(), init[:, 8 + N:].cpu())


@pytest.mark.parametrize("view", ["aligned", "odd_pitch", "misaligned"])
@pytest.mark.parametrize("kind", ["fp32", "bf16", "fp32_accumulate"])
@pytest.mark.parametrize("tile_rows", [192, 256])
def test_gemm_epilogue_layouts(tile_rows, kind, view):
    """The DMA GEMM's epilogue stages whole 32 x 32 blocks through LDS when a
    wave's part of the tile lies inside D with aligned rows (a plain fp32 D;
    on 192-row tiles also a bf16 D and accumulation), else it stores lane by
    lane.  Output views with aligned rows, with an odd row pitch, and
    starting one element past an aligned address, on both tile heights
    (some waves of the ragged last tiles outside D), against the oracle;
    the memory around the view is untouched."""
    fmt, M, N, K = "nvfp4", 400, 384, 256
    a_bits = inputs.activations((M, K), cfg_seed=81)
    b_bits = inputs.weights((N, K), cfg_seed=82)
    qa, qb = gpu_quant(a_bits, fmt, "row"), gpu_quant(b_bits, fmt, "row")
    av, sa = oracle_operand(a_bits, fmt, "row")
    bv, sb = oracle_operand(b_bits, fmt, "row")
    ref = G.gemm_ref(av, bv, sa, sb).astype(np.float64)
    bound = G.gemm_abs_bound(av, bv, sa, sb)
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    pitch = N + (9 if view == "odd_pitch" else 32)            # 393: odd
    off = 1 if view == "misaligned" else 8          # 8 elements: 16- (bf16) or 32-byte offset
    big = torch.randn((M, pitch), dtype=torch.float32, device=DEV).to(dt)
    init = big.clone()
    out = big[:, off:off + N]
    accumulate = kind == "fp32_accumulate"
    api.selftest_set_geometry(0, tile_rows)
    try:
        api.gemm(qa.operand(), qb.operand(), M, N, K, out=out, accumulate=accumulate)
        torch.cuda.synchronize()
    finally:
        api.selftest_set_geometry(0, 0)
    if kind == "bf16":
        bf16_close(out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), ref, bound)
    else:
        got = out.cpu().numpy()
        if accumulate:
            d0 = init[:, off:off + N].cpu().numpy().astype(np.float64)
            ref, bound = ref + d0, bound + np.abs(d0)
        check(got, ref, bound)
    assert torch.equal(big[:, :off].cpu(), init[:, :off].cpu())
    assert torch.equal(big[:, off + N:].cpu(), init[:, off + N:].cpu())


def test_gemm_k_zero():
    a = api.quantize(dev(inputs.activations((64, 32), cfg_seed=52)), "nvfp4")
    b = api.quantize(dev(inputs.weights((48, 32), cfg_seed=52)), "nvfp4")
    d = torch.full((64, 48), 7.0, device=DEV)
    api.gemm(a.operand(), b.operand(), 64, 48, 0, out=d)
    torch.cuda.synchronize()
    assert torch.count_nonzero(d).item() == 0
    d.fill_(7.0)
    api.gemm(a.operand(), b.operand(), 64, 48, 0, out=d, accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(d == 7.0).item()


def test_gemm_zero_operand():
    a_bits = np.zeros((64, 128), np.uint16)
    b_bits = inputs.weights((64, 128), cfg_seed=53)
    qa, qb = gpu_quant(a_bits, "nvfp4", "row"), gpu_quant(b_bits, "nvfp4", "row")
    d = api.gemm(qa.operand(), qb.operand(), 64, 64, 128, device=DEV)
    torch.cuda.synchronize()
    assert torch.count_nonzero(d).item() == 0


@pytest.mark.parametrize("fmt,rel", [("ue5m3", 2.0 ** -23), ("nvfp4", 2.0 ** -17)])
def test_gemm_tiny_scales(fmt, rel):
    # Blocks far below the tensor amax get the smallest scales: UE5M3 scales
    # near 2^-17, whose 2^-5-shifted fp16 operands are subnormal; E4M3
    # subnormal scale codes (exponent field 0).  Both must be used exactly.
    rng = np.random.default_rng(54)
    a = (rng.standard_normal((64, 256)) * rel).astype(np.float32)
    a[0, 0] = 1.0
    b = (rng.standard_normal((64, 256)) * rel).astype(np.float32)
    b[0, 0] = 1.0
    a_bits, b_bits = inputs.to_bf16_bits(a), inputs.to_bf16_bits(b)
    qa, qb = gpu_quant(a_bits, fmt, "row"), gpu_quant(b_bits, fmt, "row")
    d = api.gemm(qa.operand(), qb.operand(), 64, 64, 256, device=DEV)
    torch.cuda.synchronize()
    av, sa = oracle_operand(a_bits, fmt, "row")
    bv, sb = oracle_operand(b_bits, fmt, "row")
    if fmt == "ue5m3":
        # premise: many fp16 operands are subnormal, |e2m1 * scale| * 2^-5 < 2^-14
        assert np.count_nonzero((av != 0) & (np.abs(av) * 2.0 ** -5 < 2.0 ** -14)) > 10000
    else:
        # premise: many E4M3 scale codes are subnormal (1..7)
        sc = Q.quantize(a_bits, fmt)["scales"]
        assert np.count_nonzero((sc >= 1) & (sc <= 7)) > 100
    check(d.cpu().numpy(), G.gemm_ref(av, bv, sa, sb), G.gemm_abs_bound(av, bv, sa, sb))


def test_gemm_tiny_workload_config1():
    # 256 x 256 x 256 Fprop of the tiny workload: A 1x16, W 16x16 2D
    t = inputs.linear_tensors(1)
    qa, qw = gpu_quant(t["X"], "nvfp4", "row"), gpu_quant(t["W"], "nvfp4", "2d")
    d = api.gemm(qa.operand(), qw.operand(), 256, 256, 256, device=DEV)
    torch.cuda.synchronize()
    av, sa = oracle_operand(t["X"], "nvfp4", "row")
    wv, sw = oracle_operand(t["W"], "nvfp4", "2d")
    check(d.cpu().numpy(), G.gemm_ref(av, wv, sa, sw), G.gemm_abs_bound(av, wv, sa, sw))


# ------------------------------------------------- full-size workloads ----
def _stale(name, shape):
    gen = {"X": inputs.activations, "W": inputs.weights, "dY": inputs.gradients}[name]
    b = gen(shape, cfg_seed=inputs.STALE_SEED_OFFSET)
    return np.float32(Q.tensor_amax(F.bf16_bits_to_f32(b)) / np.float32(1.5))


def _recipe(cfg, name, layout):
    """quantize() keyword arguments of one operand of a workload."""
    fmt = {2: "nvfp4", 3: "nvfp4", 4: "ue5m3", 5: "mxfp4"}[cfg]
    kw = {}
    if name == "dY":
        kw.update(rnd="sr", seed=1, offset=0 if layout == "row" else 1)
    if cfg == 3 and layout == "col":
        kw.update(rht=True, signs=SIGNS)
    if fmt == "ue5m3":
        kw["target"] = 2048.0 if name == "dY" else 448.0
    return fmt, kw


def _oracle_rows(bits, fmt, layout, sel, kw, amax):
    """Oracle operand values of rows `sel` of the [rows, K] code matrix."""
    out = []
    for r in sel:
        if layout == "row":
            q = Q.quantize(bits[r:r + 1], fmt, amax=amax, index_base=r * bits.shape[1], **kw)
            R, K = 1, bits.shape[1]
            out.append(Q.operand_values(q["codes"], q["scales"], fmt, "1d", R, K)[0])
        elif layout == "col":
            q = Q.quantize(bits[:, r:r + 1], fmt, orient="col", amax=amax,
                           index_base=r * bits.shape[0], **kw)
            out.append(Q.operand_values(q["codes"], q["scales"], fmt, "1d", 1, bits.shape[0])[0])
        elif layout == "2d":
            g = r // 16 * 16
            q = Q.quantize(bits[g:g + 16], fmt, block="2d", amax=amax, **kw)
            out.append(Q.operand_values(q["codes"], q["scales"], fmt, "2d", 16, bits.shape[1])[r - g])
        else:  # 2dT: row r of W^T is column r of W
            g = r // 16 * 16
            q = Q.quantize(bits[:, g:g + 16], fmt, block="2d", amax=amax, **kw)
            vals = Q.operand_values(q["codes"], q["scales"], fmt, "2d", bits.shape[0], 16)
            out.append(vals[:, r - g])
    return np.stack(out)


def _amax_for(bits, fmt, kw, stale):
    if fmt == "mxfp4":
        return None
    if stale is not None:
        return stale
    xf = F.bf16_bits_to_f32(bits)
    if kw.get("rht"):
        from oracle.rht import rht16_cols
        xf = rht16_cols(xf, SIGNS)
    return Q.tensor_amax(xf)


GEMMS = {
    # name: (A tensor, A layout, B tensor, B layout)
    "fprop": ("X", "row", "W", "2d"),
    "dgrad": ("dY", "row", "W", "2dT"),
    "wgrad": ("dY", "col", "X", "col"),
}

_W2D = {}


def _oracle_w2d(cfg, bits, fmt, amax, target):
    """The oracle's 16x16 quantization of a workload's whole W (cached: the
    Fprop and Dgrad cases of both scale layouts read it)."""
    if cfg not in _W2D:
        _W2D.clear()
        _W2D[cfg] = Q.quantize(bits, fmt, block="2d", emit_transpose=True, amax=amax,
                               target=target)
    return _W2D[cfg]


def _oracle_w_rows(q, fmt, layout, sel, R, C):
    """Operand values of rows `sel` of W [R, C] (layout "2d") or of W^T
    (layout "2dT") from the oracle's whole-tensor 2D quantization `q`."""
    out = []
    for r in sel:
        g = r // 16 * 16
        if layout == "2d":
            v = Q.operand_values(q["codes"][g:g + 16], q["scales"][g // 16:g // 16 + 1], fmt,
                                 "2d", 16, C)
        else:   # W^T rows g..g+15 are W's columns; their tile scales are a column of W's
            v = Q.operand_values(q["codes_t"][g:g + 16], q["scales"][:, g // 16:g // 16 + 1].T,
                                 fmt, "2d", 16, R)
        out.append(v[r - g])
    return np.stack(out)


def _one_per_32(n, rng):
    """One index in every group of 32 (every 32 x 32 output sub-tile is
    sampled once rows and columns both come from this), plus both ends."""
    idx = np.arange(0, n, 32) + rng.integers(0, 32, (n + 31) // 32)
    return np.unique(np.concatenate([[0, n - 1], np.minimum(idx, n - 1)]))


@pytest.mark.parametrize("scales", ["rowmajor", "tiled"])
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
@pytest.mark.parametrize("gemm", ["fprop", "dgrad", "wgrad"])
def test_workload_gemm(cfg, gemm, scales):
    """A full-size GEMM of a workload, in the launch configuration the
    benchmark uses: D starts as NaN and must be finite everywhere afterwards
    (every output tile written), and one entry in every 32 x 32 sub-tile is
    checked against the oracle."""
    an, la, bn, lb = GEMMS[gemm]
    fmt = {2: "nvfp4", 3: "nvfp4", 4: "ue5m3", 5: "mxfp4"}[cfg]
    if fmt == "mxfp4":   # MXFP4 weights are 1D: rowwise for Fprop, colwise for Dgrad
        lb = {"2d": "row", "2dT": "col"}.get(lb, lb)
    t = inputs.linear_tensors(cfg, which=(an, bn))
    a_bits, b_bits = t[an], t[bn]
    fa, kwa = _recipe(cfg, an, la)
    fb, kwb = _recipe(cfg, bn, lb)
    sa_stale = _stale(an, a_bits.shape) if fmt == "ue5m3" else None
    sb_stale = _stale(bn, b_bits.shape) if fmt == "ue5m3" else None

    def gq(bits, layout, kw, stale):
        amax_in = None if stale is None else torch.tensor([stale], dtype=torch.float32, device=DEV)
        x = dev(bits)
        if layout in ("2d", "2dT"):
            return api.quantize(x, fmt, block="2d", emit_transpose=True, amax_in=amax_in,
                                target=kw.get("target", 448.0))
        return api.quantize(x, fmt, orient=layout, amax_in=amax_in, scale_layout=scales, **kw)

    qa, qb = gq(a_bits, la, kwa, sa_stale), gq(b_bits, lb, kwb, sb_stale)
    M, K = qa.rows, qa.cols
    N = qb.cols if lb == "2dT" else qb.rows
    d = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    api.gemm(gpu_operand(qa, la), gpu_operand(qb, lb), M, N, K, out=d)
    torch.cuda.synchronize()
    del qa, qb
    assert bool(torch.isfinite(d).all()), "output entries left unwritten"
    rng = np.random.default_rng(100 + cfg)
    rows, cols = _one_per_32(M, rng), _one_per_32(N, rng)
    amax_a = _amax_for(a_bits, fmt, kwa, sa_stale)
    amax_b = _amax_for(b_bits, fmt, kwb, sb_stale)
    av = _oracle_rows(a_bits, fmt, la, rows, kwa, amax_a)
    if lb in ("2d", "2dT"):
        qw = _oracle_w2d(cfg, b_bits, fmt, amax_b, kwb.get("target", 448.0))
        bv = _oracle_w_rows(qw, fmt, lb, cols, *b_bits.shape)
    else:
        bv = _oracle_rows(b_bits, fmt, lb, cols, kwb, amax_b)
    if fmt == "mxfp4":
        sa = sb = 1.0
    else:
        sa = Q.global_scales(amax_a, kwa.get("target", 448.0))[1]
        sb = Q.global_scales(amax_b, kwb.get("target", 448.0))[1]
    ref = G.gemm_ref(av, bv, sa, sb)
    bound = G.gemm_abs_bound(av, bv, sa, sb)
    got = d[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
    check(got, ref, bound)


@pytest.mark.parametrize("fmt,la,lb,M,N,K", [
    ("nvfp4", "row", "row", 300, 264, 512),       # DMA kernel
    ("nvfp4", "row", "row", 130, 70, 48),         # register-staged kernel, ragged N
    ("nvfp4", "row", "2dT", 130, 80, 48),
    ("ue5m3", "row", "2d", 520, 272, 512),
    ("mxfp4", "row", "row", 280, 300, 512),       # scaled-MFMA kernel
    ("mxfp4", "row", "row", 33, 17, 32),
])
@pytest.mark.parametrize("accumulate", [False, True])
def test_gemm_bf16_output(fmt, la, lb, M, N, K, accumulate):
    """NVFP4 paper §4.1: the GEMMs may write BF16.  Each value is the fp32
    result rounded once to bf16 (accumulation adds the old bf16 value in
    fp32 first); ragged N exercises the element-wise stores."""
    a_bits = inputs.activations((M, K), cfg_seed=71)
    b_bits = (inputs.weights((K, N), cfg_seed=72) if lb == "2dT" else
              inputs.weights((N, K), cfg_seed=72) if lb == "2d" else
              inputs.gradients((N, K), cfg_seed=72))
    qa, qb = gpu_quant(a_bits, fmt, la), gpu_quant(b_bits, fmt, lb)
    av, sa = oracle_operand(a_bits, fmt, la)
    bv, sb = oracle_operand(b_bits, fmt, lb)
    if fmt == "mxfp4":
        sa = sb = 1.0
    ref = G.gemm_ref(av, bv, sa, sb).astype(np.float64)
    bound = G.gemm_abs_bound(av, bv, sa, sb)
    init = torch.randn((M, N), dtype=torch.float32, device=DEV).to(torch.bfloat16)
    out = init.clone() if accumulate else torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    api.gemm(gpu_operand(qa, la), gpu_operand(qb, lb), M, N, K, out=out, accumulate=accumulate)
    torch.cuda.synchronize()
    if accumulate:
        d0 = F.bf16_bits_to_f32(init.view(torch.int16).cpu().numpy().view(np.uint16))
        ref = ref + d0.astype(np.float64)
        bound = bound + np.abs(d0)
    bf16_close(out.view(torch.int16).cpu().numpy().view(np.uint16), ref, bound)
