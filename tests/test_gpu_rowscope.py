"""GPU parity of the per-row global scale (NVFP4 paper App. B.1, closing
remark: the global scale may span a row instead of the tensor, so the amax
needs no pass of its own) against the oracle's scope="row".

Quantizer (fp4_quantize, global_scope ROW): codes, scales, the per-row amax
and s_dec arrays, and the event counters bit-exact for NVFP4 and UE5M3, RNE
and SR, without and with a rowwise RHT (N = 4, 16, 64), row-major and TILED
scales; row lengths reach every register tiling of the kernels (a wave per
row with 1, 2 or 4 blocks per lane; a workgroup per row with 2, 4 or 8 per
thread) and rows longer than that (read in two sweeps); ragged
row counts; rows spread over 40 binades, a zero row and a one-element row;
given (stale) per-row amaxes; rows without columns.  Full size: X and dY of
the 8B FFN workload, whole amax / s_dec arrays and sampled 32-row slabs.
Dequantize with per-row s_dec: bit-exact.  GEMM with per-row s_dec on A, on
B or on both, register-staged and DMA kernels, accumulation, and Fprop at
the 8B shape on sampled entries: within 1e-5 s_A[m] s_B[n] sum_k |a b|.
"""
import numpy as np
import pytest
import torch

from fp4_block_scaled_x16_amd import api, inputs
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from scale_layout import untile

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5
TARGET = {"nvfp4": 448.0, "ue5m3": 2048.0}


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def u32(a):
    return np.asarray(a, np.float32).view(np.uint32)


def spread_rows(R, C, cfg_seed):
    """bf16 bits of [R, C]: row r is N(0, 1) * 2^(2 (r mod 21) - 20); row 1 is
    zero and row 2 holds one nonzero element (when R > 2)."""
    v = F.bf16_bits_to_f32(inputs.normal((R, C), cfg_seed=cfg_seed))
    v = v * np.exp2(2.0 * (np.arange(R) % 21) - 20.0).astype(np.float32)[:, None]
    if R > 2:
        v[1] = 0.0
        v[2] = 0.0
        v[2, C // 3] = -3.25
    return inputs.to_bf16_bits(v.astype(np.float32))


def gpu_scales(q):
    s = q.scales.cpu().numpy()
    if q.scale_layout == api.SCALES_TILED:
        return untile(s, q.rows, q.cols // 16)
    return s


def run(x, fmt, rnd, n, layout="rowmajor", amax=None, seed=3, offset=1):
    cnt = api.new_counters()
    signs = inputs.rht_sign_bits(n) if n else 0
    amax_in = None if amax is None else torch.from_numpy(np.asarray(amax, np.float32)).to(DEV)
    q = api.quantize(dev(x), fmt, rnd=rnd, seed=seed, offset=offset, rht=bool(n), signs=signs,
                     rht_n=n or 16, target=TARGET[fmt], amax_in=amax_in, counters=cnt,
                     scale_layout=layout, global_scope="row")
    torch.cuda.synchronize()
    r = Q.quantize(x, fmt, rnd=rnd, seed=seed, offset=offset, rht=bool(n), signs=signs,
                   rht_n=n or 16, target=TARGET[fmt], amax=amax, scope="row")
    return q, r, api.counters_dict(cnt)


def assert_same(q, r, cnt):
    assert np.array_equal(q.codes.cpu().numpy(), r["codes"]), "codes differ"
    assert np.array_equal(gpu_scales(q), r["scales"]), "scales differ"
    assert np.array_equal(u32(q.amax.cpu().numpy()), u32(r["amax"])), "amax differs"
    assert np.array_equal(u32(q.s_dec.cpu().numpy()), u32(r["s_dec"])), "s_dec differs"
    assert cnt == r["counters"], "counters differ"


CASES = [
    # fmt, rounding, RHT size (0: none), rows, cols, scale layout
    ("nvfp4", "rne", 0, 37, 64, "rowmajor"),        # 1 block per thread, most idle
    ("nvfp4", "sr", 0, 19, 4112, "tiled"),          # 257 blocks: workgroup, 2 per thread
    ("ue5m3", "rne", 0, 9, 16000, "rowmajor"),      # 4 per thread
    ("ue5m3", "sr", 0, 5, 21504, "tiled"),          # 8 per thread (the 8B dY row)
    ("nvfp4", "rne", 0, 3, 33600, "rowmajor"),      # 2100 blocks: two sweeps
    ("nvfp4", "sr", 16, 3, 33600, "tiled"),         # two sweeps with the RHT
    ("nvfp4", "rne", 16, 33, 4096, "rowmajor"),
    ("ue5m3", "sr", 4, 17, 2048, "rowmajor"),
    ("nvfp4", "rne", 64, 12, 1024, "tiled"),        # N / 16 = 4 lanes per group
    ("ue5m3", "rne", 0, 300, 128, "rowmajor"),      # 300 short rows
]


@pytest.mark.parametrize("fmt,rnd,n,R,C,layout", CASES)
def test_row_scope_quantize(fmt, rnd, n, R, C, layout):
    x = spread_rows(R, C, cfg_seed=R + C)
    assert_same(*run(x, fmt, rnd, n, layout))


@pytest.mark.parametrize("fmt,rnd,n,R,C", [("nvfp4", "rne", 0, 5000, 96),
                                            ("ue5m3", "sr", 0, 5000, 96),
                                            ("ue5m3", "rne", 0, 3000, 4096),
                                            ("nvfp4", "sr", 16, 1200, 2048),
                                            ("nvfp4", "rne", 0, 2500, 4608)])
def test_row_scope_many_rows(fmt, rnd, n, R, C):
    """More rows than resident waves / workgroups: each walks several rows,
    the wave kernel loading the next row while it encodes the current one."""
    x = spread_rows(R, C, cfg_seed=7)
    assert_same(*run(x, fmt, rnd, n))


@pytest.mark.parametrize("fmt,rnd,C", [("nvfp4", "rne", 256), ("ue5m3", "sr", 33600)])
def test_row_scope_given_amax(fmt, rnd, C):
    """Given (stale) per-row amaxes: 1.5x the row amaxes of another tensor, so
    some blocks saturate; the row is then read once even when it does not fit
    the registers."""
    x = spread_rows(21, C, cfg_seed=31)
    other = F.bf16_bits_to_f32(spread_rows(21, C, cfg_seed=32))
    stale = (Q.row_amax(other) * np.float32(1.5)).astype(np.float32)
    stale[5] = np.float32(0.0)                    # a zero amax: s_enc = 1
    q, r, cnt = run(x, fmt, rnd, 0, amax=stale)
    assert_same(q, r, cnt)
    assert np.array_equal(u32(q.amax.cpu().numpy()), u32(stale))     # read, not written


def test_row_scope_rows_without_columns():
    q = api.quantize(torch.zeros((7, 0), dtype=torch.int16, device=DEV), "nvfp4",
                     global_scope="row")
    torch.cuda.synchronize()
    assert np.all(q.amax.cpu().numpy() == 0.0) and np.all(q.s_dec.cpu().numpy() == 1.0)


@pytest.mark.parametrize("fmt", ["nvfp4", "ue5m3"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_row_scope_dequantize(fmt, out):
    x = spread_rows(45, 320, cfg_seed=41)
    q = api.quantize(dev(x), fmt, target=TARGET[fmt], global_scope="row")
    d = api.dequantize(q, out)
    torch.cuda.synchronize()
    r = Q.quantize(x, fmt, target=TARGET[fmt], scope="row")
    want = Q.dequantize(r["codes"], r["scales"], fmt, "1d", r["s_dec"], 45, 320,
                        out="f32" if out == torch.float32 else "bf16")
    got = d.cpu()
    if out == torch.float32:
        assert np.array_equal(got.numpy().view(np.uint32), want.view(np.uint32))
    else:
        assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), want)


# ------------------------------------------------------------- full size --
@pytest.mark.parametrize("name", ["X", "dY"])
def test_row_scope_workload(name):
    """The 8B FFN workload's X [8192, 4096] (RNE) and dY [8192, 21504] (SR),
    rowwise with per-row scales: the whole amax and s_dec arrays, then
    sampled 32-row slabs (each row is its own tensor, so a slab is exact)."""
    fmt, rnd = "ue5m3", ("sr" if name == "dY" else "rne")
    xb = inputs.linear_tensors(4, which=(name,))[name]
    R, C = xb.shape
    q = api.quantize(dev(xb), fmt, rnd=rnd, seed=1, target=TARGET[fmt], global_scope="row",
                     scale_layout="tiled")
    torch.cuda.synchronize()
    am = Q.row_amax(F.bf16_bits_to_f32(xb))
    assert np.array_equal(u32(q.amax.cpu().numpy()), u32(am))
    want_sdec = np.array([Q.global_scales(a, TARGET[fmt])[1] for a in am], np.float32)
    assert np.array_equal(u32(q.s_dec.cpu().numpy()), u32(want_sdec))
    codes = q.codes.cpu().numpy()
    scales = untile(q.scales.cpu().numpy(), R, C // 16)
    rng = np.random.default_rng(4)
    for a in sorted({0, R - 32, *(int(v) // 16 * 16 for v in rng.integers(0, R - 32, 5))}):
        r = Q.quantize(xb[a:a + 32], fmt, rnd=rnd, seed=1, target=TARGET[fmt], scope="row",
                       index_base=a * C)
        assert np.array_equal(codes[a:a + 32], r["codes"]), a
        assert np.array_equal(scales[a:a + 32], r["scales"]), a


# ------------------------------------------------------------------ GEMM --
def check(d_gpu, ref, bound):
    err = np.abs(d_gpu.astype(np.float64) - ref.astype(np.float64))
    bad = err > TOL * bound
    assert not bad.any(), "max err/bound %.3g at %s" % (
        float((err / np.maximum(bound, 1e-300)).max()), np.argwhere(bad)[:5].tolist())


def operand(bits, fmt, scope, layout="rowmajor"):
    """(GPU Quantized, oracle values, oracle s_dec) of a rowwise 1D operand."""
    q = api.quantize(dev(bits), fmt, target=TARGET[fmt], global_scope=scope,
                     scale_layout=layout)
    r = Q.quantize(bits, fmt, target=TARGET[fmt], scope=scope)
    R, Ch = r["codes"].shape
    return q, Q.operand_values(r["codes"], r["scales"], fmt, "1d", R, 2 * Ch), r["s_dec"]


GEMM_CASES = [
    # fmt, scope of A, scope of B, M, N, K (K % 512 == 0 -> DMA kernel)
    ("nvfp4", "row", "row", 600, 520, 208),
    ("nvfp4", "row", "tensor", 300, 264, 512),
    ("nvfp4", "tensor", "row", 272, 300, 1024),
    ("ue5m3", "row", "row", 520, 272, 512),
    ("ue5m3", "row", "tensor", 130, 70, 48),
    ("ue5m3", "tensor", "row", 256, 516, 256),
]


@pytest.mark.parametrize("fmt,sa,sb,M,N,K", GEMM_CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_row_scope_gemm(fmt, sa, sb, M, N, K, accumulate):
    a_bits = spread_rows(M, K, cfg_seed=M)
    b_bits = spread_rows(N, K, cfg_seed=N + 1)
    qa, av, s_a = operand(a_bits, fmt, sa, layout="tiled")
    qb, bv, s_b = operand(b_bits, fmt, sb)
    init = torch.randn((M, N), dtype=torch.float32, device=DEV) if accumulate else None
    d0 = init.cpu().numpy().astype(np.float64) if accumulate else 0.0
    out = init.clone() if accumulate else None
    d = api.gemm(qa.operand(), qb.operand(), M, N, K, out=out, accumulate=accumulate,
                 device=DEV)
    torch.cuda.synchronize()
    ref = G.gemm_ref(av, bv, s_a, s_b).astype(np.float64) + d0
    bound = G.gemm_abs_bound(av, bv, s_a, s_b) + np.abs(d0)
    check(d.cpu().numpy(), ref, bound)


def test_row_scope_fprop_8b_sampled():
    """Fprop of the 8B FFN shape (M = 8192 tokens, N = 21504, K = 4096) with
    per-row scales on X and on the rowwise W: a grid of sampled entries,
    the oracle quantizing only the rows they need (each row is its own
    tensor under per-row scales)."""
    fmt = "ue5m3"
    t = inputs.linear_tensors(4, which=("X", "W"))
    xb, wb = t["X"], t["W"]
    M, K = xb.shape
    N = wb.shape[0]
    qx = api.quantize(dev(xb), fmt, target=TARGET[fmt], global_scope="row", scale_layout="tiled")
    qw = api.quantize(dev(wb), fmt, target=TARGET[fmt], global_scope="row", scale_layout="tiled")
    d = api.gemm(qx.operand(), qw.operand(), M, N, K, device=DEV)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 14)]))
    ra = Q.quantize(xb[rows], fmt, target=TARGET[fmt], scope="row")
    rb = Q.quantize(wb[cols], fmt, target=TARGET[fmt], scope="row")
    av = Q.operand_values(ra["codes"], ra["scales"], fmt, "1d", len(rows), K)
    bv = Q.operand_values(rb["codes"], rb["scales"], fmt, "1d", len(cols), K)
    ref = G.gemm_ref(av, bv, ra["s_dec"], rb["s_dec"])
    bound = G.gemm_abs_bound(av, bv, ra["s_dec"], rb["s_dec"])
    got = d[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
    check(got, ref, bound)
