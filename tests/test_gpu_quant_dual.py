"""GPU parity of fp4_quantize_dual, the one-read rowwise + colwise quantizer.

Bar: both outputs bit-exact with the oracle -- the rowwise side with the
oracle's rowwise quantization of X, the colwise side with its colwise
quantization (X^T, optionally RHT-rotated) -- in codes, scales, tensor amax
and s_dec, and the event counters equal to the sum of the two sides'.
Small cases span several 8BS x 64 tiles with ragged tails in both
dimensions; the full-size cases run the workloads' X and dY and compare
sampled slabs of each output with the oracle and the whole outputs with the
single-orientation kernels.
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


def scales_of(q):
    s = q.scales.cpu().numpy()
    if q.scale_layout == api.SCALES_TILED:
        return untile(s, q.rows, q.cols // api.BLOCK_LEN[q.fmt])
    return s


def check_side(q, r):
    assert np.array_equal(q.codes.cpu().numpy(), r["codes"]), "codes differ"
    assert np.array_equal(scales_of(q), r["scales"]), "scales differ"
    if r["amax"] is not None:
        assert f32_bits(q.amax.item()) == f32_bits(r["amax"]), "amax differs"
    assert f32_bits(q.s_dec.item()) == f32_bits(r["s_dec"]), "s_dec differs"


CASES = [
    # fmt, rnd, rht, rows, cols, scale layout
    ("nvfp4", "rne", False, 304, 208, "rowmajor"),   # 2 tiles + 48 rows; 3 tiles + 16 cols
    ("nvfp4", "sr", True, 304, 208, "tiled"),
    ("nvfp4", "rne", True, 128, 64, "rowmajor"),     # exactly one tile
    ("ue5m3", "rne", True, 272, 144, "rowmajor"),
    ("ue5m3", "sr", False, 304, 208, "tiled"),
    ("mxfp4", "rne", False, 320, 224, "rowmajor"),   # 256-row tile + 64; 3 tiles + 32 cols
    ("mxfp4", "sr", False, 320, 224, "tiled"),
    ("nvfp4", "sr", False, 16, 16, "rowmajor"),      # one block each way
]


@pytest.mark.parametrize("fmt,rnd,rht,rows,cols,layout", CASES)
def test_dual_small(fmt, rnd, rht, rows, cols, layout):
    xb = (inputs.gradients((rows, cols), cfg_seed=61) if rnd == "sr"
          else inputs.activations((rows, cols), cfg_seed=61))
    cnt = api.new_counters()
    qr, qc = api.quantize_dual(dev(xb), fmt, rnd=rnd, seed=3, offset=0, offset_t=1, rht=rht,
                               signs=SIGNS if rht else 0, counters=cnt, scale_layout=layout)
    torch.cuda.synchronize()
    rr = Q.quantize(xb, fmt, orient="row", rnd=rnd, seed=3, offset=0)
    rc = Q.quantize(xb, fmt, orient="col", rnd=rnd, seed=3, offset=1, rht=rht,
                    signs=SIGNS if rht else 0)
    check_side(qr, rr)
    check_side(qc, rc)
    want = {k: rr["counters"][k] + rc["counters"][k] for k in rr["counters"]}
    assert api.counters_dict(cnt) == want


@pytest.mark.parametrize("T", [448.0, 2048.0])
def test_dual_stale_amax_shared_buffer(T):
    """UE5M3 with a given (stale) amax passed once for both sides (one
    buffer), so that scales saturate and the counters see it."""
    xb = inputs.activations((256, 192), cfg_seed=62)
    stale = np.float32(Q.tensor_amax(F.bf16_bits_to_f32(xb)) / np.float32(1.5))
    am = torch.tensor([stale], dtype=torch.float32, device=DEV)
    cnt = api.new_counters()
    qr, qc = api.quantize_dual(dev(xb), "ue5m3", target=T, amax_in=am, amax_t_in=am, counters=cnt)
    torch.cuda.synchronize()
    rr = Q.quantize(xb, "ue5m3", orient="row", target=T, amax=stale)
    rc = Q.quantize(xb, "ue5m3", orient="col", target=T, amax=stale)
    check_side(qr, rr)
    check_side(qc, rc)
    assert api.counters_dict(cnt) == {k: rr["counters"][k] + rc["counters"][k]
                                      for k in rr["counters"]}


def test_dual_empty():
    x = dev(np.zeros((16, 64), np.uint16))[:0]
    qr, qc = api.quantize_dual(x, "nvfp4")
    torch.cuda.synchronize()
    assert qr.codes.shape == (0, 32) and qc.codes.shape == (64, 0)
    assert qr.amax.item() == 0.0 and qr.s_dec.item() == 1.0 and qc.s_dec.item() == 1.0


def _slabs(n, k, rng):
    starts = np.concatenate([[0, n - k], rng.integers(0, n - k, 4)]) // 32 * 32
    return [(int(a), int(a) + k) for a in np.unique(starts)]


FMT = {2: "nvfp4", 3: "nvfp4", 4: "ue5m3", 5: "mxfp4"}


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
@pytest.mark.parametrize("name", ["X", "dY"])
def test_dual_workload(cfg, name):
    """The workloads' X and dY in the configuration a step would use (TILED
    scales; SR on dY with offsets 0 / 1; RHT on the colwise side of the 12B
    workload; UE5M3 with a stale amax): equal to the two single-orientation
    kernels everywhere, and to the oracle on sampled 32-row slabs."""
    fmt = FMT[cfg]
    xb = inputs.linear_tensors(cfg, which=(name,))[name]
    rnd = "sr" if name == "dY" else "rne"
    rht = cfg == 3
    target, am = 448.0, None
    if fmt == "ue5m3":
        target = 2048.0 if name == "dY" else 448.0
        gen = {"X": inputs.activations, "dY": inputs.gradients}[name]
        st = gen(xb.shape, cfg_seed=inputs.STALE_SEED_OFFSET)
        am = np.float32(Q.tensor_amax(F.bf16_bits_to_f32(st)) / np.float32(1.5))
    am_dev = None if am is None else torch.tensor([am], dtype=torch.float32, device=DEV)
    xd = dev(xb)
    qr, qc = api.quantize_dual(xd, fmt, rnd=rnd, seed=1, offset=0, offset_t=1, rht=rht,
                               signs=SIGNS if rht else 0, target=target, amax_in=am_dev,
                               amax_t_in=am_dev, scale_layout="tiled")
    sr = api.quantize(xd, fmt, orient="row", rnd=rnd, seed=1, offset=0, target=target,
                      amax_in=am_dev, scale_layout="tiled")
    sc = api.quantize(xd, fmt, orient="col", rnd=rnd, seed=1, offset=1, rht=rht,
                      signs=SIGNS if rht else 0, target=target, amax_in=am_dev,
                      scale_layout="tiled")
    torch.cuda.synchronize()
    for a, b in ((qr, sr), (qc, sc)):
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
        assert torch.equal(a.s_dec, b.s_dec)
    del sr, sc
    xf = F.bf16_bits_to_f32(xb)
    want_r = want_c = None
    if fmt != "mxfp4":
        want_r = am if am is not None else Q.tensor_amax(xf)
        want_c = am if am is not None else Q.tensor_amax(rht16_cols(xf, SIGNS) if rht else xf)
        assert f32_bits(qr.amax.item()) == f32_bits(want_r)
        assert f32_bits(qc.amax.item()) == f32_bits(want_c)
    rng = np.random.default_rng(70 + cfg)
    for q, orient, off, want in ((qr, "row", 0, want_r), (qc, "col", 1, want_c)):
        full = scales_of(q)
        for a, b in _slabs(q.rows, 32, rng):
            xs = xb[a:b] if orient == "row" else xb[:, a:b]
            r = Q.quantize(xs, fmt, orient=orient, rnd=rnd, seed=1, offset=off,
                           rht=rht and orient == "col", signs=SIGNS if rht else 0,
                           target=target, amax=want, index_base=a * q.cols)
            assert np.array_equal(q.codes[a:b].cpu().numpy(), r["codes"]), (orient, a)
            assert np.array_equal(full[a:b], r["scales"]), (orient, a)


def test_dual_fused_amax_keeps_nan_like_k_amax():
    """With the 16-point RHT on the colwise side and both amaxes computed,
    the plain amax comes from the rotated-amax kernel's read.  Its rowwise
    amax must equal what the plain amax kernel (the unfused path) returns,
    also for a tensor holding a NaN (outside the value contract, but the two
    paths must not differ)."""
    x = inputs.activations((64, 128), cfg_seed=49)
    x[5, 17] = 0x7FC0                                   # bf16 quiet NaN
    xd = dev(x)
    qr, _ = api.quantize_dual(xd, "nvfp4", rht=True, signs=SIGNS)       # fused amax pass
    plain = api.amax(xd)                                                 # k_amax
    torch.cuda.synchronize()
    assert f32_bits(qr.amax.item()) == f32_bits(plain.item())
    assert np.isnan(plain.item())
