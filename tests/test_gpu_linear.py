"""GPU parity of QuantizedLinear (forward + backward of one FP4 linear layer)
against the same layer composed from the oracle.

Per step: Y = Fprop, dX = Dgrad, and the fp32 main gradient accumulating
Wgrad, each within 1e-5 * s_A s_B sum|a b| per element (summed over the
steps for the accumulated gradient) of the oracle's fp64 GEMMs of its own
quantized operands; event counters equal to the oracle's.  Cases: NVFP4
with and without the RHT (16-point, with the amax refreshed every step and
every second step, and 64-point refreshed every second step), the RHT
along K on the Fprop / Dgrad operands too (16- and 4-point), UE5M3 with the
tensor amax refreshed every second step (steps in between reuse it on new
data), MXFP4, and the 2D-block recipe (16x16 blocks for X and dY too, SR
on dY, rounded-up scales).
"""
import numpy as np
import pytest
import torch

from fp4_block_scaled_x16_amd import inputs
from fp4_block_scaled_x16_amd.linear import QuantizedLinear, Recipe
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from oracle.rht import rht_cols
from bf16_check import bf16_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5
SIGNS = inputs.rht_sign_mask()


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def vals(q, fmt, block="1d"):
    R, C2 = q["codes"].shape
    return Q.operand_values(q["codes"], q["scales"], fmt, block, R, 2 * C2)


def s_dec(q, fmt):
    return 1.0 if fmt == "mxfp4" else q["s_dec"]


def oracle_step(x, w, dy, r: Recipe, step, amax):
    """Oracle Y, dX, dW (+ abs bounds) and counters of one step, with the
    tensor amax values `amax` (dict; None entries for MXFP4)."""
    fmt, cnt, sr_mode = r.fmt, [], r.scale_round
    if r.act_block == "2d":
        # one 16x16-block quantization per tensor; the transposed operand is
        # the same values transposed (2D-block page)
        q2 = Q.quantize(x, fmt, block="2d", target=r.target_x, amax=amax["x"],
                        scale_round=sr_mode)
        xv = vals(q2, fmt, "2d")
        x_ops = ((xv, q2["s_dec"]), (xv.T.copy(), q2["s_dec"]))
        cnt.append(q2["counters"])
    else:
        qx = Q.quantize(x, fmt, orient="row", target=r.target_x, amax=amax["x"],
                        scale_round=sr_mode, rht=r.rht_kd, signs=r.rht_kd_signs, rht_n=r.rht_kd_n)
        qxt = Q.quantize(x, fmt, orient="col", rht=r.rht, signs=r.rht_signs, target=r.target_x,
                         amax=amax["x_t"], rht_n=r.rht_n, scale_round=sr_mode)
        x_ops = ((vals(qx, fmt), s_dec(qx, fmt)), (vals(qxt, fmt), s_dec(qxt, fmt)))
        cnt += [qx["counters"], qxt["counters"]]
    if r.rht_kd:
        kd = dict(rht=True, signs=r.rht_kd_signs, rht_n=r.rht_kd_n, target=r.target_w,
                  scale_round=sr_mode)
        qw = Q.quantize(w, fmt, orient="row", amax=amax["w"], **kd)
        qwt = Q.quantize(w, fmt, orient="col", amax=amax["w_t"], **kd)
        wv, wtv, sw, swt = vals(qw, fmt), vals(qwt, fmt), qw["s_dec"], qwt["s_dec"]
        cnt += [qw["counters"], qwt["counters"]]
    elif r.two_level:
        qw = Q.quantize(w, fmt, block="2d", emit_transpose=True, target=r.target_w,
                        amax=amax["w"], scale_round=sr_mode)
        wv = vals(qw, fmt, "2d")
        wtv, sw, swt = wv.T.copy(), qw["s_dec"], qw["s_dec"]
        cnt.append(qw["counters"])
    else:
        qw, qwt = Q.quantize(w, fmt, orient="row"), Q.quantize(w, fmt, orient="col")
        wv, wtv, sw, swt = vals(qw, fmt), vals(qwt, fmt), 1.0, 1.0
        cnt += [qw["counters"], qwt["counters"]]
    if r.act_block == "2d":
        q2 = Q.quantize(dy, fmt, block="2d", rnd="sr", seed=r.sr_seed, offset=2 * step,
                        target=r.target_dy, amax=amax["dy"], scale_round=sr_mode)
        dv = vals(q2, fmt, "2d")
        dy_ops = ((dv, q2["s_dec"]), (dv.T.copy(), q2["s_dec"]))
        cnt.append(q2["counters"])
    else:
        qdy = Q.quantize(dy, fmt, orient="row", rnd="sr", seed=r.sr_seed, offset=2 * step,
                         target=r.target_dy, amax=amax["dy"], scale_round=sr_mode,
                         rht=r.rht_kd, signs=r.rht_kd_signs, rht_n=r.rht_kd_n)
        qdyt = Q.quantize(dy, fmt, orient="col", rnd="sr", seed=r.sr_seed, offset=2 * step + 1,
                          rht=r.rht, signs=r.rht_signs, target=r.target_dy, amax=amax["dy_t"],
                          rht_n=r.rht_n, scale_round=sr_mode)
        dy_ops = ((vals(qdy, fmt), s_dec(qdy, fmt)), (vals(qdyt, fmt), s_dec(qdyt, fmt)))
        cnt += [qdy["counters"], qdyt["counters"]]
    out = {}
    for name, (a, sa), (b, sb) in (("y", x_ops[0], (wv, sw)),
                                   ("dx", dy_ops[0], (wtv, swt)),
                                   ("dw", dy_ops[1], x_ops[1])):
        out[name] = (G.gemm_ref(a, b, sa, sb), G.gemm_abs_bound(a, b, sa, sb))
    counters = {k: sum(c[k] for c in cnt) for k in cnt[0]}
    return out, counters


def tensor_amaxes(x, w, dy, r):
    if not r.two_level:
        return dict(x=None, x_t=None, w=None, w_t=None, dy=None, dy_t=None)
    xf, wf, dyf = F.bf16_bits_to_f32(x), F.bf16_bits_to_f32(w), F.bf16_bits_to_f32(dy)

    def along_k(v):     # rotated along the rows (the K axis of Fprop / Dgrad)
        return rht_cols(v.T, r.rht_kd_signs, r.rht_kd_n).T if r.rht_kd else v

    a = dict(x=Q.tensor_amax(along_k(xf)), w=Q.tensor_amax(along_k(wf)),
             dy=Q.tensor_amax(along_k(dyf)))
    a["x_t"] = Q.tensor_amax(rht_cols(xf, r.rht_signs, r.rht_n)) if r.rht else Q.tensor_amax(xf)
    a["dy_t"] = Q.tensor_amax(rht_cols(dyf, r.rht_signs, r.rht_n)) if r.rht else Q.tensor_amax(dyf)
    a["w_t"] = Q.tensor_amax(rht_cols(wf, r.rht_kd_signs, r.rht_kd_n)) if r.rht_kd else a["w"]
    return a


def check(got, ref_bound):
    ref, bound = ref_bound
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= TOL * bound), float((err / np.maximum(bound, 1e-300)).max())


RECIPES = {
    "nvfp4": (Recipe("nvfp4"), 1),
    "nvfp4_rht": (Recipe("nvfp4", rht=True, rht_signs=SIGNS), 1),
    "nvfp4_rht64_periodic": (Recipe("nvfp4", rht=True, rht_n=64, rht_signs=inputs.rht_sign_bits(64),
                                    amax_interval=2), 3),
    "ue5m3_periodic": (Recipe("ue5m3", target_dy=2048.0, amax_interval=2), 3),
    "mxfp4": (Recipe("mxfp4"), 1),
    "nvfp4_2d_blocks_up": (Recipe("nvfp4", act_block="2d", scale_round="up"), 2),
    "ue5m3_2d_blocks_periodic": (Recipe("ue5m3", target_dy=2048.0, act_block="2d",
                                        amax_interval=2), 2),
    "nvfp4_1d_up": (Recipe("nvfp4", scale_round="up"), 1),
    # the fused plain + rotated amax pass on refreshes, kept for the next step
    "nvfp4_rht16_periodic": (Recipe("nvfp4", rht=True, rht_signs=SIGNS, amax_interval=2), 3),
    # RHT along K on the Fprop / Dgrad operands as well (1D W)
    "nvfp4_rht_all_gemms": (Recipe("nvfp4", rht=True, rht_signs=SIGNS, rht_kd=True,
                                   rht_kd_signs=SIGNS), 1),
    "ue5m3_rht4_kd_periodic": (Recipe("ue5m3", target_dy=2048.0, rht_kd=True, rht_kd_n=4,
                                      rht_kd_signs=inputs.rht_sign_bits(4), amax_interval=2), 3),
}


@pytest.mark.parametrize("name", list(RECIPES))
def test_linear_layer(name):
    r, steps = RECIPES[name]
    tokens, d_in, d_out = 272, 128, 208          # 2D W tiles; two GEMM tiles in two dims
    if r.fmt == "mxfp4":
        tokens, d_in, d_out = 320, 128, 224      # 32-multiples for 1x32 blocks
    if r.rht and r.rht_n > 16:
        tokens = 320                             # a multiple of the RHT size
    w = inputs.weights((d_out, d_in), cfg_seed=80)
    layer = QuantizedLinear(dev(w), r)
    dw_ref = np.zeros((d_out, d_in))
    dw_bound = np.zeros((d_out, d_in))
    want_cnt = {k: 0 for k in ("scale_saturated", "scale_underflow", "scale_subnormal",
                               "elem_saturated", "elem_underflow")}
    amax = None
    for s in range(steps):
        x = inputs.activations((tokens, d_in), cfg_seed=81 + s)
        dy = inputs.gradients((tokens, d_out), cfg_seed=81 + s)
        if amax is None or s % r.amax_interval == 0:
            amax = tensor_amaxes(x, w, dy, r)       # refreshed on this step
        y = layer.forward(dev(x))
        dx = layer.backward(dev(dy))
        torch.cuda.synchronize()
        ref, cnt = oracle_step(x, w, dy, r, s, amax)
        check(y, ref["y"])
        check(dx, ref["dx"])
        dw_ref += ref["dw"][0]
        dw_bound += ref["dw"][1]
        check(layer.main_grad, (dw_ref, dw_bound))
        for k in want_cnt:
            want_cnt[k] += cnt[k]
    got = dict(zip(want_cnt, [int(v) for v in layer.counters.cpu().tolist()]))
    assert got == want_cnt
    assert layer.step == steps


def test_backward_needs_forward():
    layer = QuantizedLinear(dev(inputs.weights((32, 32), cfg_seed=1)))
    with pytest.raises(RuntimeError):
        layer.backward(torch.zeros((16, 32), dtype=torch.bfloat16, device=DEV))


@pytest.mark.parametrize("name,steps", [("nvfp4_rht", 2), ("ue5m3_periodic", 3)])
def test_linear_autograd_bf16(name, steps):
    """The layer under autograd with bf16 outputs (NVFP4 paper §4.1: FP4
    inputs, BF16 outputs): y = layer(x); y.backward(dy) gives x.grad = dX and
    accumulates dW into main_grad.  Y and dX are the oracle's fp32 values
    rounded once to bf16 (within the GEMM bound plus half a bf16 ulp)."""
    import dataclasses
    r0, _ = RECIPES[name]
    r = dataclasses.replace(r0, out_dtype="bf16")
    tokens, d_in, d_out = 272, 128, 208
    w = inputs.weights((d_out, d_in), cfg_seed=80)
    layer = QuantizedLinear(dev(w), r)
    dw_ref = np.zeros((d_out, d_in))
    dw_bound = np.zeros((d_out, d_in))
    amax = None
    for s in range(steps):
        x = inputs.activations((tokens, d_in), cfg_seed=91 + s)
        dy = inputs.gradients((tokens, d_out), cfg_seed=91 + s)
        if amax is None or s % r.amax_interval == 0:
            amax = tensor_amaxes(x, w, dy, r)
        xt = dev(x).view(torch.bfloat16).requires_grad_()
        y = layer(xt)
        assert y.dtype == torch.bfloat16 and y.requires_grad
        y.backward(dev(dy).view(torch.bfloat16))
        torch.cuda.synchronize()
        ref, _ = oracle_step(x, w, dy, r, s, amax)
        bf16_close(y.detach().view(torch.int16).cpu().numpy().view(np.uint16), *ref["y"])
        assert xt.grad.dtype == torch.bfloat16
        bf16_close(xt.grad.view(torch.int16).cpu().numpy().view(np.uint16), *ref["dx"])
        dw_ref += ref["dw"][0]
        dw_bound += ref["dw"][1]
        check(layer.main_grad, (dw_ref, dw_bound))
    assert layer.weight.grad is None and layer.step == steps


def test_autograd_needs_bf16_output():
    layer = QuantizedLinear(dev(inputs.weights((32, 32), cfg_seed=1)))
    with pytest.raises(ValueError):
        layer(torch.zeros((16, 32), dtype=torch.bfloat16, device=DEV))
