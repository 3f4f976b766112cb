"""A linear layer whose three GEMMs run on FP4 operands.

NVFP4 paper §4.1 and Fig. 5: in a linear layer Y = X W^T, the forward
product (Fprop) and both backward products -- Dgrad (dX = dY W) and Wgrad
(dW = dY^T X) -- consume FP4-quantized operands and accumulate in fp32.
This class composes the library's entry points into that layer:

  forward(X)    X  -> rowwise codes (Fprop A) and colwise codes of X^T
                      (Wgrad B) from one read; RHT on the colwise side when
                      the recipe asks for it (§4.2, App. C)
                W  -> 16x16 2D codes of W and W^T with one scale per tile
                      (§4.3; MXFP4: 1D rowwise and colwise codes)
                Y  = Fprop(X, W)                          fp32 [tokens, out]
  backward(dY)  dY -> rowwise codes (Dgrad A) and colwise codes of dY^T
                      (Wgrad A) with stochastic rounding (§4.4)
                dX = Dgrad(dY, W^T)                       fp32 [tokens, in]
                main_grad += Wgrad(dY^T, X^T)             fp32 [out, in]

With rht_kd (§4.2: Fprop and Dgrad "may also benefit" from the RHT) the
Fprop and Dgrad operands are rotated along their K axis as well: X and W
rowwise along the input features (Fprop), dY rowwise and W colwise along
the output features (Dgrad), each pair with the same signs so the rotation
cancels in the product.  W is then quantized in 1D blocks (a rowwise and a
colwise code matrix, rotated along different axes) instead of 16x16 tiles:
one rotated W cannot serve both products (§4.3 on keeping Fprop and Dgrad
consistent; the rotated layer trades that consistency for the rotation).

With act_block = "2d" (the 2D-block FP4 recipe) X and dY are quantized in
16x16 blocks as well, each once with its transpose (dY with stochastic
rounding, the same random bits for both orientations), so every operand a
tensor contributes holds the same values in Fprop / Dgrad and in Wgrad;
scale_round = "up" rounds block scales up (truncation-free scaling).

Tensor amax: current scaling (recomputed every step, the NVFP4 recipe) or,
with amax_interval = N > 1, recomputed every N-th step and reused in
between (the periodic tensor scaling of the UE5M3 recipe).  The SR random
stream of step s uses Philox counter offsets 2s (rowwise dY) and 2s + 1
(colwise dY), so no two steps or orientations share random bits.

Outputs: Y and dX are fp32 or bf16 (out_dtype; §4.1: the GEMMs write BF16
or FP32, rounded once from the fp32 result in the GEMM's epilogue); the
weight gradient accumulates in fp32 (main_grad).

Calling the layer (`layer(x)`) runs it under autograd: a torch.autograd.
Function whose forward is Fprop and whose backward is Dgrad (the gradient
of x) and Wgrad (added to main_grad; the weight gets no .grad).  Its
gradient dY is quantized from bf16, so the autograd path takes bf16 x and
writes bf16 Y and dX (out_dtype "bf16").  `forward` / `backward` are the
same steps called explicitly, one backward per forward.

Every computation runs in the library's kernels; this module only
allocates outputs and passes pointers (through `api`).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import api


@dataclass
class Recipe:
    fmt: str = "nvfp4"            # "nvfp4", "ue5m3" or "mxfp4"
    target_x: float = 448.0       # T of s_enc = 6 T / amax, per tensor
    target_w: float = 448.0
    target_dy: float = 448.0
    rht: bool = False             # RHT on the Wgrad operands (colwise X and dY)
    rht_n: int = 16               # RHT size N: 4, 16, 32, 64 or 128
    rht_signs: int = 0            # N-bit sign mask D_r
    sr_seed: int = 1              # Philox key of the stochastic rounding of dY
    amax_interval: int = 1        # recompute each tensor amax every this many steps
    scale_layout: str = "tiled"   # storage of the 1D block scales
    act_block: str = "1d"         # "1d" (1x16 / 1x32) or "2d" (16x16) for X and dY
    scale_round: str = "rne"      # block scales: "rne" or "up" (truncation-free)
    rht_kd: bool = False          # RHT along K on the Fprop / Dgrad operands too
    rht_kd_n: int = 16            # its size N: 4 or 16
    rht_kd_signs: int = 0         # its N-bit sign mask
    out_dtype: str = "fp32"       # Y and dX: "fp32" or "bf16"

    @property
    def two_level(self):
        return self.fmt != "mxfp4"


class QuantizedLinear:
    """Y = X W^T with FP4 Fprop / Dgrad / Wgrad (see the module docstring).

    weight: bf16 [out, in] device tensor (the master copy stays in bf16);
    main_grad: fp32 [out, in], accumulated by every backward (zero it
    between optimizer steps).
    """

    def __init__(self, weight: torch.Tensor, recipe: Recipe = Recipe()):
        if weight.dim() != 2:
            raise ValueError("weight must be [out, in]")
        if recipe.act_block == "2d" and (recipe.rht or recipe.rht_kd or not recipe.two_level):
            raise ValueError("2D activation blocks need NVFP4 or UE5M3 and no RHT")
        if recipe.rht_kd and (not recipe.two_level or recipe.rht_kd_n not in (4, 16)):
            raise ValueError("the RHT along K needs NVFP4 or UE5M3 and N = 4 or 16")
        if recipe.out_dtype not in _OUT_DTYPES:
            raise ValueError("out_dtype must be 'fp32' or 'bf16'")
        self.weight = weight
        self.recipe = recipe
        self.out_features, self.in_features = weight.shape
        dev = weight.device
        self.main_grad = torch.zeros((self.out_features, self.in_features), dtype=torch.float32,
                                     device=dev)
        names = ("x", "x_t", "w", "w_t", "dy", "dy_t")
        self.amax = {n: torch.zeros(1, dtype=torch.float32, device=dev) for n in names}
        self.step = 0
        self.counters = api.new_counters(dev)
        self._saved = None

    def _refresh(self):
        r = self.recipe
        return r.two_level and (r.amax_interval <= 1 or self.step % r.amax_interval == 0)

    def _amax_args(self, x, name, rht):
        """amax buffers (rowwise, colwise) for a dual quantization of x,
        refreshed on this step if due; without an RHT on either side both
        share one buffer.  MXFP4 has none.  With an RHT a refresh leaves both
        to the quantizer (None, None: each side's amax in its own rotated
        space; the plain and the 16-point-rotated one from one read), and
        `_keep_amax` keeps what it computed."""
        r = self.recipe
        if not r.two_level:
            return None, None
        if self._refresh():
            if rht:
                return None, None
            api.amax(x, out=self.amax[name])
        return self.amax[name], self.amax[name + "_t" if rht else name]

    def _kd(self):
        """Keyword arguments of the rowwise side's RHT along K (or none)."""
        r = self.recipe
        if not r.rht_kd:
            return {}
        return dict(rht_row=True, signs_row=r.rht_kd_signs, rht_n_row=r.rht_kd_n)

    def _keep_amax(self, name, q, q_t, given):
        if self.recipe.two_level and given is None:
            self.amax[name], self.amax[name + "_t"] = q.amax, q_t.amax

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        """Y = X W^T under autograd (bf16 x, bf16 Y; see the module docstring)."""
        if self.recipe.out_dtype != "bf16":
            raise ValueError("the autograd path needs Recipe(out_dtype='bf16'): its gradient "
                             "dY is quantized from bf16")
        return _Fp4LinearFunction.apply(x, self.weight, self)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """Fprop of one step; the operands Dgrad / Wgrad need are kept for
        the next `backward`."""
        y, self._saved = self._forward(x)
        return y

    def backward(self, dy: torch.Tensor) -> torch.Tensor:
        """Dgrad (returned) and Wgrad (added to main_grad) of the last forward."""
        if self._saved is None:
            raise RuntimeError("backward() needs a preceding forward()")
        saved, self._saved = self._saved, None
        return self._backward(dy, saved)

    def _forward(self, x):
        r = self.recipe
        if x.dim() != 2 or x.shape[1] != self.in_features:
            raise ValueError("x must be [tokens, in_features]")
        am, am_t = self._amax_args(x, "x", r.rht or r.rht_kd)
        if r.act_block == "2d":
            qx2 = api.quantize(x, r.fmt, block="2d", emit_transpose=True, target=r.target_x,
                               amax_in=am, counters=self.counters, scale_round=r.scale_round)
            x_op, xt_op = qx2.operand(), qx2.operand(transposed=True)
        else:
            qx, qx_t = api.quantize_dual(x, r.fmt, rht=r.rht, signs=r.rht_signs, rht_n=r.rht_n,
                                         target=r.target_x, amax_in=am, amax_t_in=am_t,
                                         counters=self.counters, scale_layout=r.scale_layout,
                                         scale_round=r.scale_round, **self._kd())
            self._keep_amax("x", qx, qx_t, am)
            x_op, xt_op = qx.operand(), qx_t.operand()
        if r.rht_kd:
            # 1D W: rowwise along the inputs (Fprop B), colwise along the
            # outputs (Dgrad B), each rotated along its own K
            am, am_t = self._amax_args(self.weight, "w", True)
            qw, qw_t = api.quantize_dual(self.weight, r.fmt, rht=True, signs=r.rht_kd_signs,
                                         rht_n=r.rht_kd_n, target=r.target_w, amax_in=am,
                                         amax_t_in=am_t, counters=self.counters,
                                         scale_layout=r.scale_layout, scale_round=r.scale_round,
                                         **self._kd())
            self._keep_amax("w", qw, qw_t, am)
            w_op, wt_op = qw.operand(), qw_t.operand()
        elif r.two_level:
            if self._refresh():
                api.amax(self.weight, out=self.amax["w"])
            qw = api.quantize(self.weight, r.fmt, block="2d", emit_transpose=True,
                              target=r.target_w, amax_in=self.amax["w"], counters=self.counters,
                              scale_round=r.scale_round)
            w_op, wt_op = qw.operand(), qw.operand(transposed=True)
        else:
            qw, qw_t = api.quantize_dual(self.weight, r.fmt, counters=self.counters,
                                         scale_layout=r.scale_layout)
            w_op, wt_op = qw.operand(), qw_t.operand()
        tokens = x.shape[0]
        y = api.gemm(x_op, w_op, tokens, self.out_features, self.in_features, device=x.device,
                     out_dtype=_OUT_DTYPES[r.out_dtype])
        return y, (xt_op, wt_op, tokens)

    def _backward(self, dy, saved):
        r = self.recipe
        xt_op, wt_op, tokens = saved
        if dy.dim() != 2 or tuple(dy.shape) != (tokens, self.out_features):
            raise ValueError("dy must be [tokens, out_features]")
        am, am_t = self._amax_args(dy, "dy", r.rht or r.rht_kd)
        if r.act_block == "2d":
            qdy2 = api.quantize(dy, r.fmt, block="2d", rnd="sr", seed=r.sr_seed,
                                offset=2 * self.step, emit_transpose=True, target=r.target_dy,
                                amax_in=am, counters=self.counters, scale_round=r.scale_round)
            dy_op, dyt_op = qdy2.operand(), qdy2.operand(transposed=True)
        else:
            qdy, qdy_t = api.quantize_dual(dy, r.fmt, rnd="sr", seed=r.sr_seed,
                                           offset=2 * self.step, offset_t=2 * self.step + 1,
                                           rht=r.rht, signs=r.rht_signs, rht_n=r.rht_n,
                                           target=r.target_dy, amax_in=am, amax_t_in=am_t,
                                           counters=self.counters, scale_layout=r.scale_layout,
                                           scale_round=r.scale_round, **self._kd())
            self._keep_amax("dy", qdy, qdy_t, am)
            dy_op, dyt_op = qdy.operand(), qdy_t.operand()
        dx = api.gemm(dy_op, wt_op, tokens, self.in_features, self.out_features, device=dy.device,
                      out_dtype=_OUT_DTYPES[r.out_dtype])
        api.gemm(dyt_op, xt_op, self.out_features, self.in_features, tokens,
                 out=self.main_grad, accumulate=True)
        self.step += 1
        return dx


_OUT_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


class _Fp4LinearFunction(torch.autograd.Function):
    """Autograd wrapper of one QuantizedLinear step: forward = Fprop (the
    quantized operands for the backward GEMMs are kept on the context),
    backward = Dgrad (the gradient of x) and Wgrad (added to the layer's
    main_grad; no gradient is returned for the weight or the layer)."""

    @staticmethod
    def forward(ctx, x, weight, layer):
        y, ctx.saved = layer._forward(x)
        ctx.layer = layer
        return y

    @staticmethod
    def backward(ctx, dy):
        saved, ctx.saved = ctx.saved, None
        dx = ctx.layer._backward(dy.contiguous(), saved)
        return dx, None, None
