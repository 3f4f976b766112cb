"""ctypes binding of libfp4_mi355x.so (include/fp4.h).

Argument marshalling only: torch tensors provide device memory, the current
torch stream is passed as the hipStream_t, and every computation runs in the
library's HIP kernels.  The library is loaded on first use; if it is missing
(not built) every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp4_mi355x.so")

NVFP4, UE5M3, MXFP4, MXFP8 = 0, 1, 2, 3
FORMATS = {"nvfp4": NVFP4, "ue5m3": UE5M3, "mxfp4": MXFP4, "mxfp8": MXFP8}
BLOCK_LEN = {NVFP4: 16, UE5M3: 16, MXFP4: 32, MXFP8: 32}
RNE, SR = 0, 1
BLOCK_1D, BLOCK_2D16 = 0, 1
ROWWISE, COLWISE = 0, 1
SCALES_ROWMAJOR, SCALES_TILED = 0, 1
SCALE_LAYOUTS = {"rowmajor": SCALES_ROWMAJOR, "tiled": SCALES_TILED}
GLOBAL_TENSOR, GLOBAL_ROW = 0, 1
COUNT_LEVELS = {"all": 0, "scales": 1}
GLOBAL_SCOPES = {"tensor": GLOBAL_TENSOR, "row": GLOBAL_ROW}
COUNTER_NAMES = ("scale_saturated", "scale_underflow", "scale_subnormal",
                 "elem_saturated", "elem_underflow")


class Fp4Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class QuantDesc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("block", ctypes.c_int), ("orient", ctypes.c_int),
                ("round", ctypes.c_int), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
                ("rht", ctypes.c_int), ("rht_signs", ctypes.c_uint32), ("target", ctypes.c_float),
                ("amax_given", ctypes.c_int), ("emit_transpose", ctypes.c_int),
                ("scale_layout", ctypes.c_int), ("rht_n", ctypes.c_int),
                ("rht_signs_hi", ctypes.c_uint32 * 3), ("scale_round", ctypes.c_int),
                ("global_scope", ctypes.c_int), ("count_level", ctypes.c_int)]


SCALE_ROUND = {"rne": 0, "up": 1}


def _sign_words(signs):
    """An up-to-128-bit sign mask as (bits 0-31, [bits 32-63, 64-95, 96-127])."""
    signs = int(signs)
    m = 0xFFFFFFFF
    return signs & m, (ctypes.c_uint32 * 3)((signs >> 32) & m, (signs >> 64) & m, (signs >> 96) & m)


class Operand(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("scale_stride_row", ctypes.c_int64),
                ("scale_stride_kblk", ctypes.c_int64), ("scale_row_group", ctypes.c_int32),
                ("s_dec", ctypes.c_void_p), ("scale_layout", ctypes.c_int),
                ("s_dec_scope", ctypes.c_int)]


_lib = None
EXPORTS = ("fp4_amax", "fp4_quantize", "fp4_dequantize", "fp4_rht16", "fp4_gemm",
           "fp4_status_string", "fp4_last_error")


def load_library(path=None):
    """Load (once) and return the ctypes library; raises if it is not built.
    The path defaults to $FP4_LIB if set (e.g. the sanitized host build of
    the argument checks), else the in-tree library."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("FP4_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise Fp4Error(-1, "%s is missing: build it with __graft_entry__.build() "
                           "(python fp4_block_scaled_x16_amd/build.py)" % path)
    lib = ctypes.CDLL(path)
    i64, vp, u32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
    lib.fp4_amax.argtypes = [ctypes.POINTER(QuantDesc), vp, i64, i64, i64, vp, vp]
    lib.fp4_quantize.argtypes = [ctypes.POINTER(QuantDesc), vp, i64, i64, i64, vp, vp, vp, vp,
                                 vp, vp, vp]
    lib.fp4_quantize_dual.argtypes = [ctypes.POINTER(QuantDesc), ctypes.POINTER(QuantDesc), vp, i64,
                                      i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fp4_dequantize.argtypes = [i32, i32, i32, vp, vp, vp, i32, i64, i64, vp, i32, vp]
    lib.fp4_rht16.argtypes = [ctypes.POINTER(QuantDesc), vp, i64, i64, i64, vp, vp]
    lib.fp4_gemm.argtypes = [ctypes.POINTER(Operand), ctypes.POINTER(Operand), i64, i64, i64, vp,
                             i32, i64, i32, vp]
    lib.fp4_selftest_sweep.argtypes = [i32, vp, i32, vp, vp]
    lib.fp4_selftest_gemm_decode.argtypes = [i32, vp, vp]
    lib.fp4_selftest_set_geometry.argtypes = [i32, i32]
    for f in ("fp4_amax", "fp4_quantize", "fp4_quantize_dual", "fp4_dequantize", "fp4_rht16",
              "fp4_gemm", "fp4_selftest_sweep", "fp4_selftest_gemm_decode",
              "fp4_selftest_set_geometry"):
        getattr(lib, f).restype = ctypes.c_int
    lib.fp4_status_string.argtypes = [ctypes.c_int]
    lib.fp4_status_string.restype = ctypes.c_char_p
    lib.fp4_last_error.argtypes = []
    lib.fp4_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status, what):
    if status != 0:
        lib = load_library()
        raise Fp4Error(status, "%s: %s (%s)" % (what, lib.fp4_status_string(status).decode(),
                                               lib.fp4_last_error().decode()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _as_bf16_bits(x):
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    if x.dtype not in (torch.int16, torch.uint16):
        raise TypeError("x must be bfloat16 (or its int16 bit view)")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D row-major tensor")
    return x


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ------------------------------------------------------------------ amax --
def _rht_desc(orient, rht, signs, rht_n):
    s_lo, s_hi = _sign_words(signs)
    return QuantDesc(NVFP4, BLOCK_1D, COLWISE if orient == "col" else ROWWISE, RNE, 0, 0,
                     int(bool(rht)), s_lo, 448.0, 0, 0, SCALES_ROWMAJOR, int(rht_n), s_hi, 0)


def amax(x, rht=False, signs=0, out=None, rht_n=16, orient="col"):
    """Tensor amax -> device fp32 [1]; with rht, of the tensor rotated along
    the blocked axis of `orient` ("col": N-row groups of each column, the
    Wgrad operands; "row": N-column groups of each row, Fprop / Dgrad)."""
    x = _as_bf16_bits(x)
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    desc = _rht_desc(orient, rht, signs, rht_n)
    lib = load_library()
    _check(lib.fp4_amax(ctypes.byref(desc), _ptr(x), x.shape[0], x.shape[1], x.stride(0),
                        _ptr(out), _stream(x.device)), "fp4_amax")
    return out


# -------------------------------------------------------------- quantize --
@dataclass
class Quantized:
    """Codes and scales of one quantized matrix, plus what a GEMM needs."""
    fmt: int
    block: int
    rows: int               # rows of the code matrix
    cols: int               # cols of the code matrix (the blocked axis for 1D)
    codes: torch.Tensor     # uint8 [rows, cols/2] (MXFP8: [rows, cols], a byte per element)
    scales: torch.Tensor    # uint8 1D: [rows, cols/BS] (TILED: flat, tiled_scale_bytes);
                            # 2D: [rows/16, cols/16]
    s_dec: torch.Tensor     # fp32 [1], or [rows] with per-row global scales
    amax: torch.Tensor      # fp32 [1] or [rows] (two-level formats)
    codes_t: torch.Tensor = None   # 2D with emit_transpose: [cols, rows/2]
    scale_layout: int = SCALES_ROWMAJOR
    scope: int = GLOBAL_TENSOR     # GLOBAL_ROW: one global scale per row

    def operand(self, transposed=False):
        """GEMM operand over the K-major code matrix (K = cols), or for 2D
        weights with transposed=True over the codes of the transpose.

        The operand holds raw device pointers; it keeps this object (and so
        its tensors) alive for as long as the operand itself is referenced.
        """
        bs = BLOCK_LEN[self.fmt]
        if self.fmt == MXFP8:
            raise ValueError("no GEMM takes MXFP8 operands")
        if self.block == BLOCK_1D:
            assert not transposed
            op = Operand(self.fmt, self.codes.data_ptr(), self.cols // 2, self.scales.data_ptr(),
                         self.cols // bs, 1, 1, self.s_dec.data_ptr(), self.scale_layout,
                         self.scope)
        elif not transposed:
            op = Operand(self.fmt, self.codes.data_ptr(), self.cols // 2, self.scales.data_ptr(),
                         self.cols // 16, 1, 16, self.s_dec.data_ptr(), SCALES_ROWMAJOR)
        else:
            assert self.codes_t is not None
            op = Operand(self.fmt, self.codes_t.data_ptr(), self.rows // 2, self.scales.data_ptr(),
                         1, self.cols // 16, 16, self.s_dec.data_ptr(), SCALES_ROWMAJOR)
        op._owner = self
        return op


def tiled_scale_bytes(rows, blocks_per_row):
    """Size of the TILED scale buffer of a [rows, blocks_per_row] scale matrix:
    2 KiB atoms of 256 rows x 8 blocks."""
    return -(-rows // 256) * -(-blocks_per_row // 8) * 2048


def quantize(x, fmt="nvfp4", block="1d", orient="row", rnd="rne", seed=0, offset=0, rht=False,
             signs=0, target=448.0, amax_in=None, emit_transpose=False, counters=None,
             scale_layout="rowmajor", rht_n=16, scale_round="rne", global_scope="tensor",
             count="all"):
    """Quantize a bf16 [R, C] matrix.  orient="col" quantizes X^T ([C, R]).
    scale_layout: "rowmajor" or "tiled" (1D blocks only).  rht_n: size of
    the RHT (4, 16, 32, 64, 128); signs: its sign mask, up to 128 bits.
    scale_round: "rne" or "up" (truncation-free block scales).
    global_scope: "tensor" or "row" (rowwise 1D NVFP4 / UE5M3: one global
    scale per row, amax and s_dec of R entries, no separate amax pass).

    amax_in: None -> computed on the device; else a device fp32 [1] tensor read
    as the (possibly stale) tensor amax ([R] per-row amaxes with "row").
    counters: optional device uint64 [5] tensor, accumulated; count: "all"
    or "scales" (block-scale events only).
    """
    x = _as_bf16_bits(x)
    f = _fmt(fmt)
    R, C = x.shape
    blk = BLOCK_2D16 if block == "2d" else BLOCK_1D
    col = orient == "col"
    rows, cols = (C, R) if col else (R, C)
    bs = 16 if blk == BLOCK_2D16 else BLOCK_LEN[f]
    dev = x.device
    code_cols = cols if f == MXFP8 else cols // 2
    codes = torch.empty((rows, code_cols), dtype=torch.uint8, device=dev)
    layout = SCALE_LAYOUTS[scale_layout] if isinstance(scale_layout, str) else int(scale_layout)
    if blk == BLOCK_2D16:
        scales = torch.empty((rows // 16, cols // 16), dtype=torch.uint8, device=dev)
    elif layout == SCALES_TILED:
        scales = torch.empty(tiled_scale_bytes(rows, cols // bs), dtype=torch.uint8, device=dev)
    else:
        scales = torch.empty((rows, cols // bs), dtype=torch.uint8, device=dev)
    codes_t = (torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev)
               if emit_transpose else None)
    scope = GLOBAL_SCOPES[global_scope]
    n_g = rows if scope == GLOBAL_ROW else 1
    s_dec = torch.empty(n_g, dtype=torch.float32, device=dev)
    am = amax_in if amax_in is not None else torch.empty(n_g, dtype=torch.float32, device=dev)
    s_lo, s_hi = _sign_words(signs)
    desc = QuantDesc(f, blk, COLWISE if col else ROWWISE, SR if rnd == "sr" else RNE,
                     int(seed), int(offset), int(bool(rht)), s_lo, float(target),
                     int(amax_in is not None), int(bool(emit_transpose)), layout, int(rht_n), s_hi,
                     SCALE_ROUND[scale_round], scope, COUNT_LEVELS[count])
    lib = load_library()
    _check(lib.fp4_quantize(ctypes.byref(desc), _ptr(x), R, C, x.stride(0), _ptr(codes),
                            _ptr(scales), _ptr(codes_t), _ptr(am), _ptr(s_dec), _ptr(counters),
                            _stream(dev)), "fp4_quantize")
    return Quantized(f, blk, rows, cols, codes, scales, s_dec, am, codes_t, layout, scope)


def _scales_1d(rows, blocks, layout, dev):
    if layout == SCALES_TILED:
        return torch.empty(tiled_scale_bytes(rows, blocks), dtype=torch.uint8, device=dev)
    return torch.empty((rows, blocks), dtype=torch.uint8, device=dev)


def quantize_dual(x, fmt="nvfp4", rnd="rne", seed=0, offset=0, offset_t=None, rht=False, signs=0,
                  target=448.0, amax_in=None, amax_t_in=None, counters=None,
                  scale_layout="rowmajor", scale_layout_t=None, rht_n=16, scale_round="rne",
                  rht_row=False, signs_row=0, rht_n_row=16, count="all"):
    """Rowwise and colwise 1D quantization of a bf16 [R, C] matrix from one
    read: returns (rowwise Quantized [R, C], colwise Quantized of X^T [C, R]).

    Both sides use `rnd` and `seed`; the colwise side uses offset_t (default
    offset + 1), the RHT (rht/signs/rht_n, along the columns) and
    scale_layout_t (default scale_layout); the rowwise side may rotate along
    the rows (rht_row/signs_row, rht_n_row 4 or 16).  amax_in / amax_t_in:
    None -> computed on the device, else device fp32 [1] tensors read as
    the given amax of each side.  count: "all" or "scales" (block-scale
    events only).
    """
    x = _as_bf16_bits(x)
    f = _fmt(fmt)
    R, C = x.shape
    bs = BLOCK_LEN[f]
    dev = x.device
    lay = SCALE_LAYOUTS[scale_layout] if isinstance(scale_layout, str) else int(scale_layout)
    lay_t = lay if scale_layout_t is None else (
        SCALE_LAYOUTS[scale_layout_t] if isinstance(scale_layout_t, str) else int(scale_layout_t))
    if offset_t is None:
        offset_t = offset + 1
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
    codes_t = torch.empty((C, R // 2), dtype=torch.uint8, device=dev)
    scales = _scales_1d(R, C // bs, lay, dev)
    scales_t = _scales_1d(C, R // bs, lay_t, dev)
    s_dec = torch.empty(1, dtype=torch.float32, device=dev)
    s_dec_t = torch.empty(1, dtype=torch.float32, device=dev)
    am = amax_in if amax_in is not None else torch.empty(1, dtype=torch.float32, device=dev)
    am_t = amax_t_in if amax_t_in is not None else torch.empty(1, dtype=torch.float32, device=dev)
    r = SR if rnd == "sr" else RNE
    s_lo, s_hi = _sign_words(signs)
    sr_mode = SCALE_ROUND[scale_round]
    r_lo, r_hi = _sign_words(signs_row)
    cl = COUNT_LEVELS[count]
    d_row = QuantDesc(f, BLOCK_1D, ROWWISE, r, int(seed), int(offset), int(bool(rht_row)), r_lo,
                      float(target), int(amax_in is not None), 0, lay, int(rht_n_row), r_hi,
                      sr_mode, GLOBAL_TENSOR, cl)
    d_col = QuantDesc(f, BLOCK_1D, COLWISE, r, int(seed), int(offset_t), int(bool(rht)), s_lo,
                      float(target), int(amax_t_in is not None), 0, lay_t, int(rht_n), s_hi,
                      sr_mode, GLOBAL_TENSOR, cl)
    lib = load_library()
    _check(lib.fp4_quantize_dual(ctypes.byref(d_row), ctypes.byref(d_col), _ptr(x), R, C,
                                 x.stride(0), _ptr(codes), _ptr(scales), _ptr(codes_t),
                                 _ptr(scales_t), _ptr(am), _ptr(am_t), _ptr(s_dec), _ptr(s_dec_t),
                                 _ptr(counters), _stream(dev)), "fp4_quantize_dual")
    return (Quantized(f, BLOCK_1D, R, C, codes, scales, s_dec, am, None, lay),
            Quantized(f, BLOCK_1D, C, R, codes_t, scales_t, s_dec_t, am_t, None, lay_t))


def new_counters(device="cuda"):
    return torch.zeros(5, dtype=torch.int64, device=device)


def counters_dict(c):
    return dict(zip(COUNTER_NAMES, [int(v) for v in c.cpu().tolist()]))


# ------------------------------------------------------------ dequantize --
def dequantize(q: Quantized, out_dtype=torch.float32, out=None):
    """Values of a quantized matrix as fp32 or bf16 [rows, cols] (into `out`,
    a contiguous tensor of that shape and dtype, when given)."""
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=out_dtype, device=q.codes.device)
    elif (out.dtype != out_dtype or tuple(out.shape) != (q.rows, q.cols)
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous %s tensor of shape (%d, %d)"
                         % (out_dtype, q.rows, q.cols))
    lib = load_library()
    _check(lib.fp4_dequantize(q.fmt, q.block, q.scale_layout, _ptr(q.codes), _ptr(q.scales),
                              _ptr(q.s_dec), q.scope,
                              q.rows, q.cols, _ptr(out), int(out_dtype == torch.float32),
                              _stream(out.device)), "fp4_dequantize")
    return out


# ------------------------------------------------------------------- RHT --
def rht16(x, signs, rht_n=16, orient="col", out=None):
    """The RHT alone (fp32 [R, C]) along the blocked axis of `orient` (into
    `out`, a contiguous fp32 tensor of x's shape, when given)."""
    x = _as_bf16_bits(x)
    if out is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    elif out.dtype != torch.float32 or out.shape != x.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor of the input's shape")
    else:
        y = out
    desc = _rht_desc(orient, True, signs, rht_n)
    lib = load_library()
    _check(lib.fp4_rht16(ctypes.byref(desc), _ptr(x), x.shape[0], x.shape[1], x.stride(0),
                         _ptr(y), _stream(x.device)), "fp4_rht16")
    return y


# ------------------------------------------------------------------ GEMM --
OUT_TYPES = {torch.float32: 0, torch.bfloat16: 1}


def gemm(a: Operand, b: Operand, M, N, K, out=None, accumulate=False, device=None,
         out_dtype=torch.float32):
    """D[M, N] (+)= s_A s_B sum_k a[m, k] b[n, k], written as fp32 or bf16
    (the dtype of `out` when given, else out_dtype)."""
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=device or "cuda")
    if out.dtype not in OUT_TYPES or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be a row-major 2-D fp32 or bf16 tensor")
    lib = load_library()
    _check(lib.fp4_gemm(ctypes.byref(a), ctypes.byref(b), M, N, K, _ptr(out), OUT_TYPES[out.dtype],
                        out.stride(0), int(bool(accumulate)), _stream(out.device)), "fp4_gemm")
    return out


# ------------------------------------------------------------- self-test --
SWEEPS = {"e2m1_rne": 0, "e4m3_scale": 1, "ue5m3_scale": 2, "e2m1_sr": 3, "e4m3_elem": 4}


def selftest_sweep(kind, thresholds, device="cuda"):
    """Run one of the library's conversions over its whole input domain
    against the step function `thresholds` (ascending fp32 bit patterns,
    uint32): returns (mismatches, smallest mismatching pattern or None,
    inputs checked)."""
    if len(thresholds) and int(max(thresholds)) >= 2 ** 31:
        raise ValueError("thresholds are magnitudes: patterns below 2^31")
    thr = torch.tensor([int(t) for t in thresholds], dtype=torch.int32).to(device)
    res = torch.empty(3, dtype=torch.int64, device=device)
    lib = load_library()
    _check(lib.fp4_selftest_sweep(SWEEPS[kind], _ptr(thr), thr.numel(), _ptr(res),
                                  _stream(res.device)), "fp4_selftest_sweep")
    bad, first, checked = (int(v) & (2 ** 64 - 1) for v in res.cpu().tolist())
    return bad, (None if bad == 0 else first), checked


def selftest_gemm_decode(fmt, device="cuda"):
    """The GEMM's operand decode of every (scale code, E2M1 code) pair:
    uint16 fp16 patterns [256, 4, 16] (see fp4_selftest_gemm_decode)."""
    out = torch.empty((256, 4, 16), dtype=torch.int16, device=device)
    lib = load_library()
    _check(lib.fp4_selftest_gemm_decode(_fmt(fmt), _ptr(out), _stream(out.device)),
           "fp4_selftest_gemm_decode")
    return out.cpu().numpy().view("uint16")


def selftest_set_geometry(max_workgroups=0, gemm_tile_rows=0):
    """Launch-geometry controls for race guards (0, 0: the defaults)."""
    _check(load_library().fp4_selftest_set_geometry(int(max_workgroups), int(gemm_tile_rows)),
           "fp4_selftest_set_geometry")
