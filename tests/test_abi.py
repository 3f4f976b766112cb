"""The C-ABI library: it loads, exports every function include/*.h declares,
and rejects invalid arguments on the host (no GPU is touched: these calls
return before any HIP API call)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from fp4_block_scaled_x16_amd import api
from conftest import ROOT

HEADERS = glob.glob(os.path.join(ROOT, "include", "*.h"))
DECL = re.compile(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fp4_[a-z0-9_]+)\s*\(", re.M)


def declared():
    names = set()
    for h in HEADERS:
        names |= set(DECL.findall(open(h).read()))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return api.load_library()


def test_header_declares_the_boundary():
    assert {"fp4_amax", "fp4_quantize", "fp4_quantize_dual", "fp4_dequantize", "fp4_rht16",
            "fp4_gemm", "fp4_status_string", "fp4_last_error"} <= declared()


def test_exports_every_declared_symbol(lib):
    path = os.environ.get("FP4_LIB") or api.LIB_PATH      # the library `lib` loaded
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing but the declared API is exported
    assert {e for e in exported if e.startswith("fp4")} == declared()


def _err(lib):
    return lib.fp4_last_error().decode()


def desc(**kw):
    d = dict(format=0, block=0, orient=0, round=0, seed=0, offset=0, rht=0, rht_signs=0,
             target=448.0, amax_given=0, emit_transpose=0, scale_layout=0)
    d.update(kw)
    return api.QuantDesc(**d)


FAKE = ctypes.c_void_p(0x10000)          # 16-byte aligned, never dereferenced


def quant(lib, d, rows=32, cols=64, ld=None, x=FAKE, codes=FAKE, scales=FAKE, codes_t=None,
          amax=FAKE):
    return lib.fp4_quantize(ctypes.byref(d), x, rows, cols, cols if ld is None else ld, codes,
                            scales, codes_t, amax, None, None, None)


@pytest.mark.parametrize("kw,rows,cols,status", [
    (dict(format=7), 32, 64, 1),
    (dict(block=3), 32, 64, 1),
    (dict(round=2), 32, 64, 1),
    (dict(format=2, block=1), 32, 64, 3),            # 2D needs NVFP4/UE5M3
    (dict(block=1, orient=1), 32, 64, 3),            # 2D is rowwise only
    (dict(scale_round=2), 32, 64, 1),                # bad scale rounding
    (dict(rht=1, block=1), 32, 64, 3),               # RHT needs 1D blocks
    (dict(rht=1, rht_n=128), 32, 64, 2),             # rowwise RHT: cols % rht_n
    (dict(rht=1, orient=1, format=2), 32, 64, 3),    # RHT needs two-level formats
    (dict(format=2, amax_given=1), 32, 64, 3),       # MXFP4 has no tensor amax
    (dict(emit_transpose=1), 32, 64, 3),             # emit_transpose needs 2D
    (dict(target=0.0), 32, 64, 1),
    (dict(target=float("inf")), 32, 64, 1),
    (dict(), 32, 40, 2),                             # cols % 16
    (dict(format=2), 32, 48, 2),                     # cols % 32
    (dict(orient=1), 24, 64, 2),                     # rows % 16 (colwise)
    (dict(block=1), 40, 64, 2),                      # 2D rows % 16
    (dict(), -1, 64, 2),
    (dict(scale_layout=2), 32, 64, 1),
    (dict(block=1, scale_layout=1), 32, 64, 3),      # TILED scales are 1D only
    (dict(format=3, round=1), 32, 64, 3),            # MXFP8 is RNE only
    (dict(format=3, block=1), 32, 64, 3),            # MXFP8 is 1D
    (dict(format=3, rht=1, orient=1), 32, 64, 3),    # no RHT for MXFP8
    (dict(format=3, amax_given=1), 32, 64, 3),       # no tensor amax
    (dict(format=3), 32, 48, 2),                     # cols % 32
    (dict(format=3, orient=1), 48, 64, 2),           # rows % 32 (colwise)
    (dict(global_scope=1, format=3), 32, 64, 3),     # no per-row scales
    (dict(global_scope=2), 32, 64, 1),               # bad global scope
    (dict(count_level=2), 32, 64, 1),                # bad counting level
    (dict(global_scope=1, format=2), 32, 64, 3),     # per-row scales: two-level formats
    (dict(global_scope=1, orient=1), 32, 64, 3),     # per-row scales: ROWWISE only
    (dict(global_scope=1, block=1), 32, 64, 3),      # per-row scales: 1D only
])
def test_quantize_rejects(lib, kw, rows, cols, status):
    assert quant(lib, desc(**kw), rows, cols) == status
    assert _err(lib)


def _hi(*w):
    return (ctypes.c_uint32 * 3)(*w)


@pytest.mark.parametrize("kw,rows,status", [
    (dict(rht_n=8), 64, 1),                                  # not a supported size
    (dict(rht_n=256), 256, 1),
    (dict(rht_n=32), 48, 2),                                 # rows % N
    (dict(rht_n=128), 192, 2),
    (dict(rht_n=4, rht_signs=0x10), 32, 1),                  # sign bit at or above N
    (dict(rht_n=16, rht_signs=1 << 16), 32, 1),
    (dict(rht_n=32, rht_signs_hi=_hi(1, 0, 0)), 64, 1),
    (dict(rht_n=64, rht_signs_hi=_hi(0, 1, 0)), 64, 1),
])
def test_quantize_rejects_rht_sizes(lib, kw, rows, status):
    assert quant(lib, desc(orient=1, rht=1, **kw), rows, 64) == status
    assert _err(lib)


def test_quantize_rht_size_is_unchecked_without_rht(lib):
    # rht_n and the high sign words only matter with rht on: an RNE rowwise
    # call with them set passes validation up to the (missing) device
    d = desc(rht_n=8, rht_signs_hi=_hi(7, 7, 7))
    assert quant(lib, d, codes=None) == 1 and "codes" in _err(lib)


def test_quantize_rejects_pointers(lib):
    assert quant(lib, desc(), x=None) == 1
    assert quant(lib, desc(), x=ctypes.c_void_p(0x10008)) == 1      # misaligned
    assert quant(lib, desc(), ld=60) == 1                           # ld < cols
    assert quant(lib, desc(), ld=68) == 1                           # ld % 8
    assert quant(lib, desc(), codes=None) == 1
    assert quant(lib, desc(), amax=None) == 1
    assert quant(lib, desc(block=1, emit_transpose=1)) == 1         # codes_t null
    assert lib.fp4_quantize(None, FAKE, 32, 64, 64, FAKE, FAKE, None, FAKE, None, None, None) == 1
    # TILED scales must be 16-byte aligned (row-major ones need not be)
    assert quant(lib, desc(scale_layout=1), scales=ctypes.c_void_p(0x10004)) == 1


def dual(lib, rd, cd, rows=32, cols=64, x=FAKE, codes=FAKE, scales=FAKE, codes_t=FAKE,
         scales_t=FAKE, amax=FAKE, amax_t=ctypes.c_void_p(0x10010)):
    return lib.fp4_quantize_dual(ctypes.byref(rd), ctypes.byref(cd), x, rows, cols, cols, codes,
                                 scales, codes_t, scales_t, amax, amax_t, None, None, None, None)


@pytest.mark.parametrize("rkw,ckw,rows,cols,status", [
    (dict(format=7), dict(orient=1), 32, 64, 1),
    (dict(), dict(orient=1, round=2), 32, 64, 1),
    (dict(orient=1), dict(orient=1), 32, 64, 3),              # first desc must be ROWWISE
    (dict(), dict(), 32, 64, 3),                              # second desc must be COLWISE
    (dict(), dict(orient=1, format=1), 32, 64, 3),            # formats differ
    (dict(), dict(orient=1, rht=1, rht_n=64), 32, 64, 2),     # rows % rht_n
    (dict(), dict(orient=1, rht=1, rht_n=5), 64, 64, 1),
    (dict(), dict(orient=1, round=1), 32, 64, 3),             # rounding modes differ
    (dict(rht=1, rht_n=32), dict(orient=1), 32, 64, 3),       # rowwise-side RHT: N 4 or 16
    (dict(rht=1, rht_n=4, rht_signs=1 << 4), dict(orient=1), 32, 64, 1),   # bits above N
    (dict(rht=1, format=2), dict(orient=1, format=2), 64, 64, 3),   # RHT with MXFP4
    (dict(format=2), dict(orient=1, format=2, rht=1), 64, 64, 3),   # RHT with MXFP4
    (dict(block=1), dict(orient=1), 32, 64, 3),               # 2D
    (dict(), dict(orient=1, emit_transpose=1), 32, 64, 3),
    (dict(format=2, amax_given=1), dict(orient=1, format=2), 64, 64, 3),
    (dict(target=-1.0), dict(orient=1), 32, 64, 1),
    (dict(), dict(orient=1, scale_layout=4), 32, 64, 1),
    (dict(), dict(orient=1), 24, 64, 2),                      # rows % 16
    (dict(), dict(orient=1), 32, 40, 2),                      # cols % 16
    (dict(format=2), dict(orient=1, format=2), 48, 64, 2),    # rows % 32
    (dict(format=3), dict(orient=1, format=3), 64, 64, 3),    # MXFP8: single quantizations
    (dict(count_level=1), dict(orient=1), 32, 64, 3),         # both sides count the same
    (dict(), dict(orient=1, count_level=5), 32, 64, 1),
    (dict(global_scope=1), dict(orient=1), 32, 64, 3),        # per-row scales: fp4_quantize
    (dict(), dict(orient=1, global_scope=1), 32, 64, 3),
])
def test_quantize_dual_rejects(lib, rkw, ckw, rows, cols, status):
    assert dual(lib, desc(**rkw), desc(**ckw), rows, cols) == status
    assert _err(lib)


def test_quantize_dual_rejects_pointers(lib):
    r, c = desc(), desc(orient=1)
    assert dual(lib, r, c, x=None) == 1
    assert dual(lib, r, c, codes_t=None) == 1
    assert dual(lib, r, c, scales_t=None) == 1
    assert dual(lib, r, c, codes_t=ctypes.c_void_p(0x10008)) == 1       # misaligned
    assert dual(lib, r, c, amax_t=None) == 1
    # a shared amax buffer is only allowed without RHT and with equal amax_given
    assert dual(lib, r, desc(orient=1, rht=1), amax_t=FAKE) == 1
    assert dual(lib, r, desc(orient=1, amax_given=1), amax_t=FAKE) == 1
    assert dual(lib, r, desc(orient=1, scale_layout=1), scales_t=ctypes.c_void_p(0x10004)) == 1
    assert lib.fp4_quantize_dual(None, ctypes.byref(c), FAKE, 32, 64, 64, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, None, None, None, None) == 1


def amax_call(lib, d, rows=32, cols=64, amax=FAKE):
    return lib.fp4_amax(None if d is None else ctypes.byref(d), FAKE, rows, cols, cols, amax, None)


def rht_call(lib, d, rows=32, cols=64, y=FAKE):
    return lib.fp4_rht16(None if d is None else ctypes.byref(d), FAKE, rows, cols, cols, y, None)


def test_other_entry_points_reject(lib):
    assert amax_call(lib, None) == 1                                          # no desc
    assert amax_call(lib, desc(orient=1, rht=1), amax=None) == 1
    assert amax_call(lib, desc(orient=1, rht=1), rows=24) == 2                # rows % 16
    assert amax_call(lib, desc(orient=0, rht=1), cols=40) == 2                # cols % 16
    assert amax_call(lib, desc(orient=0, rht=1, rht_n=128), cols=64) == 2     # cols % 128
    assert amax_call(lib, desc(orient=1, rht=1, rht_signs=1 << 16)) == 1      # bits above N
    assert amax_call(lib, desc(orient=1, rht=1, rht_n=8)) == 1                # bad size
    assert amax_call(lib, desc(orient=5)) == 1
    assert amax_call(lib, desc(orient=0), rows=1 << 31) == 2                  # too many rows
    assert amax_call(lib, desc(orient=0, global_scope=1)) == 3                # tensor amax only
    assert lib.fp4_dequantize(0, 0, 0, FAKE, FAKE, FAKE, 0, 32, 40, FAKE, 1, None) == 2
    assert lib.fp4_dequantize(2, 1, 0, FAKE, FAKE, FAKE, 0, 32, 64, FAKE, 1, None) == 3
    assert lib.fp4_dequantize(0, 0, 0, FAKE, FAKE, None, 0, 32, 64, FAKE, 1, None) == 1
    assert lib.fp4_dequantize(0, 0, 5, FAKE, FAKE, FAKE, 0, 32, 64, FAKE, 1, None) == 1
    assert lib.fp4_dequantize(0, 1, 1, FAKE, FAKE, FAKE, 0, 32, 64, FAKE, 1, None) == 3
    assert lib.fp4_dequantize(0, 0, 1, FAKE, ctypes.c_void_p(0x10008), FAKE, 0, 32, 64, FAKE, 1,
                              None) == 1
    assert lib.fp4_dequantize(0, 0, 0, FAKE, FAKE, FAKE, 2, 32, 64, FAKE, 1, None) == 1
    assert lib.fp4_dequantize(3, 1, 0, FAKE, FAKE, None, 0, 32, 64, FAKE, 1, None) == 3
    assert lib.fp4_dequantize(3, 0, 0, FAKE, FAKE, None, 1, 32, 64, FAKE, 1, None) == 3
    assert lib.fp4_dequantize(3, 0, 0, FAKE, FAKE, None, 0, 32, 48, FAKE, 1, None) == 2
    assert lib.fp4_dequantize(4, 0, 0, FAKE, FAKE, None, 0, 32, 64, FAKE, 1, None) == 1
    assert lib.fp4_dequantize(2, 0, 0, FAKE, FAKE, FAKE, 1, 32, 64, FAKE, 1, None) == 3
    assert lib.fp4_dequantize(0, 1, 0, FAKE, FAKE, FAKE, 1, 32, 64, FAKE, 1, None) == 3
    assert rht_call(lib, desc(orient=1), rows=40) == 2
    assert rht_call(lib, desc(orient=1), y=None) == 1
    assert rht_call(lib, desc(orient=1), y=ctypes.c_void_p(0x10008)) == 1    # 16-byte aligned
    assert rht_call(lib, desc(orient=0, rht_n=32), cols=48) == 2
    assert rht_call(lib, desc(orient=1, rht_n=4, rht_signs=1 << 4)) == 1
    assert rht_call(lib, None) == 1


def op(fmt=0, codes=0x10000, ld=32, rg=1, layout=0, scales=0x20000, s_dec=0x30000, scope=0):
    return api.Operand(fmt, codes, ld, scales, 4, 1, rg, s_dec, layout, scope)


@pytest.mark.parametrize("a,b,M,N,K,status", [
    (op(0), op(2), 16, 16, 64, 3),          # formats differ
    (op(0), op(0), 16, 16, 40, 2),          # K % 16
    (op(2), op(2), 16, 16, 48, 2),          # K % 32
    (op(0), op(0), -1, 16, 64, 2),
    (op(0, rg=3), op(0), 16, 16, 64, 1),
    (op(2, rg=16), op(2), 16, 16, 64, 3),   # 2D scales with MXFP4
    (op(0, ld=16), op(0), 16, 16, 64, 1),   # ld_codes < K/2
    (op(0, codes=0x10004), op(0), 16, 16, 64, 1),
    (op(0, codes=0), op(0), 16, 16, 64, 1),
    (op(0, layout=3), op(0), 16, 16, 64, 1),
    (op(0, layout=1, rg=16), op(0), 16, 16, 64, 3),          # TILED scales are 1D
    (op(2, layout=1, scales=0x20008), op(2), 16, 16, 64, 1),  # TILED misaligned
    (op(3), op(3), 16, 16, 64, 3),                            # no MXFP8 GEMM
    (op(0, scope=2), op(0), 16, 16, 64, 1),                   # bad s_dec scope
    (op(2, scope=1), op(2), 16, 16, 64, 3),                   # per-row s_dec with MXFP4
    (op(0), op(0, scope=1, s_dec=0), 16, 16, 64, 3),          # per-row s_dec is required
])
def test_gemm_rejects(lib, a, b, M, N, K, status):
    assert lib.fp4_gemm(ctypes.byref(a), ctypes.byref(b), M, N, K, FAKE, 0, N, 0, None) == status
    assert _err(lib)


def test_empty_calls_are_noops(lib):
    # nothing to do: accepted without any device work
    a, b = op(0), op(0)
    assert lib.fp4_gemm(ctypes.byref(a), ctypes.byref(b), 0, 16, 64, None, 0, 16, 0, None) == 0
    assert lib.fp4_gemm(ctypes.byref(a), ctypes.byref(b), 0, 16, 64, None, 1, 16, 0, None) == 0
    assert lib.fp4_dequantize(0, 0, 0, None, None, None, 0, 0, 64, None, 1, None) == 0


def test_gemm_rejects_output_type(lib):
    a, b = op(0), op(0)
    assert lib.fp4_gemm(ctypes.byref(a), ctypes.byref(b), 16, 16, 64, FAKE, 2, 16, 0, None) == 1
    assert "d_type" in _err(lib)


def test_geometry_control_rejects(lib):
    assert lib.fp4_selftest_set_geometry(-1, 0) == 1
    assert lib.fp4_selftest_set_geometry(0, 128) == 1
    assert lib.fp4_selftest_set_geometry(5, 192) == 0      # accepted: no device work
    assert lib.fp4_selftest_set_geometry(0, 0) == 0


def test_selftest_sweep_rejects(lib):
    # validation happens on the host before any device work
    assert lib.fp4_selftest_sweep(5, FAKE, 7, FAKE, None) == 1
    assert lib.fp4_selftest_sweep(4, FAKE, 7, FAKE, None) == 1      # E4M3 elements take 126
    assert "126 thresholds" in _err(lib)
    assert lib.fp4_selftest_sweep(-1, FAKE, 7, FAKE, None) == 1
    assert lib.fp4_selftest_sweep(3, FAKE, 6, FAKE, None) == 1      # E2M1 SR takes 7
    assert "7 thresholds" in _err(lib)
    assert lib.fp4_selftest_sweep(3, None, 7, FAKE, None) == 1
    assert lib.fp4_selftest_sweep(3, FAKE, 7, None, None) == 1


def test_status_strings(lib):
    assert lib.fp4_status_string(0) == b"ok"
    assert lib.fp4_status_string(3) == b"unsupported combination"


def test_operand_keeps_its_storage_alive():
    """A GEMM operand carries raw device pointers, so it must keep the
    quantized tensors it points into alive: dropping the Quantized object
    right after .operand() must not free them (a later allocator flush would
    unmap memory the GEMM still reads)."""
    import gc
    import weakref
    import torch
    codes = torch.zeros((32, 16), dtype=torch.uint8)
    scales = torch.zeros((32, 2), dtype=torch.uint8)
    s_dec = torch.ones(1)
    q = api.Quantized(api.NVFP4, api.BLOCK_1D, 32, 32, codes, scales, s_dec, s_dec.clone())
    ref = weakref.ref(codes)
    op = q.operand()
    del q, codes, scales
    gc.collect()
    assert ref() is not None and op.codes == ref().data_ptr()
    del op
    gc.collect()
    assert ref() is None


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of the ABI structs have the C header's size and
    field offsets (compiled with the host C compiler)."""
    exe = tmp_path / "abi_layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_layout.c"), "-o", str(exe)], check=True)
    c = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines():
        k, v = line.split()
        c[k] = int(v)
    for name, cls in (("fp4_quant_desc", api.QuantDesc), ("fp4_operand", api.Operand)):
        assert ctypes.sizeof(cls) == c[name + ".__size__"], name
        for field, _ in cls._fields_:
            assert getattr(cls, field).offset == c["%s.%s" % (name, field)], (name, field)
    assert c["fp4_counters.__size__"] == 5 * 8
