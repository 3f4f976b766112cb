"""Build libfp4_mi355x.so (gfx950) in-tree with hipcc.

Every translation unit is compiled with:
  --offload-arch=gfx950 -O3      the only target
  -ffp-contract=off              no fused multiply-add: the quantizer's fp32
                                 scale arithmetic must round after every op
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                 no packed fp32 instructions
fp32 denormals stay enabled and fp32 division stays correctly rounded
(hipcc's defaults; neither -ffast-math nor flush-to-zero is used).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libfp4_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

# (source, object name, extra flags): gemm_nv.hip is built once per
# block-scale format and gemm_nv_dma.hip once per format and tile height, so
# the kernel families compile in parallel
SOURCES = [("quant.hip", "quant", []), ("quant_rowscope.hip", "quant_rowscope", []),
           ("quant_mxfp8.hip", "quant_mxfp8", []),
           ("gemm.hip", "gemm", [])] + [
    ("gemm_nv.hip", "gemm_nv_%d" % f, ["-DFP4_NV_FMT=%d" % f]) for f in (0, 1)] + [
    ("gemm_nv_dma.hip", "gemm_nv_dma_%d_%d" % (f, mi), ["-DFP4_DMA_FMT=%d" % f, "-DFP4_DMA_MI=%d" % mi])
    for f in (0, 1) for mi in (4, 3)] + [
    ("gemm_mx.hip", "gemm_mx", []), ("gemm_mx_dma.hip", "gemm_mx_dma", []),
    ("selftest.hip", "selftest", []), ("fp4_api.cpp", "fp4_api", [])]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-fvisibility=hidden", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in p.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), p.stdout, err))
    return err


def _stale(obj, src):
    """True if obj is missing or older than its source or any header."""
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    deps += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose=False, incremental=False):
    """Compile every source (incremental=True: only those whose object is
    older than the source or any header) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src, name, extra in SOURCES:
        obj = os.path.join(BUILD, name + ".o")
        objs.append(obj)
        if incremental and not _stale(obj, os.path.join(CSRC, src)):
            continue
        cmds.append([HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, len(cmds))) as ex:
        for err in ex.map(_run, cmds):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


CLANG = "/opt/rocm/llvm/bin/clang++"
SANITIZED_LIB = os.path.join(BUILD, "sanitize", "libfp4_mi355x_sanitized.so")


def build_sanitized():
    """The C ABI's host code (fp4_api.cpp: every argument check) built as
    plain host C++ with AddressSanitizer and UndefinedBehaviorSanitizer
    (every UB report fatal), linked against host-only stand-ins for the
    kernel launchers (csrc/sanitize_stubs.cpp).  Loaded in place of the real
    library (FP4_LIB) by tests that never reach a device.  Returns the
    library path."""
    out_dir = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-std=c++17", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")]
    objs = []
    for src in ("fp4_api.cpp", "sanitize_stubs.cpp"):
        obj = os.path.join(out_dir, src.replace(".cpp", ".o"))
        _run([CLANG] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    _run([CLANG, "-shared", "-shared-libasan", "-fsanitize=address,undefined", "-o",
          SANITIZED_LIB] + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return SANITIZED_LIB


def sanitizer_runtime():
    """Path of clang's shared ASan runtime (to LD_PRELOAD into a process that
    loads the sanitized library)."""
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
