"""Benchmark: one step = the whole FP4 hot path of one linear layer.

Default workload: the 8B hybrid model's FFN up-projection (X [8192, 4096],
W [21504, 4096], dY [8192, 21504]) with UE5M3 block scales and stale tensor
amaxes (T = 448 for X and W, 2048 for dY), on synthetic seeded tensors
already resident in HBM.  A step runs:

  quantize X rowwise + colwise (RNE, one read)   -> Fprop A, Wgrad B
  quantize W 16x16 2D (+ W^T)                    -> Fprop B, Dgrad B
  quantize dY rowwise + colwise (SR, one read)   -> Dgrad A, Wgrad A
  GEMMs Fprop, Dgrad, Wgrad                      (fp32 outputs)

(NVFP4 workloads, --config 2|3|5, add the tensor amax passes; --separate-quant
quantizes each orientation with its own read.)  Event counters are kept on
every quantization.  The step is captured once as a HIP graph and replayed
(after a bitwise check of replays against the eager step).  Per-kernel
durations come from graphs that run each op after a 512 MiB read (which
evicts the 256 MB Infinity Cache), minus the same graph without the op,
timed with events on the launch stream.  Printed: one JSON line whose
`value` is the step's GEMM throughput (3 x 2MNK / step time, TFLOP/s),
per-kernel timings and rates (`parts`), the roofline of the dominant kernel
and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--config 2|3|4|5] [--no-cpu] [--separate-quant]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantize GB/s (% HBM peak); FP4 block-scaled GEMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp16": 2500.0, "fp4": 10100.0}   # dense MFMA, MI355X
# rocprofv3 counter summaries of the dominant (GEMM) kernel, per workload
PROFILE_TRAFFIC = {2: os.path.join(ROOT, "profiles", "traffic_gemm_nvfp4_1.2b_ffn.txt"),
                   4: os.path.join(ROOT, "profiles", "traffic_gemm_ue5m3_8b_ffn.txt")}
FLUSH_BYTES = 512 << 20     # read before each timed op: more than the 256 MB Infinity Cache

# algorithmic bytes per element
B_AMAX = 2.0
B_Q1D = {"nvfp4": 2.0 + 0.5 + 1.0 / 16, "ue5m3": 2.0 + 0.5 + 1.0 / 16, "mxfp4": 2.0 + 0.5 + 1.0 / 32}
B_Q2D_T = 2.0 + 0.5 + 0.5 + 1.0 / 256
# one read, rowwise and colwise codes + scales written
B_DUAL = {"nvfp4": 2.0 + 2 * (0.5 + 1.0 / 16), "ue5m3": 2.0 + 2 * (0.5 + 1.0 / 16),
          "mxfp4": 2.0 + 2 * (0.5 + 1.0 / 32)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, choices=(2, 3, 4, 5))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the CPU oracle's sample (W is quantized in full)")
    ap.add_argument("--layer", action="store_true",
                    help="time QuantizedLinear.forward + backward (the layer a user calls) "
                         "instead of the step's kernel list")
    ap.add_argument("--rht-n", type=int, default=16, choices=(4, 16, 32, 64, 128),
                    help="--layer on the 12B workload: size of the RHT")
    ap.add_argument("--act-2d", action="store_true",
                    help="--layer: 16x16 blocks for X and dY too (the 2D-block recipe; no RHT)")
    ap.add_argument("--scale-up", action="store_true",
                    help="--layer: truncation-free (rounded-up) block scales")
    ap.add_argument("--no-rht", action="store_true",
                    help="--layer on the 12B workload: leave out the RHT of the Wgrad operands")
    ap.add_argument("--serial", action="store_true",
                    help="run the step's kernels one after another on one stream")
    ap.add_argument("--separate-quant", action="store_true",
                    help="quantize X and dY rowwise and colwise in separate kernels (two reads "
                         "each) instead of one dual kernel per tensor")
    ap.add_argument("--counters-run", action="store_true",
                    help="run each op of the step once, eagerly, then a 512 MiB calibration "
                         "kernel, for rocprofv3 --pmc; prints nothing else")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="per-kernel durations from a rocprofv3 kernel trace of a default run: "
                         "all launches, and the isolated launches of the per-op timing graphs")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of two --counters-run passes (FETCH_SIZE, "
                         "WRITE_SIZE) into the GEMM traffic summary")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PASS_A_CSV", "PASS_B_CSV"),
                    help="per-kernel SQ counter summary of two --counters-run passes (the "
                         "counters of SQ_PASS_A and SQ_PASS_B); needs --ops-json")
    ap.add_argument("--ops-json", metavar="PATH",
                    help="--counters-run: write the step's ops in launch order here; "
                         "--summarize-sq: read them")
    return ap.parse_args()


CAL_BYTES = 512 << 20       # calibration kernel: reads and writes this many bytes
# Events the step's quantizations count: the block-scale saturation and
# underflow events the UE5M3 workload asks for ("scales"; "all" adds the
# per-element events, about a quarter more quantizer work).
COUNT = "scales"


def counters_run(ops, host, ops_json=None):
    """One eager pass of the step's ops, then y = 2 x on CAL_BYTES of fp32
    (a plain streaming kernel of known traffic) to calibrate the counters.
    ops_json: also write the ops in launch order (name, kind, algorithmic
    units, elements of the tensor a quantization reads) for --summarize-sq."""
    import torch
    if ops_json:
        numel = {k: int(v.numel()) for k, v in host["device"].items()}
        rows = []
        for (name, kind, units, _) in ops:
            tensor = next((t for t in ("dY", "X", "W") if (" " + t + " ") in (name + " ")), None)
            rows.append({"name": name, "kind": kind, "units": units,
                         "elements": numel.get(tensor) if not name.startswith("gemm") else None})
        with open(ops_json, "w") as f:
            json.dump(rows, f)
    for (_, _, _, f) in ops:
        f()
    x = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        torch.mul(x, 2.0, out=y)
    torch.cuda.synchronize()


def summarize_pmc(fetch_csv, write_csv, cfg):
    """Per-launch HBM bytes of every library kernel of the step from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the same
    counter reads for the calibration kernel of known size; the GEMM line
    (mean over its launches) is what the roofline's `traffic` reports."""
    import csv

    def per_dispatch(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = int(r["Dispatch_Id"])
                rows[key] = (r["Kernel_Name"], rows.get(key, ("", 0.0))[1] + float(r["Counter_Value"]))
        return [rows[k] for k in sorted(rows)]

    def short(n):
        n = n.replace("void ", "").replace("fp4gemm::", "").replace("(anonymous namespace)::", "")
        return n.split("(")[0]

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = per_dispatch(path, counter)
        lib = [(short(n), v) for (n, v) in d if "k_gemm" in n or "k_quant" in n or "k_amax" in n]
        cal = [v for (n, v) in d if "elementwise" in n.lower() and "mul" in n.lower()]
        if not lib or not cal:
            raise SystemExit("no library or calibration dispatches in %s" % path)
        factor = CAL_BYTES / (np.mean(cal[-2:]) * 1024.0)     # bytes per counted byte
        out[counter] = (lib, factor)
    fetch, f_fac = out["FETCH_SIZE"]
    write, w_fac = out["WRITE_SIZE"]
    lines = ["kernel_source_sha256_16=%s" % source_hash(*GEMM_SOURCES),
             "calibration_fetch_factor=%.4f" % f_fac, "calibration_write_factor=%.4f" % w_fac]
    gemm_tot = []
    gnames = iter(["fprop", "dgrad", "wgrad"])
    for (n, fv), (_, wv) in zip(fetch, write):
        fb, wb = fv * 1024.0 * f_fac, wv * 1024.0 * w_fac
        tag = next(gnames) if "k_gemm" in n else "quant"
        if "k_gemm" in n:
            gemm_tot.append(fb + wb)
        lines.append("%s %s fetch_bytes=%.0f write_bytes=%.0f" % (tag, n, fb, wb))
    lines.append("hbm_bytes_per_launch=%.0f" % float(np.mean(gemm_tot)))
    print("\n".join(lines))


# SQ counters of the two passes --summarize-sq reads (8 SQ counters each)
SQ_PASS_A = ("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
             "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY")
SQ_PASS_B = ("SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_ANY",
             "SQ_WAIT_ANY", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_VMEM", "SQ_INSTS_VMEM_RD")
SQ_INSTANCES = 32      # SQ_BUSY_CYCLES sums the 32 shader engines (8 XCDs x 4)
SIMDS = 1024           # 256 CUs x 4 SIMDs


def summarize_sq(csv_a, csv_b, ops_json):
    """Per-kernel SQ counter summary of one eager pass of the step (the
    dispatches of --counters-run, matched to the ops in launch order).

    clock_GHz      SQ_BUSY_CYCLES / 32 engines / kernel duration
    valu_busy      SQ_INSTS_VALU x 4 cycles (a wave64 VALU op on a 16-lane
                   SIMD) / (1024 SIMDs x busy cycles per engine)
    mfma_busy      SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x busy cycles per engine)
    valu_ops/elem  64 x SQ_INSTS_VALU / elements of the quantized tensor
    wait_frac      SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave-cycles waiting on s_waitcnt)
    lds_conflict   SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS
    (durations are those of the profiled pass: counters slow kernels down)."""
    import csv

    def load(path):
        d = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = int(r["Dispatch_Id"])
                e = d.setdefault(key, {"name": r["Kernel_Name"],
                                       "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [d[k] for k in sorted(d)]

    def short(n):
        n = n.replace("void ", "").replace("fp4gemm::", "").replace("(anonymous namespace)::", "")
        return n.split("(")[0]
    lib = lambda rows: [r for r in rows if any(k in r["name"] for k in ("k_quant", "k_gemm", "k_amax"))]
    a, b = lib(load(csv_a)), lib(load(csv_b))
    with open(ops_json) as f:
        ops = json.load(f)
    a, b = a[-len(ops):], b[-len(ops):]
    lines = ["%-22s %-40s %8s %6s %6s %6s %9s %6s %6s" % (
        "op", "kernel", "us", "GHz", "valu", "mfma", "valu/elem", "wait", "ldsbc")]
    for op, ra, rb in zip(ops, a, b):
        cyc = ra["SQ_BUSY_CYCLES"] / SQ_INSTANCES
        valu = ra["SQ_INSTS_VALU"] * 4.0 / (SIMDS * cyc)
        mfma = ra["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc)
        per_elem = ("%9.1f" % (64.0 * ra["SQ_INSTS_VALU"] / op["elements"])
                    if op["elements"] else "%9s" % "-")
        wait = ra["SQ_WAIT_INST_ANY"] / max(ra["SQ_WAVE_CYCLES"], 1.0)
        bc = rb["SQ_LDS_BANK_CONFLICT"] / max(rb["SQ_ACTIVE_INST_LDS"], 1.0)
        lines.append("%-22s %-40s %8.1f %6.2f %6.3f %6.3f %s %6.3f %6.3f" % (
            op["name"][:22], short(ra["name"])[:40], ra["ns"] / 1e3, cyc / ra["ns"], valu, mfma,
            per_elem, wait, bc))
    print("\n".join(lines))


# every source the GEMM kernels are built from
GEMM_SOURCES = ("gemm.hip", "gemm_common.hpp", "gemm_nv.hip", "gemm_nv_dma.hip", "gemm_mx.hip",
                "gemm_mx_dma.hip", "fp4_device.hpp")


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp4_block_scaled_x16_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(cfg, kernel_hash):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary of this workload, if it was taken on the current kernel
    source."""
    path = PROFILE_TRAFFIC.get(cfg)
    if path is None or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and " " not in line.split("=", 1)[0] and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_step(cfg, dev, dual=True):
    """Inputs on the device and the list of (name, kind, units, fn) ops."""
    import torch
    from fp4_block_scaled_x16_amd import api, inputs
    
    c = inputs.CONFIGS[cfg]
    fmt = c["fmt"]
    T, din, dout = c["tokens"], c["d_in"], c["d_out"]
    t = inputs.linear_tensors(cfg)
    X = torch.from_numpy(t["X"].view(np.int16)).to(dev)
    W = torch.from_numpy(t["W"].view(np.int16)).to(dev)
    dY = torch.from_numpy(t["dY"].view(np.int16)).to(dev)
    cnt = api.new_counters(dev)
    rht = cfg == 3
    target_x = target_w = target_dy = 448.0
    stale, host_stale = {}, {}
    if fmt == "ue5m3":
        # the stale amax: from the same distribution drawn 50 steps earlier
        # (seed offset 50), divided by 1.5 so the current tensors overshoot it
        target_dy = 2048.0
        for name, gen, shape in (("X", inputs.activations, X.shape), ("W", inputs.weights, W.shape),
                                 ("dY", inputs.gradients, dY.shape)):
            host_stale["stale_" + name] = gen(tuple(shape), cfg_seed=inputs.STALE_SEED_OFFSET)
            b = torch.from_numpy(host_stale["stale_" + name].view(np.int16)).to(dev)
            stale[name] = (api.amax(b) / 1.5).contiguous()
            del b
    D_f = torch.empty((T, dout), dtype=torch.float32, device=dev)
    D_d = torch.empty((T, din), dtype=torch.float32, device=dev)
    D_w = torch.empty((dout, din), dtype=torch.float32, device=dev)
    st = {}
    sig = inputs.rht_sign_mask()

    def amax_op(name, x):
        def f():
            if name in stale:
                st["amax_" + name] = stale[name]
            else:
                st["amax_" + name] = api.amax(x)
        return f

    def amax_rot_op(name, x):
        def f():
            st["amax_rot_" + name] = api.amax(x, rht=True, signs=sig)
        return f

    ops = []
    two_level = fmt != "mxfp4"
    # With the RHT and dual quantization, X's and dY's plain and rotated
    # amax come from one read inside the dual quantizer (no separate ops).
    fused_amax = rht and dual
    if two_level:
        ops += [("amax W", "hbm", B_AMAX * W.numel(), amax_op("W", W))]
        if not fused_amax:
            ops += [("amax X", "hbm", B_AMAX * X.numel(), amax_op("X", X)),
                    ("amax dY", "hbm", B_AMAX * dY.numel(), amax_op("dY", dY))]
        if fmt == "ue5m3":     # stale amaxes given: nothing to compute in the step
            for name in ("X", "W", "dY"):
                st["amax_" + name] = stale[name]
            ops = []
        if rht and not fused_amax:
            ops += [("amax rot X", "hbm", B_AMAX * X.numel(), amax_rot_op("X", X)),
                    ("amax rot dY", "hbm", B_AMAX * dY.numel(), amax_rot_op("dY", dY))]
    b1 = B_Q1D[fmt]

    def q(name, x, out, **kw):
        def f():
            if two_level:
                key = ("amax_rot_" if kw.get("rht") else "amax_") + name
                kw2 = dict(kw, amax_in=st[key])
            else:
                kw2 = kw
            if kw2.get("block") != "2d":
                kw2 = dict(kw2, scale_layout="tiled")   # the GEMM-friendly 1D scale layout
            st[out] = api.quantize(x, fmt, counters=cnt, count=COUNT, **kw2)
        return f

    def qd(name, x, out_r, out_c, **kw):
        """Rowwise and colwise codes of x from one read (RHT on the colwise side)."""
        def f():
            kw2 = dict(kw, scale_layout="tiled")
            if two_level and not fused_amax:
                kw2["amax_in"] = st["amax_" + name]
                kw2["amax_t_in"] = st[("amax_rot_" if kw.get("rht") else "amax_") + name]
            st[out_r], st[out_c] = api.quantize_dual(x, fmt, counters=cnt, count=COUNT, **kw2)
        return f

    bd = B_DUAL[fmt] + (B_AMAX if fused_amax else 0.0)   # + the amax read when fused
    if dual:
        ops.append(("quant X row+col", "hbm", bd * X.numel(),
                    qd("X", X, "qx", "qxc", rht=rht, signs=sig if rht else 0, target=target_x)))
    else:
        ops.append(("quant X row", "hbm", b1 * X.numel(), q("X", X, "qx", target=target_x)))
    if two_level:
        ops.append(("quant W 2d+T", "hbm", B_Q2D_T * W.numel(),
                    q("W", W, "qw", block="2d", emit_transpose=True, target=target_w)))
    elif dual:
        ops.append(("quant W row+col", "hbm", bd * W.numel(), qd("W", W, "qw", "qwc")))
    else:
        ops.append(("quant W row", "hbm", b1 * W.numel(), q("W", W, "qw")))
        ops.append(("quant W col", "hbm", b1 * W.numel(), q("W", W, "qwc", orient="col")))
    if dual:
        ops.append(("quant dY row+col SR", "hbm", bd * dY.numel(),
                    qd("dY", dY, "qdy", "qdyc", rnd="sr", seed=1, offset=0, offset_t=1, rht=rht,
                       signs=sig if rht else 0, target=target_dy)))
    else:
        ops.append(("quant dY row SR", "hbm", b1 * dY.numel(),
                    q("dY", dY, "qdy", rnd="sr", seed=1, offset=0, target=target_dy)))
        ops.append(("quant dY col SR", "hbm", b1 * dY.numel(),
                    q("dY", dY, "qdyc", orient="col", rnd="sr", seed=1, offset=1, rht=rht,
                      signs=sig if rht else 0, target=target_dy)))
        ops.append(("quant X col", "hbm", b1 * X.numel(),
                    q("X", X, "qxc", orient="col", rht=rht, signs=sig if rht else 0,
                      target=target_x)))

    def g(a, la, b, lb, M, N, K, out):
        def f():
            A = st[a].operand()
            B = st[b].operand(transposed=(lb == "T")) if two_level else st[b].operand()
            api.gemm(A, B, M, N, K, out=out)
        return f

    fl = lambda M, N, K: 2.0 * M * N * K
    ops.append(("gemm fprop", "mfma", fl(T, dout, din), g("qx", "r", "qw", "r", T, dout, din, D_f)))
    ops.append(("gemm dgrad", "mfma", fl(T, din, dout),
                g("qdy", "r", "qw" if two_level else "qwc", "T", T, din, dout, D_d)))
    ops.append(("gemm wgrad", "mfma", fl(dout, din, T), g("qdyc", "r", "qxc", "r", dout, din, T, D_w)))
    return ops, cnt, dict(X=t["X"], W=t["W"], dY=t["dY"], gpu_outputs=(D_f, D_d, D_w),
                          device=dict(X=X, W=W, dY=dY), fprop_out=D_f,
                          targets=dict(X=target_x, W=target_w, dY=target_dy), **host_stale), fmt


def cpu_cores():
    """Host cores this process may run on (at most 16, the host share of one GPU)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_chunk(task):
    """Pool worker: the oracle's quantization of one chunk and its exactly
    dequantized GEMM operand values (fp64) -> (values, s_dec)."""
    from oracle import quantize as Q
    bits, fmt, layout, kw = task
    if layout == "2d":
        q = Q.quantize(bits, fmt, block="2d", emit_transpose=True, **kw)
        R, C = bits.shape
        return Q.operand_values(q["codes"], q["scales"], fmt, "2d", R, C), q["s_dec"]
    q = Q.quantize(bits, fmt, orient=layout, **kw)
    R, Cc = q["codes"].shape
    return Q.operand_values(q["codes"], q["scales"], fmt, "1d", R, 2 * Cc), q["s_dec"]


def _oracle_amax_chunk(task):
    from oracle import formats as F
    from oracle import quantize as Q
    bits, rht, signs = task
    xf = F.bf16_bits_to_f32(bits)
    if rht:
        from oracle.rht import rht16_cols
        xf = rht16_cols(xf, signs)
    return float(Q.tensor_amax(xf))


def _pooled_quantize(pool, n, bits, fmt, layout, **kw):
    """Operand values of one quantized operand, chunked over the pool: rows
    for rowwise and 2D (16-row groups), columns for colwise (each chunk
    keeps its Philox indices through index_base)."""
    if fmt != "mxfp4" and "amax" not in kw:
        raise ValueError("chunks of a two-level quantization need the tensor amax")
    R, C = bits.shape
    tasks = []
    if layout == "col":
        step = -(-C // n)
        for c0 in range(0, C, step):
            tasks.append((np.ascontiguousarray(bits[:, c0:c0 + step]), fmt, "col",
                          dict(kw, index_base=c0 * R)))
        parts = pool.map(_oracle_chunk, tasks)
        return np.concatenate([p[0] for p in parts], axis=0), parts[0][1]
    unit = 16 if layout == "2d" else 1
    step = -(-R // (n * unit)) * unit
    for r0 in range(0, R, step):
        k = dict(kw) if layout == "2d" else dict(kw, index_base=r0 * C)
        tasks.append((bits[r0:r0 + step], fmt, layout, k))
    parts = pool.map(_oracle_chunk, tasks)
    return np.concatenate([p[0] for p in parts], axis=0), parts[0][1]


def cpu_baseline(cfg, host, fmt, tokens, pool):
    """The CPU oracle on a token slab of the same step (W quantized in full):
    quantizers over a process pool of the host's cores, fp64 BLAS GEMMs on
    the same number of threads."""
    from threadpoolctl import threadpool_limits
    from oracle import formats as F
    from oracle import quantize as Q
    from oracle import gemm as G
    from fp4_block_scaled_x16_amd import inputs

    n = cpu_cores()
    X, W, dY = host["X"][:tokens], host["W"], host["dY"][:tokens]
    rht = cfg == 3
    sig = inputs.rht_sign_mask()
    two_level = fmt != "mxfp4"
    tgt_dy = 2048.0 if fmt == "ue5m3" else 448.0
    # stale amaxes (UE5M3) are inputs of the step, not part of it
    stale = {}
    if fmt == "ue5m3":
        for name in ("X", "W", "dY"):
            stale[name] = np.float32(Q.tensor_amax(F.bf16_bits_to_f32(host["stale_" + name]))
                                     / np.float32(1.5))

    def amax(name, bits, rot=False):
        if not two_level:
            return {}
        if name in stale:
            return {"amax": stale[name]}
        step = -(-bits.shape[0] // (16 * n)) * 16
        parts = pool.map(_oracle_amax_chunk, [(bits[r:r + step], rot, sig)
                                              for r in range(0, bits.shape[0], step)])
        return {"amax": np.float32(max(parts))}

    t0 = time.perf_counter()
    kx = dict(amax("X", X))
    kxc = dict(amax("X", X, rht), rht=rht, signs=sig) if rht else kx
    kdy = dict(amax("dY", dY), rnd="sr", seed=1, target=tgt_dy)
    kdyc = dict(amax("dY", dY, rht), rnd="sr", seed=1, target=tgt_dy, rht=rht, signs=sig) \
        if rht else kdy
    kw_ = dict(amax("W", W))
    xv, sx = _pooled_quantize(pool, n, X, fmt, "row", **kx)
    xcv, sxc = _pooled_quantize(pool, n, X, fmt, "col", **kxc)
    dyv, sdy = _pooled_quantize(pool, n, dY, fmt, "row", offset=0, **kdy)
    dycv, sdyc = _pooled_quantize(pool, n, dY, fmt, "col", **dict(kdyc, offset=1))
    if two_level:
        wv, sw = _pooled_quantize(pool, n, W, fmt, "2d", **kw_)
        wtv = wv.T
    else:
        wv, sw = _pooled_quantize(pool, n, W, fmt, "row")
        wtv, _ = _pooled_quantize(pool, n, W, fmt, "col")
    t_q = time.perf_counter() - t0
    s = (lambda v: v) if two_level else (lambda v: 1.0)
    with threadpool_limits(limits=n, user_api="blas"):
        d_f = G.gemm_ref(xv, wv, s(sx), s(sw))
        d_d = G.gemm_ref(dyv, np.ascontiguousarray(wtv), s(sdy), s(sw))
        d_w = G.gemm_ref(np.ascontiguousarray(dycv), np.ascontiguousarray(xcv), s(sdyc), s(sxc))
    dt = time.perf_counter() - t0
    T = tokens
    din, dout = X.shape[1], W.shape[0]
    flops = 2.0 * T * dout * din * 3
    del d_f, d_d, d_w
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "sample": "the same step on %d of %d tokens (W quantized in full), %.1f s: "
                      "quantizers %.1f s over a pool of %d processes, GEMMs %.1f s in fp64 BLAS "
                      "on %d threads" % (tokens, host["X"].shape[0], dt, t_q, n, dt - t_q, n),
            "seconds": round(dt, 3), "cpu_model": cpu_model()}


def layer_main(args, dev):
    """Forward + backward of QuantizedLinear on a workload's tensors, captured
    as one graph: the end-to-end time of the FP4 layer (amax, quantization,
    three GEMMs, fp32 Wgrad accumulation)."""
    import torch
    from fp4_block_scaled_x16_amd import inputs
    from fp4_block_scaled_x16_amd.linear import QuantizedLinear, Recipe

    cfg = args.config
    c = inputs.CONFIGS[cfg]
    fmt = c["fmt"]
    t = inputs.linear_tensors(cfg)
    X, W, dY = (torch.from_numpy(t[n].view(np.int16)).to(dev) for n in ("X", "W", "dY"))
    rht = cfg == 3 and not args.no_rht and not args.act_2d
    r = Recipe(fmt, target_dy=2048.0 if fmt == "ue5m3" else 448.0, rht=rht, rht_n=args.rht_n,
               rht_signs=inputs.rht_sign_bits(args.rht_n) if rht else 0,
               act_block="2d" if args.act_2d else "1d",
               scale_round="up" if args.scale_up else "rne")
    layer = QuantizedLinear(W, r)

    def step():
        layer.forward(X)
        layer.backward(dY)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 3 * 2.0 * c["tokens"] * c["d_in"] * c["d_out"]
    print(json.dumps({
        "metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "data": "synthetic (seeded PCG64, bf16 inputs resident in HBM)",
        "config": {"workload": c["name"].replace("-rht", "") + ("-rht" if rht else "") + "-layer",
                   "format": fmt, "rht": rht, "rht_n": args.rht_n if rht else None,
                   "act_block": r.act_block, "scale_round": r.scale_round,
                   "tokens": c["tokens"], "d_in": c["d_in"], "d_out": c["d_out"],
                   "amax": "current (recomputed every step)", "wgrad": "fp32 accumulate"},
        "counters_all_runs": {k: int(v) for k, v in zip(("scale_saturated", "scale_underflow",
                                                 "scale_subnormal", "elem_saturated",
                                                 "elem_underflow"),
                                                layer.counters.cpu().tolist())},
    }))


OP_TIMING_LAUNCHES = 40     # per op and graph: R = 10 launches, replayed 1 + 3 times


def summarize_trace(path):
    """Average duration of each library kernel over all its launches, and
    over the per-op timing graphs (each kernel alone on the GPU): the first
    OP_TIMING_LAUNCHES launches of the kernel after the first cache flush
    (torch's row-wise max over the 512 MiB buffer), each after a flush
    (`parts`), and the next OP_TIMING_LAUNCHES, back to back (`parts_warm`);
    as opposed to the step replays before them, where independent kernels
    run side by side.  A kernel that several ops launch (k_amax in a
    current-amax step) reports the graphs of the first of them; kernels the
    step does not launch (the per-row-scale comparison's, the stale amaxes'
    setup) get no per-op columns."""
    import csv
    import collections
    by = collections.defaultdict(list)
    flush_t = []
    with open(path) as f:
        for r in csv.DictReader(f):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            if "reduce_kernel" in r["Kernel_Name"] and "MaxNanFunctor" in r["Kernel_Name"]:
                flush_t.append(t0)
                continue
            n = r["Kernel_Name"].replace("void ", "").replace("fp4gemm::", "")
            n = n.replace("(anonymous namespace)::", "").split("(")[0]
            if n.startswith(("k_gemm", "k_quant", "k_amax")):
                by[n].append((t0, (t1 - t0) / 1e3))
    if not flush_t:
        raise SystemExit("no cache-flush launches in %s" % path)
    first_flush = min(flush_t)
    L = OP_TIMING_LAUNCHES
    print("| kernel | calls | avg us, all | avg us, alone after a cache flush | avg us, alone back to back |")
    print("|---|---:|---:|---:|---:|")
    for n, v in by.items():
        v = sorted(v)
        d = [x[1] for x in v]
        after = [x[1] for x in v if x[0] >= first_flush]
        # the step ran it: an eager warmup, two checked replays and the timed
        # ones, so at least 4 launches before the flushes (the three amax
        # launches that set up stale amaxes do not count)
        if len(d) - len(after) >= 4 and len(after) >= 2 * L:
            cold, warm = after[:L], after[L:2 * L]
            cols = "%.1f | %.1f" % (sum(cold) / L, sum(warm) / L)
        else:
            cols = "- | -"
        print("| %s | %d | %.1f | %s |" % (n, len(d), sum(d) / len(d), cols))


def format_comparison(dev):
    """MXFP4 against NVFP4 on the 8B workload's identical tensors, every
    operand 1D in both formats (W rowwise for Fprop, colwise for Dgrad), RNE
    for X and W, SR for dY: each format's relative Frobenius quantization
    error ||dq(q(x)) - x||_F / ||x||_F per tensor, and its three GEMMs'
    durations (graphs of 10 launches on the launch stream)."""
    import torch
    from fp4_block_scaled_x16_amd import api, inputs

    c = inputs.CONFIGS[5]
    T, din, dout = c["tokens"], c["d_in"], c["d_out"]
    t = inputs.linear_tensors(5)
    ten = {n: torch.from_numpy(t[n].view(np.int16)).to(dev) for n in ("X", "W", "dY")}
    del t
    out = {}
    for fmt in ("mxfp4", "nvfp4"):
        qx, qxc = api.quantize_dual(ten["X"], fmt, scale_layout="tiled")
        qw, qwc = api.quantize_dual(ten["W"], fmt, scale_layout="tiled")
        qdy, qdyc = api.quantize_dual(ten["dY"], fmt, rnd="sr", seed=1, offset=0, offset_t=1,
                                      scale_layout="tiled")
        err = {}
        for name, q in (("X", qx), ("W", qw), ("dY", qdy)):
            xf = ten[name].view(torch.bfloat16).double()
            dq = api.dequantize(q).double()
            err[name] = float(torch.linalg.vector_norm(dq - xf) / torch.linalg.vector_norm(xf))
            del xf, dq
        gemms = {"fprop": (qx, qw, T, dout, din), "dgrad": (qdy, qwc, T, din, dout),
                 "wgrad": (qdyc, qxc, dout, din, T)}
        ms, tf = {}, {}
        for name, (qa, qb, M, N, K) in gemms.items():
            a, b = qa.operand(), qb.operand()
            D = torch.empty((M, N), dtype=torch.float32, device=dev)
            api.gemm(a, b, M, N, K, out=D)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(10):
                    api.gemm(a, b, M, N, K, out=D)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms[name] = round(e0.elapsed_time(e1) / 30, 4)
            tf[name] = round(2.0 * M * N * K / (ms[name] * 1e-3) / 1e12, 1)
            del g, D
        peak = PEAK_TFLOPS["fp4" if fmt == "mxfp4" else "fp16"]
        out[fmt] = {"frobenius_rel_error": {k: round(v, 6) for k, v in err.items()},
                    "gemm_ms": ms, "gemm_TFLOPs": tf,
                    "gemm_frac_peak": {k: round(v / peak, 4) for k, v in tf.items()}}
        del qx, qxc, qw, qwc, qdy, qdyc
    return out


def row_scope_parts(fmt, host, graph_ms, flush, R=10):
    """The per-row global scale (NVFP4 paper App. B.1, closing remark) on the
    rowwise operands of Fprop and Dgrad, cache-flushed like `parts`: for X,
    W (RNE) and dY (SR), the tensor-scope route -- an amax pass, then the
    rowwise quantizer -- against the one-pass rowwise quantizer with one
    global scale per row; and Fprop on 1D operands with per-row decode
    scales on both against the same with tensor scales.  (The colwise Wgrad
    operands keep the tensor scope: a row of X^T spans every token.)"""
    import torch
    from fp4_block_scaled_x16_amd import api

    dev_t, tg = host["device"], host["targets"]
    dev = host["fprop_out"].device
    cnt = api.new_counters(dev)
    buf = torch.empty(1, dtype=torch.float32, device=dev)

    def cold_ms(f):
        def body():
            for _ in range(R):
                flush()
                f()

        def flush_only():
            for _ in range(R):
                flush()
        return max(graph_ms(body) - graph_ms(flush_only), 0.0) / R

    res = {}
    for name, rnd in (("X", "rne"), ("W", "rne"), ("dY", "sr")):
        x = dev_t[name]
        kw = dict(rnd=rnd, seed=1, target=tg[name], scale_layout="tiled", counters=cnt, count=COUNT)

        def two():
            api.amax(x, out=buf, orient="row")
            api.quantize(x, fmt, amax_in=buf, **kw)

        def one():
            api.quantize(x, fmt, global_scope="row", **kw)
        t2, t1 = cold_ms(two), cold_ms(one)
        res[name] = {"amax_pass_plus_rowwise_ms": round(t2, 4), "rowwise_per_row_ms": round(t1, 4),
                     "rowwise_per_row_GBps": round(B_Q1D[fmt] * x.numel() / (t1 * 1e-3) / 1e9, 1)}
    X, W = dev_t["X"], dev_t["W"]
    M, K = X.shape
    N = W.shape[0]
    out = host["fprop_out"]
    for scope in ("tensor", "row"):
        # both operands 1D with TILED scales, so only the global scope differs
        qx = api.quantize(X, fmt, global_scope=scope, target=tg["X"], scale_layout="tiled")
        qw = api.quantize(W, fmt, global_scope=scope, target=tg["W"], scale_layout="tiled")
        t_g = cold_ms(lambda: api.gemm(qx.operand(), qw.operand(), M, N, K, out=out))
        res["fprop_1d_%s_scales_ms" % scope] = round(t_g, 4)
        del qx, qw
    res["note"] = ("rowwise operands of Fprop/Dgrad; Wgrad's colwise operands keep the tensor "
                   "scope")
    return res


def other_kernels(fmt, host, graph_ms, flush, R=10):
    """The hot path's kernels that the step does not launch, cold like
    `parts`, against HBM with their algorithmic bytes per element: the
    dequantization of X's rowwise codes to bf16 (2.5625 B) and fp32
    (4.5625 B; NVFP4 paper App. B.3), the RHT alone on X along tokens, 16-
    and 64-point (bf16 in, fp32 out: 6 B; §4.2), and MXFP8 quantization of
    an X-sized input rowwise and colwise (3.03125 B; 2D-block FP4 page, the
    Q/K projections) and the dequantization of its rowwise codes to bf16
    (3.03125 B) and fp32 (5.03125 B).  Two-level workloads dequantize their
    own format; the MXFP4 workload dequantizes NVFP4 codes of X."""
    import torch
    from fp4_block_scaled_x16_amd import api, inputs

    X = host["device"]["X"]
    dev = X.device
    n = X.numel()
    signs = inputs.rht_sign_mask()
    qx = api.quantize(X, fmt if fmt != "mxfp4" else "nvfp4")
    qm = api.quantize(X, "mxfp8")
    out_bf = torch.empty(X.shape, dtype=torch.bfloat16, device=dev)
    out_f = torch.empty(X.shape, dtype=torch.float32, device=dev)
    work = [("dequantize X to bf16", 2.5625, lambda: api.dequantize(qx, torch.bfloat16, out=out_bf)),
            ("dequantize X to fp32", 4.5625, lambda: api.dequantize(qx, torch.float32, out=out_f)),
            ("rht X 16-point", 6.0, lambda: api.rht16(X, signs, out=out_f)),
            ("rht X 64-point", 6.0, lambda: api.rht16(X, signs, rht_n=64, out=out_f)),
            ("mxfp8 X rowwise", 3.03125, lambda: api.quantize(X, "mxfp8")),
            ("mxfp8 X colwise", 3.03125, lambda: api.quantize(X, "mxfp8", orient="col")),
            ("mxfp8 dequantize X to bf16", 3.03125, lambda: api.dequantize(qm, torch.bfloat16, out=out_bf)),
            ("mxfp8 dequantize X to fp32", 5.03125, lambda: api.dequantize(qm, torch.float32, out=out_f))]

    def flush_only():
        for _ in range(R):
            flush()
    t_flush = graph_ms(flush_only)
    res = {}
    for name, bpe, f in work:
        def body():
            for _ in range(R):
                flush()
                f()

        def warm():
            for _ in range(R):
                f()
        ms = max(graph_ms(body) - t_flush, 0.0) / R
        gbs = bpe * n / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "GBps": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "ms_warm": round(graph_ms(warm) / R, 4)}
    res["elements"] = n
    return res


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.config)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq[0], args.summarize_sq[1], args.ops_json)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU (--gpus 1); runs on several GPUs are not "
              "part of this benchmark.", file=sys.stderr)
        sys.exit(2)
    # the CPU oracle's worker processes are forked before anything touches the GPU
    pool = None
    if not (args.no_cpu or args.layer or args.counters_run):
        import multiprocessing
        pool = multiprocessing.get_context("fork").Pool(cpu_cores())
    import torch
    from fp4_block_scaled_x16_amd import api, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    api.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.layer:
        layer_main(args, dev)
        return
    cfg = args.config
    ops, cnt, host, fmt = build_step(cfg, dev, dual=not args.separate_quant)
    if args.counters_run:
        counters_run(ops, host, args.ops_json)
        return

    def run_step():
        for (_, _, _, f) in ops:
            f()

    # The amax + quantize work of X, W and dY is independent: each tensor's
    # runs on its own stream (default priority), Fprop starts as soon as X
    # and W are quantized (beside dY's VALU-bound stochastic rounding), and
    # Dgrad / Wgrad follow on the main stream once everything has joined.
    # Every side stream first waits for the main stream, so memory the
    # previous step's GEMMs read is not reused before they finish.
    side = [torch.cuda.Stream(dev) for _ in range(3)]

    def tensor_of(name):
        if name.startswith("gemm"):
            return name
        return next(t for t in ("dY", "X", "W") if (" " + t + " ") in (name + " "))

    def run_step_concurrent():
        main = torch.cuda.current_stream(dev)
        ev = {}
        for i, t in enumerate(("X", "W", "dY")):
            side[i].wait_stream(main)
            with torch.cuda.stream(side[i]):
                for (n, _, _, f) in ops:
                    if tensor_of(n) == t:
                        f()
                ev[t] = torch.cuda.Event()
                ev[t].record(side[i])
        with torch.cuda.stream(side[0]):
            side[0].wait_event(ev["W"])
            next(f for (n, _, _, f) in ops if n == "gemm fprop")()
        for s_ in side:
            main.wait_stream(s_)
        for (n, _, _, f) in ops:
            if n in ("gemm dgrad", "gemm wgrad"):
                f()

    if not args.serial:
        run_step = run_step_concurrent  # noqa: F811

    # eager warmup (also performs the library's one-time kernel attribute setup)
    for _ in range(max(1, args.warmup)):
        run_step()
    torch.cuda.synchronize()
    outs = [t for t in host["gpu_outputs"]]
    eager = [t.clone() for t in outs]

    # the step as one HIP graph: no host launch gaps inside the timed region
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_step()
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager step")
    for _ in range(args.warmup):
        graph.replay()
    cnt.zero_()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    counters = api.counters_dict(cnt)

    # Per-kernel durations, timed with events on the stream the kernels run
    # on: a graph of R x (512 MiB read, op) minus a graph of R x (512 MiB
    # read), so every op starts with the Infinity Cache holding none of its
    # inputs and no dirty lines of other work (a write flush would leave
    # 256 MB of them for the op to write back); the op's own output lines
    # are written back under the next flush, which the difference charges
    # to the op.  `parts_warm`: a graph of R back-to-back launches.
    R = 10
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_buf.fill_(1.0)
    flush_rows = flush_buf.view(-1, 4096)
    flush_out = torch.empty(flush_rows.shape[0], dtype=torch.float32, device=dev)

    def flush():
        # reads the 512 MiB buffer (a row-wise max: one small output, and a
        # kernel of torch's own, so kernel traces tell it from the library's)
        torch.amax(flush_rows, dim=1, out=flush_out)

    def graph_ms(body, reps=3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / reps

    def flushes():
        for _ in range(R):
            flush()

    op_ms, op_ms_warm = [], []
    for (_, _, _, f) in ops:
        def cold():
            for _ in range(R):
                flush()
                f()

        def warm():
            for _ in range(R):
                f()
        t_flush = graph_ms(flushes)
        op_ms.append(max(graph_ms(cold) - t_flush, 0.0) / R)
        op_ms_warm.append(graph_ms(warm) / R)

    def rates(times):
        out = {}
        for i, (name, kind, units, _) in enumerate(ops):
            ms = times[i]
            p = {"ms": round(ms, 4)}
            if kind == "hbm" and units > 0:
                gbs = units / (ms * 1e-3) / 1e9
                p.update(GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
            elif kind == "mfma":
                tf = units / (ms * 1e-3) / 1e12
                peak = PEAK_TFLOPS["fp4" if fmt == "mxfp4" else "fp16"]
                p.update(TFLOPs=round(tf, 1), frac_peak=round(tf / peak, 4))
            out[name] = p
        return out
    parts, parts_warm = rates(op_ms), rates(op_ms_warm)
    # side measurements after the per-op graphs, whose launches come first
    # after the step's (what --summarize-trace reads)
    row_scope = None
    if fmt != "mxfp4":
        row_scope = row_scope_parts(fmt, host, graph_ms, flush)
    fmt_cmp = format_comparison(dev) if cfg == 5 else None
    others = other_kernels(fmt, host, graph_ms, flush)
    q_bytes = sum(u for (_, k, u, _) in ops if k == "hbm")
    q_ms = sum(parts[n]["ms"] for (n, k, u, _) in ops if k == "hbm" and u > 0)
    g_flops = sum(u for (_, k, u, _) in ops if k == "mfma")
    g_ms = sum(parts[n]["ms"] for (n, k, _, _) in ops if k == "mfma")
    value = g_flops / (ms_step * 1e-3) / 1e12

    # dominant kernel: the block-scaled GEMM (all three launches run the same kernel)
    gemm_names = [n for (n, k, _, _) in ops if k == "mfma"]
    avg_ms = float(np.mean([parts[n]["ms"] for n in gemm_names]))
    per_launch = g_flops / len(gemm_names)
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["fp4" if fmt == "mxfp4" else "fp16"]
    khash = source_hash(*GEMM_SOURCES)
    traffic = read_traffic(cfg, khash)
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "k_gemm_two_level_dma<NVFP4>" if fmt == "nvfp4" else
                          ("k_gemm_two_level_dma<UE5M3>" if fmt == "ue5m3" else "k_gemm_mx_tiled"),
                "flops_per_launch": per_launch, "avg_launch_ms": round(avg_ms, 4),
                "kernel_source_sha256_16": khash}

    c = inputs.CONFIGS[cfg]
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4(e2m1)+%s scales; %s MFMA, fp32 accumulate" % (
            {"nvfp4": "e4m3", "ue5m3": "ue5m3", "mxfp4": "ue8m0"}[fmt],
            "fp4 scaled" if fmt == "mxfp4" else "fp16 (exact dequant)"),
        "data": "synthetic (seeded PCG64, bf16 inputs resident in HBM)",
        "config": {"workload": c["name"], "format": fmt, "tokens": c["tokens"], "d_in": c["d_in"],
                   "d_out": c["d_out"], "gemms": "fprop, dgrad, wgrad", "scales_1d": "tiled",
                   "quantize_kernels": len([1 for (n, k, u, _) in ops if n.startswith("quant")]),
                   "counters": "block-scale events" if COUNT == "scales" else "all events",
                   "streams": 1 if args.serial else 4,
                   "dual_quantize": not args.separate_quant},
        "quantize": {"GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "ms": round(q_ms, 4)},
        "gemm": {"TFLOPs": round(g_flops / (g_ms * 1e-3) / 1e12, 1),
                 "frac_peak": round(g_flops / (g_ms * 1e-3) / 1e12 / peak, 4), "ms": round(g_ms, 4)},
        "roofline": roofline,
        "parts": parts,
        "parts_warm": parts_warm,
        "counters": counters,
        "wall_s_timed": round(wall, 3),
    }
    if row_scope is not None:
        out["row_scope"] = row_scope
    del flush_buf, flush_rows, flush_out
    out["other_kernels"] = others
    if fmt_cmp is not None:
        out["format_comparison"] = fmt_cmp
    if pool is not None:
        out["cpu_baseline"] = cpu_baseline(cfg, host, fmt, args.cpu_tokens, pool)
        pool.close()
        pool.join()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
