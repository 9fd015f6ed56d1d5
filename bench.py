"""Benchmark of the ConvRot quantized linear on one MI355X.

One step = one pass of the hot path over one batch: for every linear of the workload,
rotate + quantize the activations (HIP kernel 1), int8 MFMA GEMM with the fused dequantizing
epilogue (HIP kernel 2). The default workload is ViT-L attention projections at batch 8:
X f16 [41472, 1024] through qkv (N = 3072) and out-proj (N = 1024), both W8A8; weights are
quantized once, offline, before timing (reported separately).

Prints ONE JSON line. `value` = whole-step throughput in TOPS (2*M*N*K summed over the calls,
divided by the wall time of the timed steps, inputs already resident in HBM). A ring of input /
output buffer sets larger than the 256 MB Infinity Cache is rotated so that no step reads what
the previous one left in the cache. Per-kernel durations come from HIP events recorded on the
launch stream between the kernels of the same hot path (split into its two calls); they feed the
`roofline` object of the dominant kernel (the GEMM of the largest call) and the per-call
breakdown. `cpu_baseline` times the CPU oracle (never tuned) on a bounded row sample of the
same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
       python bench.py --copy-calibration        (a plain 1 GiB copy, for counter calibration)
       python bench.py --pmc-summary FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
                                                 (rocprofv3 counters -> profiles/pmc_traffic.json)
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense fp6 / fp4 MFMA, TFLOP/s (the W4A4 path's matrix cores)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20
PEAK_F64_OPS = 39.3e12       # MI355X vector fp64, non-fused ops/s (78.6 TFLOP/s counts an FMA as 2)
NCLIP = 51                   # clipping candidates of the MSE weight-scale rule
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gemm_common.h", "gemm_i8.hip", "gemm_rw.hip", "gemm_i8_wide.hip", "gemm_fp6.hip",
              "rotate_quant.hip"):
        with open(os.path.join(ROOT, "w4a4_integer_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters(workload, kernel):
    """Memory-side bytes per launch (L2 fetch + write) of `kernel` ("gemm" or "rotate_quant")
    from committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by a copy-kernel calibration;
    None if absent or taken on different kernel sources."""
    try:
        with open(PMC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("workloads", {}).get(workload, {}).get(kernel)


COPY_BYTES = 1 << 30         # size of the plain copy that calibrates the byte counters


def copy_calibration(reps=5):
    """A plain device-to-device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES), repeated;
    run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to scale those counters to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": reps}))


def _read_counter_csv(path):
    """rocprofv3 counter_collection.csv -> {dispatch_id: (kernel_name, grid, {counter: value})}."""
    import csv
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            d = out.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], int(r["Grid_Size"]), {}])
            # A counter reported per hardware instance arrives as several rows: sum them.
            d[2][r["Counter_Name"]] = d[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _is_gemm(kernel_name):
    """The library's GEMM kernels: gemm_kernel, gemm_xr_kernel, gemm_rw_kernel, gemm_n2_kernel,
    gemm_wide_kernel and gemm_fp6_kernel (template arguments follow the name)."""
    import re
    return re.search(r"(?:^|::|\s)gemm_\w*kernel\s*[<(]", kernel_name) is not None


def gemm_kernel_name(M, N, K, bits, x_layout, w_layout=0, act=0, s32=False):
    """The GEMM kernel the launcher picks for a call, by the dispatch rule of gemm_i8.hip,
    gemm_rw.hip, gemm_i8_wide.hip and gemm_fp6.hip (a label for the roofline record)."""
    from w4a4_integer_quantized_amd import binding as rq
    if w_layout == rq.RQ_W_FP6:
        return "gemm_fp6_kernel"
    Kb = K if bits == 8 else K // 2
    tiles = -(-M // 256) * -(-N // 128)
    if bits == 8 and x_layout == rq.RQ_X_TILED and Kb == 1024 and N == 32 * 96 and -(-M // 64) >= 64 \
            and -(-M // 256) * 256 * 1024 < 2 ** 31:
        return "gemm_rw_kernel"
    if x_layout == rq.RQ_X_ROWS and act == 0 and 1536 <= Kb < 3072 and -(-M // 256) * -(-N // 256) >= 192:
        return "gemm_wide_kernel"
    if tiles <= 256 and (Kb // 64) % 2 == 0 and Kb // 64 >= 16:
        return "gemm_kernel (8 waves, split K)"
    if bits == 8 and x_layout == rq.RQ_X_TILED and tiles > 256 and Kb in (1024, 1536, 2048):
        return "gemm_xr_kernel"
    if tiles > 256 and Kb >= 3072:
        return "gemm_n2_kernel"
    return "gemm_kernel"


def rq_kernel_name(K, fp6=False):
    """The rotate+quantize kernel the launcher picks, by the dispatch rule of rotate_quant.hip:
    the coalesced kernel when nb = K / 128 blocks split as G * NI with G in {1, 2, 4, 8, 12, 16}
    and NI <= 4 (int codes only), else the quad kernel, else the generic one."""
    nb = K // 128
    if not fp6 and any(nb % g == 0 and nb // g <= 4 for g in (1, 2, 4, 8, 12, 16)):
        return "rotate_quant_coalesced_kernel"
    for bpq in range(1, 5):
        if nb % bpq:
            continue
        lanes = 4 * (nb // bpq)
        if lanes <= 64 or (lanes % 64 == 0 and lanes <= 256):
            return "rotate_quant_kernel"
    return "rotate_quant_generic_kernel"


def dominant_gemm_kernel(key):
    """Symbol stem of the GEMM kernel that runs the workload's largest linear inside
    rq_rotq_linear (tiled activation codes), e.g. "gemm_rw_kernel"."""
    from w4a4_integer_quantized_amd import binding as rq
    from w4a4_integer_quantized_amd import synth
    cfg = synth.CONFIGS[key]
    dom = max(cfg.linears, key=lambda l: l.N * l.K)
    return gemm_kernel_name(cfg.M, dom.N, dom.K, cfg.bits, rq.RQ_X_TILED).split()[0]


def _matches(name, stem):
    return stem is None or ("::%s<" % stem) in name or name.startswith(stem + "<")


def mfma_summary(counter_csv, trace_csv, n_simd=1024, n_xcc=8, gemm_kernel=None):
    """Reduce a rocprofv3 run with --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES
    SQ_INSTS_VALU_MFMA_MOPS_I8 GRBM_GUI_ACTIVE --kernel-trace to per-launch figures of the GEMM's
    largest launch (of the kernel `gemm_kernel` names, when given): MFMA busy fraction, int8 MFMA
    ops, GPU-active cycles per XCD and the shader clock they imply over the traced duration."""
    import csv
    import numpy as np
    dur = {}
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    rows = {}
    for did, (name, grid, vals) in _read_counter_csv(counter_csv).items():
        if _is_gemm(name) and _matches(name, gemm_kernel) and did in dur:
            rows.setdefault(grid, []).append((name, vals, dur[did]))
    grid = max(rows)
    name = rows[grid][0][0]
    util = [v.get("MfmaUtil", float("nan")) for _, v, _ in rows[grid]]
    busy = [v.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) for _, v, _ in rows[grid]]
    mops = [v.get("SQ_INSTS_VALU_MFMA_MOPS_I8", float("nan")) for _, v, _ in rows[grid]]
    gui = [v.get("GRBM_GUI_ACTIVE", float("nan")) / n_xcc for _, v, _ in rows[grid]]
    secs = [d for _, _, d in rows[grid]]
    doc = {"kernel": name, "grid_threads": grid, "dispatches": len(secs),
           "duration_us_median": round(float(np.median(secs)) * 1e6, 2),
           "MfmaUtil_pct_median": round(float(np.median(util)), 2),
           "mfma_busy_cycles_per_simd_median": round(float(np.median(busy)) / n_simd, 1),
           "gui_active_cycles_per_xcd_median": round(float(np.median(gui)), 1),
           "implied_clock_GHz": round(float(np.median(gui)) / float(np.median(secs)) / 1e9, 3),
           "int8_mfma_ops_median": float(np.median(mops)) * 512}
    print(json.dumps(doc))
    return doc


def _median_by_group(csv_path, counter, select):
    """Median of one counter over the dispatches of each (kernel family, grid) group."""
    import numpy as np
    groups = {}
    for name, grid, vals in _read_counter_csv(csv_path).values():
        fam = select(name)
        if fam and counter in vals:
            groups.setdefault((fam, grid), []).append(vals[counter])
    return {k: (float(np.median(v)), len(v)) for k, v in groups.items()}


def pmc_summary(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_path=None,
                gemm_kernel=None):
    """Reduce four rocprofv3 --pmc runs (bench FETCH_SIZE, bench WRITE_SIZE, copy FETCH_SIZE,
    copy WRITE_SIZE; counters in KiB per dispatch) to bytes per launch of the dominant GEMM (the
    largest launch of `gemm_kernel`, when given, else of any GEMM) and of the rotate+quantize
    kernel, scaled by what the same counters read for the plain copy of COPY_BYTES. Writes
    out_path (default profiles/pmc_traffic.json), keyed by the kernel sources' hash, and returns
    the document."""
    out_path = out_path or PMC_FILE
    def fam(name):
        if _is_gemm(name):
            return "gemm" if _matches(name, gemm_kernel) else None
        if "rotate_quant" in name:
            return "rotate_quant"
        return None

    def copy_fam(name):
        return "copy" if "copy" in name.lower() else None

    cf = _median_by_group(copy_fetch_csv, "FETCH_SIZE", copy_fam)
    cw = _median_by_group(copy_write_csv, "WRITE_SIZE", copy_fam)
    cf_kib = max(cf.values())[0]
    cw_kib = max(cw.values())[0]
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    fetch = _median_by_group(fetch_csv, "FETCH_SIZE", fam)
    write = _median_by_group(write_csv, "WRITE_SIZE", fam)
    res = {}
    for kind in ("gemm", "rotate_quant"):
        # The dominant launch of each kernel is its largest grid (the largest call of the step).
        keys = [k for k in fetch if k[0] == kind and k in write]
        if not keys:
            continue
        k = max(keys, key=lambda t: t[1])
        fb = fetch[k][0] * 1024.0 * f_scale
        wb = write[k][0] * 1024.0 * w_scale
        res[kind] = {"grid_threads": k[1], "dispatches": fetch[k][1], "fetch_bytes": round(fb),
                     "write_bytes": round(wb), "bytes": round(fb + wb),
                     "fetch_kib_raw": fetch[k][0], "write_kib_raw": write[k][0]}
    doc = {"kernel_source_hash": kernel_source_hash(),
           "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "workloads": {workload: res}}
    try:
        with open(out_path) as fh:
            old = json.load(fh)
        if old.get("kernel_source_hash") == doc["kernel_source_hash"]:
            old["workloads"].update(doc["workloads"])
            old["calibration"] = doc["calibration"]
            doc = old
    except (OSError, ValueError):
        pass
    with open(out_path, "w") as fh:
        json.dump(doc, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(doc))
    return doc


def cpu_baseline(g, cfg, target_s, act_of=None):
    """The CPU oracle as it stands on a bounded sample of the same workload's rows (with the
    fused activation where the GPU step has one), on all host cores, then single-threaded on a
    smaller sample."""
    import numpy as np
    import oracle
    dt = oracle.F16 if cfg.io == "f16" else oracle.BF16
    act_of = act_of or {}
    wq = {lin.name: oracle.quantize_weights(g["W"][lin.name], cfg.bits)[0::2] for lin in cfg.linears}

    split = {"rq_s": 0.0, "rq_bytes": 0, "gemm_s": 0.0, "gemm_ops": 0}

    def run(rows):
        # The oracle's linear, step by step: rotate+quantize, integer GEMM, epilogue.
        t0 = time.perf_counter()
        ops = 0
        for lin in cfg.linears:
            src = np.ascontiguousarray((g["x_bits"] if lin.source == "x" else g["x2_bits"][lin.name])[:rows])
            wc, ws = wq[lin.name]
            t1 = time.perf_counter()
            xc, xs, _ = oracle.quantize_rows(src, dt, cfg.bits)
            t2 = time.perf_counter()
            acc = oracle.gemm_s32(xc, wc)
            act = act_of.get(lin.name, 0)
            if act:
                oracle.epilogue_act(acc, xs, ws, g["bias"][lin.name], dt, act)
            else:
                oracle.epilogue(acc, xs, ws, g["bias"][lin.name], dt)
            t3 = time.perf_counter()
            split["rq_s"] += t2 - t1
            split["rq_bytes"] += rows * lin.K * 2 + rows * lin.K * cfg.bits // 8 + 4 * rows
            split["gemm_s"] += t3 - t2
            split["gemm_ops"] += 2 * rows * lin.N * lin.K
            ops += 2 * rows * lin.N * lin.K
        return time.perf_counter() - t0, ops

    # Grow the token sample until one pass takes a tenth of the target (or covers the whole
    # step), then repeat passes until the target time is spent.
    rows = min(cfg.M, 256)
    while True:
        t, ops = run(rows)
        if rows == cfg.M or t >= 0.1 * target_s:
            break
        rows = int(min(cfg.M, max(2 * rows, rows * 0.1 * target_s / max(t, 1e-6))))
    total_t, total_ops, passes = t, ops, 1
    while total_t < target_s:
        t, ops = run(rows)
        total_t += t
        total_ops += ops
        passes += 1
    out = {"value": total_ops / total_t / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
           "kind": "oracle",
           "rotate_quant_GBps": round(split["rq_bytes"] / split["rq_s"] / 1e9, 3),
           "gemm_epilogue_TOPS": round(split["gemm_ops"] / split["gemm_s"] / 1e12, 5),
           "sample": "first %d of %d tokens, every linear of the step (rotate+quantize, int GEMM, "
                     "epilogue%s), %d passes, %.1f s" % (rows, cfg.M, " with the fused GELU" if any(act_of.values())
                                                          else "", passes, total_t)}
    # One single-threaded pass on a smaller sample (about a fifth of the target time).
    cores = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        rows1 = max(1, min(rows, int(rows * 0.2 * target_s / max(total_t / passes * cores, 1e-6))))
        t1, ops1 = run(rows1)
    finally:
        oracle.set_num_threads(cores)
    out["single_thread"] = {"value": ops1 / t1 / 1e12, "unit": "TOPS", "cores": 1,
                            "sample": "first %d tokens, one pass, %.1f s" % (rows1, t1)}
    return out


def offline_weight_quant(rq, torch, W_np, bits, dev, reps=5):
    """Times rq_quantize_weights under each weight-scale rule on one weight matrix, with the
    weight quantization error of each rule (row sample, against the exact rotation in float64:
    plain numpy block-Hadamard, W_rot = W blockdiag(H_128) / sqrt(128))."""
    import numpy as np
    import scipy.linalg
    N, K = W_np.shape
    Wd = torch.from_numpy(W_np).to(dev)
    rows = np.random.default_rng(7).choice(N, min(N, 256), replace=False)
    Hn = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128.0)
    wr = W_np[rows].astype(np.float64).reshape(len(rows), K // 128, 128) @ Hn
    wr = wr.reshape(len(rows), K)
    out = {"N": N, "K": K, "bits": bits, "w_dtype": "f32"}
    alg_bytes = 4 * N * K + N * K * bits // 8 + 4 * N
    for name, mode in (("absmax", rq.RQ_W_ABSMAX), ("mse", rq.RQ_W_MSE), ("tensor", rq.RQ_W_TENSOR)):
        rq.quantize_weights(Wd, bits=bits, w_scale_mode=mode)     # warm-up
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            Wq, ws = rq.quantize_weights(Wd, bits=bits, w_scale_mode=mode)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        codes = Wq.cpu().numpy()
        if bits == 4:
            lo = (codes.view(np.uint8) & 0xF).astype(np.int8)
            hi = (codes.view(np.uint8) >> 4).astype(np.int8)
            lo[lo >= 8] -= 16
            hi[hi >= 8] -= 16
            codes = np.stack([lo, hi], axis=-1).reshape(N, K)
        deq = codes[rows].astype(np.float64) * ws.cpu().numpy()[rows, None].astype(np.float64)
        d = {"ms": round(ms, 4), "GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
             "w_err_rel_frobenius": round(float(np.linalg.norm(deq - wr) / np.linalg.norm(wr)), 6)}
        if mode == rq.RQ_W_MSE:
            # Each candidate evaluation is 5 binary64 operations by definition (two exact
            # products, a difference, a square, a sum); the search evaluates NCLIP * N * K.
            f64 = 5.0 * NCLIP * N * K / (ms * 1e-3)
            d["roofline"] = {"bound": "alu", "achieved": round(f64 / 1e12, 2), "peak": PEAK_F64_OPS / 1e12,
                             "unit": "T fp64 op/s", "frac": round(f64 / PEAK_F64_OPS, 4)}
        out[name] = d
    return out


def library_int8_gemm(torch, M, N, K, reps=20):
    """Context only: the vendor library's int8 GEMM (hipBLASLt through torch._int_mm) on the
    dominant call's shape. It writes int32 (4 B per output, twice this path's fp16/bf16 Y) and
    applies no scales or bias; it is a sanity point, not a target."""
    A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
    Bt = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda").t()
    for _ in range(3):
        torch._int_mm(A, Bt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch._int_mm(A, Bt)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"shape": [M, N, K], "us": round(us, 2), "TOPS": round(2 * M * N * K / us / 1e6, 1),
            "out": "int32, no epilogue", "via": "torch._int_mm (hipBLASLt)"}


def hbm_ceilings(torch, M, K, rq_us=None, reps=20):
    """Memory ceilings of the rotate+quantize kernel's access pattern on X [M, K] fp16, in
    algorithmic GB/s: libconvrot_ceiling.so's kernels issue the coalesced kernel's exact loads
    and stores (tiled code layout) without its arithmetic -- 2:1 (read X, write one byte per
    element), read-only and write-only -- each over a ring of buffers larger than the
    Infinity Cache (as the workload's ring). `rq_us`: the rotate+quantize kernel's time on the same shape, reported as a
    fraction of the 2:1 ceiling."""
    import ctypes
    from w4a4_integer_quantized_amd import build as B
    lib = ctypes.CDLL(B.CEILING_LIB)
    fn = lib.rqc_hbm_pattern
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    R = max(4, math.ceil(3 * MALL_BYTES / (3 * M * K)))      # >= 3x the Infinity Cache per cycle
    xs = [torch.randn((M, K), device="cuda").half() for _ in range(R)]
    q = [torch.empty((-(-M // 256) * 256, K), dtype=torch.int8, device="cuda") for _ in range(R)]
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for mode, name, nbytes in ((0, "copy_2to1_same_pattern", 3 * M * K), (1, "read_only", 2 * M * K),
                               (2, "write_only", M * K)):
        def call(i):
            assert fn(mode, xs[i % R].data_ptr(), q[i % R].data_ptr(), M, K, 1, stream) == 0
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    out["shape"] = [M, K]
    out["via"] = "libconvrot_ceiling.so rqc_hbm_pattern (the coalesced kernel's loads and stores, no arithmetic)"
    if rq_us:
        out["rotate_quant_us"] = rq_us
        out["rotate_quant_vs_2to1_ceiling"] = round(out["copy_2to1_same_pattern"]["us"] / rq_us, 4)
    return out


def gpu_state():
    """rocm-smi's view of clocks and power right after the timed work (context)."""
    import shutil
    import subprocess
    if any(k.startswith("ROCPROF") for k in os.environ):
        return {"skipped": "running under a profiler"}
    tool = shutil.which("rocm-smi")
    if tool is None:
        return {"error": "rocm-smi not found"}
    try:
        # The tool is a Python script: run it with this interpreter as a plain child process.
        r = subprocess.run([sys.executable, tool, "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=20)
        doc = json.loads(r.stdout) if r.returncode == 0 else {}
    except Exception as ex:  # the tool may be absent or print no JSON
        return {"error": str(ex)[:200]}
    out = {}
    for card, d in doc.items():
        out[card] = {k: v for k, v in d.items() if any(t in k.lower() for t in ("sclk", "mclk", "fclk", "power"))}
    return out


def synth_workload_name(key):
    from w4a4_integer_quantized_amd import synth
    return synth.CONFIGS[key].workload


GELU_ACT = {"gelu_erf": 1, "gelu_tanh": 2}     # rq.RQ_ACT_GELU_ERF / RQ_ACT_GELU_TANH


class WorkloadRun:
    """One workload on the GPU: its weights quantized offline, a ring of input / output buffer
    sets larger than the Infinity Cache, and the hot path's calls with every argument marshalled
    once, before any timing. A step is rq_rotq_linear for each linear of the workload, in
    order, on one dedicated stream."""

    def __init__(self, key, stream, w4_fp6=False, unfused_gelu=False, min_sets=3):
        import numpy as np
        import torch
        import w4a4_integer_quantized_amd as rq
        from w4a4_integer_quantized_amd import synth
        self.rq, self.torch, self.np = rq, torch, np
        self.key = key
        self.cfg = cfg = synth.CONFIGS[key]
        log("generating %s" % cfg.workload)
        self.g = g = synth.generate(key)
        self.tdt = tdt = torch.float16 if cfg.io == "f16" else torch.bfloat16
        self.dev = dev = torch.device("cuda:0")
        self.stream, self.sptr = stream, stream.cuda_stream
        self.bits, self.M = bits, M = cfg.bits, cfg.M
        self.unfused_gelu = unfused_gelu
        # 4-bit codes run on the int8 matrix cores by default; --w4-fp6 runs them on the FP6 ones
        # (weights and activations stored as FP6 tiles; identical results).
        self.wl = wl = rq.RQ_W_FP6 if bits == 4 and w4_fp6 else rq.RQ_W_ROWS
        self.xl = rq.RQ_X_FP6 if wl == rq.RQ_W_FP6 else rq.RQ_X_TILED
        # Offline weight quantization (timed once, reported separately).
        self.Wq, self.Ws, self.B = {}, {}, {}
        self.wq_ms = 0.0
        for lin in cfg.linears:
            Wd = torch.from_numpy(g["W"][lin.name]).to(dev)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            self.Wq[lin.name], self.Ws[lin.name] = rq.quantize_weights(Wd, bits=bits, w_layout=wl)
            torch.cuda.synchronize()
            self.wq_ms += (time.perf_counter() - t0) * 1e3
            self.B[lin.name] = torch.from_numpy(g["bias"][lin.name]).to(dev)
            del Wd
        # MLP pairs: the GELU between the linears runs in the first linear's epilogue (or, with
        # unfused_gelu, as a torch op on the GPU between the two calls, inside the step).
        self.act_of = {lin.name: rq.RQ_ACT_NONE for lin in cfg.linears}
        if not unfused_gelu:
            for lin in cfg.linears:
                if lin.source in GELU_ACT:
                    self.act_of[lin.producer] = GELU_ACT[lin.source]
        self.cfgc = {lin.name: rq.make_cfg(bits, w_layout=wl, act=self.act_of[lin.name]) for lin in cfg.linears}
        self.cfg_split = {lin.name: rq.make_cfg(bits, x_layout=self.xl, w_layout=wl, act=self.act_of[lin.name])
                          for lin in cfg.linears}
        self.xdt = rq.RQ_F16 if cfg.io == "f16" else rq.RQ_BF16
        # Ring of buffer sets (X copies, outputs, workspace) larger than the Infinity Cache.
        x_host = torch.from_numpy(g["x_bits"].view(np.int16)).view(tdt)
        ws_bytes = {lin.name: rq.workspace_size(M, lin.K, bits, w_layout=wl) for lin in cfg.linears}
        set_bytes = x_host.numel() * 2 + sum(M * lin.N * 2 + ws_bytes[lin.name] for lin in cfg.linears)
        # Enough sets that every kernel, timed alone over the ring, cycles through at least 3x
        # the Infinity Cache: the smallest per-kernel footprint (rotate+quantize: X and its codes;
        # GEMM: the codes and Y) sets the count, within 8 GB of device memory.
        kern_bytes = min(min(M * lin.K * 2 + M * lin.K * bits // 8, M * lin.K * bits // 8 + M * lin.N * 2)
                         for lin in cfg.linears)
        cap = max(min_sets, min(256, (8 << 30) // set_bytes))
        self.R = R = max(min_sets, min(cap, math.ceil(3 * MALL_BYTES / kern_bytes)))
        self.set_bytes = set_bytes
        self.sets = []
        for _ in range(R):
            st = {"X": x_host.to(dev), "Y": {}, "ws": {}}
            for lin in cfg.linears:
                st["Y"][lin.name] = torch.empty((M, lin.N), dtype=tdt, device=dev)
                st["ws"][lin.name] = torch.empty((ws_bytes[lin.name],), dtype=torch.uint8, device=dev)
            self.sets.append(st)
        log("%s: ring of %d buffer sets, %.0f MB each" % (key, R, set_bytes / 1e6))
        self._marshal(ws_bytes)

    def _input(self, st, lin):
        if lin.source == "x":
            return st["X"]
        if self.act_of[lin.producer] != self.rq.RQ_ACT_NONE:
            return st["Y"][lin.producer]            # the producer's epilogue applied the GELU
        return None                                 # computed by a torch op inside the step

    def _marshal(self, ws_bytes):
        """Every buffer's shape is checked here, once; the timed loop then passes the stored
        integer pointers and ctypes configs straight to the C entry points."""
        import ctypes
        rq, torch, M = self.rq, self.torch, self.M
        lib = rq.load()
        self.fn_linear, self.fn_rq, self.fn_gemm = lib.rq_rotq_linear, lib.rq_rotate_quantize, lib.rq_gemm_dequant
        self.calls = []          # per set: [(lin, gelu_src or None, args of rq_rotq_linear)]
        self.split = []          # per set: [(lin, gelu_src, args of rq_rotate_quantize, args of rq_gemm_dequant)]
        for st in self.sets:
            calls, split = [], []
            for lin in self.cfg.linears:
                X = self._input(st, lin)
                gelu_src = None
                if X is None:
                    # The torch op writes into a buffer of its own, allocated once per set.
                    X = torch.empty((M, lin.K), dtype=self.tdt, device=self.dev)
                    st.setdefault("G", {})[lin.name] = X
                    gelu_src = (st["Y"][lin.producer], X, "tanh" if lin.source == "gelu_tanh" else "none")
                assert X.shape == (M, lin.K) and X.dtype == self.tdt and X.is_contiguous(), (lin.name, X.shape)
                Y, ws = st["Y"][lin.name], st["ws"][lin.name]
                assert Y.shape == (M, lin.N) and Y.dtype == self.tdt and Y.is_contiguous(), lin.name
                assert ws.numel() >= ws_bytes[lin.name], lin.name
                wq, wsc, b = self.Wq[lin.name], self.Ws[lin.name], self.B[lin.name]
                assert wq.numel() * wq.element_size() == rq.rq_weight_bytes(lin.N, lin.K, self.cfgc[lin.name]), lin.name
                assert wsc.shape == (lin.N,) and b.shape == (lin.N,) and wsc.dtype == b.dtype == torch.float32
                cfg_ref = ctypes.byref(self.cfgc[lin.name])
                calls.append((lin, gelu_src, (X.data_ptr(), self.xdt, M, lin.K, wq.data_ptr(), wsc.data_ptr(),
                                              lin.N, b.data_ptr(), cfg_ref, Y.data_ptr(), ws.data_ptr(),
                                              ws.numel(), self.sptr)))
                # The split calls use the fused call's own workspace layout: [codes | x_scale].
                cs = self.cfg_split[lin.name]
                xq = ws.data_ptr()
                xs = xq + (rq.rq_codes_bytes(M, lin.K, cs) + 255) // 256 * 256
                cs_ref = ctypes.byref(cs)
                split.append((lin, gelu_src,
                              (X.data_ptr(), self.xdt, M, lin.K, cs_ref, xq, xs, self.sptr),
                              (xq, xs, wq.data_ptr(), wsc.data_ptr(), b.data_ptr(), M, lin.N, lin.K, cs_ref,
                               Y.data_ptr(), self.xdt, self.sptr)))
            self.calls.append(calls)
            self.split.append(split)

    def _gelu(self, src):
        Yp, out, approx = src
        self.torch.ops.aten.gelu.out(Yp, approximate=approx, out=out)

    def step(self, i):
        fn = self.fn_linear
        for lin, gelu_src, a in self.calls[i % self.R]:
            if gelu_src is not None:
                self._gelu(gelu_src)
            st = fn(*a)
            if st:
                raise self.rq.ConvRotError(st, "rq_rotq_linear", self.rq.load().rq_last_error_detail().decode())

    def split_step(self, i, evs):
        """The same two kernels per call through the split entry points, with HIP events
        recorded on the launch stream between them."""
        for c, (lin, gelu_src, a_rq, a_gm) in enumerate(self.split[i % self.R]):
            if gelu_src is not None:
                self._gelu(gelu_src)
            evs[3 * c].record(self.stream)
            st = self.fn_rq(*a_rq)
            evs[3 * c + 1].record(self.stream)
            st |= self.fn_gemm(*a_gm)
            evs[3 * c + 2].record(self.stream)
            if st:
                raise self.rq.ConvRotError(st, "split step", self.rq.load().rq_last_error_detail().decode())

    def ops_per_step(self):
        return sum(2 * self.M * lin.N * lin.K for lin in self.cfg.linears)

    def time(self, steps, warmup, peak_gemm):
        """Timed steps (wall clock between device synchronizations) and per-kernel event times."""
        torch, np, M, bits = self.torch, self.np, self.M, self.bits
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / steps
        tops = self.ops_per_step() * steps / wall / 1e12
        log("%s: timed %d steps: %.4f ms/step, %.1f TOPS" % (self.key, steps, ms_per_step, tops))
        nl = len(self.cfg.linears)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3 * nl)] for _ in range(steps)]
        for i in range(min(warmup, 3)):
            self.split_step(i, ev[0])
        torch.cuda.synchronize()
        for i in range(steps):
            self.split_step(i, ev[i])
        torch.cuda.synchronize()
        # Each kernel alone, `steps` back-to-back launches over the buffer ring between two
        # events on the launch stream: its average launch duration without per-launch event
        # overhead. rotate+quantize reads X from HBM here as in a step, and this is its roofline
        # time. The GEMM alone finds its codes out of the caches (written several launches
        # earlier), unlike in a step, where they were just written by rotate+quantize and sit in
        # the Infinity Cache: its roofline time is the split steps' event time, and the
        # cold-codes time is reported beside it.
        loop_ms = {}
        for c, lin in enumerate(self.cfg.linears):
            for kind, idx, fn in (("rq", 2, self.fn_rq), ("gemm", 3, self.fn_gemm)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
                st = 0
                for i in range(steps):
                    st |= fn(*self.split[i % self.R][c][idx])
                e1.record(self.stream)
                torch.cuda.synchronize()
                if st:
                    raise self.rq.ConvRotError(st, "kernel loop", self.rq.load().rq_last_error_detail().decode())
                loop_ms[(lin.name, kind)] = e0.elapsed_time(e1) / steps
        calls = {}
        kern_us = 0.0
        for c, lin in enumerate(self.cfg.linears):
            rq_t = np.array([ev[i][3 * c].elapsed_time(ev[i][3 * c + 1]) for i in range(steps)])
            gm_t = np.array([ev[i][3 * c + 1].elapsed_time(ev[i][3 * c + 2]) for i in range(steps)])
            rq_ms, gm_ms = loop_ms[(lin.name, "rq")], float(gm_t.mean())
            kern_us += (rq_ms + gm_ms) * 1e3
            ops = 2 * M * lin.N * lin.K
            rq_bytes = M * lin.K * 2 + M * lin.K * bits // 8 + 4 * M
            gemm_bytes = M * lin.K * bits // 8 + lin.N * lin.K * bits // 8 + 8 * lin.N + 4 * M + M * lin.N * 2
            calls[lin.name] = {
                "M": M, "N": lin.N, "K": lin.K,
                "gemm_kernel": gemm_kernel_name(M, lin.N, lin.K, bits, self.xl, self.wl, self.act_of[lin.name]),
                "act": self.act_of[lin.name],
                "rotate_quant_kernel": rq_kernel_name(lin.K, fp6=self.wl != 0),
                "rotate_quant_us": round(rq_ms * 1e3, 2),
                "rotate_quant_GBps": round(rq_bytes / (rq_ms * 1e-3) / 1e9, 1),
                "rotate_quant_hbm_frac": round(rq_bytes / (rq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "gemm_us": round(gm_ms * 1e3, 2),
                "gemm_TOPS": round(ops / (gm_ms * 1e-3) / 1e12, 1),
                "gemm_mfma_frac": round(ops / (gm_ms * 1e-3) / 1e12 / peak_gemm, 4),
                "call_us": round((rq_ms + gm_ms) * 1e3, 2),
                "call_TOPS": round(ops / ((rq_ms + gm_ms) * 1e-3) / 1e12, 1),
                "call_int8_peak_frac": round(ops / ((rq_ms + gm_ms) * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                "rotate_quant_alg_bytes": rq_bytes, "gemm_alg_bytes": gemm_bytes, "gemm_alg_ops": ops,
                "gemm_us_codes_not_cached": round(loop_ms[(lin.name, "gemm")] * 1e3, 2),
                "timing": "rotate_quant_us: back-to-back launches of the kernel alone; gemm_us: HIP events "
                          "around the GEMM in split steps (right after its rotate+quantize); split_*: "
                          "HIP events around each kernel of a split step",
                "split_rotate_quant_us_mean_p10_p50_p90": [round(float(rq_t.mean()) * 1e3, 2)] + [
                    round(float(np.percentile(rq_t, p)) * 1e3, 2) for p in (10, 50, 90)],
                "split_gemm_us_mean_p10_p50_p90": [round(float(gm_t.mean()) * 1e3, 2)] + [
                    round(float(np.percentile(gm_t, p)) * 1e3, 2) for p in (10, 50, 90)],
            }
        return {"ms_per_step": ms_per_step, "tops": tops, "calls": calls,
                "kernel_us_per_step": round(kern_us, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="vit_attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the headline workload (the default also runs every other one)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (vendor library GEMM, weight-quantizer rules)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--unfused-gelu", action="store_true",
                    help="MLP pairs: apply GELU as a separate torch op between the linears "
                         "instead of in the first linear's epilogue (for comparison)")
    ap.add_argument("--w4-fp6", action="store_true",
                    help="run 4-bit codes on the FP6 matrix cores (FP6 code tiles) instead of the int8 ones")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("COUNTER_CSV", "KERNEL_TRACE_CSV"),
                    help="reduce a rocprofv3 MFMA-utilization run of the GEMM and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="reduce rocprofv3 counter CSVs into profiles/pmc_traffic.json (no GPU)")
    args = ap.parse_args()
    if args.mfma_summary:
        mfma_summary(*args.mfma_summary, gemm_kernel=dominant_gemm_kernel(args.workload))
        return
    if args.pmc_summary:
        pmc_summary(synth_workload_name(args.workload), *args.pmc_summary,
                    gemm_kernel=dominant_gemm_kernel(args.workload))
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the quantized linear "
              "shards over tokens with no exchange; see the design notes). Run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch
    import w4a4_integer_quantized_amd as rq
    from w4a4_integer_quantized_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    # All work goes to one dedicated stream (default priority). Dependent kernels on the legacy
    # null stream measured ~10% slower per step here (extra synchronization between launches).
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)

    run = WorkloadRun(args.workload, stream, w4_fp6=args.w4_fp6, unfused_gelu=args.unfused_gelu)
    cfg, g, M, bits = run.cfg, run.g, run.M, run.bits
    peak_gemm = PEAK_FP6_TOPS if run.wl == rq.RQ_W_FP6 else PEAK_INT8_TOPS
    res = run.time(args.steps, args.warmup, peak_gemm)
    calls, tops, ms_per_step = res["calls"], res["tops"], res["ms_per_step"]

    dom = max(cfg.linears, key=lambda l: l.N * l.K)
    dc = calls[dom.name]
    tr = traffic_from_counters(cfg.workload, "gemm")
    traffic = tr["bytes"] if tr else None
    roofline = {"bound": "mfma", "kernel": "%s (%s: %dx%dx%d, W%dA%d)" % (dc["gemm_kernel"], dom.name, M, dom.N, dom.K,
                                                                           bits, bits),
                "achieved": dc["gemm_TOPS"], "peak": peak_gemm, "unit": "TOP/s",
                "frac": dc["gemm_mfma_frac"], "traffic": traffic,
                "avg_launch_us": dc["gemm_us"], "alg_ops_per_launch": dc["gemm_alg_ops"],
                "alg_bytes_per_launch": dc["gemm_alg_bytes"], "traffic_detail": tr}
    rtr = traffic_from_counters(cfg.workload, "rotate_quant")
    rq_traffic = rtr["bytes"] if rtr else None
    roofline_rq = {"bound": "hbm", "kernel": "%s (%s input %dx%d)" % (rq_kernel_name(dom.K), dom.name, M, dom.K),
                   "achieved": dc["rotate_quant_GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": dc["rotate_quant_hbm_frac"], "traffic": rq_traffic,
                   "avg_launch_us": dc["rotate_quant_us"], "alg_bytes_per_launch": dc["rotate_quant_alg_bytes"],
                   "traffic_detail": rtr}

    # Quantization error as context (not parity): GPU outputs on a row sample against the
    # unquantized linear X W^T + b in float64 (plain numpy), relative Frobenius norm.
    qerr = {}
    rs = np.random.default_rng(12345).choice(M, min(M, 512), replace=False)
    for lin in cfg.linears:
        if lin.source != "x":
            continue          # second-layer inputs come from the GPU's own GELU; skip
        xr = torch.from_numpy(g["x_bits"][rs].view(np.int16)).view(run.tdt).float().numpy().astype(np.float64)
        ref = xr @ g["W"][lin.name].astype(np.float64).T + g["bias"][lin.name].astype(np.float64)
        if run.act_of[lin.name] != rq.RQ_ACT_NONE:
            ref = synth.gelu(ref, "gelu_erf" if run.act_of[lin.name] == rq.RQ_ACT_GELU_ERF else "gelu_tanh")
        got = run.sets[0]["Y"][lin.name][torch.from_numpy(rs).to(dev)].float().cpu().numpy().astype(np.float64)
        qerr[lin.name] = round(float(np.linalg.norm(got - ref) / np.linalg.norm(ref)), 6)

    gelu_cfg = {}
    if any(l.source in GELU_ACT for l in cfg.linears):
        gelu_cfg = {"gelu": "torch op between the linears" if args.unfused_gelu else
                    "fused into the first linear's epilogue"}
    out = {
        "metric": "rotq_linear TOPS (rotate+quant+GEMM) and % of MI355X INT8 MFMA peak",
        "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 codes as fp6 e2m3" if run.wl == rq.RQ_W_FP6 else "int8",
        "data": "synthetic",
        "config": {"workload": cfg.workload, "M": M, "K": cfg.K, "N": [l.N for l in cfg.linears],
                   "io": cfg.io, "bits": bits, "calls_per_step": len(cfg.linears), **gelu_cfg},
        "int8_peak_frac": round(tops / PEAK_INT8_TOPS, 4),
        "kernel_us_per_step": res["kernel_us_per_step"],
        "roofline": roofline, "roofline_rotate_quant": roofline_rq, "calls": calls,
        "weight_quant_ms_offline": round(run.wq_ms, 3), "buffer_sets": run.R,
        "quant_error_rel_frobenius_vs_fp64": qerr,
    }
    out["gpu_state_after_timing"] = gpu_state()

    # Every other workload, each timed the same way (fewer steps; not part of `value`), and the
    # 4-bit workload once more on the other code path (FP6 matrix cores, or the int8 ones when
    # --w4-fp6 made FP6 the default), under the key "<key>_fp6" / "<key>_int8".
    if not args.no_other_workloads:
        others = {}
        runs = [(key, args.w4_fp6, key) for key in synth.CONFIGS if key != args.workload]
        runs += [(key, not args.w4_fp6, key + ("_int8" if args.w4_fp6 else "_fp6"))
                 for key in synth.CONFIGS if synth.CONFIGS[key].bits == 4]
        for key, fp6, label in runs:
            other = WorkloadRun(key, stream, w4_fp6=fp6, unfused_gelu=args.unfused_gelu)
            pg = PEAK_FP6_TOPS if other.wl == rq.RQ_W_FP6 else PEAK_INT8_TOPS
            r = other.time(max(20, args.steps // 2), max(5, args.warmup // 2), pg)
            others[label] = {"workload": other.cfg.workload, "ms_per_step": round(r["ms_per_step"], 4),
                             "step_TOPS": round(r["tops"], 1),
                             "step_int8_peak_frac": round(r["tops"] / PEAK_INT8_TOPS, 4),
                             "kernel_us_per_step": r["kernel_us_per_step"],
                             "four_bit_codes_on": ("fp6 matrix cores" if other.wl == rq.RQ_W_FP6 else
                                                   "int8 matrix cores") if other.bits == 4 else None,
                             "calls": r["calls"]}
            del other
            torch.cuda.empty_cache()
        out["workloads"] = others

    if not args.no_context:
        log("HBM ceilings of plain elementwise kernels on X's shape (context)")
        out["context_hbm_ceilings"] = hbm_ceilings(torch, M, cfg.K, rq_us=out["roofline_rotate_quant"]["avg_launch_us"])
        log("library int8 GEMM on the %s shape (context)" % dom.name)
        out["context_library_int8_gemm"] = library_int8_gemm(torch, M, dom.N, dom.K)
        log("offline weight quantizer rules on %s" % dom.name)
        out["weight_quantizer"] = offline_weight_quant(rq, torch, g["W"][dom.name], bits, dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, ~%.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(g, cfg, args.cpu_seconds, run.act_of)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
