"""Benchmark of the SharQ linear-layer hot path on one MI355X.

One step = the whole hot path over one batch: sharq_prepare (RMSNorm, 2:4
mask, FP4 backbone, residual, FP4 residual; one HBM pass) followed by
sharq_dual_gemm (sparse-path + dense-path FP4 GEMM into one fp32 Y), on the
Llama-3.1-8B QKV-projection prefill shape (X 2048x4096 bf16, W 6144x4096).
The weight is quantized once before timing (it is not per-token work).

Inputs are synthetic and seeded (synth_inputs); several independent buffer
sets are rotated so that every step reads X and W from HBM rather than from
the 256 MB last-level cache.

Prints ONE JSON line.  `value` is the step's throughput in algorithmic
TFLOP/s (3*M*N*K: the backbone GEMM multiplies two of every four k, the
residual GEMM all of them).  `roofline` describes the dominant kernel (the
dual GEMM) against the dense MFMA peak of its operand type (HBM bandwidth
for the decode shape, whose GEMM streams the weight once); `roofline_prep`
the preparation kernel(s) against HBM bandwidth.  The timed region holds the
steps only, with one HIP event pair around it; each kernel's average launch
duration comes from the same launches of that kernel run back to back over
the same buffer sets, one event pair around the batch.
`traffic` is the HBM bytes per launch measured with rocprofv3 counters
(FETCH_SIZE and WRITE_SIZE, scaled by what the same counters read for a
device copy of known size), read from profiles/traffic.json when it was
taken on the current kernel source, else null.  `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.

Other modes, each printing one JSON line of its own: --chain times one
Llama-3.1-8B decoder layer's four linears with SharQ against the vendor bf16
and FP8 GEMMs (and the residual-add and SiLU fusions against their unfused
forms); --moe times one Qwen3-30B-A3B mixture-of-experts layer on the
grouped dual GEMM.

Traffic measurement (two counter runs, then the conversion on any host):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o pmc -- \
      python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline --calibrate-copy [--workload W]
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR_W -o pmc -- \
      python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline --calibrate-copy [--workload W]
  python3 bench.py --traffic-from DIR_F DIR_W [--workload W] [--variant V]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth_inputs as si  # noqa: E402

PEAK_FP4_TFLOPS = 10100.0        # MI355X dense MXFP4 MFMA
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
LLC_BYTES = 256 << 20            # MI355X Infinity Cache

PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20           # the counter-calibration copy


def prep_bytes_per_elem(fmt: int) -> float:
    # read bf16 (2 B); write backbone codes 1/4, meta 1/8, residual codes 1/2, and the
    # two scale arrays (1/32 each for MXFP4, 1/16 each for NVFP4)
    return 2.0 + 0.25 + 0.125 + 0.5 + (2.0 / 32 if fmt == si.MXFP4 else 2.0 / 16)


def gemm_bytes(w: si.Workload, y_bytes: float = 4.0) -> float:
    m, n, k = w.m, w.n, w.k
    blk = 32 if w.fmt == si.MXFP4 else 16
    a = m * k * (0.25 + 0.125 + 0.5) + 2 * m * k / blk
    wb = n * k * 0.5 + n * k / blk
    return a + wb + y_bytes * m * n


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparsity_fp4_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_sources(fmt: int):
    gemm = ("gemm_mx.hip", "prep_block.h") if fmt == si.MXFP4 else ("gemm_nv.hip",)
    return ((*gemm, "gemm_common.h", "fp4_device.h", "kernels.h"),
            ("prep.hip", "prep_block.h", "fp4_device.h", "kernels.h"))


def traffic_key(kind: str, w: si.Workload, variant: int, dense_view: bool, bf16_out: bool = False) -> str:
    if kind == "dual_gemm":
        return f"dual_gemm/{w.name}/v{variant}" + ("/bf16_out" if bf16_out else "")
    return f"prepare/{w.name}/{'dense' if dense_view else 'nodense'}"


def _pmc_rows(d: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no rocprofv3 counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter: str):
    """{dispatch id: (kernel name, grid size, counter value summed over instances)}"""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        name, grid, val = r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])
        if key in out:
            out[key] = (name, grid, out[key][2] + val)
        else:
            out[key] = (name, grid, val)
    return out


def traffic_convert(args, w: si.Workload):
    """Counter runs -> HBM bytes per launch of the GEMM and of one preparation
    (all its kernels), each counter scaled by its reading for the copy."""
    res = {}
    for counter, d in (("FETCH_SIZE", args.traffic_from[0]), ("WRITE_SIZE", args.traffic_from[1])):
        disp = _per_dispatch(_pmc_rows(d), counter)
        copies = [v for v in disp.values() if "copyBuffer" in v[0]]
        if not copies:
            raise SystemExit(f"{d}: no calibration copy (run the bench with --calibrate-copy)")
        # the calibration copy is by far the largest copy of the run
        factor = COPY_BYTES / (max(c[2] for c in copies) * 1024.0)
        # one preparation = its prep_* kernel plus the NVFP4 amax kernels
        # launched right before it; any other kernel (the weight
        # quantization's amax pass included) drops the pending amax kernels
        gemm, prep, pending = [], [], []
        for key in sorted(disp):
            name, _, val = disp[key]
            if "dual_gemm" in name:
                gemm.append(val)
                pending = []
            elif "prep_" in name:
                prep.append(sum(pending) + val)
                pending = []
            elif "amax" in name:
                pending.append(val)
            else:
                pending = []
        res[counter] = {"factor": factor, "gemm_kib": float(np.mean(gemm)),
                        "prep_kib": float(np.mean(prep)), "launches": len(gemm)}
    f, wr = res["FETCH_SIZE"], res["WRITE_SIZE"]
    gemm_src, prep_src = kernel_sources(w.fmt)
    entries = {
        traffic_key("dual_gemm", w, args.variant, not args.no_dense_view, args.bf16_out): {
            "source_hash": source_hash(*gemm_src),
            "fetch_kib": round(f["gemm_kib"], 1), "write_kib": round(wr["gemm_kib"], 1),
            "bytes_per_launch": round(f["gemm_kib"] * 1024 * f["factor"] + wr["gemm_kib"] * 1024 * wr["factor"]),
            "launches": f["launches"]},
        traffic_key("prepare", w, args.variant, not args.no_dense_view): {
            "source_hash": source_hash(*prep_src),
            "fetch_kib": round(f["prep_kib"], 1), "write_kib": round(wr["prep_kib"], 1),
            "bytes_per_launch": round(f["prep_kib"] * 1024 * f["factor"] + wr["prep_kib"] * 1024 * wr["factor"])},
    }
    path = os.path.join(PROFILES, "traffic.json")
    d = {}
    if os.path.exists(path):
        with open(path) as fh:
            d = json.load(fh)
    d["copy_calibration"] = {"bytes": COPY_BYTES, "fetch_factor": round(f["factor"], 4),
                             "write_factor": round(wr["factor"], 4)}
    d.update(entries)
    with open(path, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(entries))


def traffic_from_profiles(kernel_key: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or
    None when absent or taken on another version of the kernel source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


def yardsticks(w: si.Workload, torch, dev) -> dict:
    """What plain work of the same size takes on this GPU (context, not targets):
    a device copy that reads 2 B and writes 1 B per element of X (the
    preparation's traffic), and the vendor MXFP4 GEMM (hipBLASLt through
    torch._scaled_mm) on the dual GEMM folded into one GEMM with K' = 2K.
    Each is the mean of 20 back-to-back launches between two events."""
    out = {}

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    n_el = w.m * w.k
    src = torch.empty(2 * n_el, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n_el, dtype=torch.uint8, device=dev)
    # reads both halves of src (2 B / element), writes dst (1 B / element)
    us = timed(lambda: torch.maximum(src[:n_el], src[n_el:], out=dst))
    out["copy_like_prep"] = {"us": round(us, 3), "bytes": 3 * n_el,
                             "GB/s": round(3 * n_el / (us * 1e-6) / 1e9, 1)}
    del src, dst
    if w.fmt == si.MXFP4 and w.m > 64:
        try:
            K2 = 2 * w.k
            a = torch.randint(0, 255, (w.m, K2 // 2), dtype=torch.uint8, device=dev).view(torch.float4_e2m1fn_x2)
            b = torch.randint(0, 255, (w.n, K2 // 2), dtype=torch.uint8, device=dev).view(torch.float4_e2m1fn_x2)
            sa = torch.full((w.m, K2 // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
            sb = torch.full((w.n, K2 // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
            us = timed(lambda: torch._scaled_mm(a, b.t(), sa, sb, out_dtype=torch.bfloat16))
            out["vendor_mxfp4_gemm_folded"] = {"us": round(us, 3), "m": w.m, "n": w.n, "k": K2,
                                               "dense_TFLOP/s": round(2.0 * w.m * w.n * K2 / (us * 1e-6) / 1e12, 1)}
        except Exception as e:  # not every torch build routes MX formats to hipBLASLt
            out["vendor_mxfp4_gemm_folded"] = {"error": str(e)[:200]}
    if w.fmt == si.MXFP4 and w.m > 64:
        out["mfma_fp4_random_operands"] = mfma_yardstick(torch, dev)
    if w.m <= 64:
        out["stream_read_gemm_bytes"] = stream_read_yardstick(torch, dev, gemm_bytes(w))
    return out


def stream_read_yardstick(torch, dev, nbytes: float) -> dict:
    """A kernel that only reads (csrc/yardstick.hip), over as many bytes as the
    decode GEMM's algorithmic traffic: the rate a plain read of that size
    reaches from HBM.  Five buffers are read in turn (more than the 256 MB
    Infinity Cache holds), 20 launches between two events."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "sparsity_fp4_quantized_amd", "libsharq_yardstick.so"))
    L.sharq_yardstick_stream_read.restype = ctypes.c_int
    L.sharq_yardstick_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    size = int((nbytes + 16383) // 16384 * 16384)
    bufs = [torch.ones(size, dtype=torch.uint8, device=dev) for _ in range(5)]
    out = torch.empty(size // 16384, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    reps = 20

    def launch(i):
        rc = L.sharq_yardstick_stream_read(bufs[i % 5].data_ptr(), size, out.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"stream read yardstick: launch returned {rc}")

    for i in range(5):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"us": round(us, 3), "bytes": size, "GB/s": round(size / (us * 1e-6) / 1e9, 1)}


def mfma_yardstick(torch, dev) -> dict:
    """A kernel doing nothing but FP4 scaled MFMAs on random operands (two
    workgroups of four wavefronts per CU, as the tiled dual GEMM): its
    FLOP/s and the engine clock it ran at (s_memtime against the 100 MHz
    s_memrealtime), i.e. the MFMA rate this GPU sustains on FP4 data."""
    import ctypes
    path = os.path.join(ROOT, "sparsity_fp4_quantized_amd", "libsharq_yardstick.so")
    L = ctypes.CDLL(path)
    L.sharq_yardstick_mfma_fp4.restype = ctypes.c_int
    L.sharq_yardstick_mfma_fp4.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    wgs, iters = 512, 4000
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    ticks = torch.empty(2 * wgs, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for label, rnd in (("random", 1), ("constant", 0)):
        for _ in range(2):   # the second launch is the one reported
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = L.sharq_yardstick_mfma_fp4(wgs, iters, rnd, out.data_ptr(), ticks.data_ptr(), stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                return {"error": f"launch returned {rc}"}
        t = ticks.view(wgs, 2).double().sum(0).cpu().numpy()
        flops = wgs * 4 * iters * 24 * 2.0 * 32 * 32 * 64
        us = e0.elapsed_time(e1) * 1e3
        res[label] = {"us": round(us, 1), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                      "clock_MHz": round(100.0 * t[1] / t[0])}
    return res


def _host_cpu():
    """(CPU model name, CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc


def cpu_baseline(w: si.Workload, x, W, g, reps: int = 3) -> dict:
    """The CPU oracle as committed, built for this host (gcc -O3 -march=native
    -fopenmp -ffp-contract=off, no fast-math: the same values as the test
    build), timed on one thread and on all the threads this process may use:
    the preparation on the whole X, the dual GEMM on a sample of whole rows of
    Y (every column), each the median of `reps` runs.  The full step's time is
    the preparation's plus the GEMM sample's scaled to all rows; `value` is
    the all-threads figure in the unit of the GPU line."""
    import statistics

    import oracle
    try:
        L = oracle.omp_lib_built()
        build = "gcc " + " ".join(oracle.OMP_CFLAGS)
    except Exception as e:                      # no compiler: the plain build, one thread
        L, build = None, f"plain build ({type(e).__name__} building the OpenMP one)"
    model, nproc = _host_cpu()
    env = os.environ.get("OMP_NUM_THREADS")
    all_threads = int(env) if env and env.isdigit() else nproc
    q = oracle.quantize_weight(w.fmt, W)      # the weight is quantized offline: untimed
    flops = 3.0 * w.m * w.n * w.k

    def run(threads):
        used = L.oracle_threads(threads) if L is not None else 1
        rows = min(w.m, -(-max(8, used) // used) * used)
        tp, tg = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            p = oracle.prepare(w.fmt, x, g, L=L)
            tp.append(time.perf_counter() - t0)
            ps = oracle.gather_rows(p, np.arange(rows))
            t0 = time.perf_counter()
            oracle.dual_gemm(w.fmt, ps, q, L=L)
            tg.append(time.perf_counter() - t0)
        prep_s, gemm_rows_s = statistics.median(tp), statistics.median(tg)
        gemm_s = gemm_rows_s * w.m / rows
        step_s = prep_s + gemm_s
        pbytes = w.m * w.k * prep_bytes_per_elem(w.fmt)
        return {"threads": used, "prep_s": round(prep_s, 4), "prep_GB/s": round(pbytes / prep_s / 1e9, 3),
                "gemm_rows_sampled": rows, "gemm_sample_s": round(gemm_rows_s, 4),
                "gemm_s_projected": round(gemm_s, 2), "gemm_TFLOP/s": flops / gemm_s / 1e12,
                "step_s_projected": round(step_s, 2), "TFLOP/s": flops / step_s / 1e12}

    one = run(1)
    many = run(all_threads) if L is not None and all_threads > 1 else one
    return {"value": many["TFLOP/s"], "unit": "TFLOP/s", "cores": many["threads"], "kind": "oracle",
            "sample": (f"oracle preparation of the whole X ({w.m}x{w.k}) and dual GEMM of the first "
                       f"{many['gemm_rows_sampled']} (all threads) / {one['gemm_rows_sampled']} (one thread) "
                       f"rows of Y against all {w.n} columns (K={w.k}); median of {reps} runs each; the "
                       f"full step's time is the preparation's plus the GEMM sample's scaled to {w.m} rows"),
            "single_thread": one, "all_threads": many, "nproc": nproc, "OMP_NUM_THREADS": env,
            "cpu_model": model, "build": build}


CHAIN_LAYERS = 3     # weight copies cycled, so that no linear's W stays in the 256 MB cache


def chain_main(args):
    """Decoder-layer linear chain: Llama-3.1-8B's QKV -> O -> gate+up -> down,
    at prefill (2048 tokens) and decode (16 tokens), with SharQ (preparation +
    dual GEMM, MXFP4, fp32 Y) against the vendor GEMMs on the same shapes:
    bf16 (torch.nn.functional.linear -> hipBLASLt, bf16 out) and FP8 E4M3
    with per-tensor scales (torch._scaled_mm, bf16 out), the latter also with
    the activation's dynamic quantization (amax, scale, cast) counted.  The
    baselines get no RMSNorm, SharQ's preparation includes it where the layer
    has one.  Speed only: accuracy needs the model's weights.  Weights: one
    seeded N(0, 0.02) draw per linear, and CHAIN_LAYERS row-rotated copies that
    the timed loop cycles through.  ``sharq_with_silu_fused`` is the layer as
    SharQ runs it: QKV and O as above, then gate+up with SiLU(gate) * up and
    down's preparation in its epilogue, and down without a preparation of its
    own (it does the SiLU the other chains leave out).  Prints one JSON line."""
    import torch
    import torch.nn.functional as F
    import sparsity_fp4_quantized_amd as sq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    reps, warm = max(args.steps // 4, 10), max(args.warmup // 4, 5)
    fp8 = torch.float8_e4m3fn
    one = torch.ones((), dtype=torch.float32, device=dev)

    def batch_us(fn):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    # weights: bf16, FP8 (per-tensor scale) and the SharQ payload, per layer copy
    wts = {}
    for lin in si.LAYER_LINEARS:
        w = si.layer_workload(lin, 16)
        W0 = torch.from_numpy(si.workload_w(w).view(np.int16)).to(dev).view(torch.bfloat16)
        copies = [torch.roll(W0, shifts=7 * l, dims=0).contiguous() for l in range(CHAIN_LAYERS)]
        ws = [(Wl.abs().amax().float() / 448.0) for Wl in copies]
        w8 = [(Wl.float() / sc).to(fp8) for Wl, sc in zip(copies, ws)]
        wq = [sq.quantize_weight(Wl.view(torch.int16)) for Wl in copies]
        wts[lin] = (copies, w8, ws, wq)
    torch.cuda.synchronize()

    result = {"metric": "Llama-3.1-8B decoder-layer linear chain (QKV, O, gate+up, down) time",
              "unit": "us", "higher_is_better": False, "layers_cycled": CHAIN_LAYERS,
              "steps": reps, "warmup": warm, "data": "synthetic (seeded activations, N(0,0.02) weights)"}
    for phase, m in (("prefill", 2048), ("decode", 16)):
        runs = {"sharq": [], "sharq_bf16_out": [], "bf16": [], "fp8": [], "fp8_with_act_quant": []}
        per = {}
        for lin in si.LAYER_LINEARS:
            w = si.layer_workload(lin, m)
            copies, w8, ws, wq = wts[lin]
            x = torch.from_numpy(si.workload_x(w).view(np.int16)).to(dev)
            g = None if not w.norm else torch.from_numpy(si.workload_gamma(w).view(np.int16)).to(dev)
            xb = x.view(torch.bfloat16)
            xs = xb.abs().amax().float() / 448.0
            x8 = (xb.float() / xs).to(fp8)
            sp, rs = sq.alloc_prepared(sq.MXFP4, m, w.k, dev, dense_backbone=True)
            y = torch.empty((m, w.n), dtype=torch.float32, device=dev)
            calls = [(sq.bind_prepare(x, g, 1e-5, sp, rs), sq.bind_dual_gemm(sp, rs, wq[l], y))
                     for l in range(CHAIN_LAYERS)]
            # the same with Y stored in bf16 (sharq_dual_gemm_bf16), the
            # output type the vendor GEMMs below write
            y16 = torch.empty((m, w.n), dtype=torch.bfloat16, device=dev)
            calls16 = [(sq.bind_prepare(x, g, 1e-5, sp, rs), sq.bind_dual_gemm(sp, rs, wq[l], y16))
                       for l in range(CHAIN_LAYERS)]

            def sharq(i, calls=calls):
                p, q = calls[i % CHAIN_LAYERS]
                p()
                q()

            def sharq16(i, calls=calls16):
                p, q = calls[i % CHAIN_LAYERS]
                p()
                q()

            def bf16(i, xb=xb, copies=copies):
                F.linear(xb, copies[i % CHAIN_LAYERS])

            def f8(i, x8=x8, xs=xs, w8=w8, ws=ws):
                torch._scaled_mm(x8, w8[i % CHAIN_LAYERS].t(), xs, ws[i % CHAIN_LAYERS], out_dtype=torch.bfloat16)

            def f8q(i, xb=xb, w8=w8, ws=ws):
                s_ = xb.abs().amax().float() / 448.0
                q8 = (xb / s_).to(fp8)
                torch._scaled_mm(q8, w8[i % CHAIN_LAYERS].t(), s_, ws[i % CHAIN_LAYERS], out_dtype=torch.bfloat16)

            fns = {"sharq": sharq, "sharq_bf16_out": sharq16, "bf16": bf16, "fp8": f8, "fp8_with_act_quant": f8q}
            per[lin] = {}
            for k, fn in fns.items():
                try:
                    per[lin][k] = round(batch_us(fn), 2)
                    if runs[k] is not None:
                        runs[k].append(fn)
                except (RuntimeError, TypeError) as e:   # a torch build without this vendor path
                    per[lin][k] = {"error": str(e)[:200]}
                    runs[k] = None
        # the residual add in front of QKV's norm: fused into the preparation
        # (one kernel) against torch's bf16 add followed by the preparation
        w = si.layer_workload("qkv", m)
        h = torch.from_numpy(si.workload_x(w).view(np.int16)).to(dev)
        o = torch.from_numpy(si.activations("normal", m, w.k, 0, 1.0, 40).view(np.int16)).to(dev)
        g = torch.from_numpy(si.workload_gamma(w).view(np.int16)).to(dev)
        xsum = torch.empty_like(h)
        sp, rs = sq.alloc_prepared(sq.MXFP4, m, w.k, dev, dense_backbone=True)
        fused = sq.bind_prepare_residual(h, o, g, 1e-5, sp, rs, xsum)
        plain = sq.bind_prepare(xsum, g, 1e-5, sp, rs)
        hb, ob, xb_ = h.view(torch.bfloat16), o.view(torch.bfloat16), xsum.view(torch.bfloat16)

        def unfused(i):
            torch.add(hb, ob, out=xb_)
            plain()

        residual_add = {"fused_us": round(batch_us(lambda i: fused()), 2),
                        "torch_add_then_prepare_us": round(batch_us(unfused), 2)}
        # SiLU(gate) * up in front of down: fused into the preparation, reading
        # the two halves of the gate+up projection's fp32 output, against
        # torch's silu, multiply and bf16 cast followed by the preparation
        F_ = si.LAYER_LINEARS["down"][0]
        g_, u_ = si.gate_up_output(m, F_, 42)
        gu = torch.from_numpy(np.concatenate([g_, u_], axis=1)).to(dev)
        gate, up = gu[:, :F_], gu[:, F_:]
        spd, rsd = sq.alloc_prepared(sq.MXFP4, m, F_, dev, dense_backbone=True)
        xd = torch.empty((m, F_), dtype=torch.bfloat16, device=dev)
        fused_s = sq.bind_prepare_silu_mul(gate, up, spd, rsd)
        plain_s = sq.bind_prepare(xd.view(torch.int16), None, 1e-5, spd, rsd)

        def unfused_s(i):
            torch.mul(F.silu(gate), up, out=xd)
            plain_s()

        silu_mul = {"fused_us": round(batch_us(lambda i: fused_s()), 2),
                    "torch_silu_mul_then_prepare_us": round(batch_us(unfused_s), 2)}
        # the SharQ layer as it runs: gate+up's epilogue forms SiLU(gate) * up
        # and prepares it for down (sharq_dual_gemm_silu_prepare; at decode,
        # where 128-row tiles waste the GEMM, the fp32 product goes through
        # sharq_prepare_silu_mul), so down has no preparation of its own.  It
        # does the SiLU work that the chains above leave out.
        wgu = si.layer_workload("gate_up", m)
        inter = wgu.n // 2
        xg = torch.from_numpy(si.workload_x(wgu).view(np.int16)).to(dev)
        gg = torch.from_numpy(si.workload_gamma(wgu).view(np.int16)).to(dev)
        spg, rsg = sq.alloc_prepared(sq.MXFP4, m, wgu.k, dev, dense_backbone=True)
        spx, rsx = sq.alloc_prepared(sq.MXFP4, m, inter, dev, dense_backbone=True)
        yd = torch.empty((m, si.LAYER_LINEARS["down"][1]), dtype=torch.float32, device=dev)
        prep_g = sq.bind_prepare(xg, gg, 1e-5, spg, rsg)
        if m > 32:
            gu_calls = [sq.bind_dual_gemm_silu_prepare(spg, rsg, wts["gate_up"][3][l], spx, rsx)
                        for l in range(CHAIN_LAYERS)]
        else:
            ygu = torch.empty((m, wgu.n), dtype=torch.float32, device=dev)
            silu_p = sq.bind_prepare_silu_mul(ygu[:, :inter], ygu[:, inter:], spx, rsx)
            gu_calls = [(lambda q=sq.bind_dual_gemm(spg, rsg, wts["gate_up"][3][l], ygu): (q(), silu_p()))
                        for l in range(CHAIN_LAYERS)]
        down_calls = [sq.bind_dual_gemm(spx, rsx, wts["down"][3][l], yd) for l in range(CHAIN_LAYERS)]
        yd16 = torch.empty((m, si.LAYER_LINEARS["down"][1]), dtype=torch.bfloat16, device=dev)
        down_calls16 = [sq.bind_dual_gemm(spx, rsx, wts["down"][3][l], yd16) for l in range(CHAIN_LAYERS)]

        def mlp(i):
            prep_g()
            gu_calls[i % CHAIN_LAYERS]()
            down_calls[i % CHAIN_LAYERS]()

        def mlp16(i):
            prep_g()
            gu_calls[i % CHAIN_LAYERS]()
            down_calls16[i % CHAIN_LAYERS]()

        per["gate_up_silu_down"] = {"sharq_fused": round(batch_us(mlp), 2),
                                    "sharq_fused_bf16_out": round(batch_us(mlp16), 2)}
        chain = {}
        for k, fns in runs.items():
            if fns is not None and len(fns) == len(si.LAYER_LINEARS):
                chain[k] = round(batch_us(lambda i, fns=fns: [fn(i) for fn in fns]), 2)
        if runs["sharq"] is not None:
            layer = runs["sharq"][:2] + [mlp]
            chain["sharq_with_silu_fused"] = round(batch_us(lambda i: [fn(i) for fn in layer]), 2)
        if runs["sharq_bf16_out"] is not None:
            layer16 = runs["sharq_bf16_out"][:2] + [mlp16]
            chain["sharq_with_silu_fused_bf16_out"] = round(batch_us(lambda i: [fn(i) for fn in layer16]), 2)
        speed = {f"sharq_speedup_vs_{k}": round(chain[k] / chain["sharq"], 3)
                 for k in chain if not k.startswith("sharq")}
        if "sharq_bf16_out" in chain:
            speed.update({f"sharq_bf16_out_speedup_vs_{k}": round(chain[k] / chain["sharq_bf16_out"], 3)
                          for k in chain if not k.startswith("sharq")})
        result[phase] = {"m": m, "chain_us": chain, "per_linear_us": per, **speed,
                         "qkv_residual_add_and_prepare": residual_add,
                         "down_silu_mul_and_prepare": silu_mul}
    print(json.dumps(result), flush=True)


def moe_main(args):
    """One Qwen3-30B-A3B mixture-of-experts layer at prefill (4096 tokens, 128
    experts, 8 a token, hidden 2048, expert intermediate 768): the tokens'
    preparation (RMSNorm, once per token), the grouped gate+up dual GEMM over
    the gathered rows (n 1536, k 2048), SiLU(gate) * up fused into the down
    projection's preparation, and the grouped down dual GEMM (n 2048, k 768);
    ``layer_silu_fused`` runs SiLU(gate) * up and that preparation in the
    grouped gate+up GEMM's epilogue instead.
    Seeded routing with uneven expert loads.  Against torch's bf16 grouped GEMM
    (torch._grouped_mm) on the same groups where this torch build has one.
    Prints one JSON line."""
    import torch
    import sparsity_fp4_quantized_amd as sq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = si.MOE_QWEN3_30B_A3B
    T, H, I, E, K8 = 4096, cfg["hidden"], cfg["intermediate"], cfg["experts"], cfg["top_k"]
    reps, warm = max(args.steps // 4, 10), max(args.warmup // 4, 5)

    def batch_us(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    x = torch.from_numpy(si.activations("student_t4", T, H, 20, 50.0, 101).view(np.int16)).to(dev)
    g = torch.from_numpy(si.gamma(H, None).view(np.int16)).to(dev)
    row_index, offsets = si.moe_routing(T, E, K8, 102)
    rows = int(offsets[-1])
    idx_d = torch.from_numpy(row_index).to(dev)
    off_d = torch.from_numpy(offsets).to(dev)
    w13 = torch.from_numpy(si.weights(E * 2 * I, H, 103).view(np.int16)).to(dev)
    w2 = torch.from_numpy(si.weights(E * H, I, 104).view(np.int16)).to(dev)
    q13, q2 = sq.quantize_weight(w13), sq.quantize_weight(w2)
    sp, rs = sq.alloc_prepared(sq.MXFP4, T, H, dev, dense_backbone=True)
    y13 = torch.empty((rows, 2 * I), dtype=torch.float32, device=dev)
    sp2, rs2 = sq.alloc_prepared(sq.MXFP4, rows, I, dev, dense_backbone=True)
    y2 = torch.empty((rows, H), dtype=torch.float32, device=dev)
    prep = sq.bind_prepare(x, g, 1e-5, sp, rs)
    gemm13 = sq.bind_grouped_dual_gemm(sp, rs, q13, off_d, rows, y13, row_index=idx_d)
    prep2 = sq.bind_prepare_silu_mul(y13[:, :I], y13[:, I:], sp2, rs2)
    gemm2 = sq.bind_grouped_dual_gemm(sp2, rs2, q2, off_d, rows, y2)

    # the same with SiLU(gate) * up and down's preparation in the grouped
    # gate+up GEMM's epilogue (no fp32 gate+up output)
    sp3, rs3 = sq.alloc_prepared(sq.MXFP4, rows, I, dev, dense_backbone=True)
    fused13 = sq.bind_grouped_dual_gemm_silu_prepare(sp, rs, q13, off_d, rows, sp3, rs3, row_index=idx_d)
    gemm2f = sq.bind_grouped_dual_gemm(sp3, rs3, q2, off_d, rows, y2)

    if args.power:
        # the grouped gate+up GEMM back to back (its operands prepared first),
        # then the tokens' preparation, beside the FP4 MFMA yardstick
        import types
        power_main(types.SimpleNamespace(name="qwen3_30b_a3b_moe_grouped_gate_up"), torch, dev,
                   [prep], [gemm13], 1)
        return

    def layer():
        prep()
        gemm13()
        prep2()
        gemm2()

    def layer_fused():
        prep()
        fused13()
        gemm2f()

    t = {"prepare": batch_us(prep), "grouped_gate_up": batch_us(gemm13),
         "silu_mul_prepare": batch_us(prep2), "grouped_down": batch_us(gemm2), "layer": batch_us(layer),
         "grouped_gate_up_silu_prepare": batch_us(fused13), "layer_silu_fused": batch_us(layer_fused)}
    f13, f2 = 3.0 * rows * 2 * I * H, 3.0 * rows * H * I
    res = {"metric": "Qwen3-30B-A3B MoE layer (prefill, 4096 tokens): grouped dual-path FP4 GEMMs",
           "unit": "us", "higher_is_better": False, "steps": reps, "warmup": warm,
           "data": "synthetic (seeded activations and routing, N(0,0.02) weights)",
           "config": {"workload": "qwen3_30b_a3b_moe_prefill", "tokens": T, "experts": E, "top_k": K8,
                      "hidden": H, "intermediate": I, "rows": rows,
                      "group_rows_min_max": [int(np.diff(offsets).min()), int(np.diff(offsets).max())]},
           "times_us": {k: round(v, 2) for k, v in t.items()},
           "grouped_gate_up_TFLOP/s": round(f13 / (t["grouped_gate_up"] * 1e-6) / 1e12, 1),
           "grouped_gate_up_frac_of_fp4_peak": round(f13 / (t["grouped_gate_up"] * 1e-6) / 1e12 / PEAK_FP4_TFLOPS, 4),
           "grouped_down_TFLOP/s": round(f2 / (t["grouped_down"] * 1e-6) / 1e12, 1),
           "grouped_down_frac_of_fp4_peak": round(f2 / (t["grouped_down"] * 1e-6) / 1e12 / PEAK_FP4_TFLOPS, 4)}
    # vendor bf16 grouped GEMM on the same groups (gate+up), where available
    try:
        xb = x.view(torch.bfloat16)[idx_d.long()]
        wb = w13.view(torch.bfloat16).view(E, 2 * I, H).transpose(1, 2).contiguous()   # [E, k, n], dense
        ends = off_d[1:].to(torch.int32)
        us = batch_us(lambda: torch._grouped_mm(xb, wb, offs=ends, out_dtype=torch.bfloat16))
        res["bf16_grouped_mm_gate_up_us"] = round(us, 2)
    except (RuntimeError, AttributeError, TypeError) as e:
        res["bf16_grouped_mm_gate_up_us"] = {"error": str(e)[:200]}
    print(json.dumps(res), flush=True)


def parse_amd_smi_power(text: str):
    """(socket power W, mean gfx clock MHz over the XCDs) from the CSV that
    `amd-smi metric -p -c --csv` prints for one GPU (a header line starting
    `gpu,` and one data line), or None when either is missing."""
    ls = text.strip().splitlines()
    hdr = next((l.split(",") for l in ls if l.startswith("gpu,")), None)
    row = next((l.split(",") for l in ls if l[:1].isdigit()), None)
    if not hdr or not row or len(hdr) != len(row):
        return None
    d = dict(zip(hdr, row))
    try:
        clk = [float(d[f"gfx_{i}_clk"]) for i in range(8) if f"gfx_{i}_clk" in d]
        return float(d["socket_power"]), sum(clk) / len(clk)
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def power_main(w: si.Workload, torch, dev, preps, gemms, nsets: int) -> None:
    """Socket power and engine clocks while one kernel runs back to back.

    A sampler thread reads `amd-smi metric -p -c --csv` (socket power, the
    eight XCDs' gfx clocks; the reading refreshes about once a second; the
    board's limit from `rocm-smi -M`) while
    the dual GEMM, the preparation and the FP4 MFMA yardstick (random and
    constant operands) each run for a few seconds, with an idle gap between
    them.  Per phase: the launch time and the median of the samples taken
    after its first second (the settled state).  This tells whether a kernel
    runs at the board's power limit, where the engine clock, not the
    schedule, sets its speed."""
    import ctypes
    import statistics
    import subprocess
    import threading

    samples, phase, stop = [], ["start"], threading.Event()

    def read():
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--csv"], capture_output=True, text=True)
        return parse_amd_smi_power(r.stdout)

    def sampler():
        while not stop.is_set():
            v = read()
            if v is not None:
                samples.append((time.time(), phase[0], v[0], v[1]))
            time.sleep(0.1)

    cap = subprocess.run(["rocm-smi", "-M", "--csv"], capture_output=True, text=True)
    if read() is None:
        raise SystemExit("amd-smi gave no socket power reading on this machine")
    path = os.path.join(ROOT, "sparsity_fp4_quantized_amd", "libsharq_yardstick.so")
    L = ctypes.CDLL(path)
    L.sharq_yardstick_mfma_fp4.restype = ctypes.c_int
    L.sharq_yardstick_mfma_fp4.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    out = torch.empty(512 * 256, dtype=torch.float32, device=dev)
    ticks = torch.empty(1024, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def yard(rnd):
        def f(i):
            if L.sharq_yardstick_mfma_fp4(512, 4000, rnd, out.data_ptr(), ticks.data_ptr(), stream) != 0:
                raise RuntimeError("yardstick launch failed")
        return f

    for p in preps:   # every set's GEMM operands prepared from its X
        p()
    torch.cuda.synchronize()
    phases = [("dual_gemm", lambda i: gemms[i % nsets](), 4.0, 200),
              ("prepare", lambda i: preps[i % nsets](), 3.0, 1000),
              ("mfma_fp4_random_operands", yard(1), 4.0, 20),
              ("mfma_fp4_constant_operands", yard(0), 3.0, 20)]
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    res, spans = {}, {}
    time.sleep(1.5)
    for name, fn, secs, per in phases:
        phase[0] = name
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0, n = time.time(), 0
        e0.record()
        while time.time() - t0 < secs:
            for _ in range(per):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        spans[name] = (t0 + 1.0, time.time())
        res[name] = {"launches": n, "us_per_launch": round(e0.elapsed_time(e1) * 1e3 / n, 2)}
        phase[0] = "idle"
        time.sleep(1.5)
    stop.set()
    th.join()
    for name, (a, b) in spans.items():
        ps = [p for t, ph, p, c in samples if ph == name and a <= t <= b]
        cs = [c for t, ph, p, c in samples if ph == name and a <= t <= b]
        if ps:
            res[name]["socket_power_W"] = round(statistics.median(ps), 1)
            res[name]["gfx_clock_MHz"] = round(statistics.median(cs), 1)
            res[name]["samples"] = len(ps)
    idle = [p for t, ph, p, c in samples if ph == "start"]
    cap_w = None
    for l in cap.stdout.splitlines():
        f = l.split(",")
        if len(f) == 2 and f[0].startswith("card"):
            try:
                cap_w = float(f[1])
            except ValueError:
                pass
    print(json.dumps({"metric": "socket power and engine clock per kernel, back to back", "workload": w.name,
                      "power_cap_W": cap_w,
                      "idle_socket_power_W": round(statistics.median(idle), 1) if idle else None,
                      "phases": res, "sampler": "amd-smi metric -p -c --csv, every ~0.1 s"}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 200 untimed steps: after 20 the qkv step still ran 8% slower than after
    # 200 (67-68 against 62 us, the same kernels) while the GPU settled
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="qkv_prefill", choices=sorted(si.WORKLOADS))
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--no-dense-view", action="store_true",
                    help="prepare writes only the 2:4 backbone; the GEMM expands it")
    ap.add_argument("--bf16-out", action="store_true",
                    help="the dual GEMM writes Y in bf16 (sharq_dual_gemm_bf16) instead of fp32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="time only the CPU oracle on the workload (no GPU work) and print its JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help=f"run one {COPY_BYTES >> 20} MiB device copy first (counter calibration)")
    ap.add_argument("--no-yardsticks", action="store_true",
                    help="skip the plain-copy and vendor FP4 GEMM reference timings")
    ap.add_argument("--moe", action="store_true",
                    help="time one Qwen3-30B-A3B mixture-of-experts layer (grouped dual GEMMs) instead")
    ap.add_argument("--chain", action="store_true",
                    help="time the decoder-layer linear chain (SharQ vs bf16 / FP8 vendor GEMMs) instead")
    ap.add_argument("--power", action="store_true",
                    help="sample socket power and engine clocks (amd-smi) while the workload's dual GEMM, "
                         "its preparation and the FP4 MFMA yardstick each run back to back, and exit "
                         "(with --moe: the grouped gate+up GEMM and the tokens' preparation)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="convert two rocprofv3 --pmc runs into profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_convert(args, si.WORKLOADS[args.workload])
        return
    if args.cpu_baseline_only:
        w = si.WORKLOADS[args.workload]
        out = {"workload": w.name, "cpu_baseline": cpu_baseline(w, si.workload_x(w), si.workload_w(w),
                                                               si.workload_gamma(w))}
        print(json.dumps(out), flush=True)
        return

    if args.moe and args.gpus == 1:
        moe_main(args)
        return
    if args.chain and args.gpus == 1:
        chain_main(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the SharQ path here "
              "is single-GPU, and its sharding is described, not run.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparsity_fp4_quantized_amd as sq

    w = si.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x_np, W_np, g_np = si.workload_x(w), si.workload_w(w), si.workload_gamma(w)
    blk = sq.BLOCK[w.fmt]
    y_bytes = 2.0 if args.bf16_out else 4.0
    per_set = w.m * w.k * (2 + 0.9375) + w.n * w.k * 0.53 + y_bytes * w.m * w.n
    nsets = int(min(16, max(2, np.ceil(2 * LLC_BYTES / per_set))))

    x0 = torch.from_numpy(x_np.view(np.int16)).to(dev)
    W0 = torch.from_numpy(W_np.view(np.int16)).to(dev)
    g = None if g_np is None else torch.from_numpy(g_np.view(np.int16)).to(dev)
    sets = []
    for i in range(nsets):
        xi = x0.clone()
        wq = sq.quantize_weight(W0.clone() if i else W0, w.fmt)
        sp, rs = sq.alloc_prepared(w.fmt, w.m, w.k, dev, dense_backbone=not args.no_dense_view)
        y = torch.empty((w.m, w.n), dtype=torch.bfloat16 if args.bf16_out else torch.float32, device=dev)
        sets.append((xi, wq, sp, rs, y))
    torch.cuda.synchronize()

    # each set's two library calls with their arguments marshalled once, so
    # that a step costs the host two calls into the library (unbound, the
    # Python marshalling took about 9 us a call: more than a decode step's
    # kernels and about as long as the qkv preparation)
    preps = [sq.bind_prepare(xi, g, 1e-5, sp, rs) for (xi, wq, sp, rs, y) in sets]
    gemms = [sq.bind_dual_gemm(sp, rs, wq, y, variant=args.variant) for (xi, wq, sp, rs, y) in sets]

    def step(i):
        preps[i % nsets]()
        gemms[i % nsets]()

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.power:
        power_main(w, torch, dev, preps, gemms, nsets)
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronized on both sides, with one
    # event pair around it (events between kernels would add ~4 us each)
    stream = torch.cuda.current_stream()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    step_ms_events = e_start.elapsed_time(e_end) / args.steps

    # per-kernel average launch duration: the timed region's launches of one
    # kernel, back to back on the same stream over the same buffer sets, one
    # event pair around the batch
    def batch_ms(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def prep_only(i):
        preps[i % nsets]()

    def gemm_only(i):
        gemms[i % nsets]()

    prep_ms = batch_ms(prep_only, args.steps)
    gemm_ms = batch_ms(gemm_only, args.steps)

    flops = 3.0 * w.m * w.n * w.k
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    pbytes = w.m * w.k * (prep_bytes_per_elem(w.fmt) + (0.0 if args.no_dense_view else 0.5))
    prep_gbps = pbytes / (prep_ms * 1e-3) / 1e9
    peak = PEAK_FP4_TFLOPS if w.fmt == sq.MXFP4 else PEAK_BF16_TFLOPS

    gemm_src, prep_src = kernel_sources(w.fmt)
    dense_view = not args.no_dense_view
    gemm_traffic = traffic_from_profiles(traffic_key("dual_gemm", w, args.variant, dense_view, args.bf16_out),
                                         source_hash(*gemm_src))
    prep_traffic = traffic_from_profiles(traffic_key("prepare", w, args.variant, dense_view),
                                         source_hash(*prep_src))
    gbytes = gemm_bytes(w, y_bytes)
    if w.m <= 64:
        # decode: the GEMM streams W once; HBM bandwidth bounds it
        gemm_gbps = gbytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "dual_gemm", "achieved": round(gemm_gbps, 1),
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gemm_gbps / PEAK_HBM_GBPS, 4),
                    "traffic": gemm_traffic, "avg_launch_us": round(gemm_ms * 1e3, 3),
                    "algorithmic_bytes_per_launch": gbytes, "algorithmic_flops_per_launch": flops}
    else:
        roofline = {"bound": "mfma", "kernel": "dual_gemm", "achieved": round(gemm_tflops, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                    "traffic": gemm_traffic, "avg_launch_us": round(gemm_ms * 1e3, 3),
                    "algorithmic_flops_per_launch": flops,
                    # the structured-sparse MFMA skips the backbone's zero half
                    # (SPARSE_MFMA, and AUTO for NVFP4, which resolves to it)
                    "executed_TFLOP/s": round((1.0 if (args.variant == 3 or (w.fmt == sq.NVFP4 and args.variant == 0))
                                               else 4.0 / 3.0) * gemm_tflops, 2),
                    "dense_equivalent_TFLOP/s": round(2.0 / 3.0 * gemm_tflops, 2)}

    out = {
        "metric": "dual-path FP4 GEMM TFLOP/s + prep GB/s (Llama-8B shapes), % of roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if w.fmt == sq.MXFP4 else "nvfp4 operands, fp16 mfma",
        "data": "synthetic (seeded Llama-3.1-8B-shaped activations with outlier channels, "
                "N(0,0.02) weights)",
        "config": {"workload": f"{w.name}: X {w.m}x{w.k} bf16, W {w.n}x{w.k}, "
                               f"{'RMSNorm, ' if w.norm else ''}2:4 mask, "
                               f"{'MXFP4' if w.fmt == sq.MXFP4 else 'NVFP4-style'}",
                   "m": w.m, "n": w.n, "k": w.k, "gemm_variant": args.variant,
                   "backbone_dense_view": not args.no_dense_view,
                   "y_dtype": "bf16" if args.bf16_out else "fp32",
                   "buffer_sets": nsets},
        "roofline": roofline,
        "roofline_prep": {"bound": "hbm", "kernel": "prepare", "achieved": round(prep_gbps, 1),
                          "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                          "frac": round(prep_gbps / PEAK_HBM_GBPS, 4), "traffic": prep_traffic,
                          "avg_launch_us": round(prep_ms * 1e3, 3),
                          "algorithmic_bytes_per_launch": pbytes},
        "gemm_bytes_per_launch": gbytes,
        "step_ms_events": round(step_ms_events, 5),
    }
    if not args.no_yardsticks:
        out["yardsticks"] = yardsticks(w, torch, dev)
        mf = out["yardsticks"].get("mfma_fp4_random_operands", {}).get("random")
        if mf and "executed_TFLOP/s" in roofline:
            # executed MFMA rate against the rate FP4 MFMAs alone sustain on data
            roofline["executed_vs_fp4_mfma_yardstick"] = round(roofline["executed_TFLOP/s"] / mf["TFLOP/s"], 4)
            # the published peak assumes the 2.4 GHz peak engine clock; the
            # same peak at the clock the yardstick ran at under FP4 MFMA load
            sclk = mf["clock_MHz"]
            roofline["sclk_MHz_under_fp4_mfma_load"] = sclk
            roofline["peak_at_that_sclk"] = round(peak * sclk / 2400.0, 1)
            roofline["frac_at_that_sclk"] = round(roofline["achieved"] / (peak * sclk / 2400.0), 4)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, x_np, W_np, g_np)
        # the step's rate on the GPU over the oracle's on every host thread
        if cb.get("value"):
            cb["gpu_over_cpu"] = round(value / cb["value"], 1)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
