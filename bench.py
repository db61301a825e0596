#!/usr/bin/env python3
"""Throughput of the pair-biased attention hot path on one MI355X.

A step is one forward + backward pass of pair-biased gated attention over one
batch of the triangle-attention workload (B=384 rows, N=384 tokens, H=4
heads, d=32, bf16 in / fp32 accumulate, last 19 keys masked): pba_forward then
pba_backward, i.e. every kernel of the attention path.  The pair-weighted
average (S=1024 MSA rows, N=768, H=8, d=32), the MSA row attention with pair
bias (B=1024 rows, N=768, H=8, d=32) and the pair-bias projection
Linear(LayerNorm(z)) (z [768, 768, 128], H=16) and the windowed atom
attention (B=48, N=3072 atoms, H=4, d=32) are timed in loops of their own and
reported in the same JSON line under "pair_avg", "msa_row_attn", "bias_proj"
and "local_attn".

Prints one JSON line: the step figures, per-kernel times, a roofline object for
the dominant kernel and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def attn_flops(B, H, N, d):
    """Algorithmic flops of forward + backward: 4 + 10 = 14 * B*H*N^2*d."""
    return 14.0 * B * H * N * N * d


def attn_fwd_flops(B, H, N, d):
    return 4.0 * B * H * N * N * d


# Algorithmic work credited to each kernel of the attention path (flops), per
# launch.  The backward's 10*B*H*N^2*d runs in one launch that carries the
# dK/dV tiles (S recomputed; dP, dV and dK formed) and the dQ tiles (dQ; their
# own recomputation of S and dP is not credited).
def attn_kernel_flops(B, H, N, d):
    u = float(B) * H * N * N * d
    return {"attn_fwd": 4 * u, "bwd_pre": 0.0, "bwd_dkdv_dq": 10 * u, "bwd_dbias_reduce": 0.0}


ATTN_BWD_KERNELS = ["bwd_pre", "bwd_dkdv_dq", "bwd_dbias_reduce"]
PWA_FWD_KERNELS = ["pwa_softmax", "pwa_weighted_sum"]
PWA_BWD_KERNELS = ["pwa_bwd_softmax", "pwa_bwd_pre", "pwa_bwd_dv_dw", "pwa_bwd_db"]


def proj_fwd_bytes(N, H, c):
    """Algorithmic HBM bytes of the pair-bias projection forward: read z
    [N,N,c] bf16, write bias [H,N,N] bf16, read gamma, beta, w (fp32)."""
    P = N * N
    return P * (2 * c + 2 * H) + 4 * (2 * c + H * c)


def proj_bwd_bytes(N, H, c):
    """Backward: read z and dbias, write dz (bf16), read and write the fp32
    parameters and their gradients; the per-workgroup partial sums are the
    kernels' own traffic, not algorithmic."""
    P = N * N
    return P * (4 * c + 2 * H) + 8 * (2 * c + H * c)


def proj_main_bwd_bytes(N, H, c):
    """The backward's main kernel alone: z and dbias in, dz out."""
    return N * N * (4 * c + 2 * H)


LOCAL_BWD_KERNELS = ["local_bwd_pre", "local_bwd_dkdv_dq", "local_bwd_dbias_reduce"]


def local_units(B, H, N, d):
    """Window score elements times d: every query against its 128 window slots."""
    return float(B) * H * N * 128 * d


def local_kernel_flops(B, H, N, d):
    """Algorithmic flops credited per launch, as for the dense path: forward
    4 (QK^T, PV); backward 10 in the one launch that carries the
    key-stationary role (S recompute, dP, dV, dK: 8) and the query-stationary
    role (dQ: 2; its own recompute of S and dP is not credited)."""
    u = local_units(B, H, N, d)
    return {"local_fwd": 4 * u, "local_bwd_pre": 0.0, "local_bwd_dkdv_dq": 10 * u, "local_bwd_dbias_reduce": 0.0}


PROJ_FWD_KERNELS = ["bias_proj_fwd"]
PROJ_BWD_KERNELS = ["bias_proj_bwd", "bias_proj_reduce"]


def pwa_bytes(S, N, H, d, elt=2):
    """Algorithmic HBM bytes of PWA forward + backward.

    forward reads V, G, b and writes O (3T + b); backward reads dO, O, G, V and
    b and writes dV, dG and db (6T + 2b).  T = S*N*H*d elements.
    """
    T = S * N * H * d * elt
    b = H * N * N * elt
    return 9 * T + 3 * b


def pwa_fwd_bytes(S, N, H, d, elt=2):
    T = S * N * H * d * elt
    return 3 * T + H * N * N * elt


def pwa_flops(S, N, H, d):
    return 6.0 * S * H * N * N * d


def to_dev(arr, torch):
    if arr.dtype == np.uint8:
        return torch.from_numpy(arr).cuda()
    return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()


SPINUP_S = 0.25


def time_loop(fn, steps, warmup, torch, spinup_s=SPINUP_S):
    """Spin up, warm up, then time `steps` calls with HIP events on the
    current stream.

    The spin-up runs untimed calls for `spinup_s` seconds (synchronized every
    four calls) so the GPU leaves its idle clock state first: timed straight
    after process start or host-side input generation, the first loop reads
    about 15 % slow (0.444 vs 0.387 ms per attention step at B=384 N=384).
    Then `warmup` untimed calls, then exactly `steps` timed calls."""
    t_end = time.perf_counter() + spinup_s
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return t0.elapsed_time(t1) / steps, wall


def call_dist(fn, calls, torch, before=None):
    """Per-call HIP-event durations on the current stream: median, p10, p90
    (ms).  `before` runs ahead of each call, outside the timed interval."""
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(calls):
        if before is not None:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    q = np.percentile(ms, [50, 10, 90])
    return {"median_ms": round(float(q[0]), 4), "p10_ms": round(float(q[1]), 4), "p90_ms": round(float(q[2]), 4),
            "calls": calls}


def graph_call_dist(step, outputs, calls, torch):
    """Per-replay HIP-event durations of one `step` captured in a HIP graph:
    the same kernel launches without Python's per-call work (argument checks,
    output allocation, ctypes), which sets the pace of the eager calls of a
    small workload.  Every replay's outputs (`outputs()` after the captured
    step) are compared bit for bit with an eager step's, with eager work and
    synchronisation between the replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
        step()
        ref = [x.clone() for x in outputs()]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    got = outputs()
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(calls):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
        for a, b in zip(got, ref):
            if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
                raise SystemExit(f"graph replay {i} differs from the eager step")
    del graph
    q = np.percentile(ms, [50, 10, 90])
    return {"median_ms": round(float(q[0]), 4), "p10_ms": round(float(q[1]), 4), "p90_ms": round(float(q[2]), 4),
            "calls": calls, "replays_checked": calls}


COLD_BYTES = 512 << 20


def call_protocols(fwd, bwd, step, torch, calls):
    """Warm (back-to-back calls, caches as the previous call left them) and
    cold (a 512 MiB buffer is written before each call, evicting L2 and most
    of the 256 MB MALL) per-call distributions of fwd, bwd and fwd+bwd."""
    fwd()
    torch.cuda.synchronize()
    out = {"warm": {"fwd": call_dist(fwd, calls, torch), "bwd": call_dist(bwd, calls, torch),
                    "fwd_bwd": call_dist(step, calls, torch)}}
    scratch = torch.empty(COLD_BYTES // 4, dtype=torch.float32, device="cuda")
    flush = lambda: scratch.fill_(1.0)  # noqa: E731
    out["cold"] = {"fwd": call_dist(fwd, calls, torch, flush), "bwd": call_dist(bwd, calls, torch, flush),
                   "fwd_bwd": call_dist(step, calls, torch, flush)}
    del scratch
    return out


def sclk_during(fn, torch, seconds=1.0):
    """Shader clock read from the amdgpu sysfs files (current DPM level of
    pp_dpm_sclk, or hwmon freq1_input) every few ms while `fn` runs back to
    back for about `seconds`; None where the files are not readable."""
    import glob
    import threading
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    hw = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/freq1_input"))

    def read_mhz():
        vals = []
        for pth in paths:
            try:
                with open(pth) as f:
                    for line in f:
                        if "*" in line:
                            vals.append(float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz")))
            except (OSError, ValueError, IndexError):
                pass
        if not vals:
            for pth in hw:
                try:
                    with open(pth) as f:
                        vals.append(float(f.read().strip()) / 1e6)
                except (OSError, ValueError):
                    pass
        return max(vals) if vals else None

    if read_mhz() is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_mhz()
            if v is not None:
                samples.append(v)
            time.sleep(0.005)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    a = np.array(samples)
    return {"source": "pp_dpm_sclk" if paths else "hwmon freq1_input", "samples": int(a.size),
            "median_mhz": round(float(np.median(a)), 1), "min_mhz": round(float(a.min()), 1),
            "max_mhz": round(float(a.max()), 1)}


def attn_bytes(B, H, N, d, elt):
    """Minimum HBM bytes of one forward + backward call pair: 15 T + 3 |bias| +
    4 |LSE| (forward reads Q, K, V, G, bias and writes O, LSE; backward reads
    Q, K, V, G, O, dO, LSE, bias, writes dQ, dK, dV, dG, dBias and writes and
    reads the D workspace)."""
    T = B * H * N * d * elt
    return 15 * T + 3 * H * N * N * elt + 4 * B * H * N * 4


PEAK_FP32_MFMA_TFLOPS = 157.3


def bench_attn_config(name, torch, pba, calls):
    """fwd+bwd per-call median of one attention config, with %MFMA (against the
    peak of its dtype), %HBM and the fraction of roofline max(MFMA floor, HBM
    floor) / measured time."""
    c = workloads.CONFIGS[name]
    inp = workloads.attention_inputs(c, with_f64=False)
    f32 = c.dtype == "f32"
    dev = (lambda a: torch.from_numpy(a).cuda()) if f32 else (lambda a: to_dev(a, torch))
    t = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "bias", "dout")}
    km = None if inp["key_mask"] is None else to_dev(inp["key_mask"], torch)
    dt = torch.float32 if f32 else torch.bfloat16
    ws = torch.empty(pba.pba_backward_workspace_bytes(c.B, c.H, c.N, c.d, dt), dtype=torch.uint8, device="cuda")
    st = {}

    def step():
        st["out"], st["lse"] = pba.pba_forward(t["q"], t["k"], t["v"], t["g"], t["bias"], km)
        st["grads"] = pba.pba_backward(t["q"], t["k"], t["v"], t["g"], t["bias"], km, st["out"], st["lse"],
                                       t["dout"], workspace=ws)

    # the same spin-up as the timed loops: untimed calls until the GPU has
    # left its idle clock state, then the per-call distribution
    t_end = time.perf_counter() + SPINUP_S
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    dist = call_dist(step, calls, torch)
    try:
        gdist = graph_call_dist(step, lambda: [st["out"], st["lse"]] + list(st["grads"].values()), calls, torch)
    except RuntimeError as ex:  # no graph capture here: the eager per-call time stands
        gdist = {"error": str(ex)[:200]}
    # the faster of the two ways to issue the same step (graph replay wins
    # where Python's per-call work outlasts the kernels, eager elsewhere)
    mode = "graph" if gdist.get("median_ms", float("inf")) < dist["median_ms"] else "eager"
    ms = gdist["median_ms"] if mode == "graph" else dist["median_ms"]
    flops = attn_flops(c.B, c.H, c.N, c.d)
    nbytes = attn_bytes(c.B, c.H, c.N, c.d, 4 if f32 else 2)
    peak = PEAK_FP32_MFMA_TFLOPS if f32 else PEAK_BF16_TFLOPS
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    floor_ms = max(flops / (peak * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e3
    return {"B": c.B, "H": c.H, "N": c.N, "d": c.d, "dtype": c.dtype, "fwd_bwd": dist, "fwd_bwd_graph": gdist,
            "tflops": round(tf, 2), "mfma_frac": round(tf / peak, 4), "mfma_peak": peak,
            "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
            "timing": mode, "roofline_frac": round(floor_ms / ms, 4),
            "roofline_frac_eager": round(floor_ms / dist["median_ms"], 4)}


def host_info():
    """Cores this process may use, the CPU model, and the BLAS library NumPy
    calls with its thread count (threadpoolctl, when importable)."""
    cores = len(os.sched_getaffinity(0))
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = i.get("num_threads")
                break
    except Exception:
        pass
    return {"cores": cores, "cpu": model, "blas": blas, "blas_threads": threads}


def cpu_baseline(cfg, target_s=15.0):
    """The fp64 oracle on a bounded sample of the attention workload (rows of
    B), forward and backward timed separately; the backward recomputes the
    forward as the plain definition does."""
    import oracle  # test infrastructure: used only for this baseline leg
    hi = host_info()
    B = 4
    while True:
        sub = workloads.scaled_attention_config(cfg, B=B)
        inp = workloads.attention_inputs(sub)
        args = (inp["q64"], inp["k64"], inp["v64"], inp["g64"], inp["bias64"], inp["key_mask"])
        t0 = time.perf_counter()
        oracle.attention_forward(*args)
        t1 = time.perf_counter()
        oracle.attention_backward(*args, inp["dout64"])
        t2 = time.perf_counter()
        dt = t2 - t0
        if dt * 2 > target_s or B >= cfg.B:
            break
        B = min(cfg.B, max(B * 2, int(B * target_s / max(dt, 1e-3) * 0.9)))
    flops = attn_flops(B, cfg.H, cfg.N, cfg.d)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": hi["blas_threads"] or hi["cores"],
            "kind": "oracle",
            "fwd_s": round(t1 - t0, 3), "bwd_s": round(t2 - t1, 3),
            "fwd_tflops": attn_fwd_flops(B, cfg.H, cfg.N, cfg.d) / (t1 - t0) / 1e12,
            "sample": f"{B} of {cfg.B} rows (B) of the triangle workload, fwd then bwd, fp64 NumPy, "
                      f"{dt:.2f} s (fwd {t1 - t0:.2f} s, bwd {t2 - t1:.2f} s, bwd recomputing the forward); "
                      f"{hi['cpu']}, {hi['cores']} cores visible, BLAS {hi['blas']} with {hi['blas_threads']} "
                      f"threads, NumPy elementwise ops single-threaded"}


def cpu_baseline_pwa(pc, target_s=10.0):
    """The fp64 pair-weighted-average oracle on a bounded sample of the MSA
    rows (each row's output depends on that row alone), forward and backward
    timed separately; reported in GB/s of the algorithmic bytes of the
    sample."""
    import oracle  # test infrastructure: used only for this baseline leg
    hi = host_info()
    S = 16
    while True:
        sub = workloads.scaled_pwa_config(pc, S=S)
        inp = workloads.pwa_inputs(sub)
        t0 = time.perf_counter()
        oracle.pwa_forward(inp["b64"], inp["v64"], inp["g64"], inp["key_mask"])
        t1 = time.perf_counter()
        oracle.pwa_backward(inp["b64"], inp["v64"], inp["g64"], inp["key_mask"], inp["dout64"])
        t2 = time.perf_counter()
        dt = t2 - t0
        if dt * 2 > target_s or S >= pc.S:
            break
        S = min(pc.S, max(S * 2, int(S * target_s / max(dt, 1e-3) * 0.9)))
    nbytes = pwa_bytes(S, pc.N, pc.H, pc.d)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": hi["blas_threads"] or hi["cores"], "kind": "oracle",
            "fwd_s": round(t1 - t0, 3), "bwd_s": round(t2 - t1, 3),
            "tflops": pwa_flops(S, pc.N, pc.H, pc.d) / dt / 1e12,
            "sample": f"{S} of {pc.S} MSA rows of the pair-weighted-average workload, fwd then bwd, fp64 NumPy, "
                      f"{dt:.2f} s (fwd {t1 - t0:.2f} s, bwd {t2 - t1:.2f} s); {hi['cpu']}, {hi['cores']} cores "
                      f"visible, BLAS {hi['blas']} with {hi['blas_threads']} threads"}


COPY_BYTES = 256 << 20
CALIBRATION_KERNEL = "neg"  # torch's elementwise negation: one dispatch, reads and writes COPY_BYTES

# kernel of each timed phase: (symbol prefix in the HIP library, source file)
KERNEL_SOURCES = {
    "attn_fwd": ("attn_fwd_res_kernel", "attn_fwd.hip"),
    "bwd_pre": ("attn_bwd_pre_bf16_kernel", "attn_bwd.hip"),
    "bwd_dkdv_dq": ("attn_bwd_dq_bf16_kernel", "attn_bwd.hip"),
    "bwd_dbias_reduce": ("bias_grad_reduce_kernel", "attn_bwd.hip"),
    "pwa_weighted_sum": ("pwa_gemm_dl_kernel<32, true>", "pwa.hip"),
    "pwa_bwd_pre": ("pwa_bwd_pre_kernel", "pwa.hip"),
    "pwa_bwd_dv_dw": ("pwa_gemm_kernel<32, false", "pwa.hip"),
    "bias_proj_fwd": ("bias_proj_fwd_kernel<4>", "bias_proj.hip"),
    "local_fwd": ("local_fwd_kernel", "local_attn.hip"),
    "local_bwd_dkdv_dq": ("local_bwd_kernel", "local_attn.hip"),
    "bias_proj_bwd": ("bias_proj_bwd_kernel<4, true>", "bias_proj.hip"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(fname):
    import hashlib
    path = os.path.join(ROOT, "pair_biased_attention_amd", "csrc", fname)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from(fetch_dir, write_dir):
    """Per-dispatch HBM bytes from a FETCH_SIZE pass and a WRITE_SIZE pass of
    `bench.py --counters`, each scaled by what the counter reads for the
    calibration copy of COPY_BYTES; written to profiles/traffic.json with the
    digest of each kernel's source file."""
    import csv
    import glob

    def per_dispatch(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals, disp = {}, {}
        for row in csv.DictReader(open(files[0])):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"].replace("void ", "")
            vals[name] = vals.get(name, 0.0) + float(row["Counter_Value"])
            disp.setdefault(name, set()).add(row["Dispatch_Id"])
        return {n: vals[n] / len(disp[n]) for n in vals}

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    cal = [n for n in fetch if CALIBRATION_KERNEL in n.split("(")[0].lower()]
    if not cal:
        raise SystemExit("calibration copy kernel not found in the FETCH_SIZE pass")
    ff = COPY_BYTES / (fetch[cal[0]] * 1024.0)
    fw = COPY_BYTES / (write[cal[0]] * 1024.0)
    out = {"calibration": {"kernel": cal[0][:120], "bytes": COPY_BYTES,
                           "fetch_size_kib": fetch[cal[0]], "write_size_kib": write[cal[0]],
                           "fetch_factor": ff, "write_factor": fw},
           "kernels": {}}
    for phase, (prefix, src) in KERNEL_SOURCES.items():
        names = [n for n in fetch if n.startswith("pba::" + prefix) or n.startswith(prefix)]
        if not names:
            continue
        n = names[0]
        out["kernels"][phase] = {"kernel": n.split("(")[0], "source": src, "source_digest": source_digest(src),
                                 "fetch_bytes": fetch[n] * 1024.0 * ff, "write_bytes": write.get(n, 0.0) * 1024.0 * fw}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def traffic_for(phase):
    """HBM bytes per launch of a phase's kernel from profiles/traffic.json, or
    None when none were taken or the kernel's source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)["kernels"][phase]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_digest") != source_digest(t["source"]):
        return None
    return round(t["fetch_bytes"] + t["write_bytes"])


def counters_pass(args, torch, pba):
    """Run each kernel of interest a few times under a counter profiler."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)  # calibration: reads and writes exactly COPY_BYTES
    torch.cuda.synchronize()
    print(f"copy {COPY_BYTES} bytes done", flush=True)
    del src, dst
    cfg = workloads.CONFIGS["tri_attn_n384"]
    inp = workloads.attention_inputs(cfg, with_f64=False)
    t = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "bias", "dout")}
    km = to_dev(inp["key_mask"], torch)
    ws = torch.empty(pba.pba_backward_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    for _ in range(args.steps):
        out, lse = pba.pba_forward(t["q"], t["k"], t["v"], t["g"], t["bias"], km)
        pba.pba_backward(t["q"], t["k"], t["v"], t["g"], t["bias"], km, out, lse, t["dout"], workspace=ws)
    torch.cuda.synchronize()
    print(f"attention steps done: {args.steps}", flush=True)
    if args.no_pwa:
        return
    del t, ws
    pc = workloads.CONFIGS["msa_pwa"]
    pin = workloads.pwa_inputs(pc, with_f64=False)
    pt = {n: to_dev(pin[n], torch) for n in ("b", "v", "g", "dout")}
    del pin
    for _ in range(args.pwa_steps):
        o, l = pba.pair_weighted_avg(pt["b"], pt["v"], pt["g"], None)
        pba.pair_weighted_avg_backward(pt["b"], pt["v"], pt["g"], None, o, l, pt["dout"])
    torch.cuda.synchronize()
    print(f"pair-average steps done: {args.pwa_steps}", flush=True)
    del pt
    jc = workloads.CONFIGS["bias_proj_pairformer"]
    jin = workloads.bias_proj_inputs(jc, with_f64=False)
    z, dbias = to_dev(jin["z"], torch), to_dev(jin["dbias"], torch)
    prm = {n: torch.from_numpy(jin[n]).cuda() for n in ("gamma", "beta", "w")}
    for _ in range(args.pwa_steps):
        pba.pba_bias_proj_forward(z, prm["gamma"], prm["beta"], prm["w"], 1e-5)
        pba.pba_bias_proj_backward(z, prm["gamma"], prm["beta"], prm["w"], dbias, 1e-5)
    torch.cuda.synchronize()
    print(f"projection steps done: {args.pwa_steps}", flush=True)
    del z, dbias, prm
    lc = workloads.CONFIGS["local_atom_attn"]
    lin = workloads.local_inputs(lc, with_f64=False)
    lt = {n: to_dev(lin[n], torch) for n in ("q", "k", "v", "g", "bias", "dout")}
    lkm = to_dev(lin["key_mask"], torch)
    del lin
    for _ in range(args.pwa_steps):
        o, l = pba.pba_local_forward(lt["q"], lt["k"], lt["v"], lt["g"], lt["bias"], lkm)
        pba.pba_local_backward(lt["q"], lt["k"], lt["v"], lt["g"], lt["bias"], lkm, o, l, lt["dout"])
    torch.cuda.synchronize()
    print(f"windowed attention steps done: {args.pwa_steps}", flush=True)
    del lt, lkm
    # the other attention configs (c1 tiny fp32, c3 Pairformer B = 1 d = 24, c4
    # DiT 48 copies d = 48): their own kernel instances
    for name in ("tiny_fp32", "pairformer_apb", "dit_apb_x48"):
        c = workloads.CONFIGS[name]
        cin = workloads.attention_inputs(c, with_f64=False)
        f32 = c.dtype == "f32"
        dev = (lambda a: torch.from_numpy(a).cuda()) if f32 else (lambda a: to_dev(a, torch))
        ct = {n: dev(cin[n]) for n in ("q", "k", "v", "g", "bias", "dout")}
        ckm = None if cin["key_mask"] is None else to_dev(cin["key_mask"], torch)
        for _ in range(args.pwa_steps):
            o, l = pba.pba_forward(ct["q"], ct["k"], ct["v"], ct["g"], ct["bias"], ckm)
            pba.pba_backward(ct["q"], ct["k"], ct["v"], ct["g"], ct["bias"], ckm, o, l, ct["dout"])
        torch.cuda.synchronize()
        print(f"{name} steps done: {args.pwa_steps}", flush=True)
        del ct, ckm


def bench_proj(args, torch, pba):
    """Pair-bias projection bias = Linear(LayerNorm(z)) forward + backward on the
    Pairformer pair bias (z [768, 768, 128] bf16, H = 16)."""
    jc = workloads.CONFIGS["bias_proj_pairformer"]
    N, H, c = jc.N, jc.H, jc.c
    jin = workloads.bias_proj_inputs(jc, with_f64=False)
    z = to_dev(jin["z"], torch)
    dbias = to_dev(jin["dbias"], torch)
    prm = {n: torch.from_numpy(jin[n]).cuda() for n in ("gamma", "beta", "w")}
    del jin
    eps = 1e-5
    jws = torch.empty(pba.pba_bias_proj_backward_workspace_bytes(N, H, c), dtype=torch.uint8, device="cuda")
    bias = torch.empty((H, N, N), dtype=torch.bfloat16, device="cuda")
    grads = {"dz": torch.empty_like(z), "dgamma": torch.empty_like(prm["gamma"]),
             "dbeta": torch.empty_like(prm["beta"]), "dw": torch.empty_like(prm["w"])}

    def jfwd():
        pba.pba_bias_proj_forward(z, prm["gamma"], prm["beta"], prm["w"], eps)

    def jstep():
        jfwd()
        pba.pba_bias_proj_backward(z, prm["gamma"], prm["beta"], prm["w"], dbias, eps, workspace=jws)

    ms_j, _ = time_loop(jstep, args.proj_steps, 3, torch)
    ms_jf, _ = time_loop(jfwd, args.proj_steps, 3, torch)
    acc_f, acc_b = [0.0], [0.0] * len(PROJ_BWD_KERNELS)
    for i in range(args.proj_steps + 1):
        f = pba.pba_bias_proj_forward_timed(z, prm["gamma"], prm["beta"], prm["w"], eps, bias)
        b = pba.pba_bias_proj_backward_timed(z, prm["gamma"], prm["beta"], prm["w"], dbias, eps, jws, grads)
        if i:  # the first pass is a warm-up
            acc_f = [x + y for x, y in zip(acc_f, f)]
            acc_b = [x + y for x, y in zip(acc_b, b)]
    kms = {n: a / args.proj_steps for n, a in zip(PROJ_FWD_KERNELS + PROJ_BWD_KERNELS, acc_f + acc_b)}
    step_bytes = proj_fwd_bytes(N, H, c) + proj_bwd_bytes(N, H, c)
    gbs = step_bytes / (ms_j * 1e-3) / 1e9
    gbs_f = proj_fwd_bytes(N, H, c) / (ms_jf * 1e-3) / 1e9
    kb = proj_main_bwd_bytes(N, H, c)
    kgbs = kb / (kms["bias_proj_bwd"] * 1e-3) / 1e9
    fgbs = proj_fwd_bytes(N, H, c) / (kms["bias_proj_fwd"] * 1e-3) / 1e9
    out = {
        "workload": "bias_proj_pairformer: bias = Linear(LayerNorm(z)), z [768,768,128] bf16 -> bias [16,768,768] "
                    "bf16, fp32 gamma/beta/w, fwd+bwd (dz, dgamma, dbeta, dw)",
        "value": round(gbs, 1), "unit": "GB/s", "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "ms_per_step": round(ms_j, 4), "steps": args.proj_steps,
        "fwd": {"ms": round(ms_jf, 4), "value": round(gbs_f, 1), "unit": "GB/s",
                "hbm_frac": round(gbs_f / PEAK_HBM_GBS, 4),
                "kernel_gbs": round(fgbs, 1), "traffic": traffic_for("bias_proj_fwd")},
        "roofline": {"kernel": "bias_proj_bwd", "bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "ms_per_launch": round(kms["bias_proj_bwd"], 4), "bytes_per_launch": kb,
                     "traffic": traffic_for("bias_proj_bwd")},
        "kernels_ms": {n: round(v, 4) for n, v in kms.items()},
    }
    del z, dbias, prm, jws, bias, grads
    torch.cuda.empty_cache()
    return out


def bench_local(args, torch, pba):
    """Windowed atom attention fwd + bwd on B=48 copies, N=3072 atoms, H=4, d=32."""
    lc = workloads.CONFIGS["local_atom_attn"]
    B, H, N, d = lc.B, lc.H, lc.N, lc.d
    lin = workloads.local_inputs(lc, with_f64=False)
    t = {n: to_dev(lin[n], torch) for n in ("q", "k", "v", "g", "bias", "dout")}
    km = to_dev(lin["key_mask"], torch)
    del lin
    ws = torch.empty(pba.pba_local_backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    st = {}

    def lfwd():
        st["out"], st["lse"] = pba.pba_local_forward(t["q"], t["k"], t["v"], t["g"], t["bias"], km)

    def lstep():
        lfwd()
        pba.pba_local_backward(t["q"], t["k"], t["v"], t["g"], t["bias"], km, st["out"], st["lse"], t["dout"],
                               workspace=ws)

    ms_l, _ = time_loop(lstep, args.local_steps, 3, torch)
    ms_lf, _ = time_loop(lfwd, args.local_steps, 3, torch)
    grads = {n: torch.empty_like(t["q"]) for n in ("dq", "dk", "dv", "dg")}
    grads["dbias"] = torch.empty_like(t["bias"])
    out, lse = torch.empty_like(t["q"]), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    acc_f, acc_b = [0.0], [0.0] * len(LOCAL_BWD_KERNELS)
    for i in range(args.local_steps + 1):
        f = pba.pba_local_forward_timed(t["q"], t["k"], t["v"], t["g"], t["bias"], km, out, lse)
        b = pba.pba_local_backward_timed(t["q"], t["k"], t["v"], t["g"], t["bias"], km, out, lse, t["dout"], ws,
                                         grads)
        if i:  # the first pass is a warm-up
            acc_f = [x + y for x, y in zip(acc_f, f)]
            acc_b = [x + y for x, y in zip(acc_b, b)]
    kms = {n: a / args.local_steps for n, a in zip(["local_fwd"] + LOCAL_BWD_KERNELS, acc_f + acc_b)}
    kfl = local_kernel_flops(B, H, N, d)
    dom = max(kms, key=kms.get)
    dom_tf = kfl[dom] / (kms[dom] * 1e-3) / 1e12
    u = local_units(B, H, N, d)
    val = 14 * u / (ms_l * 1e-3) / 1e12
    out_obj = {
        "workload": "local_atom_attn: windowed atom attention with pair bias, B=48 copies, N=3072 atoms, H=4, "
                    "d=32, bf16, 32-query blocks x 128-key windows, local bias [4,96,32,128], last 154 atoms "
                    "masked, fwd+bwd",
        "value": round(val, 2), "unit": "TFLOP/s", "mfma_frac": round(val / PEAK_BF16_TFLOPS, 4),
        "ms_per_step": round(ms_l, 4), "steps": args.local_steps,
        "fwd": {"ms": round(ms_lf, 4), "value": round(4 * u / (ms_lf * 1e-3) / 1e12, 2), "unit": "TFLOP/s"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(dom_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "ms_per_launch": round(kms[dom], 4), "flops_per_launch": kfl[dom],
                     "traffic": traffic_for(dom)},
        "kernels_ms": {n: round(v, 4) for n, v in kms.items()},
    }
    del t, ws, st, grads, out, lse
    torch.cuda.empty_cache()
    return out_obj


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pwa-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calls", type=int, default=30,
                    help="per-call timings (warm and cold, median/p10/p90), the sampled shader clock and the "
                         "all-config table use this many calls each; 0 skips them")
    ap.add_argument("--no-pwa", action="store_true")
    ap.add_argument("--next-steps", type=int, default=5,
                    help="timed steps of the MSA row attention workload (0 skips it)")
    ap.add_argument("--local-steps", type=int, default=20,
                    help="timed steps of the windowed atom attention (0 skips it)")
    ap.add_argument("--proj-steps", type=int, default=20,
                    help="timed steps of the pair-bias projection Linear(LayerNorm(z)) (0 skips it)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn a FETCH_SIZE and a WRITE_SIZE pass of --counters into profiles/traffic.json")
    ap.add_argument("--counters", action="store_true",
                    help="hardware-counter pass: a 256 MiB device copy (calibration kernel of known size), then "
                         "--steps attention steps and --pwa-steps steps of the pair average, the projection and "
                         "the windowed attention; no timing, no JSON line")
    args = ap.parse_args()
    if args.traffic_from:
        return traffic_from(*args.traffic_from)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (no sharding, no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import pair_biased_attention_amd as pba
    from pair_biased_attention_amd import _lib

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    _lib.load()  # fails loudly without the HIP library

    if args.counters:
        return counters_pass(args, torch, pba)

    cfg = workloads.CONFIGS["tri_attn_n384"]
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    inp = workloads.attention_inputs(cfg, with_f64=False)
    t = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "g", "bias", "dout")}
    km = to_dev(inp["key_mask"], torch)
    ws = torch.empty(pba.pba_backward_workspace_bytes(B, H, N, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    state = {}

    def fwd():
        state["out"], state["lse"] = pba.pba_forward(t["q"], t["k"], t["v"], t["g"], t["bias"], km)

    def step():
        fwd()
        pba.pba_backward(t["q"], t["k"], t["v"], t["g"], t["bias"], km, state["out"], state["lse"], t["dout"],
                         workspace=ws)

    ms_step, wall = time_loop(step, args.steps, args.warmup, torch)
    ms_fwd, _ = time_loop(fwd, args.steps, 2, torch)
    flops = attn_flops(B, H, N, d)
    value = flops / (ms_step * 1e-3) / 1e12

    # per-kernel durations: HIP events recorded between the backward's launches
    # on the stream they are launched on (pba_backward_timed), averaged
    grads = {n: torch.empty_like(t["q"]) for n in ("dq", "dk", "dv", "dg")}
    grads["dbias"] = torch.empty_like(t["bias"])
    timed_args = (t["q"], t["k"], t["v"], t["g"], t["bias"], km, state["out"], state["lse"], t["dout"], ws, grads)
    pba.pba_backward_timed(*timed_args)
    acc = [0.0] * len(ATTN_BWD_KERNELS)
    for _ in range(args.steps):
        acc = [a + b for a, b in zip(acc, pba.pba_backward_timed(*timed_args))]
    kernel_ms = {"attn_fwd": ms_fwd}
    kernel_ms.update({n: a / args.steps for n, a in zip(ATTN_BWD_KERNELS, acc)})
    kflops = attn_kernel_flops(B, H, N, d)
    dom = max(kernel_ms, key=kernel_ms.get)
    dom_tflops = kflops[dom] / (kernel_ms[dom] * 1e-3) / 1e12

    result = {
        "metric": "fwd+bwd TFLOP/s & %MFMA peak (N=384 tri-attn); GB/s & %HBM (pair-avg)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "tri_attn_n384: triangle attention fwd+bwd, B=384 rows, N=384, H=4, d=32, "
                               "bf16 in / fp32 accumulate, last 19 keys masked, bias [4,384,384] broadcast over rows",
                   "B": B, "H": H, "N": N, "d": d, "global_batch": B, "seq_len": N, "parallelism": "single GPU"},
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "spinup_s_untimed": SPINUP_S,
        # dominant kernel of the step; algorithmic flops per launch as credited
        # in attn_kernel_flops, over its HIP-event duration
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(dom_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
                     "ms_per_launch": round(kernel_ms[dom], 4), "flops_per_launch": kflops[dom],
                     "traffic": traffic_for(dom)},
        "kernels_ms": {n: round(v, 4) for n, v in kernel_ms.items()},
    }

    def bwd():
        pba.pba_backward(t["q"], t["k"], t["v"], t["g"], t["bias"], km, state["out"], state["lse"], t["dout"],
                         workspace=ws)

    if args.calls > 0:
        result["calls"] = call_protocols(fwd, bwd, step, torch, args.calls)
        result["sclk"] = sclk_during(step, torch)
        print("call protocols done", file=sys.stderr, flush=True)

    pcalls = None
    if not args.no_pwa:
        del t, state, ws, timed_args, grads
        torch.cuda.empty_cache()
        pc = workloads.CONFIGS["msa_pwa"]
        pin = workloads.pwa_inputs(pc, with_f64=False)
        pt = {n: to_dev(pin[n], torch) for n in ("b", "v", "g", "dout")}
        del pin
        pws_f = torch.empty(pba.pair_weighted_avg_workspace_bytes(pc.S, pc.N, pc.H, pc.d, torch.bfloat16),
                            dtype=torch.uint8, device="cuda")
        pws_b = torch.empty(pba.pair_weighted_avg_backward_workspace_bytes(pc.S, pc.N, pc.H, pc.d, torch.bfloat16),
                            dtype=torch.uint8, device="cuda")
        pst = {}

        def pfwd():
            pst["out"], pst["lse"] = pba.pair_weighted_avg(pt["b"], pt["v"], pt["g"], None, workspace=pws_f)

        def pstep():
            pfwd()
            pba.pair_weighted_avg_backward(pt["b"], pt["v"], pt["g"], None, pst["out"], pst["lse"], pt["dout"],
                                           workspace=pws_b)

        ms_p, _ = time_loop(pstep, args.pwa_steps, 2, torch)
        ms_pf, _ = time_loop(pfwd, args.pwa_steps, 2, torch)

        def pbwd():
            pba.pair_weighted_avg_backward(pt["b"], pt["v"], pt["g"], None, pst["out"], pst["lse"], pt["dout"],
                                           workspace=pws_b)

        pcalls = call_protocols(pfwd, pbwd, pstep, torch, args.calls) if args.calls > 0 else None
        psclk = sclk_during(pstep, torch) if args.calls > 0 else None
        gbs = pwa_bytes(pc.S, pc.N, pc.H, pc.d) / (ms_p * 1e-3) / 1e9
        gbs_f = pwa_fwd_bytes(pc.S, pc.N, pc.H, pc.d) / (ms_pf * 1e-3) / 1e9
        pgr = {"dv": torch.empty_like(pt["v"]), "dg": torch.empty_like(pt["g"]), "db": torch.empty_like(pt["b"])}
        pout, plse = torch.empty_like(pt["v"]), torch.empty((pc.H, pc.N), dtype=torch.float32, device="cuda")
        pk_f = [0.0] * len(PWA_FWD_KERNELS)
        pk_b = [0.0] * len(PWA_BWD_KERNELS)
        for i in range(args.pwa_steps + 1):
            f = pba.pair_weighted_avg_timed(pt["b"], pt["v"], pt["g"], None, pout, plse, pws_f)
            bk = pba.pair_weighted_avg_backward_timed(pt["b"], pt["v"], pt["g"], None, pout, plse, pt["dout"],
                                                      pws_b, pgr)
            if i:  # the first pass is a warm-up
                pk_f = [a + b for a, b in zip(pk_f, f)]
                pk_b = [a + b for a, b in zip(pk_b, bk)]
        pkms = {n: a / args.pwa_steps for n, a in zip(PWA_FWD_KERNELS + PWA_BWD_KERNELS, pk_f + pk_b)}
        # the weighted sum + gate kernel moves exactly the forward's algorithmic bytes (3T + b)
        ws_gbs = pwa_fwd_bytes(pc.S, pc.N, pc.H, pc.d) / (pkms["pwa_weighted_sum"] * 1e-3) / 1e9
        # the dominant kernel of the step is the backward's dV + dw launch:
        # 4 S H N^2 d flops (dV = w^T dA and dw = dA^T V) over 3 T bytes (reads
        # dA and V, writes dV), an intensity above the ridge, so its roofline is
        # the matrix cores'
        dvdw_flops = 4.0 * pc.S * pc.H * pc.N * pc.N * pc.d
        dvdw_bytes = 3 * pc.S * pc.N * pc.H * pc.d * 2
        dvdw_ms = pkms["pwa_bwd_dv_dw"]
        dvdw_tf = dvdw_flops / (dvdw_ms * 1e-3) / 1e12
        result["pair_avg"] = {
            "workload": "msa_pwa: S=1024 MSA rows, N=768, H=8, d=32, bf16, fwd+bwd",
            "value": round(gbs, 1), "unit": "GB/s", "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "ms_per_step": round(ms_p, 4),
            "tflops": round(pwa_flops(pc.S, pc.N, pc.H, pc.d) / (ms_p * 1e-3) / 1e12, 2),
            "fwd": {"ms": round(ms_pf, 4), "value": round(gbs_f, 1), "unit": "GB/s",
                    "hbm_frac": round(gbs_f / PEAK_HBM_GBS, 4)},
            "roofline": {"kernel": "pwa_bwd_dv_dw", "bound": "mfma", "achieved": round(dvdw_tf, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dvdw_tf / PEAK_BF16_TFLOPS, 4),
                         "ms_per_launch": round(dvdw_ms, 4), "flops_per_launch": dvdw_flops,
                         "bytes_per_launch": dvdw_bytes,
                         "gbs": round(dvdw_bytes / (dvdw_ms * 1e-3) / 1e9, 1),
                         "traffic": traffic_for("pwa_bwd_dv_dw")},
            "fwd_roofline": {"kernel": "pwa_weighted_sum", "bound": "hbm", "achieved": round(ws_gbs, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ws_gbs / PEAK_HBM_GBS, 4),
                             "ms_per_launch": round(pkms["pwa_weighted_sum"], 4),
                             "bytes_per_launch": pwa_fwd_bytes(pc.S, pc.N, pc.H, pc.d),
                             "traffic": traffic_for("pwa_weighted_sum")},
            "kernels_ms": {n: round(v, 4) for n, v in pkms.items()},
        }
        if pcalls is not None:
            result["pair_avg"]["calls"] = pcalls
            result["pair_avg"]["sclk"] = psclk
            med = pcalls["warm"]["fwd_bwd"]["median_ms"]
            pflops, pb = pwa_flops(pc.S, pc.N, pc.H, pc.d), pwa_bytes(pc.S, pc.N, pc.H, pc.d)
            floor_ms = max(pflops / (PEAK_BF16_TFLOPS * 1e12), pb / (PEAK_HBM_GBS * 1e9)) * 1e3
            pair_cfg = {"S": pc.S, "H": pc.H, "N": pc.N, "d": pc.d, "dtype": "bf16",
                        "fwd_bwd": pcalls["warm"]["fwd_bwd"],
                        "tflops": round(pflops / (med * 1e-3) / 1e12, 2),
                        "mfma_frac": round(pflops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "gbs": round(pb / (med * 1e-3) / 1e9, 1), "hbm_frac": round(pb / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "bytes": pb, "roofline_frac": round(floor_ms / med, 4)}
        del pt, pst, pws_f, pws_b, pgr, pout, plse
        torch.cuda.empty_cache()

    if args.next_steps > 0:
        # MSA row attention with pair bias: the same kernels on the row attention
        # the pair-weighted average replaces (1024 MSA rows, N = 768)
        mc = workloads.CONFIGS["msa_row_attn"]
        minp = workloads.attention_inputs(mc, with_f64=False)
        mt = {n: to_dev(minp[n], torch) for n in ("q", "k", "v", "g", "bias", "dout")}
        mkm = to_dev(minp["key_mask"], torch)
        del minp
        mws = torch.empty(pba.pba_backward_workspace_bytes(mc.B, mc.H, mc.N, mc.d, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        mst = {}

        def mfwd():
            mst["out"], mst["lse"] = pba.pba_forward(mt["q"], mt["k"], mt["v"], mt["g"], mt["bias"], mkm)

        def mstep():
            mfwd()
            pba.pba_backward(mt["q"], mt["k"], mt["v"], mt["g"], mt["bias"], mkm, mst["out"], mst["lse"],
                             mt["dout"], workspace=mws)

        ms_m, _ = time_loop(mstep, args.next_steps, 2, torch)
        ms_mf, _ = time_loop(mfwd, args.next_steps, 2, torch)
        mval = attn_flops(mc.B, mc.H, mc.N, mc.d) / (ms_m * 1e-3) / 1e12
        mval_f = 4.0 * mc.B * mc.H * mc.N * mc.N * mc.d / (ms_mf * 1e-3) / 1e12
        result["msa_row_attn"] = {
            "workload": "msa_row_attn: MSA row attention with pair bias, B=1024 MSA rows, N=768, H=8, d=32, "
                        "bf16, last 38 keys masked, bias [8,768,768] broadcast over rows, fwd+bwd",
            "value": round(mval, 2), "unit": "TFLOP/s", "mfma_frac": round(mval / PEAK_BF16_TFLOPS, 4),
            "ms_per_step": round(ms_m, 4), "steps": args.next_steps,
            "fwd": {"ms": round(ms_mf, 4), "value": round(mval_f, 2), "unit": "TFLOP/s"},
        }
        del mt, mws, mst

    if args.calls > 0:
        # every config of the path: fwd+bwd per-call median, %MFMA, %HBM and the
        # fraction of roofline (the other configs run only here)
        table = {}
        for name in ("tiny_fp32", "tri_attn_n384", "pairformer_apb", "dit_apb_x48"):
            table[name] = bench_attn_config(name, torch, pba, args.calls)
            torch.cuda.empty_cache()
        if not args.no_pwa and pcalls is not None:
            table["msa_pwa"] = pair_cfg
        result["configs_table"] = table
        print("config table done", file=sys.stderr, flush=True)

    if args.proj_steps > 0:
        result["bias_proj"] = bench_proj(args, torch, pba)
    if args.local_steps > 0:
        result["local_attn"] = bench_local(args, torch, pba)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg)
        if "pair_avg" in result:
            result["pair_avg"]["cpu_baseline"] = cpu_baseline_pwa(workloads.CONFIGS["msa_pwa"])

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
