"""Benchmark of the attention forward pass on one MI355X.

A step is one call of the whole forward pass (one fused kernel launch) over
the long-sequence causal workload: B=1, H=16, N=16384, d=256, bf16 inputs
drawn i.i.d. N(0,1) with seed 42, scale 1/sqrt(256), lower-triangular mask.
The metric is attention TFLOP/s with 4*B*H*N^2*d flops, halved for causal.
Inputs are resident in HBM before the timed region starts.

Before timing, every output of one call (all rows of all heads) is checked
against the fp64 oracle, and beside it against a CPU model of the kernel's
roundings (tests/kernel_model.py). The oracle's run on the headline workload
is timed on the host cores and reported as the CPU baseline. The other five
workloads' outputs are checked the same way before they are timed, and the
SHA-256 of every input tensor is reported. After them, the headline and a plain bf16
matrix product run back to back for 2 s each with the board's socket power
read beside them (the "power" entry; --no-power skips it).

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS at N=2k-16k fp16/bf16; % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA, published
PRIMARY = 5                # long-sequence causal d=256 workload
SECONDARY = 4              # GPT-3-shaped causal d=128 workload (reported beside)
FP32 = 3                   # fp32-input workload (reported beside, against the fp32 matrix peak)
PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd16_bf16_d256_causal_n16384_traffic.json")
MFMA_FLOP_PER_CLK_CU = 4096  # dense bf16/fp16 MFMA flops per clock per compute unit
N_CU = 256
TOL_O = {"f16": 2e-3, "bf16": 1e-2, "f32": 1e-5}
TOL_LSE = 1e-3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def metric_flops(c):
    f = 4.0 * c["B"] * c["H"] * c["N"] ** 2 * c["D"]
    return f / 2 if c["causal"] else f


def kernel_source_digest():
    """SHA-256 of the forward kernel sources with comments and blank space
    removed, so that an edit of a comment does not void measured counters."""
    import re

    h = hashlib.sha256()
    for rel in ("transformer_exact_attention_flashattention_amd/csrc/fa_kernels.h",
                "transformer_exact_attention_flashattention_amd/csrc/fa_fwd.hip"):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.strip() for line in text.splitlines() if line.strip())
        h.update(text.encode())
    return h.hexdigest()


def _load_counters():
    """The committed rocprofv3 counter summary of the headline kernel, or None
    if it is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256") != kernel_source_digest():
        return None
    return t


N_XCD = 8  # GRBM_GUI_ACTIVE comes summed over the XCDs


def counter_rows(root):
    """Per dispatch of every kernel in the rocprofv3 CSVs under `root`:
    {(file, dispatch id): {"kernel": name, "ns": duration, counter: value
    summed over its instances}} from counter-collection files, or with the
    duration alone from kernel-trace files."""
    import csv
    import glob

    out = {}
    for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                key = (path, r["Dispatch_Id"])
                d = out.setdefault(key, {"kernel": r["Kernel_Name"],
                                         "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    for path in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                out[(path, r["Dispatch_Id"])] = {"kernel": r["Kernel_Name"],
                                                 "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])}
    return out


def counter_means(root, match, skip=0, first=None):
    """Mean of each counter (and of the duration, "ns") over the dispatches
    whose kernel name contains `match`, in dispatch order: `skip` of them
    left out, then the next `first` if given; also their count
    ("dispatches")."""
    rows = [d for _, d in sorted(counter_rows(root).items(), key=lambda kv: (kv[0][0], int(kv[0][1])))
            if match in d["kernel"]]
    rows = rows[skip:]
    if first:
        rows = rows[:first]
    if not rows:
        raise SystemExit(f"no dispatch of a kernel matching {match!r} under {root}")
    keys = {k for d in rows for k in d if k != "kernel"}
    means = {k: sum(d.get(k, 0.0) for d in rows) / len(rows) for k in keys}
    means["dispatches"] = len(rows)
    return means


HEADLINE_KERNEL = "fwd16_kernel<fa::Bf16, 256, true"
COPY_KERNEL = "copyBuffer"  # the runtime's device-to-device copy (bench.py --calibrate-copy: 1 GiB)


def ingest_counters(fetch_dir, write_dir, grbm_dir):
    """Writes TRAFFIC_FILE from three rocprofv3 runs of
    `bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-parity --no-secondary --calibrate-copy`:
    FETCH_SIZE, WRITE_SIZE and GRBM_GUI_ACTIVE of the headline kernel. HBM
    bytes per launch = FETCH_SIZE and WRITE_SIZE (KiB) each scaled by what
    they read for the calibration copy of 1 GiB; clock = GRBM_GUI_ACTIVE per
    XCD over the dispatch's traced duration."""
    fetch = counter_means(fetch_dir, HEADLINE_KERNEL)
    write = counter_means(write_dir, HEADLINE_KERNEL)
    grbm = counter_means(grbm_dir, HEADLINE_KERNEL)
    cf = counter_means(fetch_dir, COPY_KERNEL)
    cw = counter_means(write_dir, COPY_KERNEL)
    gib = float(1 << 30)
    fetch_scale = gib / (cf["FETCH_SIZE"] * 1024)
    write_scale = gib / (cw["WRITE_SIZE"] * 1024)
    hbm = fetch["FETCH_SIZE"] * 1024 * fetch_scale + write["WRITE_SIZE"] * 1024 * write_scale
    sclk = grbm["GRBM_GUI_ACTIVE"] / N_XCD / grbm["ns"]  # under counter collection: below the live clock
    out = {
        "kernel": "fwd16_kernel<Bf16, 256, causal>",
        "workload": "long-causal-d256 B=1 H=16 N=16384 d=256",
        "kernel_sha256": kernel_source_digest(),
        "fetch_size_kib": fetch["FETCH_SIZE"], "write_size_kib": write["WRITE_SIZE"],
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "hbm_bytes_per_launch": hbm,
        "grbm_gui_active_per_dispatch": grbm["GRBM_GUI_ACTIVE"], "grbm_dispatch_ns": grbm["ns"],
        "sclk_ghz_profiled": round(sclk, 4),
        "dispatches": {"fetch": fetch["dispatches"], "write": write["dispatches"], "grbm": grbm["dispatches"]},
        "source": "profiles/fwd16_bf16_causal_counters.md",
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def load_traffic(launch_bytes_alg):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    they are missing or were taken on different kernel sources."""
    t = _load_counters()
    return None if t is None else t.get("hbm_bytes_per_launch")


def load_cycles():
    """GPU-busy cycles per XCD of one headline launch (GRBM_GUI_ACTIVE, summed
    over the XCDs, / 8) from the committed counter run, or None if missing
    or taken on other kernel sources. The count is stable from run to run;
    over the live launch time it gives the shader clock of the run at hand
    (under counter collection the dispatch itself runs longer)."""
    t = _load_counters()
    if t is None or "grbm_gui_active_per_dispatch" not in t:
        return None
    return t["grbm_gui_active_per_dispatch"] / N_XCD


_SETTLE = []


def gpu_settle(ms):
    """Keeps the matrix cores busy for about `ms` of wall time with a plain
    bf16 matrix product. The GPU's clocks drop while the host runs the
    oracle between workloads and take 100-150 ms of full load to come back
    (measured: the GPT-3-shaped forward runs 0.19 ms per call in its first
    25 calls after 2 s idle or after a 100 ms burn, 0.148 ms after a 500 ms
    burn or in steady state). Without this, a short kernel's timed calls
    would run at the lower clock. It uses another kernel than the one timed,
    so the timed kernel's own dispatch counts stay exactly W + K."""
    import torch

    if not _SETTLE:
        _SETTLE.append(torch.randn(8192, 8192, generator=torch.Generator().manual_seed(0)).to("cuda", torch.bfloat16))
    a = _SETTLE[0]
    t_end = time.perf_counter() + ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(4):
            torch.mm(a, a)
        torch.cuda.synchronize()


def time_launches(fn, stream, steps, warmup, settle_ms=600.0):
    """Per-launch kernel times (ms, sorted) from an event pair around each
    call: `warmup` untimed calls, then `steps` timed ones. settle_ms > 0
    first runs gpu_settle for that long."""
    import torch

    if settle_ms > 0:
        gpu_settle(settle_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return wall, per


def hwmon_power_dir():
    """The first GPU hwmon directory that reports the board's socket power
    (power1_input, microwatts; read-only telemetry), or None."""
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        if os.path.exists(os.path.join(d, "power1_input")):
            return d
    return None


def power_run(fn, flops, seconds, hw):
    """Runs fn back to back for about `seconds` while a thread reads the
    socket power every 20 ms; returns the rate and the mean power over the
    middle half of the samples (the first and last quarter straddle the
    ramps)."""
    import threading

    import torch

    samples, stop = [], threading.Event()

    def poll():
        path = os.path.join(hw, "power1_input")
        while not stop.is_set():
            try:
                with open(path) as fh:
                    samples.append(float(fh.read()) / 1e6)
            except (OSError, ValueError):
                pass
            stop.wait(0.02)

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    th.start()
    e0.record()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    ms = e0.elapsed_time(e1) / n
    mid = samples[len(samples) // 4: 3 * len(samples) // 4] or samples
    return {"calls": n, "ms_per_call": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "socket_w": round(sum(mid) / len(mid), 1) if mid else None, "samples": len(mid)}


def power_context(fa, c, q, k, v, scale, dev, seconds=2.0):
    """The headline forward and a plain bf16 8192^3 matrix product (the
    vendor GEMM through torch.mm), each run back to back for `seconds`, with
    the socket power beside them: what the board's power cap lets a dense
    bf16 workload reach on this GPU."""
    import torch

    hw = hwmon_power_dir()
    if hw is None:
        return None
    cap = None
    try:
        with open(os.path.join(hw, "power1_cap")) as fh:
            cap = float(fh.read()) / 1e6
    except (OSError, ValueError):
        pass
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    att = power_run(lambda: fa.fwd(qd, kd, vd, softmax_scale=scale, causal=c["causal"], out=o, lse=lse),
                    metric_flops(c), seconds, hw)
    a = torch.randn(8192, 8192, generator=torch.Generator().manual_seed(0)).to(dev, torch.bfloat16)
    b = torch.empty_like(a)
    gemm = power_run(lambda: torch.mm(a, a, out=b), 2.0 * 8192 ** 3, seconds, hw)
    del qd, kd, vd, o, lse, a, b
    return {"cap_w": cap, "headline": att, "gemm_bf16_8192": gemm,
            "gemm_frac_of_peak": round(gemm["tflops"] / PEAK_BF16_TFLOPS, 4),
            "headline_vs_gemm": round(att["tflops"] / gemm["tflops"], 4),
            "source": "hwmon power1_input (socket power) read every 20 ms over " + f"{seconds:g}"
                      + " s of back-to-back calls, middle half averaged"}


def check_parity(o, lse, q, k, v, scale, causal, rows, window=(-1, -1)):
    import numpy as np

    from oracle import attention_ref

    o_ref, l_ref = attention_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal,
                                 rows=rows, window=window)
    o_g = o[:, :, rows].double().cpu().numpy()
    l_g = lse[:, :, rows].double().cpu().numpy()
    return float(np.abs(o_g - o_ref).max()), float(np.abs(l_g - l_ref).max())


def oracle_check(o, lse, q, k, v, scale, causal, dtype, window=(-1, -1), heads=None):
    """Every row of the first `heads` heads (all by default) of one GPU
    output (CPU tensors) against the fp64 oracle, with the stated bounds.
    Also returns the oracle's wall time, which the headline workload reports
    as the CPU baseline."""
    import numpy as np

    from oracle import attention_ref

    hs = slice(None) if heads is None else slice(0, heads)
    qs, ks, vs = (t[:, hs].double().numpy() for t in (q, k, v))
    t0 = time.perf_counter()
    o_ref, l_ref = attention_ref(qs, ks, vs, scale, causal, window=window)
    dt = time.perf_counter() - t0
    o_g, l_g = o[:, hs].double().numpy(), lse[:, hs].double().numpy()
    err_o = float(np.abs(o_g - o_ref).max())
    err_l = float(np.abs(l_g - l_ref).max())
    ok = bool(np.isfinite(o_g).all()) and err_o <= TOL_O[dtype] and err_l <= TOL_LSE
    return {"max_abs_dO": err_o, "max_abs_dLSE": err_l, "ok": ok, "rows_checked": "all",
            "heads_checked": int(qs.shape[1]), "of_heads": int(q.shape[1]), "oracle_s": round(dt, 2)}


def _row_pmax(q, k, scale, causal):
    """max_j P_ij per query row (fp32 on the CPU, 1024 rows at a time): the
    weight of the row's largest score, for the model comparison's bound."""
    import torch

    qf, kf = q.float(), k.float()
    N, Nk = qf.shape[2], kf.shape[2]
    out = torch.empty(qf.shape[:3])
    for r0 in range(0, N, 1024):
        r1 = min(r0 + 1024, N)
        s = torch.matmul(qf[:, :, r0:r1], kf.transpose(-1, -2).contiguous()) * scale
        if causal:  # query i sits at key position i + Nk - N
            keys = torch.arange(Nk)[None, :]
            rows = torch.arange(r0, r1)[:, None] + (Nk - N)
            s = s.masked_fill(keys > rows, float("-inf"))
        m = s.max(dim=-1, keepdim=True).values
        out[:, :, r0:r1] = 1.0 / torch.exp(s - m).sum(dim=-1)
    return out


# The model comparison's limits (those of the GPU test of the rounding
# model): per element |O - O_model| <= 2 ulp(O_model) + 2 u' max_j P_ij
# max_j |V_jc|, with u' the spacing of [1, 2) in the input type, and at most
# this share of elements differing at all.
MODEL_SPACING_P = {"bf16": 2.0 ** -7, "f16": 2.0 ** -10}
MODEL_MAX_DIFFERING = {"bf16": 0.02, "f16": 0.05}


def model_check(o, q, k, v, scale, causal, heads=None):
    """The GPU output (CPU tensor, 16-bit) against the CPU model of the
    kernel's roundings (tests/kernel_model.py) on the first `heads` heads:
    the largest difference, in absolute terms and in units of the output
    type's spacing at the model's value (large where |O| is near 0, whose
    spacing is tiny), the share of elements that differ at all, and the
    worst ratio to the per-element bound of the GPU test of the model
    (`model_ok`: every ratio <= 1 and the differing share within its limit).
    The fp64 oracle stays the parity bar; this shows kernel errors far
    smaller than the output's own rounding."""
    import numpy as np
    import torch

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from kernel_model import forward_model, output_ulp

    hs = slice(None) if heads is None else slice(0, heads)
    om, _ = forward_model(q[:, hs], k[:, hs], v[:, hs], scale, causal)
    a, b = o[:, hs].double().numpy(), om.double().numpy()
    d = np.abs(a - b)
    ulp = output_ulp(b, q.dtype)
    dt = "bf16" if q.dtype == torch.bfloat16 else "f16"
    vmax = np.abs(v[:, hs].double().numpy()).max(axis=2, keepdims=True)
    pmax = _row_pmax(q[:, hs], k[:, hs], scale, causal).double().numpy()[..., None]
    bound = 2 * ulp + 2 * MODEL_SPACING_P[dt] * pmax * vmax
    frac = float((d > 0).mean())
    worst = float((d / bound).max())
    return {"max_abs_dO_model": float(d.max()), "max_ulps": float((d / ulp).max()),
            "frac_differing": frac, "worst_ratio_to_model_bound": round(worst, 4),
            "model_ok": bool(worst <= 1.0 and frac < MODEL_MAX_DIFFERING[dt]), "heads": int(a.shape[1])}


def blas_info():
    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info

        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max((p.get("num_threads", 0) for p in pools), default=None)
        blas = ", ".join(sorted({str(p.get("internal_api")) for p in pools})) or None
    except Exception:
        pass
    return threads, blas


def cpu_baseline_entry(c, heads, seconds):
    """The oracle's rate on the headline workload, from its timed parity run
    (`heads` whole heads, every query row)."""
    threads, blas = blas_info()
    flops = 4.0 * heads * c["N"] * c["N"] * c["D"] / (2 if c["causal"] else 1)
    return {
        "value": flops / seconds / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "cpu_count": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "blas": blas,
        "sample": f"{heads} of {c['H']} heads (all {c['N']} query rows each), fp64 numpy, {seconds:.1f} s",
    }


def cpu_baseline(q, k, v, scale, causal, heads):
    """Times the fp64 oracle (as it stands) on `heads` whole heads."""
    from oracle import attention_ref

    qs, ks, vs = (t[:, :heads].double().numpy() for t in (q, k, v))
    t0 = time.perf_counter()
    attention_ref(qs, ks, vs, scale, causal)
    dt = time.perf_counter() - t0
    N, D = q.shape[2], q.shape[3]
    return cpu_baseline_entry({"N": N, "D": D, "H": q.shape[1], "causal": causal}, heads, dt)


def cpu_small_configs(inputs):
    """The fp64 oracle as it stands, plain (three-step definition) and tiled
    (the online-softmax recurrence, Br = Bc = 64), timed on the three small
    workloads (every head, every row): seconds and TFLOP/s of metric flops."""
    from oracle import attention_ref, attention_tiled_ref

    out = {}
    for cfg in (1, 2, 3):
        c = inputs.CONFIGS[cfg]
        q, k, v = (t.double().numpy() for t in inputs.make_config(cfg))
        scale = 1.0 / math.sqrt(c["D"])
        if cfg == 1:
            attention_ref(q, k, v, scale, c["causal"])  # untimed: starts the BLAS threads
        flops = metric_flops(c)
        entry = {}
        for kind, fn in (("plain", attention_ref), ("tiled", attention_tiled_ref)):
            t0 = time.perf_counter()
            fn(q, k, v, scale, c["causal"])
            dt = time.perf_counter() - t0
            entry[kind] = {"s": round(dt, 4), "TFLOP/s": flops / dt / 1e12}
        out[c["name"]] = entry
    return out


def input_digests(q, k, v):
    from transformer_exact_attention_flashattention_amd import inputs

    return {"q": inputs.digest(q), "k": inputs.digest(k), "v": inputs.digest(v)}


def bench_backward(fa, inputs, dev, stream, steps, warmup, no_parity):
    import numpy as np
    import torch

    c = inputs.CONFIGS[SECONDARY]
    log(f"[bench] backward on config {SECONDARY} ({c['name']}): inputs")
    q, k, v = inputs.make_config(SECONDARY)
    g = torch.Generator().manual_seed(43)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    scale = 1.0 / math.sqrt(c["D"])
    o, lse = fa.fwd(qd, kd, vd, softmax_scale=scale, causal=c["causal"])
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    delta = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

    def step():
        fa.bwd(qd, kd, vd, o, lse, dod, softmax_scale=scale, causal=c["causal"], dq=dq, dk=dk, dv=dv,
               delta=delta)

    ok, err = None, float("nan")
    if not no_parity:
        from oracle import attention_bwd_ref

        step()
        torch.cuda.synchronize()
        heads = slice(0, 2)
        ref = attention_bwd_ref(*(t[:, heads].double().numpy() for t in (q, k, v, do)), scale, c["causal"])
        errs = [float(np.abs(x[:, heads].double().cpu().numpy() - r).max() / max(np.abs(r).max(), 1.0))
                for x, r in zip((dq, dk, dv), ref)]
        err = max(errs)
        ok = err <= 1e-2 and all(bool(torch.isfinite(x).all()) for x in (dq, dk, dv))
        log(f"[bench] backward: max rel err dq/dk/dv = {errs} parity={'ok' if ok else 'FAIL'}")
    _, per = time_launches(step, stream, steps, warmup)
    kms = float(np.mean(per))
    flops = 2.5 * metric_flops(c)
    tf = flops / (kms * 1e-3) / 1e12
    return {"workload": "gpt3-causal-d128 backward (dQ, dK, dV)", "B": c["B"], "H": c["H"], "N": c["N"],
            "d": c["D"], "kernel_ms_mean": round(kms, 4), "tflops": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops_counted": "2.5x the forward's metric flops",
            "parity_ok": ok, "max_rel_err_2_heads": err}


def bench_backward_d256(fa, inputs, dev, stream, steps, warmup):
    """fa_bwd on long-causal-d256 (d = 256: dQ, then dV and dK in two
    passes). The fp64 gradient oracle is too slow at N = 16384; parity at
    d = 256 is in the GPU tests (2 heads at N = 4096 and the length and
    window cases). Reported: time and finiteness of every gradient."""
    import numpy as np
    import torch

    c = inputs.CONFIGS[PRIMARY]
    log(f"[bench] backward on config {PRIMARY} ({c['name']}): inputs")
    q, k, v = inputs.make_config(PRIMARY)
    g = torch.Generator().manual_seed(44)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=True)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    delta = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

    def step():
        fa.bwd(qd, kd, vd, o, lse, dod, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)

    _, per = time_launches(step, stream, steps, warmup)
    finite = all(bool(torch.isfinite(x).all()) for x in (dq, dk, dv))
    kms = float(np.mean(per))
    tf = 2.5 * metric_flops(c) / (kms * 1e-3) / 1e12
    return {"workload": "long-causal-d256 backward (dQ, dK, dV)", "kernel_ms_mean": round(kms, 4),
            "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_counted": "2.5x the forward's metric flops", "all_finite": finite,
            "parity": "tests/test_gpu_bwd.py (d = 256: every length/window case and 2 heads at N = 4096)"}


def bench_packed(fa, inputs, dev, stream, steps, warmup):
    """The GPT-3-shaped workload stored as one packed [B, N, 3, H, d] tensor:
    the kernel reads the q, k, v slices in place and writes o [B, N, H, d].
    Timed beside the three copies that unpacking to [B, H, N, d] would cost
    and the contiguous call on those copies; the strided result must be
    bitwise equal to the contiguous one (whose parity the secondary entry
    checks)."""
    import numpy as np
    import torch

    c = inputs.CONFIGS[SECONDARY]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    log(f"[bench] packed layout of config {SECONDARY} ({c['name']}): inputs")
    qkv = inputs.make_packed_qkv(B, N, H, D, c["dtype"]).to(dev)
    sl = [qkv[:, :, i].transpose(1, 2) for i in range(3)]
    o = torch.empty((B, N, H, D), dtype=qkv.dtype, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dst = [torch.empty((B, H, N, D), dtype=qkv.dtype, device=dev) for _ in range(3)]
    oc, lsec = torch.empty_like(dst[0]), torch.empty_like(lse)

    def strided():
        fa.fwd(*sl, causal=c["causal"], out=o.transpose(1, 2), lse=lse)

    def unpack():
        for d_, s_ in zip(dst, sl):
            d_.copy_(s_)

    def contiguous():
        fa.fwd(*dst, causal=c["causal"], out=oc, lse=lsec)

    # Two alternating rounds, so that both calls see the same clock state.
    per_s, per_u, per_c = [], [], []
    for _ in range(2):
        per_c += time_launches(contiguous, stream, steps, warmup)[1]
        per_s += time_launches(strided, stream, steps, warmup)[1]
        per_u += time_launches(unpack, stream, steps, warmup)[1]
    torch.cuda.synchronize()
    same = bool(torch.equal(o.transpose(1, 2), oc)) and bool(torch.equal(lse, lsec))
    log(f"[bench] packed: strided == contiguous bitwise: {same}")
    ks, ku, kc = (float(np.mean(x)) for x in (per_s, per_u, per_c))
    tf = metric_flops(c) / (ks * 1e-3) / 1e12
    return {"workload": "gpt3-causal-d128, qkv packed [B, N, 3, H, d], o [B, N, H, d]", "kernel_ms_mean": round(ks, 4),
            "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "contiguous_kernel_ms_mean": round(kc, 4), "unpack_copy_ms_mean": round(ku, 4),
            "parity_ok": same, "parity": "bitwise equal to the contiguous call on unpacked copies"}


def bench_splitkv(fa, inputs, dev, stream, steps, warmup, no_parity):
    """A low-occupancy shape, one long causal head (B=1, H=1, N=16384,
    d=128, bf16: 128 query tiles for 256 compute units): the plain grid
    beside split-KV with the library's choice of parts (fwd kernel + merge,
    timed together). Parity of the split result on every row."""
    import numpy as np
    import torch

    B, H, N, D = 1, 1, 16384, 128
    log(f"[bench] split-KV on B={B} H={H} N={N} d={D} causal: inputs")
    q, k, v = inputs.make_qkv(B, H, N, D, "bf16", seed=42)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    splits = fa.splitkv_num_splits(B, H, N, D, True, dtype=fa.FA_BF16)
    ws = torch.empty(fa.splitkv_workspace_bytes(B, H, N, D, splits), dtype=torch.uint8, device=dev)

    def plain():
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=lse, num_splits=1)

    def split():
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=lse, num_splits=splits, workspace=ws)

    ok, err_o, err_l = None, float("nan"), float("nan")
    if not no_parity:
        o.fill_(float("nan"))
        split()
        torch.cuda.synchronize()
        chk = oracle_check(o.cpu(), lse.cpu(), q, k, v, 1.0 / math.sqrt(D), True, "bf16")
        err_o, err_l, ok = chk["max_abs_dO"], chk["max_abs_dLSE"], chk["ok"]
        log(f"[bench] split-KV: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} parity={'ok' if ok else 'FAIL'}")
    per_p, per_s = [], []
    for _ in range(2):
        per_p += time_launches(plain, stream, steps, warmup)[1]
        per_s += time_launches(split, stream, steps, warmup)[1]
    kp, ks = float(np.mean(per_p)), float(np.mean(per_s))
    flops = 4.0 * B * H * N * N * D / 2
    return {"workload": "one long causal head, B=1 H=1 N=16384 d=128 bf16", "num_splits": splits,
            "split_ms_mean": round(ks, 4), "plain_ms_mean": round(kp, 4), "speedup": round(kp / ks, 3),
            "tflops": round(flops / (ks * 1e-3) / 1e12, 2),
            "frac": round(flops / (ks * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "timed": "fwd kernel + merge kernel per call", "parity_ok": ok, "max_abs_dO": err_o,
            "max_abs_dLSE": err_l}


def bench_graph(fa, inputs, dev, stream, no_parity):
    """The two launch-bound workloads (single-head, packed-qkv) called one
    at a time from Python, and the same calls captured in a HIP graph
    (20 calls per graph) and replayed: microseconds per call. Each output
    is first checked in full against the oracle and the rounding model
    (the packed workload through its in-place strided views)."""
    import torch

    out = {}
    for cfg in (1, 2):
        c = inputs.CONFIGS[cfg]
        if c["packed"]:
            qkv_c = inputs.make_packed_qkv(c["B"], c["N"], c["H"], c["D"], c["dtype"])
            qkv = qkv_c.to(dev)
            q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
            qc, kc, vc = inputs.unpack_qkv(qkv_c)
            digests = {"qkv": inputs.digest(qkv_c)}
        else:
            qc, kc, vc = inputs.make_config(cfg)
            q, k, v = (t.to(dev) for t in (qc, kc, vc))
            digests = input_digests(qc, kc, vc)
        B, H, N, D = q.shape
        o = torch.empty((B, H, N, D), dtype=q.dtype, device=dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

        def call():
            fa.fwd(q, k, v, causal=c["causal"], out=o, lse=lse)

        entry = {"input_sha256": digests}
        if not no_parity:
            o.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            scale = 1.0 / math.sqrt(D)
            entry["parity"] = oracle_check(o.cpu(), lse.cpu(), qc, kc, vc, scale, c["causal"], c["dtype"])
            entry["parity"].update(model_check(o.cpu(), qc, kc, vc, scale, c["causal"]))
            log(f"[bench] config {cfg}: {entry['parity']}")

        for _ in range(10):
            call()
        torch.cuda.synchronize()
        n = 200
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / n
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                call()
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n // 20):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / n
        entry.update({"eager_us_per_call": round(eager_us, 2), "graph_us_per_call": round(graph_us, 2)})
        out[c["name"]] = entry
    return out


def bench_decode(fa, inputs, dev, stream, steps, warmup, no_parity):
    """A decode step: one new query per head against a key/value cache
    (B=1, H=32, Nk=32768, d=128, bf16, causal), split-KV with the library's
    choice of parts. HBM-bound: reported as GB/s of algorithmic bytes (K and
    V read once, plus q, o and lse) against the 8 TB/s peak."""
    import numpy as np
    import torch

    B, H, N, Nk, D = 1, 32, 1, 32768, 128
    log(f"[bench] decode: B={B} H={H} N={N} Nk={Nk} d={D}: inputs")
    q = inputs.make_qkv(B, H, N, D, "bf16", seed=42)[0]
    _, k, v = inputs.make_qkv(B, H, Nk, D, "bf16", seed=43)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    splits = fa.splitkv_num_splits(B, H, N, D, True, dtype=fa.FA_BF16, Nk=Nk)
    ws = torch.empty(max(fa.splitkv_workspace_bytes(B, H, N, D, splits), 16), dtype=torch.uint8, device=dev)

    def step():
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=lse, num_splits=splits, workspace=ws)

    ok, err_o, err_l = None, float("nan"), float("nan")
    if not no_parity:
        from oracle import attention_ref

        o.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        o_ref, l_ref = attention_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     1.0 / math.sqrt(D), True)
        err_o = float(np.abs(o.double().cpu().numpy() - o_ref).max())
        err_l = float(np.abs(lse.double().cpu().numpy() - l_ref).max())
        ok = err_o <= 1e-2 and err_l <= 1e-3
        log(f"[bench] decode: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} parity={'ok' if ok else 'FAIL'}")
    _, per = time_launches(step, stream, steps, warmup)
    kms = float(np.mean(per))
    nbytes = B * H * (2 * Nk * D * 2 + 2 * N * D * 2 + N * 4)
    gbs = nbytes / (kms * 1e-3) / 1e9
    return {"workload": "decode step: B=1 H=32 N=1 against Nk=32768, d=128 bf16 causal", "num_splits": splits,
            "kernel_ms_mean": round(kms, 4), "bound": "hbm", "achieved_GBps": round(gbs, 1),
            "peak_GBps": 8000.0, "frac": round(gbs / 8000.0, 4), "algorithmic_bytes": nbytes,
            "timed": "fwd kernel + merge kernel per call", "parity_ok": ok, "max_abs_dO": err_o,
            "max_abs_dLSE": err_l}


def bench_sweep(fa, inputs, dev, stream, no_parity, dtype="bf16"):
    """Forward TFLOP/s over sequence lengths 2k-16k, head dimensions 64, 128
    and 256, with and without the causal mask (bf16 or f16 inputs; one batch
    of 2^18 / N heads, so every call has 2^18 query rows). Each shape is
    first checked against the oracle on 4 rows of its first head, to the
    parity bound of its dtype."""
    import numpy as np
    import torch

    res = []
    for D in (64, 128, 256):
        for N in (2048, 4096, 8192, 16384):
            H = (1 << 18) // N
            q, k, v = inputs.make_qkv(1, H, N, D, dtype, seed=N + D)
            qd, kd, vd = (t.to(dev) for t in (q, k, v))
            o = torch.empty_like(qd)
            lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
            scale = 1.0 / math.sqrt(D)
            for causal in (False, True):
                def step():
                    fa.fwd(qd, kd, vd, softmax_scale=scale, causal=causal, out=o, lse=lse)

                ok = None
                if not no_parity:
                    step()
                    torch.cuda.synchronize()
                    rows = np.array([0, 1, N // 2, N - 1])
                    err_o, err_l = check_parity(o[:, :1].cpu(), lse[:, :1].cpu(), q[:, :1], k[:, :1], v[:, :1], scale,
                                                causal, rows)
                    ok = err_o <= TOL_O[dtype] and err_l <= TOL_LSE
                _, per = time_launches(step, stream, 10, 5, settle_ms=600.0)
                ms = float(np.mean(per))
                fl = 4.0 * H * N * N * D / (2 if causal else 1)
                res.append({"N": N, "H": H, "d": D, "causal": causal, "dtype": dtype, "kernel_ms_mean": round(ms, 4),
                            "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                            "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "parity_ok": ok})
                log(f"[sweep] {dtype} N={N} H={H} d={D} causal={causal}: {ms:.4f} ms, {res[-1]['tflops']} TFLOP/s")
            del qd, kd, vd, o, lse
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=10,
                    help="heads the CPU baseline times when the parity check (which times all of them) is off")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check (profiling runs)")
    ap.add_argument("--flush", action="store_true",
                    help="also time the main workload with a 512 MiB buffer written between calls "
                         "(outside the events): a cold-cache figure")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the standard line, print one JSON line with the forward's TFLOP/s over "
                         "N = 2k..16k, d = 64/128/256, causal or not (--sweep-dtype, bf16 by default)")
    ap.add_argument("--sweep-dtype", choices=("bf16", "f16"), default="bf16",
                    help="input type of the --sweep shapes (the fp16 and bf16 matrix peaks are the same)")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the power entry (the headline and a bf16 GEMM run back to back for 2 s each "
                         "with the socket power read beside them)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy 3 times, to scale HBM counters")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "GRBM_DIR"),
                    help="no GPU work: write the headline kernel's counter summary (HBM traffic, clock) from "
                         "three rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE, GRBM_GUI_ACTIVE)")
    ap.add_argument("--counter-means", nargs="+", metavar="ARG",
                    help="no GPU work: DIR KERNEL_SUBSTRING [SKIP [COUNT]]: the mean of each counter (and of "
                         "the duration) per dispatch of the matching kernel, from rocprofv3 CSVs under DIR")
    args = ap.parse_args()
    if args.ingest_counters:
        print(json.dumps(ingest_counters(*args.ingest_counters), indent=1))
        return
    if args.counter_means:
        a = args.counter_means
        print(json.dumps(counter_means(a[0], a[1], int(a[2]) if len(a) > 2 else 0,
                                       int(a[3]) if len(a) > 3 else None), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); each GPU box here has one GPU and "
              "the kernel needs no communication between GPUs", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_exact_attention_flashattention_amd as fa
    from transformer_exact_attention_flashattention_amd import build as fabuild
    from transformer_exact_attention_flashattention_amd import inputs

    if not fabuild.is_built():
        fabuild.build(verbose=True)
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.sweep:
        sweep = bench_sweep(fa, inputs, dev, stream, args.no_parity, args.sweep_dtype)
        print(json.dumps({"sweep": sweep, "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS, "dtype": args.sweep_dtype,
                          "data": f"synthetic: i.i.d. N(0,1) Q, K, V cast to {args.sweep_dtype}"}), flush=True)
        sys.exit(1 if any(r["parity_ok"] is False for r in sweep) else 0)

    def run_config(cfg, steps, warmup, window=(-1, -1), settle_ms=600.0, parity_heads=None, model_heads=None):
        """Inputs of one workload, one call checked in full against the oracle
        (all rows of `parity_heads` heads, all by default) and, for 16-bit
        inputs without a window, against the rounding model (`model_heads`),
        then `warmup` + `steps` timed calls."""
        c = inputs.CONFIGS[cfg]
        log(f"[bench] config {cfg} ({c['name']}): generating inputs")
        q, k, v = inputs.make_config(cfg)
        digests = input_digests(q, k, v)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        scale = 1.0 / math.sqrt(c["D"])
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

        def step():
            fa.fwd(qd, kd, vd, softmax_scale=scale, causal=c["causal"], window_size=window, out=o, lse=lse)

        if args.no_parity:
            par = {"ok": None}
        else:
            log(f"[bench] config {cfg}: every output row vs the fp64 oracle")
            o.fill_(float("nan"))
            step()
            torch.cuda.synchronize()
            o_c, l_c = o.cpu(), lse.cpu()
            par = oracle_check(o_c, l_c, q, k, v, scale, c["causal"], c["dtype"], window, parity_heads)
            if c["dtype"] != "f32" and tuple(window) == (-1, -1) and model_heads != 0:
                par.update(model_check(o_c, q, k, v, scale, c["causal"], model_heads))
            log(f"[bench] config {cfg}: {par}")
        log(f"[bench] config {cfg}: timing {steps} steps after {warmup} warmup")
        wall, per = time_launches(step, stream, steps, warmup, settle_ms)
        return c, (q, k, v, scale), par, digests, wall, per

    # The headline workload: exactly W untimed steps, then K timed ones.
    c, (q, k, v, scale), par, dig, wall, per = run_config(PRIMARY, args.steps, args.warmup, settle_ms=0.0,
                                                          model_heads=2)
    flops = metric_flops(c)
    ms_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean(per))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    value = flops * args.steps / wall / 1e12
    elem = 2
    alg_bytes = c["B"] * c["H"] * c["N"] * (4 * c["D"] * elem + 4)
    traffic = load_traffic(alg_bytes)
    cycles = load_cycles()
    sclk = None if cycles is None else round(cycles / (kern_ms * 1e-3) / 1e9, 3)
    out = {
        "metric": METRIC,
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
        "data": "synthetic: i.i.d. N(0,1) Q, K, V from torch CPU generator seed 42, cast to bf16",
        "config": {"workload": "long-causal-d256", "B": c["B"], "H": c["H"], "N": c["N"], "d": c["D"],
                   "causal": c["causal"], "input_dtype": c["dtype"]},
        "frac_of_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "at_measured_clock": None if sclk is None else {
            "sclk_ghz": sclk, "peak": round(N_CU * sclk * 1e9 * MFMA_FLOP_PER_CLK_CU / 1e12, 1),
            "frac": round(achieved / (N_CU * sclk * 1e9 * MFMA_FLOP_PER_CLK_CU / 1e12), 4),
            "source": "GRBM_GUI_ACTIVE per XCD and launch (" + os.path.relpath(TRAFFIC_FILE, ROOT)
                      + ") over this run's mean launch time"},
        "kernel_ms": {"mean": round(kern_ms, 4), "min": round(per[0], 4),
                      "median": round(per[len(per) // 2], 4), "p90": round(per[int(0.9 * (len(per) - 1))], 4)},
        "parity": par,
        "input_sha256": dig,
    }
    if args.flush:
        log("[bench] cold-cache timing: 512 MiB written between calls")
        scratch = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        q_d, k_d, v_d = (t.to(dev) for t in (q, k, v))
        o_d = torch.empty_like(q_d)
        l_d = torch.empty(q_d.shape[:3], dtype=torch.float32, device=dev)
        cold = []
        for i in range(args.warmup + args.steps):
            scratch.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fa.fwd(q_d, k_d, v_d, softmax_scale=scale, causal=c["causal"], out=o_d, lse=l_d)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= args.warmup:
                cold.append(e0.elapsed_time(e1))
        cold.sort()
        out["cold_cache"] = {"kernel_ms_median": round(cold[len(cold) // 2], 4),
                             "kernel_ms_mean": round(float(np.mean(cold)), 4),
                             "note": "512 MiB scratch written between calls, outside the events"}
        del scratch, q_d, k_d, v_d, o_d, l_d
    if not args.no_secondary:
        c4, _, par4, dig4, wall4, per4 = run_config(SECONDARY, max(args.steps, 20), args.warmup)
        k4 = float(np.mean(per4))
        a4 = metric_flops(c4) / (k4 * 1e-3) / 1e12
        out["secondary"] = {"workload": "gpt3-causal-d128", "B": 1, "H": 128, "N": 2048, "d": 128,
                            "kernel_ms_mean": round(k4, 4), "tflops": round(a4, 2),
                            "frac": round(a4 / PEAK_BF16_TFLOPS, 4), "parity_ok": par4["ok"], "parity": par4,
                            "input_sha256": dig4}
    if not args.no_secondary:
        c3, _, par3, dig3, wall3, per3 = run_config(FP32, max(args.steps, 20), args.warmup)
        k3 = float(np.mean(per3))
        a3 = metric_flops(c3) / (k3 * 1e-3) / 1e12
        out["fp32"] = {"workload": "fp32-long", "B": 4, "H": 1, "N": 4096, "d": 64, "causal": False,
                       "kernel_ms_mean": round(k3, 4), "tflops": round(a3, 2), "peak": PEAK_FP32_TFLOPS,
                       "frac": round(a3 / PEAK_FP32_TFLOPS, 4), "parity_ok": par3["ok"], "parity": par3,
                       "input_sha256": dig3}
    if not args.no_secondary:
        # Sliding-window variant of the same workload: causal, each query sees
        # itself and the 4096 keys before it. Flops count the visible pairs.
        # Parity: every row of 2 of the 16 heads.
        W = 4096
        cw, _, parw, _, wallw, perw = run_config(PRIMARY, max(args.steps // 2, 5), 2, window=(W, -1),
                                                 parity_heads=2)
        kw_ms = float(np.mean(perw))
        pairs = sum(min(i + 1, W + 1) for i in range(cw["N"]))
        flw = 4.0 * cw["B"] * cw["H"] * pairs * cw["D"]
        aw = flw / (kw_ms * 1e-3) / 1e12
        out["window"] = {"workload": "long-causal-d256, window (4096, -1)", "kernel_ms_mean": round(kw_ms, 4),
                         "tflops": round(aw, 2), "frac": round(aw / PEAK_BF16_TFLOPS, 4),
                         "flops_counted": "4*d per visible (query, key) pair", "parity_ok": parw["ok"],
                         "parity": parw}
    if not args.no_secondary:
        # Backward pass on the GPT-3-shaped workload (fa_bwd: dQ with the row sums D, and
        # dK/dV kernels), parity-checked on 2 of the 128 heads first.
        # Flops: 2.5x the forward's (the five N x N x d products of the
        # gradient, halved for causal), the usual accounting.
        out["backward"] = bench_backward(fa, inputs, dev, stream, max(args.steps, 10), args.warmup,
                                         args.no_parity)
        out["backward_d256"] = bench_backward_d256(fa, inputs, dev, stream, 5, 2)
        out["packed"] = bench_packed(fa, inputs, dev, stream, max(args.steps, 20), args.warmup)
        out["graph"] = bench_graph(fa, inputs, dev, stream, args.no_parity)
        out["decode"] = bench_decode(fa, inputs, dev, stream, max(args.steps, 20), args.warmup, args.no_parity)
        out["splitkv"] = bench_splitkv(fa, inputs, dev, stream, max(args.steps, 20), args.warmup, args.no_parity)
    if not args.no_power:
        log("[bench] power: headline and a bf16 GEMM back to back, socket power read beside them")
        out["power"] = power_context(fa, c, q, k, v, scale, dev)
    if args.calibrate_copy:
        log("[bench] copy calibration: 3 x 1 GiB device-to-device copy")
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        if "oracle_s" in par:  # the oracle already ran on every head for the parity check: its time
            out["cpu_baseline"] = cpu_baseline_entry(c, par["heads_checked"], par["oracle_s"])
        else:
            log(f"[bench] CPU baseline: fp64 oracle on {args.cpu_heads} head(s)")
            out["cpu_baseline"] = cpu_baseline(q, k, v, scale, True, args.cpu_heads)
        log("[bench] CPU baseline: plain and tiled fp64 oracle on the three small workloads")
        out["cpu_baseline"]["small_workloads"] = cpu_small_configs(inputs)
    print(json.dumps(out), flush=True)
    failed = [par["ok"]] + [out[k]["parity_ok"] for k in ("secondary", "fp32", "window", "backward", "packed",
                                                          "splitkv", "decode")
                          if k in out]
    failed += [g["parity"]["ok"] for g in out.get("graph", {}).values() if "parity" in g]
    if "backward_d256" in out:
        failed.append(out["backward_d256"]["all_finite"])
    if any(f is False for f in failed):
        sys.exit(1)


if __name__ == "__main__":
    main()
