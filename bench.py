"""Benchmark of the fused attention path on one MI355X.

A step is one call of the whole path on one batch of seeded synthetic input that is
already resident in HBM: for the default workload, dense noncausal attention with
B=1 N=4096 H=32 D=128 (BF16 in and out, FP32 accumulation), i.e. one attn_dense
call. FLOP per step = 4*B*H*Nq*Nk*D (the QK^T and PV contractions).

Output: one JSON line (rank 0) with the metric, the roofline of the dominant kernel
(timed with HIP events on the stream the kernel is launched on), the FP64 CPU oracle
timed on a bounded sample of the same workload, the timed output checked against the
oracle rows that sample computed, the inputs checked byte for byte after timing, the
shader clock held under the load (measured in this run), and the environment.

Warmup: at least --warmup steps, continued until --warmup-seconds (default 0.5 s) of
work have run: the GPU's clock takes that long under load to settle, and timed steps
on a ramping clock measure the power controller, not the kernel. The line reports
the steps and seconds actually run. Defaults: 2000 warmup steps, 500 timed steps.

Options beyond the common ones:
  --workload NAME   another workload from synth.WORKLOADS (parity sizes)
  --all             one JSON line per workload (CPU baseline on a shorter sample each)
  --no-cpu          skip the CPU oracle timing (and the output check that uses it)
  --calib-mib MiB   before the timed steps, run a plain streaming kernel (torch.neg on
                    float32: reads and writes MiB each) `steps` times; rocprofv3 counter
                    runs use it to calibrate FETCH_SIZE / WRITE_SIZE
  --ingest F W      read two rocprofv3 --pmc CSVs (FETCH_SIZE run, WRITE_SIZE run) of a
                    --calib-mib run and write profiles/traffic.json (HBM bytes per launch
                    of the attention kernel, scaled by the calibration)
  --ingest-mfma DIR read the output directory of one rocprofv3 --kernel-trace --pmc run with
                    GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_BF16
                    and add, to the same file, the attention kernel's MFMA utilisation and
                    its shader clock while it ran
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % of MI355X bf16 MFMA peak, H=32 D=128 N=4096"
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense BF16 MFMA peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
DEFAULT_WORKLOAD = "dense_b1_n4096_h32_d128"
CSRC = "transformer_attention_dense_amd/csrc/"
# the build script too: its compiler flags change the kernels' code
SHARED_SOURCES = ["attn_device.h", "attn_api.hip", "attn_launch.h", "../build.py"]
KIND_SOURCES = {"na3d": ["attn_na3d.hip"]}
DENSE_SOURCES = ["attn_kernels.hip", "attn_pingpong.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CALIBRATING = False  # set by --calib-mib


def kernel_source_hash(kind) -> str:
    """Hash of the sources (and build script) the kernels of one workload kind are built
    from: counter readings taken on other sources are stale."""
    h = hashlib.sha256()
    for rel in SHARED_SOURCES + KIND_SOURCES.get(kind, DENSE_SOURCES):
        with open(os.path.join(ROOT, CSRC, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--warmup-seconds", type=float, default=0.5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds-all", type=float, default=4.0)
    ap.add_argument("--calib-mib", type=int, default=0)
    ap.add_argument("--ingest", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--ingest-mfma", metavar="PMC_DIR")
    return ap.parse_args()


def to_device(bits, torch):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def make_call(w, dts, attn):
    if w.kind == "na3d":
        out = attn.na3d(*dts, w.kernel)
        return out, (lambda: attn.na3d(*dts, w.kernel, out=out))
    if w.kind == "block_causal":
        out = attn.block_causal(*dts)
        return out, (lambda: attn.block_causal(*dts, out=out))
    if w.kind == "dense":
        if w.Nk == w.Nq:
            out = attn.dense(*dts)
            return out, (lambda: attn.dense(*dts, out=out))
        out = attn.cross(*dts)
        return out, (lambda: attn.cross(*dts, out=out))
    out = attn.prefix(*dts)
    return out, (lambda: attn.prefix(*dts, out=out))


def counters_for(w):
    """The committed counter readings of this workload (HBM bytes per launch, MFMA
    utilisation, shader clock), if they were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    entry = t.get("workloads", {}).get(w.name)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash(w.kind):
        return {}
    return entry


def traffic_for(w):
    """HBM bytes per launch from committed counter runs, if taken on this kernel source."""
    return counters_for(w).get("hbm_bytes_per_launch")


def cpu_baseline(w, seconds, ts):
    """FP64 oracle on a bounded sample of query rows of the same workload (all keys),
    from the first row in [B, Nq, H] order. Returns the baseline record and the oracle's
    output rows [done, D] (used to check the GPU's output)."""
    import numpy as np
    import oracle
    total_rows = w.B * w.Nq * w.H
    flop_per_row = 4 * w.keys * w.D
    chunk = 256
    done = 0
    outs = []
    t0 = time.perf_counter()
    while True:
        rows = np.arange(done, min(done + chunk, total_rows), dtype=np.int64)
        if w.kind == "block_causal":
            outs.append(oracle.block_causal_rows(ts[0], ts[1], ts[2], ts[3], rows=rows))
        elif w.kind == "na3d":
            outs.append(oracle.na3d_rows(ts[0], ts[1], ts[2], w.kernel, rows=rows))
        else:
            outs.append(oracle.attention_rows(ts[0], ts[1], ts[2], *ts[3:5], rows=rows))
        done += rows.size
        el = time.perf_counter() - t0
        if el >= seconds or done >= total_rows:
            break
        chunk = min(chunk * 2, 8192)
    if w.kind == "block_causal":  # only the visible keys of the sampled rows
        vis = w.visible_per_row()
        rows_done = np.arange(done, dtype=np.int64)
        rate = 4 * w.D * int(vis[(rows_done // w.H) % w.Nq].sum()) / el / 1e12
    else:
        rate = done * flop_per_row / el / 1e12
    rec = {"value": rate, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{done} of {total_rows} query rows (first rows in [B,Nq,H] order) of "
                     f"{w.name}, every {'visible ' if w.kind == 'block_causal' else ''}key, "
                     f"FP64, {el:.1f} s"}
    return rec, np.concatenate(outs)


def check_output(out_bits, ref_rows, D):
    """The pages' acceptance step on the timed output (page "Audit SGLang interfaces
    and refresh validated kernel solutions", scripts/task_acceptance.py compare_output):
    the first ref_rows.shape[0] rows of the GPU output against the FP64 oracle, under
    the gate |err| <= 2e-2 + 2e-2 |ref| on >= 99.99% of elements, none above 1e-1, all
    finite (the pages' own BF16 rule reported beside it)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from acceptance import compare
    n = ref_rows.shape[0]
    res = compare(out_bits.reshape(-1, D)[:n], ref_rows)
    res["rows_checked"] = n
    res["rows_total"] = out_bits.size // D
    return res


def probe_library():
    """The shader-clock probe (libattn_probe.so, include/attn_probe.h), or None."""
    import ctypes
    path = os.path.join(ROOT, "transformer_attention_dense_amd", "libattn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.attn_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.attn_probe_clock.restype = ctypes.c_int
    lib.attn_probe_realtime_mhz.argtypes = []
    lib.attn_probe_realtime_mhz.restype = ctypes.c_double
    return lib


class ClockProbe:
    """The shader-clock probe (libattn_probe.so). Created before the warmup, so its code
    is loaded on the GPU before anything is measured."""

    def __init__(self, torch, workgroups=256, ticks=2000):
        self.lib = probe_library()
        self.torch = torch
        self.workgroups = workgroups
        self.ticks = ticks
        self.mhz = self.lib.attn_probe_realtime_mhz() if self.lib else 0.0
        if self.lib is not None:
            self.measure_now(torch.cuda.current_stream())  # load the module

    def enqueue(self, stream):
        """Enqueues one probe behind the launches already on `stream`; returns its output
        buffer (read it after the stream has run)."""
        buf = self.torch.zeros(self.workgroups, dtype=self.torch.float32, device="cuda")
        rc = self.lib.attn_probe_clock(buf.data_ptr(), self.workgroups, self.ticks,
                                       stream.cuda_stream)
        return buf if rc == 0 else None

    def ghz(self, bufs):
        """Median shader clock in GHz over the probes' workgroups (None if unknown)."""
        vals = [b.cpu() for b in bufs if b is not None]
        if not vals or self.mhz <= 0:
            return None
        v = self.torch.cat(vals)
        v = v[v > 0]
        return round(float(v.median()) * self.mhz / 1000.0, 3) if v.numel() else None

    def measure_now(self, stream):
        buf = self.enqueue(stream)
        self.torch.cuda.synchronize()
        return self.ghz([buf])

    def under_load(self, call, stream, rounds=4, steps=50):
        """Clock under the workload itself, outside any timed region: `rounds` times,
        `steps` more calls followed by one probe on the same stream."""
        if self.lib is None:
            return None
        bufs = []
        for _ in range(rounds):
            for _ in range(steps):
                call()
            bufs.append(self.enqueue(stream))
        self.torch.cuda.synchronize()
        return self.ghz(bufs)


def environment(torch):
    """The pages' report opens with an environment row (same page,
    scripts/audit_solutions.py); this is that row for this run."""
    import platform
    env = {"gpu": torch.cuda.get_device_name(0), "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None), "python": platform.python_version()}
    try:
        env["gpu_arch"] = torch.cuda.get_device_properties(0).gcnArchName
        env["gpu_cus"] = torch.cuda.get_device_properties(0).multi_processor_count
    except Exception:  # noqa: BLE001 - optional fields
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            env["cpu"] = next(line.split(":", 1)[1].strip() for line in f
                              if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    env["host_cores_available"] = len(os.sched_getaffinity(0))
    return env


def stream_bandwidth(torch, mib=512, reps=20):
    """Achievable HBM bandwidth on this machine for reference: a plain streaming kernel
    (torch.neg on float32, reads and writes `mib` MiB each), median of `reps` event-timed
    calls after a warmup, in GB/s of bytes read plus written."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        torch.neg(src, out=dst)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / 1000.0)
    del src, dst
    return round(2 * mib * (1 << 20) / statistics.median(times) / 1e9, 1)


def graph_timing(torch, call, out):
    """The pages' graph mode: 20 calls captured in one HIP graph (torch's capture of the
    current stream), replayed 10 times; median microseconds per call. The output after
    the replays is compared with the eager bits. Outside every timed region above;
    None if capture is not possible here."""
    try:
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                call()
        times = []
        for _ in range(10):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1000.0 / 20)
        return {"graph_call_us": round(statistics.median(times), 2),
                "graph_output_matches_eager": bool(torch.equal(out, ref))}
    except Exception as e:  # noqa: BLE001 - reported, the eager numbers stand
        return {"graph_call_us": None, "graph_error": str(e)[:200]}


def device_bits(t, torch):
    """BF16 (or int32) device tensor -> host numpy array of its raw bits."""
    import numpy as np
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bench_one(w, steps, warmup, warmup_seconds, torch, attn, ts):
    import numpy as np
    if w.kind == "block_causal":  # Q, K, V bits and the int32 image ids
        dts = [to_device(t, torch) for t in ts[:3]] + [torch.from_numpy(ts[3]).cuda()]
    else:
        dts = [to_device(t, torch) for t in ts]
    out, call = make_call(w, dts, attn)
    stream = torch.cuda.current_stream()
    probe = ClockProbe(torch)
    clock_idle = probe.measure_now(stream) if probe.lib else None
    # warmup: at least `warmup` steps and at least `warmup_seconds` of them
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - w0 < warmup_seconds:
        for _ in range(max(1, min(warmup - done, 200)) if done < warmup else 50):
            call()
            done += 1
        torch.cuda.synchronize()
    warm = {"warmup_steps_run": done, "warmup_s": round(time.perf_counter() - w0, 3)}
    # whole-job timing: exactly `steps` steps between synchronisations
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    timed_out = device_bits(out, torch)  # the output the timed steps wrote
    clock_ghz = probe.under_load(call, stream)
    inputs_unchanged = all(np.array_equal(device_bits(d, torch), np.ascontiguousarray(t))
                           for d, t in zip(dts, ts))
    # per-call event timing (the pages' eager method: median of event-bracketed calls)
    samples = []
    for _ in range(min(steps, 50)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        b.synchronize()
        samples.append(a.elapsed_time(b) * 1000.0)
    if w.kind == "block_causal":  # always one split of the 8-wave kernel
        plan = {"splits": 1, "waves": 8, "workgroups": -(-w.Nq // 256) * w.B * w.H,
                "workspace_bytes": 16 * -(-w.Nq // 32), "block_causal": True}
    elif w.kind == "na3d":  # four waves per workgroup, query tile chosen by the library
        T, Y, X = w.grid
        na = attn.attn_na3d_plan(w.B, T, Y, X, w.H, w.D, *w.kernel)
        plan = {"splits": 1, "waves": 4, "workgroups": na["workgroups"],
                "query_tile": [32 // na["query_cols"], na["query_cols"]],
                "workspace_bytes": 0, "na3d": True}
    else:
        plan = attn.attn_plan(w.B, w.Nq, w.keys, w.H, w.D)
    finite = bool(torch.isfinite(out.float()).all())
    graph = graph_timing(torch, call, out)
    # (not in counter-calibration runs: those scale by the torch.neg dispatches they see)
    stream_gbs = (stream_bandwidth(torch)
                  if w.flop / w.algorithmic_bytes < 315 and not CALIBRATING else None)
    return {"wall_s": wall, "event_ms": ev_ms, "median_call_us": statistics.median(samples),
            "plan": plan, "finite": finite, "graph": graph, "warm": warm,
            "clock_ghz": clock_ghz, "clock_idle_ghz": clock_idle, "timed_out": timed_out,
            "stream_gbs": stream_gbs,
            "inputs_unchanged": inputs_unchanged}


def kernel_name(D, plan, keys):
    """The kernel(s) a launch of this plan runs (as rocprofv3 names them)."""
    waves = plan["waves"]
    if plan.get("block_causal"):
        return f"attn_bc_meta_kernel + attn_fwd_pp_kernel<{D}, true>"
    if plan.get("na3d"):
        return f"attn_na3d_kernel<{plan['query_tile'][1]}>"
    # attn_fwd_kernel<D, waves, keys per tile, LDS slots>, as the library instantiates it:
    # one slot when every key range is one 64-key tile
    bn = 32 if (D == 128 and waves == 2) else 64
    nslot = 2 if (D == 128 and waves == 4) else 3
    if -(-keys // 64) <= plan["splits"]:
        bn, nslot = 64, 1
    main = (f"attn_fwd_pp_kernel<{D}, false>" if waves == 8 else
            f"attn_fwd_kernel<{D}, {waves}, {bn}, {nslot}>")
    return main if plan["splits"] == 1 else main + f" + attn_combine_kernel<{D}>"


def record(w, r, steps, warmup, cpu, check, env):
    ms_per_step = r["wall_s"] * 1000.0 / steps
    value = w.flop * steps / r["wall_s"] / 1e12
    launch_us = r["event_ms"] * 1000.0 / steps  # average duration per launch on the stream
    achieved = w.flop / (launch_us * 1e-6) / 1e12
    stored = counters_for(w)
    hbm = stored.get("hbm_bytes_per_launch")
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Nq": w.Nq, "Nk": w.keys, "H": w.H, "D": w.D,
                   "kind": w.kind, "description": w.description,
                   "splits": r["plan"]["splits"], "waves": r["plan"]["waves"],
                   "workgroups": r["plan"]["workgroups"]},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        **r["warm"],
        "median_call_us": round(r["median_call_us"], 2),
        **r["graph"],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": hbm,
            "traffic_source": (f"profiles/traffic.json (counter runs on kernel sources "
                               f"{stored.get('kernel_source_hash')})" if hbm else None),
            "kernel": kernel_name(w.D, r["plan"], w.keys),
            "avg_launch_us": round(launch_us, 2),
            "algorithmic_flop_per_launch": w.flop,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes,
            "hbm_gbs_algorithmic": round(w.algorithmic_bytes / (launch_us * 1e-6) / 1e9, 1),
        },
        # shader clock (s_memtime cycles per s_memrealtime tick) from probes enqueued
        # behind 4 x 50 more steps after the timed ones, and before the warmup (idle)
        "clock_ghz_under_load": r["clock_ghz"],
        "clock_ghz_idle": r["clock_idle_ghz"],
        "outputs_finite": r["finite"],
        "inputs_unchanged": r["inputs_unchanged"],
    }
    if w.flop / w.algorithmic_bytes < 315:  # below the ridge point: HBM bound
        rec["roofline"].update({"bound": "hbm", "achieved": rec["roofline"]["hbm_gbs_algorithmic"],
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(rec["roofline"]["hbm_gbs_algorithmic"]
                                              / PEAK_HBM_GBS, 4)})
        if r.get("stream_gbs"):
            rec["roofline"]["stream_copy_gbs_this_box"] = r["stream_gbs"]
    mf = stored.get("mfma")
    if mf and rec["roofline"]["bound"] == "mfma" and mf["profiled_duration_us"] >= 100:
        # Not measured in this run: from a separate, committed counter run of the same
        # kernel sources (counters perturb timing). GRBM_GUI_ACTIVE also counts some
        # 13-16 thousand cycles per dispatch outside the kernel's own time stamps, so
        # these read a few percent off for long kernels and mean nothing for short ones,
        # which are left out.
        rec["stored_counters"] = {
            "source": "profiles/traffic.json", "kernel_source_hash": stored["kernel_source_hash"],
            "mfma_util": mf["mfma_util"], "clock_ghz": mf["clock_ghz"],
            "profiled_duration_us": mf["profiled_duration_us"]}
    if check is not None:
        rec["output_check"] = check
    if env is not None:
        rec["environment"] = env
    if w.kind == "na3d":
        rec["config"].update({"grid": list(w.grid), "kernel": list(w.kernel)})
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    return rec


def _counter_means(csv_path, counter):
    """Mean counter value per dispatch for the attention kernels and the calibration
    kernel of a rocprofv3 --pmc CSV."""
    import csv
    att, cal = [], []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if "attn_fwd" in name or "attn_na3d" in name:
                att.append(float(r["Counter_Value"]))
            elif "neg" in name:
                cal.append(float(r["Counter_Value"]))
    if not att or not cal:
        raise SystemExit(f"{csv_path}: missing attention or calibration dispatches for {counter}")
    return sum(att) / len(att), sum(cal) / len(cal)


def ingest(fetch_csv, write_csv, calib_mib, workload_name):
    """FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is scaled by what the same
    counter reads for the calibration kernel, which moves exactly calib_mib MiB each way."""
    known = calib_mib * 1024.0  # KiB
    fa, fc = _counter_means(fetch_csv, "FETCH_SIZE")
    wa, wc = _counter_means(write_csv, "WRITE_SIZE")
    ff, wf = known / fc, known / wc
    hbm = (fa * ff + wa * wf) * 1024.0
    entry = _update_entry(workload_name, {
        "hbm_bytes_per_launch": round(hbm),
        "fetch_kib_raw": fa, "write_kib_raw": wa,
        "calibration": {"kib_each_way": known, "fetch_kib_read": fc, "write_kib_read": wc,
                        "fetch_factor": ff, "write_factor": wf},
    })
    print(json.dumps(entry))


def _update_entry(workload_name, fields):
    """Merges fields into the workload's entry of the counter file; an entry taken on
    other kernel sources is dropped first."""
    import synth
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    t.pop("kernel_source_hash", None)
    h = kernel_source_hash(synth.workload(workload_name).kind)
    ws = t.setdefault("workloads", {})
    entry = ws.get(workload_name, {})
    if entry.get("kernel_source_hash") != h:
        entry = {}
    entry.update(fields)
    entry["kernel_source_hash"] = h
    ws[workload_name] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
        f.write("\n")
    return entry


def mfma_from_dir(pmc_dir, algorithmic_flop, last=100):
    """MFMA utilisation and shader clock of the attention kernel from the output
    directory of one rocprofv3 --kernel-trace --pmc run (its last `last` dispatches, i.e.
    the timed ones).

    GRBM_GUI_ACTIVE reads the busy cycles of all XCDs added together, so cycles per
    XCD = GRBM_GUI_ACTIVE / Num_Xcc, and the clock = that / the dispatch's duration.
    SQ_VALU_MFMA_BUSY_CYCLES adds the busy cycles of the matrix units of all SIMDs, so
    utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (cycles per XCD * Simd_Count).
    SQ_INSTS_VALU_MFMA_MOPS_BF16 counts BF16 MFMA work in units of 512 FLOP; it is
    reported beside the algorithmic FLOP of a launch."""
    import csv
    import glob

    def one(pattern):
        found = glob.glob(os.path.join(pmc_dir, "**", pattern), recursive=True)
        if len(found) != 1:
            raise SystemExit(f"{pmc_dir}: expected one {pattern}, found {found}")
        with open(found[0]) as f:
            return list(csv.DictReader(f))

    agent = next(a for a in one("*agent_info.csv") if a.get("Name", "").startswith("gfx"))
    xcc, simds = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    max_ghz = float(agent.get("Max_Engine_Clk_Fcompute") or 0) / 1000.0

    def is_main(name):
        return "attn_fwd" in name or "attn_na3d" in name

    per = {}
    for r in one("*counter_collection.csv"):
        if is_main(r["Kernel_Name"]):
            d = per.setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    dur = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
           for r in one("*kernel_trace.csv") if is_main(r["Kernel_Name"])}
    ids = sorted(i for i in per if i in dur)[-last:]
    if not ids:
        raise SystemExit(f"{pmc_dir}: no attention dispatches with counters and durations")
    cyc = sum(per[i]["GRBM_GUI_ACTIVE"] for i in ids) / len(ids) / xcc
    busy = sum(per[i]["SQ_VALU_MFMA_BUSY_CYCLES"] for i in ids) / len(ids)
    mops = sum(per[i]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for i in ids) / len(ids)
    ns = sum(dur[i] for i in ids) / len(ids)
    ghz = cyc / ns
    return {"mfma_util": round(busy / (cyc * simds), 4),
            "clock_ghz": round(ghz, 3),
            "dispatches": len(ids),
            "profiled_duration_us": round(ns / 1000.0, 2),
            "cycles_per_xcd": round(cyc),
            "mfma_busy_cycles": round(busy),
            "mfma_flop_counted": round(mops * 512),
            "algorithmic_flop": algorithmic_flop,
            "max_clock_ghz": max_ghz,
            "peak_at_measured_clock_tflops":
                round(PEAK_BF16_TFLOPS * ghz / max_ghz, 1) if max_ghz > 0 else None}


def ingest_mfma(pmc_dir, workload_name):
    """Adds the MFMA counter pass of one workload to the counter file."""
    import synth
    mf = mfma_from_dir(pmc_dir, synth.workload(workload_name).flop)
    entry = _update_entry(workload_name, {"mfma": mf})
    print(json.dumps(entry["mfma"]))


def main():
    args = parse()
    if args.ingest:
        ingest(args.ingest[0], args.ingest[1], args.calib_mib or 256, args.workload)
        return
    if args.ingest_mfma:
        ingest_mfma(args.ingest_mfma, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is described in the design notes, not implemented).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import transformer_attention_dense_amd as attn
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    attn.library()  # fail loudly if the HIP library is missing

    if args.calib_mib:
        global CALIBRATING
        CALIBRATING = True
        n = args.calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    env = environment(torch)
    names = [w.name for w in synth.WORKLOADS] if args.all else [args.workload]
    for name in names:
        w = synth.workload(name)
        print(f"bench: {w.name} warmup {args.warmup} steps / {args.warmup_seconds} s, "
              f"timed steps {args.steps}", file=sys.stderr, flush=True)
        ts = w.tensors()
        r = bench_one(w, args.steps, args.warmup, args.warmup_seconds, torch, attn, ts)
        cpu = check = None
        if not args.no_cpu:
            print("bench: timing the FP64 CPU oracle on a sample", file=sys.stderr, flush=True)
            cpu, ref_rows = cpu_baseline(
                w, args.cpu_seconds_all if args.all else args.cpu_seconds, ts)
            check = check_output(r["timed_out"], ref_rows, w.D)
        print(json.dumps(record(w, r, args.steps, args.warmup, cpu, check, env)), flush=True)


if __name__ == "__main__":
    main()
