"""Benchmark of the Lightning Attention chunked prefill on one MI355X.

One step = one la_prefill_fwd call over the whole workload: B=2, T=8192, H=HV=64, D=DV=128, bf16 Q/K/V/O,
FP32 state read from and written back to a 2-slot pool in place (every step sees the previous step's state;
the work per step is identical). Inputs are synthetic (la_synth recipe, seed 1) and resident in HBM before the
timed region. Prints one JSON line. --config 0/2/3 time the other prefill workloads; --config 4 times the draft
verify + commit chain through the KV buffer (B=128 requests, T=8); --config 5 times the segmented prefill of one
long prompt (B=1, T=32768, H=HV=16) and reports the unsegmented time beside it.

Timing protocol: the parent process never touches the GPU. It runs --procs fresh child processes one after the
other (default 3); each child builds the inputs, runs the kernel for --prewarm-s seconds so that the clock has
settled, W warmup steps, then K timed steps between HIP events on the launch stream, then K more steps with
events around every launch. The roofline's kernel time is the average launch duration of the back-to-back timed
launches; the separately timed launches are reported beside it. The line reports the median over the children
and the spread between them. The parent samples amd-smi clock, power and temperature every quarter second meanwhile
and reports, per child, the samples taken from late in its pre-warm to the end of its timed launches. --procs 1 measures
in-process, without amd-smi samples (for runs under rocprofv3).

  python bench.py [--steps K] [--warmup W] [--procs N] [--no-cpu-baseline] [--config {0,1,2,3,4,5}]
  python bench.py --trace-summary DIR/kernel_trace.csv --kernel NAME --skip S --count K   (no GPU)
  python bench.py --counter-summary DIR/counter_collection.csv ... --kernel NAME             (no GPU)
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LA prefill Mtok·head/s and % MFMA/HBM roofline at B=2,T=8192,H=64,D=128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6    # MI355X dense bf16 matrix peak
CHUNK = 64


def chain_bytes(w):
    """Verify + commit through the KV buffer (B requests, T drafts): verify reads q, k, v and each valid slot's
    state, writes o and copies k, v into the buffer; commit reads the first L_b buffer rows and reads and writes
    the state of every valid request with L_b > 0."""
    P = w.pool.shape[0]
    valid = [0 <= int(s) < P for s in w.state_idx]
    nvalid = sum(valid)
    tok = w.B * w.T
    verify = tok * (2 * w.H + 2 * w.HV) * 256 + nvalid * w.T * (w.H + w.HV) * 256 + nvalid * w.HV * 65536
    acc_rows = sum(int(l) for l, ok in zip(w.accepted_len, valid) if ok)
    ncommit = sum(1 for l, ok in zip(w.accepted_len, valid) if ok and int(l) > 0)
    commit = acc_rows * (w.H + w.HV) * 256 + ncommit * w.HV * 65536 * 2
    return verify + commit


def algorithmic_bytes(w):
    """Bytes the path must move at minimum: q, k read once per q/k head, v read and o written once per value
    head (bf16), plus the FP32 state read (READ) and written (WRITE) once per selected (sequence, head)."""
    tok = w.tokens
    qk = 2 * tok * w.H * 128 * 2
    vo = 2 * tok * w.HV * 128 * 2
    nstate = 0
    if w.state_idx is not None and w.pool is not None:
        P = w.pool.shape[0]
        nsel = sum(1 for s in w.state_idx if 0 <= int(s) < P)
        nstate = nsel * w.HV * 128 * 128 * 4 * ((w.flags & 1) + ((w.flags >> 1) & 1))
    return qk + vo + nstate


# MFMA instructions the chunked kernel issues per workgroup and 64-token chunk (one workgroup = one
# (sequence, value head, value half) unit). Producers: 10 lower-triangle 16x16 score tiles x 4 slices of the
# 128-wide contraction = 40 of 16x16x32. Each of the 4 consumers: history term Q S^T 4 key groups x 4 row tiles x
# (hi, lo) = 32, state update 4 key groups x 2 tiles x 2 token pairs x (hi, lo) = 32, P.V 12, all 16x16x32; and
# 16x16x16: 8 residuals of its S split (2 tiles x 4 key groups) and 4 of its V_dec split. SQ_INSTS_MFMA of a
# config-1 launch reads 392 per workgroup-chunk.
MFMA_X32_PER_WG_CHUNK = 40 + 4 * (32 + 32 + 12)      # 344 v_mfma_f32_16x16x32_bf16
MFMA_X16_PER_WG_CHUNK = 4 * (8 + 4)                  # 48 v_mfma_f32_16x16x16_bf16
FLOP_X32 = 2 * 16 * 16 * 32
FLOP_X16 = 2 * 16 * 16 * 16


def mfma_flops_executed(w):
    """Dense bf16 MFMA flops the chunked kernel issues per call: the per-workgroup-chunk instruction counts above
    times the workgroup-chunks of the call (2 value halves per (sequence, value head); a short last chunk costs a
    whole chunk)."""
    per_wg_chunk = MFMA_X32_PER_WG_CHUNK * FLOP_X32 + MFMA_X16_PER_WG_CHUNK * FLOP_X16
    chunks = sum((l + CHUNK - 1) // CHUNK for _, l in w.seq_rows())
    return per_wg_chunk * chunks * w.HV * 2


CSRC = os.path.join(ROOT, "linear_attention_decay_amd", "csrc")
TRAFFIC = {   # workload -> (committed FETCH_SIZE / WRITE_SIZE summary, kernel sources it was measured on)
    1: (os.path.join(ROOT, "profiles", "la_chunk_kernel_fixed_b2_t8192_h64_hbm_traffic.md"),
        ("la_common.h", "la_prefill.hip")),
    2: (os.path.join(ROOT, "profiles", "la_chunk_kernel_varlen_n16_h64_hbm_traffic.md"),
        ("la_common.h", "la_prefill.hip")),
    3: (os.path.join(ROOT, "profiles", "la_chunk_kernel_gva_b4_t16384_h16_hv64_hbm_traffic.md"),
        ("la_common.h", "la_prefill.hip")),
    4: (os.path.join(ROOT, "profiles", "la_short_kernel_verify_commit_b128_t8_h64_hbm_traffic.md"),
        ("la_common.h", "la_short.hip")),
    5: (os.path.join(ROOT, "profiles", "la_chunk_kernel_segmented_b1_t32768_h16_hbm_traffic.md"),
        ("la_common.h", "la_prefill.hip")),
}


def kernel_source_sha(names):
    """sha256 over the concatenated kernel sources with comments and whitespace removed (the key a traffic
    summary records: editing a comment does not change the kernel the counters were taken on)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for n in names:
        src = open(os.path.join(CSRC, n)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(config):
    """HBM bytes per step from the committed FETCH_SIZE/WRITE_SIZE summary, if it was taken on these kernel
    sources and this workload; else None."""
    if config not in TRAFFIC or not os.path.exists(TRAFFIC[config][0]):
        return None
    path, srcs = TRAFFIC[config]
    txt = open(path).read()
    if f"Kernel source sha256: {kernel_source_sha(srcs)}" not in txt:
        return None
    for line in txt.splitlines():
        if line.startswith("traffic_bytes_per_step:") or line.startswith("traffic_bytes_per_launch:"):
            return int(line.split(":")[1])
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def cpu_baseline(w, max_units=None, min_wall_s=1.2):
    """Time the FP64 oracle on a bounded sample of the same workload: whole (sequence, value head) units."""
    import oracle
    th = oracle.threads()
    n_units = max_units or 128
    rows = w.seq_rows()
    units = []
    for hv in range(w.HV):
        for n in range(w.nseq):
            units.append((rows[n][0], rows[n][1], hv))
    units = units[:n_units]
    q = w.q.reshape(-1, w.H, 128)
    k = w.k.reshape(-1, w.H, 128)
    v = w.v.reshape(-1, w.HV, 128)
    oracle.tokenwise(q, k, v, w.H, w.HV, w.scale, w.slope, units[:1])       # warm
    # whole passes over the sample until at least min_wall_s has passed (about 10 - 30 s of CPU work on a
    # many-core host)
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.tokenwise(q, k, v, w.H, w.HV, w.scale, w.slope, units)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_wall_s:
            break
    tokheads = sum(u[1] for u in units)
    return {"value": passes * tokheads / dt / 1e6, "unit": "Mtok·head/s", "cores": th, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(units)} whole (sequence, value head) units of {rows[0][1]} tokens each "
                      f"({tokheads} tok·head) x {passes} passes, FP64 tokenwise recurrence, {dt:.2f} s wall "
                      f"on {th} threads"}


# ------------------------------------------------------------------------------------------------------------
# amd-smi samples (GFX clock, socket power, hotspot temperature of GPU 0)
# ------------------------------------------------------------------------------------------------------------
def _walk(x):
    if isinstance(x, dict):
        yield x
        for v in x.values():
            yield from _walk(v)
    elif isinstance(x, list):
        for v in x:
            yield from _walk(v)


def _num(x):
    if isinstance(x, dict):
        x = x.get("value")
    try:
        return float(x)
    except (TypeError, ValueError):
        return None


def smi_sample(timeout_s=20.0):
    """One `amd-smi metric` reading of GPU 0: mean GFX clock over the gfx_N domains (MHz), socket power (W),
    hotspot temperature (C). None where amd-smi is missing or reports no such field."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "-t", "--json"], capture_output=True,
                           text=True, timeout=timeout_s)
        data = json.loads(r.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    clocks, power, temp = [], None, None
    for d in _walk(data):
        for key, val in d.items():
            if key.startswith("gfx_") and isinstance(val, dict) and "clk" in val:
                c = _num(val["clk"])
                if c is not None:
                    clocks.append(c)
            elif key == "socket_power" and power is None:
                power = _num(val)
            elif key == "hotspot" and temp is None:
                temp = _num(val)
    return {"t": round(time.time(), 2), "gfx_clock_mhz": round(sum(clocks) / len(clocks), 1) if clocks else None,
            "socket_power_w": power, "hotspot_c": temp}


class SmiPoller:
    """amd-smi samples taken by the parent (which never touches the GPU) every `period` seconds, in a thread,
    while the measurement processes run. amd-smi is itself a Python program, so it is never started from a
    process that uses the GPU."""

    def __init__(self, period=0.25):
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            s = smi_sample()
            if s is None:
                return
            self.samples.append(s)
            self._stop.wait(self.period)

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join(timeout=30)

    def window(self, t0, t1):
        return [s for s in self.samples if t0 <= s["t"] <= t1]


# ------------------------------------------------------------------------------------------------------------
# trace summary from a rocprofv3 kernel trace (no GPU)
# ------------------------------------------------------------------------------------------------------------
def trace_summary(path, kernel, skip, count):
    """Durations of the dispatches [skip, skip + count) of the kernels whose name contains `kernel`, in start
    order, from a rocprofv3 --kernel-trace CSV; prints a markdown table row (name, dispatches in the trace,
    selected range, average, median, min, max in ns)."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    sel = rows[skip:skip + count]
    if len(sel) < count:
        raise SystemExit(f"{path}: {len(rows)} dispatches of {kernel}, fewer than skip {skip} + count {count}")
    d = sorted(b - a for a, b in sel)
    avg = sum(d) / len(d)
    med = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
    print(f"| {kernel} | {len(rows)} | {skip} .. {skip + count - 1} | {avg:.1f} | {med:.1f} | {d[0]} | {d[-1]} |")
    return avg


def counter_summary(paths, kernel):
    """Median per dispatch of every counter in rocprofv3 --pmc CSVs, over the dispatches of the kernels whose name
    contains `kernel`; prints one markdown table row per counter (counter, dispatches, median)."""
    import csv
    import statistics
    vals = {}
    for path in paths:
        per = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for d in per.values():
            for k, v in d.items():
                vals.setdefault(k, []).append(v)
    for k in sorted(vals):
        print(f"| {k} | {len(vals[k])} | {statistics.median(vals[k]):,.1f} |")


# ------------------------------------------------------------------------------------------------------------
# measurement in one process
# ------------------------------------------------------------------------------------------------------------
def measure(args):
    import numpy as np
    import torch

    import la_synth
    import linear_attention_decay_amd as la

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        return {"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": args.steps}

    w = la_synth.config(args.config)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q = to_dev(w.q).view(torch.bfloat16)
    k = to_dev(w.k).view(torch.bfloat16)
    v = to_dev(w.v).view(torch.bfloat16)
    o = torch.empty_like(v)
    slope = to_dev(w.slope)
    pool = None if w.pool is None else to_dev(w.pool)
    idx = None if w.state_idx is None else to_dev(w.state_idx)
    cu = None if w.cu_seqlens is None else to_dev(w.cu_seqlens)
    flags = w.flags
    stream = torch.cuda.current_stream(dev)
    props = torch.cuda.get_device_properties(dev)

    chain = w.accepted_len is not None      # verify + commit of draft tokens through the KV buffer
    seg = args.config == 5                  # one long prompt: the segmented prefill, segment count from the CUs
    if seg:
        cus = props.multi_processor_count
        n_seg = max(1, cus // (2 * w.B * w.HV))
        ws = torch.empty(max(la.la_prefill_seg_workspace_bytes(w.B, w.HV, n_seg), 4) // 4, dtype=torch.float32,
                         device=dev)
    if chain:
        acc = to_dev(w.accepted_len)
        kb = torch.empty((w.pool.shape[0], w.T, w.H, 128), dtype=torch.bfloat16, device=dev)
        vb = torch.empty((w.pool.shape[0], w.T, w.HV, 128), dtype=torch.bfloat16, device=dev)

    def plain_step():
        la.la_prefill_fwd(q, k, v, o, slope, scale=w.scale, state_pool=pool, state_idx=idx, flags=flags, stream=stream)

    def step():
        if seg:
            la.la_prefill_fwd_seg(q, k, v, o, slope, scale=w.scale, state_pool=pool, state_idx=idx, flags=flags,
                                  segments=0, workspace=ws, stream=stream)
        elif chain:
            la.la_verify_kvbuffer(q, k, v, o, slope, pool, idx, k_buf=kb, v_buf=vb, scale=w.scale, stream=stream)
            la.la_state_commit_kvbuffer(kb, vb, slope, pool, idx, acc, stream=stream)
        elif cu is None:
            la.la_prefill_fwd(q, k, v, o, slope, scale=w.scale, state_pool=pool, state_idx=idx, flags=flags,
                              stream=stream)
        else:
            la.la_prefill_fwd_varlen(q, k, v, o, cu, slope, scale=w.scale, state_pool=pool, state_idx=idx,
                                     flags=flags, stream=stream)

    # The GPU ramps its clock up over the first ~100 launches after idle; run the kernel for a fixed wall time
    # first so that the W warmup and K timed steps see the steady clock. Untimed, reported as clock_prewarm_s.
    launches = 0
    stamps = {"prewarm_start": time.time()}
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(20):
            step()
        launches += 20
        torch.cuda.synchronize()
    prewarm_s = time.perf_counter() - t_pre
    for _ in range(args.warmup):
        step()
    launches += args.warmup
    torch.cuda.synchronize()

    # timed region: K back-to-back launches on the launch stream, bracketed by events on that stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    stamps["timed_start"] = time.time()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps

    # per-launch kernel durations (events around each launch on the same stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    kern_ms = sum(per) / len(per)
    stamps["timed_end"] = time.time()

    plain_ms = None
    if seg:   # the same workload on the unsegmented path, for comparison
        for _ in range(3):
            plain_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            plain_step()
        e1.record(stream)
        torch.cuda.synchronize()
        plain_ms = e0.elapsed_time(e1) / args.steps

    return {"ms_per_step": ms_per_step, "kernel_ms_avg": kern_ms, "kernel_ms_median": per[len(per) // 2],
            "clock_prewarm_s": prewarm_s, "plain_ms": plain_ms, "n_seg": n_seg if seg else None,
            # dispatch index of every kernel of the step (rocprofv3 trace order): the back-to-back timed launches,
            # then the launches with per-launch events
            "dispatches": {"before_timed": launches, "timed": args.steps, "per_launch_events": args.steps},
            "gpu": {"name": props.name, "gfx_arch": getattr(props, "gcnArchName", None),
                    "cus": props.multi_processor_count, "hip_runtime": torch.version.hip},
            "stamps": stamps}


def median_iqr(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return float(np.median(a)), float(np.percentile(a, 75) - np.percentile(a, 25))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, choices=range(6))
    ap.add_argument("--procs", type=int, default=3,
                    help="fresh child processes to measure in (median reported); 1 = measure in this process")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-smi", action="store_true", help="skip the amd-smi clock / power samples")
    ap.add_argument("--prewarm-s", type=float, default=1.5,
                    help="untimed seconds of launches before warmup, so the timed steps run at the steady clock")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy_) --steps times: the reference kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarize dispatches of --kernel from a rocprofv3 kernel trace and exit (no GPU)")
    ap.add_argument("--counter-summary", metavar="CSV", nargs="+",
                    help="median per dispatch of each counter of --kernel in rocprofv3 --pmc CSVs, then exit (no GPU)")
    ap.add_argument("--kernel", default="la_chunk_kernel<0>")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--count", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              f"sharding over several GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.trace_summary:
        trace_summary(args.trace_summary, args.kernel, args.skip, args.count)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.kernel)
        return
    if args.child or args.copy_calibration:
        print(json.dumps(measure(args)), flush=True)
        return

    # One measurement per fresh child process; this process starts no GPU work itself.
    runs = []
    poller = None
    if args.procs <= 1:
        runs.append(measure(args))
    else:
        poller = None if args.no_smi else SmiPoller().start()
        cmd = [sys.executable, os.path.abspath(__file__), "--child", "--config", str(args.config), "--steps",
               str(args.steps), "--warmup", str(args.warmup), "--prewarm-s", str(args.prewarm_s)]
        for i in range(args.procs):
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
            if r.returncode != 0:
                print(f"bench.py: measurement process {i} exited with status {r.returncode}", file=sys.stderr)
                sys.exit(r.returncode if r.returncode > 0 else 1)
            runs.append(json.loads(r.stdout.strip().splitlines()[-1]))
        if poller is not None:
            poller.stop()

    import la_synth
    w = la_synth.config(args.config)
    chain = w.accepted_len is not None
    seg = args.config == 5
    ms_per_step, ms_iqr = median_iqr([r["ms_per_step"] for r in runs])
    ev_ms, ev_iqr = median_iqr([r["kernel_ms_avg"] for r in runs])
    tokheads = w.tokens * w.HV
    value = tokheads / (ms_per_step * 1e-3) / 1e6
    alg_bytes = chain_bytes(w) if chain else algorithmic_bytes(w)
    # The roofline uses the average launch duration of the timed back-to-back launches (the HIP events around the
    # timed region, on the launch stream): the rate the kernel sustains. The per-launch events of the second pass
    # separate the launches by a few microseconds, which lets the clock rise above its sustained value, so they
    # are reported beside it but not used.
    kern_ms = ms_per_step
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    short = chain or seg or 1 <= w.T <= 16     # MFMA count below is for the plain chunked kernel only
    mfma_tfs = None if short else mfma_flops_executed(w) / (kern_ms * 1e-3) / 1e12
    r0 = runs[0]

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Mtok·head/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "HV": w.HV, "D": 128, "DV": 128,
                   "chunk": CHUNK, "state_flags": w.flags, "tokens": w.tokens},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
                     "kernel": ("la_chunk_kernel<3> + la_seg_scan_kernel + la_chunk_kernel<4> (segmented)" if seg else
                                "la_short_kernel<false> + la_short_kernel<true> (verify + commit)" if chain else
                                "la_short_kernel<false>" if 1 <= w.T <= 16 else
                                "la_chunk_kernel<1>" if w.cu_seqlens is not None else "la_chunk_kernel<0>"),
                     "kernel_ms_avg": round(kern_ms, 6), "kernel_ms_separate_launches": round(ev_ms, 6),
                     "algorithmic_bytes": alg_bytes},
        "mfma": None if short else {"executed_tflops": round(mfma_tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                                    "frac": round(mfma_tfs / MFMA_BF16_PEAK_TFS, 4),
                                    "insts_per_workgroup_chunk": {"16x16x32_bf16": MFMA_X32_PER_WG_CHUNK,
                                                                  "16x16x16_bf16": MFMA_X16_PER_WG_CHUNK}},
        "timing": {"processes": len(runs), "ms_per_step_each": [round(r["ms_per_step"], 6) for r in runs],
                   "ms_per_step_iqr": round(ms_iqr, 6),
                   "kernel_ms_separate_launches_each": [round(r["kernel_ms_avg"], 6) for r in runs],
                   "kernel_ms_separate_launches_iqr": round(ev_iqr, 6),
                   "clock_prewarm_s_each": [round(r["clock_prewarm_s"], 3) for r in runs],
                   "dispatches_per_process": r0["dispatches"]},
        "machine": {"gpu": r0["gpu"]["name"], "gfx_arch": r0["gpu"]["gfx_arch"], "cus": r0["gpu"]["cus"],
                    "rocm": rocm_version(), "hip_runtime": r0["gpu"]["hip_runtime"], "cpu_model": cpu_model(),
                    # per process: samples returned from 0.8 s into the pre-warm (amd-smi reports power and clock
                    # averaged over its last few hundred ms) to the end of the timed launches
                    "smi_under_load_each": None if poller is None else [
                        poller.window(r["stamps"]["prewarm_start"] + 0.8, r["stamps"]["timed_end"]) for r in runs]},
    }
    if seg:
        plain, _ = median_iqr([r["plain_ms"] for r in runs])
        out["segmented"] = {"segments_requested": r0["n_seg"], "unsegmented_ms_per_step": round(plain, 6),
                            "speedup": round(plain / ms_per_step, 3)}
    if not args.no_cpu_baseline and args.config in (0, 1):
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
