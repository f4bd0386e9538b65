"""Benchmark of the Lightning Attention chunked prefill on one MI355X.

One step = one la_prefill_fwd call over the whole workload: B=2, T=8192, H=HV=64, D=DV=128, bf16 Q/K/V/O,
FP32 state read from and written back to a 2-slot pool in place (every step sees the previous step's state;
the work per step is identical). Inputs are synthetic (la_synth recipe, seed 1) and resident in HBM before the
timed region. Prints one JSON line. --config 0/2/3 time the other prefill workloads; --config 4 times the draft
verify + commit chain through the KV buffer (B=128 requests, T=8); --config 5 times the segmented prefill of one
long prompt (B=1, T=32768, H=HV=16) and reports the unsegmented time beside it.

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--config {0,1,2,3,4,5}]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
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


def mfma_flops_executed(w):
    """Dense bf16 MFMA flops the kernel issues per call: per 64-token chunk and value head, scores 64x64x128 (by
    both workgroups of a head), P.V 64x128x64 (block lower triangle, P as hi+lo), Q.S^T 64x128x128 (S as hi+lo),
    state update 128x128x64 (V_dec as hi+lo), plus the identity transposes."""
    per_chunk_head = (
        2 * (10 / 16) * 64 * 64 * 128 * 2        # scores: 10 of 16 tiles, computed in each of the 2 value halves
        + 2 * (12 / 16) * 64 * 128 * 64 * 2     # P.V: 6 of 8 32-token blocks per column tile, hi + lo
        + 2 * 64 * 128 * 128 * 2                # Q.S^T with S hi + lo
        + 2 * 128 * 128 * 64 * 2                # state update with V_dec hi + lo
        + 2 * (32 + 8) * 16 * 16 * 16 * 2       # identity transposes of K (both halves) and V
    )
    chunks = sum((l + CHUNK - 1) // CHUNK for _, l in w.seq_rows())
    return per_chunk_head * chunks * w.HV


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


def cpu_baseline(w, max_units=None, min_wall_s=1.2):
    """Time the FP64 oracle on a bounded sample of the same workload: whole (sequence, value head) units."""
    import numpy as np
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
            "sample": f"{len(units)} whole (sequence, value head) units of {rows[0][1]} tokens each "
                      f"({tokheads} tok·head) x {passes} passes, FP64 tokenwise recurrence, {dt:.2f} s wall "
                      f"on {th} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, choices=range(6))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="untimed seconds of launches before warmup, so the timed steps run at the steady clock")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy_) --steps times: the reference kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              f"sharding over several GPUs)", file=sys.stderr)
        sys.exit(2)

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
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": args.steps}), flush=True)
        return

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

    chain = w.accepted_len is not None      # verify + commit of draft tokens through the KV buffer
    seg = args.config == 5                  # one long prompt: the segmented prefill, segment count from the CUs
    if seg:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
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
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    prewarm_s = time.perf_counter() - t_pre
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back launches on the launch stream, bracketed by events on that stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
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

    tokheads = w.tokens * w.HV
    value = tokheads / (ms_per_step * 1e-3) / 1e6
    alg_bytes = chain_bytes(w) if chain else algorithmic_bytes(w)
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    short = chain or seg or 1 <= w.T <= 16     # MFMA count below is for the plain chunked kernel only
    mfma_tfs = None if short else mfma_flops_executed(w) / (kern_ms * 1e-3) / 1e12

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
        "clock_prewarm_s": round(prewarm_s, 3),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "HV": w.HV, "D": 128, "DV": 128,
                   "chunk": CHUNK, "state_flags": w.flags, "tokens": w.tokens},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
                     "kernel": ("la_chunk_kernel<3> + la_seg_scan_kernel + la_chunk_kernel<4> (segmented)" if seg else
                                "la_short_kernel<false> + la_short_kernel<true> (verify + commit)" if chain else
                                "la_short_kernel<false>" if 1 <= w.T <= 16 else
                                "la_chunk_kernel<1>" if cu is not None else "la_chunk_kernel<0>"),
                     "kernel_ms_avg": round(kern_ms, 6),
                     "kernel_ms_median": round(per[len(per) // 2], 6), "algorithmic_bytes": alg_bytes},
        "mfma": None if short else {"executed_tflops": round(mfma_tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                                    "frac": round(mfma_tfs / MFMA_BF16_PEAK_TFS, 4)},
    }
    if seg:
        out["segmented"] = {"segments_requested": n_seg, "unsegmented_ms_per_step": round(plain_ms, 6),
                            "speedup": round(plain_ms / ms_per_step, 3)}
    if not args.no_cpu_baseline and args.config in (0, 1):
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
