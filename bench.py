"""Throughput of the multi-LoRA batched adapter path on one MI355X.

One step = the whole hot path over one mixed co-serving batch (seed 0):
  lora_segments_build_batch (all rows, and the fine-tuning rows) ->
  lora_shrink -> lora_expand_add -> lora_backward (dX, dA, dB),
with the forward's v of the fine-tuning rows passed to the backward as the
saved v.  `--workload` selects another of the synthetic workloads (the
backward runs only where the workload has fine-tuning rows).  Workload: 128 decode rows, 8 prefill segments of U[128, 1024]
rows, 2 fine-tuning segments of 1024 rows on the reserved adapter; 32
adapters with ranks drawn from {8, 16, 32, 64}, scale 2.0; d_in 4096 ->
d_out 14336; bf16 elements (DeltaServe section 3.2, "Mixed forward batch").

Inputs are resident in HBM before the timed region.  Consecutive steps use
different copies of every buffer (weights included): as many copies as it
takes to rotate through more than 1.2 GB, so a step never finds the previous
step's data in the 256 MB Infinity Cache (the rotation size is reported).

Prints one JSON line.  `value` = rows of the batch per second of step time.
`roofline` is for the dominant kernel (lora_expand_add: the read-modify-write
of y), timed with HIP events around its launch on the stream it runs on.
`calls` gives each library call's GPU time per call, from captured HIP graphs
of back-to-back calls over the rotating copies (no host launch overhead).
`workloads` repeats the measurement on the decode, fine-tuning and many-adapter
decode workloads (their forward path as the library's chooser picks it).
`cpu_baseline` times the fp64 oracle on the host on the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
RANKS_DESC = {2: "16", 3: "U{8,16,32,64}", 4: "16", 5: "U{8,16,32,64,128}"}
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
EVENT_EVERY = 5          # timed steps per sampled expand launch (events)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating copies of every buffer (default: enough for a rotation above 1.2 GB, at least 4)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="measure the headline workload only (no `workloads` block)")
    ap.add_argument("--workload-steps", type=int, default=50, help="timed steps per workload of the block")
    ap.add_argument("--workload", type=int, default=3, choices=(2, 3, 4, 5),
                    help="synthetic workload (workloads.config index); 3 = the mixed co-serving batch")
    ap.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    ap.add_argument("--overlap", action="store_true",
                    help="run the fine-tuning backward (v recomputed) on a second stream, concurrently with the "
                         "forward, joining at the end of each step")
    ap.add_argument("--forward", choices=("auto", "split", "fused"), default="auto",
                    help="forward of a step: lora_shrink + lora_expand_add (split), one lora_forward launch "
                         "(fused; v written for the backward), or whichever of the two has the shorter GPU "
                         "time per call on the workload (auto, measured before the timed steps)")
    ap.add_argument("--fused", action="store_true", help="same as --forward fused")
    ap.add_argument("--preemptible", action="store_true",
                    help="run the backward through lora_backward_preemptible with a granted grant word")
    ap.add_argument("--adamw", action="store_true",
                    help="end each step with the AdamW update of the fine-tuning adapter (fp32 master weights)")
    ap.add_argument("--cost-model", action="store_true",
                    help="calibrate and fit the cost model of the library's calls, then check its predictions on "
                         "the four bf16 workloads (held out); prints JSON lines, not the bench line")
    ap.add_argument("--multi-slice", action="store_true",
                    help="q/k/v projections of the decode workload (d_out 4096/1024/1024): three split forwards, "
                         "three lora_forward launches and one lora_forward_multi; prints JSON lines, not the bench line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only time a plain device copy of 256 MiB (reference for counter scaling)")
    ap.add_argument("--kernel-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="print every kernel's read / write bytes per dispatch from counter files of a run "
                         "and of --copy-calibration")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 counter_collection.csv files of FETCH_SIZE / WRITE_SIZE passes over this "
                         "bench and over --copy-calibration: write the measured HBM traffic of the expand kernel")
    args = ap.parse_args()
    if args.fused:
        args.forward = "fused"
    return args


# HBM traffic of the dominant kernel, measured with rocprofv3 counters and
# stored with a hash of the sources it was measured on; a stale file reads as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expand_kernel_mixed-coserve-4096to14336_traffic.json")
KERNEL_SOURCES = ["expand_token_adapter_amd/csrc/expand.h", "expand_token_adapter_amd/csrc/device_common.h",
                  "expand_token_adapter_amd/csrc/forward.hip", "expand_token_adapter_amd/build.py"]
EXPAND_KERNEL_PREFIX = "void lora::expand_kernel<0, false"
COPY_BYTES = 256 << 20


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _counter_means(path, counter):
    """Mean per-dispatch value of one counter for every kernel in a rocprofv3 counter_collection.csv."""
    import csv
    from collections import defaultdict
    vals = defaultdict(list)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def traffic_from(fetch, write, cfetch, cwrite):
    def pick(means, pred, what):
        hits = [(k, m) for k, m in means.items() if pred(k)]
        if not hits:
            raise SystemExit(f"no {what} dispatches in the counter file")
        return max(hits, key=lambda km: km[1][1])  # the most frequent one
    fe = pick(_counter_means(fetch, "FETCH_SIZE"), lambda k: k.startswith(EXPAND_KERNEL_PREFIX), "expand")
    wr = pick(_counter_means(write, "WRITE_SIZE"), lambda k: k.startswith(EXPAND_KERNEL_PREFIX), "expand")
    cf = pick(_counter_means(cfetch, "FETCH_SIZE"), lambda k: "copy" in k.lower(), "copy")
    cw = pick(_counter_means(cwrite, "WRITE_SIZE"), lambda k: "copy" in k.lower(), "copy")
    f_fetch = COPY_BYTES / (cf[1][0] * 1024.0)
    f_write = COPY_BYTES / (cw[1][0] * 1024.0)
    rd = fe[1][0] * 1024.0 * f_fetch
    wb = wr[1][0] * 1024.0 * f_write
    out = {"kernel": fe[0], "fetch_kib_per_dispatch": fe[1][0], "write_kib_per_dispatch": wr[1][0],
           "dispatches": [fe[1][1], wr[1][1]], "copy_kernel": cf[0], "copy_bytes_each_way": COPY_BYTES,
           "copy_fetch_kib": cf[1][0], "copy_write_kib": cw[1][0], "fetch_scale": f_fetch, "write_scale": f_write,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wb, "traffic_bytes_per_launch": rd + wb,
           "source_sha256": kernel_source_hash(), "sources": KERNEL_SOURCES}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def kernel_traffic(fetch, write, cfetch, cwrite):
    """Print, for every kernel of a FETCH_SIZE / WRITE_SIZE counter pair, its mean
    read and write bytes per dispatch, scaled by the copy calibration's counters."""
    fm, wm = _counter_means(fetch, "FETCH_SIZE"), _counter_means(write, "WRITE_SIZE")
    cf = [m for k, m in _counter_means(cfetch, "FETCH_SIZE").items() if "copy" in k.lower()]
    cw = [m for k, m in _counter_means(cwrite, "WRITE_SIZE").items() if "copy" in k.lower()]
    if not cf or not cw:
        raise SystemExit("no copy dispatches in the calibration counter files")
    f_fetch = COPY_BYTES / (max(cf, key=lambda m: m[1])[0] * 1024.0)
    f_write = COPY_BYTES / (max(cw, key=lambda m: m[1])[0] * 1024.0)
    for k in sorted(set(fm) | set(wm)):
        rd = fm[k][0] * 1024.0 * f_fetch if k in fm else None
        wb = wm[k][0] * 1024.0 * f_write if k in wm else None
        print(json.dumps({"kernel": k, "dispatches": [fm.get(k, (0, 0))[1], wm.get(k, (0, 0))[1]],
                          "read_bytes": rd, "write_bytes": wb, "fetch_scale": f_fetch, "write_scale": f_write}))


def measured_traffic():
    """Traffic per launch from the stored counter run, or None if absent or measured on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return float(t["traffic_bytes_per_launch"])


def copy_calibration(reps: int = 20):
    """A plain device-to-device copy of a known size: the achievable copy rate on
    this GPU, and the per-dispatch reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = COPY_BYTES
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    c = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        (b if i % 2 == 0 else c).copy_(a if i % 2 == 0 else b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copy_ms": ms,
                      "copy_GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def algorithmic(wl):
    """Minimum bytes / FLOPs of each kernel of one step (realized batch)."""
    e = 2
    T, d_in, d_out = wl.T, wl.d_in, wl.d_out
    ids = wl.ids
    ranks = wl.ranks.astype(np.int64)
    valid = ids >= 0
    sum_rt = int(ranks[ids[valid]].sum())            # sum over rows of r_a(t)
    used = np.unique(ids[valid])
    sum_ru = int(ranks[used].sum())                  # sum over used adapters of r_a
    n_valid = int(valid.sum())
    out = {}
    seg_bytes = lambda n: 4 * n + 4 * n + 4 * (2 * wl.num_adapters + 1)  # ids in, perm out, counts/offsets
    out["segments"] = dict(bytes=seg_bytes(T) + seg_bytes(wl.ft_count), flops=0)
    out["shrink"] = dict(bytes=e * n_valid * d_in + e * d_in * sum_ru + 4 * sum_rt, flops=2 * d_in * sum_rt)
    out["expand"] = dict(bytes=4 * sum_rt + e * d_out * sum_ru + 2 * e * n_valid * d_out, flops=2 * d_out * sum_rt)
    # the one-launch forward: the two without the v round trip (v is still written once, for the backward)
    fwd = dict(bytes=out["shrink"]["bytes"] + out["expand"]["bytes"] - 4 * sum_rt,
               flops=out["shrink"]["flops"] + out["expand"]["flops"])
    ft = wl.ft_ids
    Tf = wl.ft_count
    rft = ranks[ft].astype(np.int64)
    uft = np.unique(ft)
    r_u = int(ranks[uft].sum())
    out["backward"] = dict(
        bytes=e * Tf * d_in + e * Tf * d_out + 2 * e * Tf * d_in + e * r_u * (d_in + d_out)
        + 8 * r_u * (d_in + d_out) + 4 * int(rft.sum()),
        flops=4 * int(rft.sum()) * (d_in + d_out))
    out["step"] = dict(bytes=sum(v["bytes"] for v in out.values()), flops=sum(v["flops"] for v in out.values()))
    out["forward_fused"] = fwd
    return out


def cpu_baseline(wl, min_seconds):
    """The fp64 oracle on the host: forward of every row + backward of the fine-tuning rows."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    oracle.set_threads(threads)
    ref = oracle.from_workload(wl)
    s, n = wl.ft_start, wl.ft_count
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(ref["x"], ref["ids"], ref["ranks"], ref["scales"], ref["A"], ref["B"], ref["y0"])
        if n > 0:
            oracle.backward(ref["x"][s:s + n], ref["dy"], ref["ids"][s:s + n], ref["ranks"], ref["scales"],
                            ref["A"], ref["B"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 50:
            break
    cores = oracle.threads()
    # the same batch once on one thread (plain loops, no OpenMP split)
    oracle.set_threads(1)
    t1 = time.perf_counter()
    oracle.forward(ref["x"], ref["ids"], ref["ranks"], ref["scales"], ref["A"], ref["B"], ref["y0"])
    if n > 0:
        oracle.backward(ref["x"][s:s + n], ref["dy"], ref["ids"][s:s + n], ref["ranks"], ref["scales"],
                        ref["A"], ref["B"])
    el1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": reps * wl.T / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full batch ({wl.T} rows forward + {n} fine-tuning rows backward), "
                      f"repeated {reps}x in {el:.1f} s, fp64 plain loops, OpenMP over rows",
            "single_thread_value": wl.T / el1, "single_thread_seconds": el1,
            "host_cpu": model, "host_nproc": os.cpu_count()}


def multi_slice_report(steps: int, warmup: int, n_sets: int):
    """Forward of three projections sharing x (decode batch): split, three fused launches, one multi-slice launch."""
    import torch
    import expand_token_adapter_amd as lb
    import workloads

    dev = torch.device("cuda:0")
    wq = workloads.config(2, seed=0)
    wls = [wq] + [workloads.custom(wq.ids, wq.ranks, wq.d_in, 1024, "bf16", seed=100 + k) for k in range(2)]
    dev_e = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    sets = []
    for k in range(n_sets):
        st = {"x": dev_e(wq.x), "ids": torch.from_numpy(wq.ids).to(dev), "seg": lb.Segments(wq.T, wq.num_adapters, dev)}
        st["tables"] = [lb.AdapterTable([dev_e(a) for a in w.A], [dev_e(b) for b in w.B], w.scales.tolist())
                        for w in wls]
        st["ys"] = [dev_e(w.y0) for w in wls]
        st["vs"] = [torch.zeros((wq.T, 16), dtype=torch.float32, device=dev) for _ in wls]
        st["ws"] = torch.empty(lb.lora_shrink_workspace_bytes(torch.bfloat16, wq.T, wq.d_in, 16), dtype=torch.uint8,
                               device=dev)
        sets.append(st)

    def split(st):
        for t, y, v in zip(st["tables"], st["ys"], st["vs"]):
            lb.lora_shrink(st["x"], t, st["seg"], v=v, ws=st["ws"])
            lb.lora_expand_add(v, t, st["seg"], y)

    def fused3(st):
        for t, y, v in zip(st["tables"], st["ys"], st["vs"]):
            lb.lora_forward(st["x"], t, st["seg"], y, v=v)

    def multi(st):
        lb.lora_forward_multi(st["x"], list(zip(st["tables"], st["ys"], st["vs"])), st["seg"])

    alg = sum(algorithmic(w)["forward_fused"]["bytes"] for w in wls) - 2 * 2 * int((wq.ids >= 0).sum()) * wq.d_in  # x read once
    for name, fwd in (("split x3", split), ("lora_forward x3", fused3), ("lora_forward_multi", multi)):
        def step(st):
            lb.lora_segments_build(st["ids"], wq.num_adapters, out=st["seg"])
            fwd(st)
        # every rotating set once, then the warm-up steps (no timed step is
        # the first to touch a buffer)
        for i in range(n_sets + warmup):
            step(sets[i % n_sets])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(sets[i % n_sets])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        # GPU time per step, free of host launch costs: a captured graph of one
        # step over every set, replayed between events (outside the timed loop)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            for st in sets:
                step(st)
        torch.cuda.current_stream(dev).wait_stream(cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for st in sets:
                step(st)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 25
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        gpu_us = e0.elapsed_time(e1) * 1e3 / (reps * n_sets)
        del g
        print(json.dumps({"multi_slice": name, "workload": "decode-64x-r16-4096 q/k/v (d_out 4096/1024/1024)",
                          "rows": wq.T, "ms_per_step": ms, "rows_per_s": wq.T / (ms * 1e-3),
                          "gpu_us_per_step": gpu_us, "forward_algorithmic_bytes": alg, "steps": steps}), flush=True)


def cost_model_report(reps: int = 10):
    """Fit the cost model on synthetic calibration batches, then predict the workloads' calls."""
    import torch
    import expand_token_adapter_amd as lb
    from expand_token_adapter_amd import cost_model as cm
    import workloads

    t0 = time.perf_counter()
    samples = cm.calibrate(reps=reps)
    model = cm.fit_samples(samples)
    errs = cm.relative_errors(model, samples)
    for op in sorted(errs):
        e = np.abs(errs[op])
        print(json.dumps({"cost_model": op, "coef": dict(zip(cm.FEATURES, model.coef[op].tolist())),
                          "calibration_samples": int(e.size), "median_abs_rel_err": float(np.median(e)),
                          "max_abs_rel_err": float(e.max())}), flush=True)
    print(json.dumps({"calibration_seconds": time.perf_counter() - t0}), flush=True)
    dev = torch.device("cuda:0")
    for w in (2, 3, 4, 5):
        wl = workloads.config(w, seed=0)
        dev_e = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        A, B = [dev_e(a) for a in wl.A], [dev_e(b) for b in wl.B]
        table = lb.AdapterTable(A, B, wl.scales.tolist())
        ids = torch.from_numpy(wl.ids).to(dev)
        x, y = dev_e(wl.x), dev_e(wl.y0)
        seg = lb.Segments(wl.T, wl.num_adapters, dev)
        lb.lora_segments_build(ids, wl.num_adapters, out=seg)
        v = torch.zeros((wl.T, (table.r_max + 7) // 8 * 8), dtype=torch.float32, device=dev)
        ws = torch.empty(lb.lora_shrink_workspace_bytes(torch.bfloat16, wl.T, wl.d_in, table.r_max),
                         dtype=torch.uint8, device=dev)
        calls = {"segments": (lambda: lb.lora_segments_build(ids, wl.num_adapters, out=seg), wl.ids),
                 "forward": (lambda: (lb.lora_shrink(x, table, seg, v=v, ws=ws),
                                      lb.lora_expand_add(v, table, seg, y)), wl.ids),
                 "forward_fused": (lambda: lb.lora_forward(x, table, seg, y, v=v), wl.ids)}
        if wl.ft_count:
            s, n = wl.ft_start, wl.ft_count
            seg_ft = lb.Segments(n, wl.num_adapters, dev)
            lb.lora_segments_build(ids[s:s + n].contiguous(), wl.num_adapters, out=seg_ft)
            dy, dx = dev_e(wl.dy), torch.zeros((n, wl.d_in), dtype=torch.bfloat16, device=dev)
            grads = lb.GradTable([torch.zeros(a.shape, dtype=torch.float32, device=dev) for a in A],
                                 [torch.zeros(b.shape, dtype=torch.float32, device=dev) for b in B])
            r_ft = max(int(wl.ranks[a]) for a in set(wl.ft_ids.tolist()))
            bws = torch.empty(lb.lora_backward_workspace_bytes(torch.bfloat16, n, wl.d_in, wl.d_out, r_ft),
                              dtype=torch.uint8, device=dev)
            calls["backward"] = (lambda: lb.lora_backward(x[s:s + n], dy, table, grads, seg_ft, dx=dx,
                                                          v_saved=v[s:s + n], r_max=r_ft, ws=bws),
                                 wl.ids[s:s + n])
        for op, (f, op_ids) in calls.items():
            f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            meas = e0.elapsed_time(e1) * 1e-3 / reps
            pred = model.predict(op, op_ids, wl.ranks, wl.d_in, wl.d_out,
                                 r_max=r_ft if op == "backward" else 0, with_v=True)
            print(json.dumps({"workload": workloads.CONFIG_NAMES[w], "op": op, "measured_us": meas * 1e6,
                              "predicted_us": pred * 1e6, "rel_err": pred / meas - 1.0}), flush=True)


ROTATION_BYTES = 1.2e9  # more than the 256 MB Infinity Cache, several times over


def per_set_bytes(wl) -> int:
    """Device bytes of one rotating copy of a workload's buffers."""
    e = 2
    w = sum(a.size for a in wl.A) * e + sum(b.size for b in wl.B) * e
    io = wl.T * wl.d_in * e + wl.T * wl.d_out * e + wl.T * ((wl.r_max + 7) // 8 * 8) * 4
    ft = 0
    if wl.ft_count:
        ft = wl.ft_count * (wl.d_out + wl.d_in) * e + 2 * (w // e) * 4  # dy, dx, fp32 dA / dB of every adapter
    return w + io + ft


def auto_sets(wl) -> int:
    import math
    return max(4, int(math.ceil(ROTATION_BYTES / per_set_bytes(wl))))


class Bench:
    """One workload resident on the GPU in rotating copies, and its step."""

    def __init__(self, wl, n_sets, fused=False, preemptible=False, adamw=False, overlap=False):
        import torch
        import expand_token_adapter_amd as lb
        self.torch, self.lb = torch, lb
        self.wl = wl
        self.dev = dev = torch.device("cuda:0")
        self.fused, self.adamw = fused, adamw
        T, s, n = wl.T, wl.ft_start, wl.ft_count
        self.has_ft = has_ft = n > 0
        # The fine-tuning job knows the adapters it trains (the reserved
        # adapter), so its backward passes their largest rank as r_max.
        self.r_ft = max(int(wl.ranks[a]) for a in set(wl.ft_ids.tolist())) if has_ft else 0

        def dev_bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        base = dict(A=[dev_bf16(a) for a in wl.A], B=[dev_bf16(b) for b in wl.B], x=dev_bf16(wl.x),
                    y=dev_bf16(wl.y0), dy=dev_bf16(wl.dy) if has_ft else None)
        ids = torch.from_numpy(wl.ids).to(dev)
        ft_ids = ids[s:s + n].contiguous()
        self.sets = []
        for k in range(n_sets):
            c = (lambda t: t) if k == 0 else (lambda t: t.clone())
            A = [c(a) for a in base["A"]]
            B = [c(b) for b in base["B"]]
            st = dict(A=A, B=B, table=lb.AdapterTable(A, B, wl.scales.tolist()), x=c(base["x"]), y=c(base["y"]),
                      ids=ids.clone())
            st["v"] = torch.zeros((T, (st["table"].r_max + 7) // 8 * 8), dtype=torch.float32, device=dev)
            st["seg"] = lb.Segments(T, wl.num_adapters, dev)
            if has_ft:
                st["dy"] = c(base["dy"])
                st["ft_ids"] = ft_ids.clone()
                st["dx"] = torch.zeros((n, wl.d_in), dtype=torch.bfloat16, device=dev)
                st["dA"] = [torch.zeros(a.shape, dtype=torch.float32, device=dev) for a in A]
                st["dB"] = [torch.zeros(b.shape, dtype=torch.float32, device=dev) for b in B]
                st["grads"] = lb.GradTable(st["dA"], st["dB"])
                st["seg_ft"] = lb.Segments(n, wl.num_adapters, dev)
                st["ws"] = torch.empty(lb.lora_backward_workspace_bytes(torch.bfloat16, n, wl.d_in, wl.d_out,
                                                                        self.r_ft),
                                       dtype=torch.uint8, device=dev)
                if adamw:
                    # AdamW state of the fine-tuning adapter's A and B: fp32 master copies and moments
                    st["opt"] = [(w, gr, torch.zeros(w.shape, dtype=torch.float32, device=dev),
                                  torch.zeros(w.shape, dtype=torch.float32, device=dev), w.float())
                                 for a in sorted(set(int(i) for i in wl.ft_ids))
                                 for w, gr in ((A[a], st["dA"][a]), (B[a], st["dB"][a]))]
                    st["opt_step"] = 0
            st["ws_shrink"] = torch.empty(lb.lora_shrink_workspace_bytes(torch.bfloat16, T, wl.d_in,
                                                                         st["table"].r_max),
                                          dtype=torch.uint8, device=dev)
            self.sets.append(st)
        del base
        torch.cuda.synchronize()
        self.side = torch.cuda.Stream(device=dev) if overlap else None  # default priority
        self.grant = torch.ones(1, dtype=torch.int32, device=dev) if preemptible else None
        self.status = torch.zeros(1, dtype=torch.int32, device=dev) if preemptible else None

    # ---------------------------------------------------------------- the library calls of a step
    def seg_build(self, st):
        if self.has_ft:
            # the batch's rows and its fine-tuning rows grouped in one launch
            self.lb.lora_segments_build_batch([(st["ids"], st["seg"]), (st["ft_ids"], st["seg_ft"])],
                                              self.wl.num_adapters)
        else:
            self.lb.lora_segments_build(st["ids"], self.wl.num_adapters, out=st["seg"])

    def shrink(self, st):
        self.lb.lora_shrink(st["x"], st["table"], st["seg"], v=st["v"], ws=st["ws_shrink"])

    def expand(self, st):
        self.lb.lora_expand_add(st["v"], st["table"], st["seg"], st["y"])

    def forward_fused(self, st):
        self.lb.lora_forward(st["x"], st["table"], st["seg"], st["y"], v=st["v"])

    def forward_one_launch(self, st):
        # without v: always one launch (with v, decode batches and r_max <= 16
        # run the split kernels)
        self.lb.lora_forward(st["x"], st["table"], st["seg"], st["y"])

    def backward(self, st, v_saved=True):
        s, n = self.wl.ft_start, self.wl.ft_count
        vs = st["v"][s:s + n] if v_saved else None
        if self.grant is not None:
            self.lb.lora_backward_preemptible(st["x"][s:s + n], st["dy"], st["table"], st["grads"], st["seg_ft"],
                                              self.grant, self.status, dx=st["dx"], v_saved=vs, r_max=self.r_ft,
                                              ws=st["ws"])
            return
        self.lb.lora_backward(st["x"][s:s + n], st["dy"], st["table"], st["grads"], st["seg_ft"], dx=st["dx"],
                              v_saved=vs, r_max=self.r_ft, ws=st["ws"])

    def step(self, st, ev=None, ph=None):
        # ev: events around the dominant kernel (and the optimizer); ph: events at
        # the start, after the segment build, after the forward and at the end
        torch = self.torch
        if ph is not None:
            ph[0].record()
        side = self.side
        if side is not None and self.has_ft:
            side.wait_stream(torch.cuda.current_stream(self.dev))
            with torch.cuda.stream(side):
                self.lb.lora_segments_build(st["ft_ids"], self.wl.num_adapters, out=st["seg_ft"])
                self.backward(st, v_saved=False)
            self.lb.lora_segments_build(st["ids"], self.wl.num_adapters, out=st["seg"])
        else:
            self.seg_build(st)
        if ph is not None:
            ph[1].record()
        if self.fused:
            if ev is not None:
                ev[0].record()
            self.forward_fused(st)
            if ev is not None:
                ev[1].record()
        else:
            self.shrink(st)
            if ev is not None:
                ev[0].record()
            self.expand(st)
            if ev is not None:
                ev[1].record()
        if ph is not None:
            ph[2].record()
        if side is not None and self.has_ft:
            torch.cuda.current_stream(self.dev).wait_stream(side)
        elif self.has_ft:
            self.backward(st)
        if self.adamw and self.has_ft:
            st["opt_step"] += 1
            if ev is not None:
                ev[2].record()
            self.lb.lora_adamw_step(st["opt"], step=st["opt_step"], zero_grad=True)
            if ev is not None:
                ev[3].record()
        if ph is not None:
            ph[3].record()

    # ---------------------------------------------------------------- measurements
    def distribution(self, K, start):
        """Per-step event times of K steps (outside any timed region)."""
        torch = self.torch
        phs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(K)]
        for i in range(K):
            self.step(self.sets[(start + i) % len(self.sets)], None, phs[i])
        torch.cuda.synchronize()
        pct = lambda a: {"p10": float(np.percentile(a, 10)), "median": float(np.median(a)),
                         "p90": float(np.percentile(a, 90))}
        dist = {"steps": K, "step_ms": pct([e[0].elapsed_time(e[3]) for e in phs]),
                "forward_with_segment_build_ms": pct([e[0].elapsed_time(e[2]) for e in phs]),
                "forward_without_segment_build_ms": pct([e[1].elapsed_time(e[2]) for e in phs])}
        if self.has_ft:
            dist["backward_ms"] = pct([e[2].elapsed_time(e[3]) for e in phs])
        return dist

    def call_times(self, names, reps=None):
        """GPU time per call of each named library call: a captured HIP graph of the
        call over every rotating copy (segments built first), replayed between events."""
        torch = self.torch
        ops = {"segments": self.seg_build, "shrink": self.shrink, "expand": self.expand,
               "forward_fused": self.forward_fused, "forward_one_launch": self.forward_one_launch,
               "backward": self.backward}
        out = {}
        for st in self.sets:
            self.seg_build(st)
            self.shrink(st)
        torch.cuda.synchronize()
        for name in names:
            fn = ops[name]
            cap = torch.cuda.Stream(device=self.dev)
            cap.wait_stream(torch.cuda.current_stream(self.dev))
            with torch.cuda.stream(cap):
                for st in self.sets:
                    fn(st)
            torch.cuda.current_stream(self.dev).wait_stream(cap)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for st in self.sets:
                    fn(st)
            n_rep = reps or max(3, int(200 / len(self.sets)))
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n_rep):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) * 1e3 / (n_rep * len(self.sets))  # us per call
            del g
        return out

    def pick_forward(self, mode):
        """Set the step's forward: 'split', 'fused', or for 'auto' the one whose
        GPU time per call (captured graphs, outside any timed region) is shorter."""
        if mode != "auto":
            self.fused = mode == "fused"
            return {"mode": mode, "chosen": mode}
        from expand_token_adapter_amd.cost_model import route
        wl = self.wl
        t = self.call_times(["shrink", "expand", "forward_fused"], reps=20)
        split_us = t["shrink"] + t["expand"]
        # lora_forward given v runs the split calls' kernels on decode batches and
        # at r_max <= 16 (except the rank-16 decode kernel): then the two are one
        same = route("forward_fused", wl.ranks, wl.d_in, wl.d_out, T=wl.T, with_v=True) == "forward"
        self.fused = not same and t["forward_fused"] < split_us
        out = {"mode": "auto", "chosen": "fused" if self.fused else "split", "split_us_per_call": split_us,
               "fused_us_per_call": t["forward_fused"]}
        if same:
            out["lora_forward_runs_split_kernels"] = True
        return out

    def check_errors(self):
        errs = [int(st["seg"].err.item()) + (int(st["seg_ft"].err.item()) if self.has_ft else 0) for st in self.sets]
        if any(errs):
            raise RuntimeError(f"device-side data errors reported: {errs}")
        if self.status is not None and int(self.status.item()) != 0:
            raise RuntimeError("the granted preemptible backward reported a yield")


def call_report(wl, times, alg):
    """Per-call GPU time with its algorithmic bytes and HBM fraction."""
    out = {}
    keymap = {"segments": "segments", "shrink": "shrink", "expand": "expand", "forward_fused": "forward_fused",
              "forward_one_launch": "forward_fused", "backward": "backward"}
    for name, us in times.items():
        b = alg[keymap[name]]["bytes"]
        out[name] = {"us_per_call": us, "algorithmic_bytes": b, "GBps": b / (us * 1e-6) / 1e9,
                     "frac_of_hbm_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    return out


def workload_block(idx, steps, warmup, forward="auto"):
    """Step time and per-call GPU times of one more workload (its own rotation)."""
    import torch
    import workloads
    wl = workloads.config(idx, seed=0)
    n_sets = auto_sets(wl)
    b = Bench(wl, n_sets)
    alg = algorithmic(wl)
    choice = b.pick_forward(forward)
    for i in range(n_sets + warmup):
        b.step(b.sets[i % n_sets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        b.step(b.sets[(warmup + i) % n_sets])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    dist = b.distribution(steps, warmup + steps)
    names = ["segments", "shrink", "expand", "forward_fused", "forward_one_launch"] + (["backward"] if b.has_ft else [])
    calls = call_report(wl, b.call_times(names), alg)
    b.check_errors()
    fwd_us = calls["shrink"]["us_per_call"] + calls["expand"]["us_per_call"]
    fwd_b = alg["shrink"]["bytes"] + alg["expand"]["bytes"]
    res = {"rows": wl.T, "ft_rows": wl.ft_count, "d_in": wl.d_in, "d_out": wl.d_out, "adapters": wl.num_adapters,
           "ranks": RANKS_DESC[idx], "forward": choice["chosen"], "forward_choice": choice,
           "ms_per_step": ms, "rows_per_s": wl.T / (ms * 1e-3),
           "step_timing_distribution": dist, "calls": calls,
           "forward_split_us": fwd_us, "forward_split_algorithmic_bytes": fwd_b,
           "forward_split_frac_of_hbm_peak": fwd_b / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "input_sets": n_sets, "rotation_bytes": n_sets * per_set_bytes(wl), "steps": steps, "warmup": warmup}
    del b
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the hot path runs on "
              "one GPU's share of the batch and no multi-GPU sharding is built", file=sys.stderr)
        sys.exit(2)
    if args.adamw and args.graph:
        # the step count (bias corrections) is a launch argument: a captured
        # graph would replay the first step's constants
        print("--adamw runs eagerly only", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.cost_model:
        cost_model_report()
        return
    if args.multi_slice:
        multi_slice_report(args.steps, args.warmup, args.sets or 4)
        return
    if args.kernel_traffic:
        kernel_traffic(*args.kernel_traffic)
        return
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    import torch
    import workloads

    dev = torch.device("cuda:0")
    wl = workloads.config(args.workload, seed=0)
    T, n = wl.T, wl.ft_count
    has_ft = n > 0
    alg = algorithmic(wl)
    n_sets = args.sets or auto_sets(wl)
    b = Bench(wl, n_sets, preemptible=args.preemptible, adamw=args.adamw, overlap=args.overlap)
    choice = b.pick_forward(args.forward)
    fused = b.fused
    sets = b.sets
    r_ft = int(wl.ranks[wl.ft_ids[0]]) if has_ft else None

    graphs = None
    if args.graph:
        warm = torch.cuda.Stream(device=dev)
        warm.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(warm):
            for st in sets:
                b.step(st)
        torch.cuda.current_stream(dev).wait_stream(warm)
        torch.cuda.synchronize()
        graphs = []
        for st in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                b.step(st)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i, ev=None):
        if graphs is not None:
            graphs[i % len(sets)].replay()
        else:
            b.step(sets[i % len(sets)], ev)

    # every rotating set once, then the warm-up steps (no timed step is the
    # first to touch a buffer)
    for i in range(len(sets) + args.warmup):
        run(i)
    torch.cuda.synchronize()

    K = args.steps
    # Events around the expand launch of every EVENT_EVERY-th timed step (an
    # event record drains the stream for a few microseconds, so not every
    # step carries one).
    sampled = [i for i in range(K) if i % EVENT_EVERY == 0]
    evs = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run(args.warmup + i, None if graphs is not None else evs.get(i))
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / K

    # Dominant kernel: average duration of lora_expand_add from events recorded
    # right before and after its launch on the current stream.  Under graph
    # replay the events cannot sit inside the graph, so a separate eager loop
    # of back-to-back expand launches (same rotating buffers) is timed instead.
    if graphs is None:
        kern_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()]))
        kern_how = f"events around the launch in every {EVENT_EVERY}th timed step ({len(evs)} launches)"
    else:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(3):
            b.expand(sets[i % len(sets)])
        e0.record()
        for i in range(K):
            b.expand(sets[i % len(sets)])
        e1.record()
        torch.cuda.synchronize()
        kern_ms = e0.elapsed_time(e1) / K
        kern_how = "events around back-to-back launches"
    # Distribution of step times, outside the timed region above.
    dist = b.distribution(K, args.warmup + K) if graphs is None else None
    # Per-call GPU times from captured graphs (outside the timed region).
    names = ["segments"] + (["forward_fused"] if fused else ["shrink", "expand"]) + \
        (["backward"] if has_ft and not args.preemptible and not args.overlap else [])
    calls = call_report(wl, b.call_times(names), alg) if not args.adamw else None
    # Context: a plain 256 MiB device-to-device copy on the same GPU (read + write bytes).
    cbuf = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(cbuf)
    for _ in range(3):
        cdst.copy_(cbuf)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        cdst.copy_(cbuf)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * cbuf.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cbuf, cdst
    b.check_errors()

    ex = alg["forward_fused"] if fused else alg["expand"]
    kern_name = "lora_forward" if fused else "lora_expand_add (expand_kernel)"
    achieved = ex["bytes"] / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": "LoRA delta tokens/s + achieved HBM GB/s (or MFMA %) vs peak, mixed multi-LoRA batch",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workloads.CONFIG_NAMES[args.workload], "rows": T, "ft_rows": n, "d_in": wl.d_in,
                   "d_out": wl.d_out, "adapters": wl.num_adapters, "ranks": RANKS_DESC[args.workload],
                   "ft_adapter_rank": r_ft, "seed": 0, "input_sets": n_sets,
                   "rotation_bytes": n_sets * per_set_bytes(wl),
                   "launch": "graph" if graphs is not None else "eager",
                   "streams": 2 if args.overlap else 1, "forward": choice["chosen"],
                   "backward": "preemptible" if args.preemptible else "plain"},
        "host_enqueue_ms_per_step": (t_enq - t0) * 1e3 / K,
        "step_algorithmic_GBps": alg["step"]["bytes"] / (ms * 1e-3) / 1e9,
        "step_algorithmic_bytes": alg["step"]["bytes"],
        "step_algorithmic_TFLOPs": alg["step"]["flops"] / (ms * 1e-3) / 1e12,
        "step_timing_distribution": dist,
        "calls": calls,
        "forward_choice": choice,
        "inputs_sha256": wl.manifest(),
        "copy_256MiB_GBps": copy_gbps,
        "roofline": {"bound": "hbm", "kernel": kern_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if args.workload == 3 and not fused else None,
                     "algorithmic_bytes_per_launch": ex["bytes"], "avg_launch_ms": kern_ms, "timing": kern_how,
                     "mfma_frac": ex["flops"] / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }
    if args.adamw and has_ft:
        # per element: master, grad, m, v read (16 B); m, v, master written, the
        # gradient zeroed (16 B); the bf16 weight written (2 B)
        n_el = sum(t[0].numel() for t in sets[0]["opt"])
        opt_bytes = 34 * n_el
        line["config"]["optimizer"] = "adamw"
        if graphs is None:
            opt_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs.values()]))
            line["adamw"] = {"elements": n_el, "algorithmic_bytes_per_launch": opt_bytes, "avg_launch_ms": opt_ms,
                             "achieved_GBps": opt_bytes / (opt_ms * 1e-3) / 1e9}
    del b, sets, graphs
    torch.cuda.empty_cache()
    default_run = (args.workload == 3 and args.forward == "auto" and not (args.graph or args.overlap
                                                                          or args.preemptible or args.adamw))
    if default_run and not args.no_workloads:
        block = {}
        for idx in (2, 4, 5):
            print(f"bench: workload {workloads.CONFIG_NAMES[idx]}", file=sys.stderr, flush=True)
            block[workloads.CONFIG_NAMES[idx]] = workload_block(idx, args.workload_steps, args.warmup,
                                                                args.forward)
        line["workloads"] = block
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_min_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
