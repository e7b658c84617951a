"""Throughput of the full mixed-precision AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zero_shard]

A step is the whole hot path over one set of synthetic inputs already
resident in HBM: zero found_inf, the grad pass (inf/NaN check + binary64 sum
of squares, per-chunk partials), the one-workgroup finalize (norm), the fused
clip + AdamW + bf16 write-back pass (predicated on the device flag), and the
8-byte read of {found_inf, norm} that decides whether the step counter moves.

Default workload: one data-parallel rank's ZeRO-1 flat shard of a 70B model
over 8 ranks -- 8.75e9 elements of fp32 grad / master / exp_avg / exp_avg_sq
plus a bf16 param view (157.5 GB in HBM), grads N(0, 1e-4) so the norm (~9.35)
clips to 1.0, lr 1e-3, wd 0.1.

Prints ONE JSON line.  `value` is G params/s of the full step; HBM figures use
34 algorithmic bytes per element per step (30 for the fused update, 4 for the
grad pass).  The roofline block is for the dominant kernel (the fused update,
30 B/elem), timed with HIP events on the stream it runs on, against the
published 8 TB/s and against the practical ceiling of its read/write mix (the
library's stream probe: the same accesses with no arithmetic, timed the same
way); the shader clock under load comes from a committed counter summary.
cpu_baseline is the CPU oracle (its C routines unchanged, over the host
cores in disjoint slices) on a contiguous 1/8 slice of the same inputs, the
median of 5 steps after 1 warm-up; cpu_baseline_1thread is the same on one
core over a 1/64 slice.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "G params/s and achieved HBM GB/s (% of 8 TB/s) per full AdamW step"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E


def gradpass_bytes(w) -> int:
    """The grad pass reads each stored grad once, at its width."""
    return 2 if getattr(w, "grad_dtype", "fp32") == "bf16" else 4


def update_bytes(w) -> int:
    """Algorithmic bytes per element of the fused update for a workload's
    storage: the grad read, the master read and written, each moment read
    and written, all at their widths, and the 16-bit param written (none for
    fp32 params)."""
    mom = 2 if w.state_dtype in ("bf16", "fp16") else 4
    mst = 2 if getattr(w, "master_dtype", "fp32") == "fp16" else 4
    par = 0 if w.param_dtype == "fp32" else 2
    return gradpass_bytes(w) + 2 * mst + 4 * mom + par


def pmc_summary_path(workload_name):
    """The committed counter summary of a flat-shard workload: the default
    storage has pmc_hbm_traffic_zero_shard_70b_over_8.txt, and each other
    storage the same name with its tag (for example
    ..._bf16_grads_fp16_master.txt)."""
    return os.path.join(ROOT, "profiles", "pmc_hbm_traffic_" + workload_name.replace("zero1_shard", "zero_shard", 1)
                        + ".txt")
# the sources of the AdamW-path kernels (the counters in profiles/ name this digest)
KERNEL_SOURCES = ("mixed_precision_optimizer_amd/csrc/hpo_kernels.hip", "mixed_precision_optimizer_amd/csrc/hpo_impl.h",
                  "mixed_precision_optimizer_amd/csrc/hpo_device.h")


def kernel_digest():
    """sha256[:16] over the device sources; the counter summary records the
    digest of the kernels it measured."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name, numel):
    """HBM bytes per launch of the update kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary was taken on
    another workload or on kernels that have changed since."""
    if not workload_name.startswith("zero1_shard_70b_over_8") or numel != 8_750_000_000:
        return None
    path = pmc_summary_path(workload_name)
    if not os.path.exists(path):
        return None
    digest, traffic = None, None
    with open(path) as f:
        for line in f:
            if "kernel source digest" in line:
                digest = line.rsplit(":", 1)[1].strip()
            if line.startswith("traffic_bytes_per_launch k_adam"):
                traffic = float(line.split()[-1])
    return traffic if digest == kernel_digest() else None


CLOCK_SUMMARY = os.path.join(ROOT, "profiles", "pmc_clock_zero_shard_70b_over_8.txt")


def measured_clock(workload_name, numel):
    """Shader clock (GHz) under the update kernel and the grad pass from the
    committed rocprofv3 GRBM_GUI_ACTIVE summary of the default shard, or None
    when it was taken on kernels that have changed since."""
    if workload_name != "zero1_shard_70b_over_8" or numel != 8_750_000_000 or not os.path.exists(CLOCK_SUMMARY):
        return None
    digest, clk = None, {}
    with open(CLOCK_SUMMARY) as f:
        for line in f:
            if "kernel source digest" in line:
                digest = line.rsplit(":", 1)[1].strip()
            if line.startswith("clock_GHz "):
                _, kern, val = line.split()
                clk[kern] = float(val)
    return clk if digest == kernel_digest() and clk else None


MUON_PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_hbm_traffic_llama8b_adamw_muon_chain.txt")
MUON_SOURCES = ("mixed_precision_optimizer_amd/csrc/hpo_muon.hip", "mixed_precision_optimizer_amd/csrc/hpo_muon_impl.h")


def muon_kernel_digest():
    """sha256[:16] over the Muon device sources (named by the Muon counter summaries)."""
    import hashlib
    h = hashlib.sha256()
    for f in MUON_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_muon_traffic():
    """(measured, algorithmic) HBM bytes per launch of the X' = aX + BX GEMM on
    the Llama-8B chain from the committed rocprofv3 summary, or None when the
    Muon kernels have changed since it was taken."""
    if not os.path.exists(MUON_PMC_SUMMARY):
        return None
    digest, meas, alg = None, None, None
    with open(MUON_PMC_SUMMARY) as f:
        for line in f:
            if "kernel source digest" in line:
                digest = line.rsplit(":", 1)[1].strip()
            if line.startswith("traffic_bytes_per_launch k_ns_gemm_step"):
                meas = float(line.split()[-1])
            if line.startswith("algorithmic_bytes_per_launch k_ns_gemm_step"):
                alg = float(line.split()[-1])
    if digest != muon_kernel_digest() or meas is None or alg is None:
        return None
    return meas, alg


def host_cpu_model() -> str:
    """The host CPU's model name (lscpu's, else /proc/cpuinfo's), for the CPU baselines."""
    name = host_cpu().get("model_name")
    if name:
        return name
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpu() -> dict:
    """lscpu's model name, sockets, physical cores and logical CPUs, and the
    CPUs this process may run on."""
    import subprocess
    out = {}
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        txt = ""
    fields = {}
    for line in txt.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if "Model name" in fields:
        out["model_name"] = fields["Model name"]
    # a virtual machine may show a generic model name: the family / model /
    # stepping numbers and the hypervisor still identify the part
    for key, name in (("CPU family", "cpu_family"), ("Model", "model"), ("Stepping", "stepping"),
                      ("Hypervisor vendor", "hypervisor"), ("L3 cache", "l3_cache")):
        if key in fields:
            out[name] = fields[key]
    try:
        sockets = int(fields["Socket(s)"])
        cores = int(fields["Core(s) per socket"])
        out["sockets"] = sockets
        out["physical_cores"] = sockets * cores
        out["threads_per_core"] = int(fields.get("Thread(s) per core", "1"))
    except (KeyError, ValueError):
        pass
    if "CPU(s)" in fields:
        out["logical_cpus"] = fields["CPU(s)"]
    try:
        out["cpus_allowed"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        out["cpus_allowed"] = os.cpu_count()
    return out


def device_info(torch) -> dict:
    """Name, architecture, CU count and memory of device 0, and the HIP and
    torch versions the run used."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gb": round(p.total_memory / 1e9, 1), "hip": torch.version.hip, "torch": torch.__version__}


def spread(ms) -> dict:
    """Median, minimum and maximum of per-step kernel times (ms)."""
    return {"ms_median": round(statistics.median(ms), 4), "ms_min": round(min(ms), 4), "ms_max": round(max(ms), 4)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zero_shard",
                    choices=["zero_shard", "zero_shard_ranges", "llama8b", "ragged", "two_matrices",
                             "llama8b_muon"])
    ap.add_argument("--muon-workspace", type=int, default=0,
                    help="Muon set workspace cap in bytes (0: the library default)")
    ap.add_argument("--numel", type=int, default=None, help="override the flat shard's size")
    ap.add_argument("--state-dtype", default="fp32", choices=["fp32", "bf16"],
                    help="exp_avg / exp_avg_sq storage of the flat shard")
    ap.add_argument("--param-dtype", default="bf16", choices=["bf16", "fp16"],
                    help="model-param dtype of the flat shard")
    ap.add_argument("--grad-dtype", default="fp32", choices=["fp32", "bf16"],
                    help="main grad storage of the flat shard")
    ap.add_argument("--master-dtype", default="fp32", choices=["fp32", "fp16"],
                    help="master storage of the flat shard (fp16 needs bf16 params)")
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="elements of the workload the CPU oracle steps on all cores (-1: a contiguous 1/8 "
                         "of the workload; 0: skip); the one-core baseline takes 1/8 of that")
    ap.add_argument("--cpu-steps", type=int, default=5, help="timed oracle steps (after one warm-up step)")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="threads of the all-core oracle baseline (the host share of one GPU; capped to the "
                         "CPUs this process may use)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="N",
                    help="only run a plain device copy of N fp32 elements (known bytes: 4N read, 4N "
                         "written) five times; used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def calibrate_copy(n):
    import torch
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = min(a.elapsed_time(b) for a, b in evs)
    print(json.dumps({"calibration": "device copy", "elements": n, "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "ms": round(ms, 4), "GBps": round(8 * n / ms / 1e6, 1)}), flush=True)


def workload(args):
    from mixed_precision_optimizer_amd import inputs
    if args.workload == "zero_shard":
        return inputs.zero_shard(args.numel or 8_750_000_000, state_dtype=args.state_dtype,
                                 param_dtype=args.param_dtype, grad_dtype=args.grad_dtype,
                                 master_dtype=args.master_dtype)
    if args.workload == "zero_shard_ranges":
        return inputs.zero_shard_ranges()
    if args.workload == "llama8b":
        return inputs.llama8b()
    if args.workload == "ragged":
        w = inputs.ragged()
        w.inf_step = None
        return w
    return inputs.two_matrices()


def make_set(bufs):
    from mixed_precision_optimizer_amd import hpo
    w = bufs.workload
    if w.flat and w.n_tensors > 1:
        return hpo.hpo_set_create_flat_ranges(bufs.param, bufs.master, bufs.grad, bufs.exp_avg, bufs.exp_avg_sq,
                                              bufs.offs, [w.group_of(i) for i in range(w.n_tensors)])
    if w.flat:
        return hpo.hpo_set_create_flat(bufs.param, bufs.master, bufs.grad, bufs.exp_avg, bufs.exp_avg_sq)
    ps, ms, gs, m1, m2 = bufs.lists()
    return hpo.hpo_set_create_list(ps, ms, gs, m1, m2, [w.group_of(i) for i in range(w.n_tensors)])


def cpu_sample(bufs, n_sample):
    """Host copy of the first n_sample elements of the initial state and the
    step-1 grads (taken before any GPU step)."""
    import numpy as np
    import torch
    n = min(n_sample, bufs.total)
    host = lambda t: t[:n].detach().cpu().numpy().copy()
    bits = lambda t: t[:n].view(torch.int16).cpu().numpy().view(np.uint16).copy()
    get = lambda t: host(t) if t.dtype == torch.float32 else bits(t)
    return get(bufs.master), get(bufs.exp_avg), get(bufs.exp_avg_sq), bits(bufs.param), get(bufs.grad)


def _sample_note(n, w):
    frac = w.numel / n if n else 0
    return (f"a contiguous 1/{frac:.0f} slice ({n} elements, the first of the set) of the same workload"
            if abs(frac - round(frac)) < 1e-9 else f"the first {n} elements of the same workload")


def cpu_baseline(sample, w, steps):
    """The oracle's full step (check, norm, clip, update, RNE) on the sample,
    on one core: one warm-up step, then the median of `steps` steps."""
    import oracle
    theta, m, v, p, G = sample
    n = theta.size
    T = oracle.OTensor(theta, m, v, p, 0, w.param_dtype == "fp16", w.master_dtype == "fp16", False)
    O = oracle.OracleOptimizer([T], oracle.Hyper(w.beta1, w.beta2, w.eps, w.mode), w.groups(),
                               max_norm=w.max_norm)
    times = []
    for k in range(steps + 1):
        t0 = time.perf_counter()
        O.step([G], inv_scale=w.inv_scale())
        if k > 0:
            times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    bpe = update_bytes(w) + gradpass_bytes(w)
    return {"value": round(n / dt / 1e9, 4), "unit": "G params/s", "cores": 1, "kind": "oracle",
            "sample": f"{_sample_note(n, w)}: initial master/m/v, param and step-1 grads as stored; the full step "
                      f"(inf check, binary64 norm, clip, AdamW, RNE stores) in single-threaded C; median of {steps} "
                      f"steps after 1 warm-up; {bpe * n / dt / 1e9:.2f} GB/s at {bpe} B/elem",
            "ms_per_step": round(dt * 1e3, 2), "ms_min": round(min(times) * 1e3, 2),
            "ms_max": round(max(times) * 1e3, 2), "cpu_model": host_cpu_model()}


def cpu_baseline_threads(sample, w, steps, threads):
    """The same oracle routines on the same sample, over `threads` disjoint
    slices at once (ctypes releases the GIL in the oracle's C calls): the
    inf check and binary64 sums per slice, their sum in slice order, the
    clip decision, then each slice's update.  The oracle's code is unchanged;
    only the work is split.  One warm-up step, then the median of `steps`."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    theta, m, v, p, G = sample
    n = theta.size
    cuts = [n * k // threads for k in range(threads + 1)]
    parts = [(oracle.OTensor(theta[a:b], m[a:b], v[a:b], p[a:b], 0, w.param_dtype == "fp16",
                             w.master_dtype == "fp16", False), oracle.grad_f32(G[a:b]))
             for a, b in zip(cuts[:-1], cuts[1:])]
    hyper = oracle.Hyper(w.beta1, w.beta2, w.eps, w.mode)
    inv32 = float(np.float32(w.inv_scale()))
    times, t = [], 0
    with ThreadPoolExecutor(threads) as pool:
        for k in range(steps + 1):
            t0 = time.perf_counter()
            found = any(pool.map(lambda tg: oracle.any_nonfinite(tg[1]), parts))
            if not found:
                n2 = 0.0
                for s2 in pool.map(lambda tg: oracle.sumsq(tg[1], inv32), parts):
                    n2 = n2 + s2
                _, norm32 = oracle.norm_from_sumsq(n2)
                do_clip, C, c64 = oracle.clip_coeff(w.max_norm, norm32)
                t += 1
                list(pool.map(lambda tg: oracle.apply_update([tg[0]], [tg[1]], hyper, w.groups(), t, inv32,
                                                             do_clip, C, c64), parts))
            if k > 0:
                times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    bpe = update_bytes(w) + gradpass_bytes(w)
    hc = host_cpu()
    return {"value": round(n / dt / 1e9, 4), "unit": "G params/s", "cores": threads, "kind": "oracle",
            "sample": f"{_sample_note(n, w)}: the oracle's inf check, binary64 sums and update over {threads} "
                      f"slices in {threads} threads (its C routines unchanged); median of {steps} steps after 1 "
                      f"warm-up; {bpe * n / dt / 1e9:.2f} GB/s at {bpe} B/elem",
            "ms_per_step": round(dt * 1e3, 2), "ms_min": round(min(times) * 1e3, 2),
            "ms_max": round(max(times) * 1e3, 2), "cpu_model": host_cpu_model(),
            "host": {k: hc[k] for k in ("physical_cores", "sockets", "threads_per_core", "logical_cpus",
                                        "cpus_allowed", "cpu_family", "model", "stepping", "hypervisor",
                                        "l3_cache") if k in hc}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"bench.py runs on one GPU only (got --gpus {args.gpus}); "
                                   "the multi-GPU path (scalar all-reduces + bf16 param all-gather) is not built"}))
        sys.exit(2)
    import torch

    from mixed_precision_optimizer_amd import hpo, inputs
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    dev = torch.device("cuda", 0)
    hpo.load()
    if args.workload == "llama8b_muon":
        main_muon(args, dev)
        return
    w = workload(args)
    N = w.numel
    log(f"workload {w.name}: {N} elements, {w.n_tensors} tensors; allocating {N * 18 / 1e9:.1f} GB")
    bufs = inputs.allocate(w, dev)
    inputs.fill_grads_(bufs, 1)
    torch.cuda.synchronize()
    n_cpu = N // 8 if args.cpu_sample < 0 else args.cpu_sample
    sample = cpu_sample(bufs, n_cpu) if n_cpu > 0 else None
    hset = make_set(bufs)
    info = hset.info()
    log(f"set: chunk {info.chunk_elems} elements, {info.n_chunks} chunks, {info.device_bytes} B of tables")

    cfg = hpo.make_cfg(w.beta1, w.beta2, w.eps, w.mode)
    groups, n_groups = hpo.make_groups(w.groups())
    inv = w.inv_scale()
    buf = torch.zeros(2, dtype=torch.int32, device=dev)
    found, norm = buf[0:1], buf[1:2].view(torch.float32)
    host = torch.zeros(2, dtype=torch.int32, pin_memory=True)
    stream = torch.cuda.current_stream()
    t_applied = 0

    def step(evs=None):
        nonlocal t_applied
        if evs:
            evs[0].record(stream)
        hpo.hpo_grad_global_norm(hset, inv, norm, found, stream=stream)
        if evs:
            evs[1].record(stream)
        hpo.hpo_adamw_step(hset, cfg, groups, n_groups, t_applied + 1, inv, w.max_norm, norm, found, stream)
        if evs:
            evs[2].record(stream)
        host.copy_(buf, non_blocking=True)
        buf.zero_()   # found_inf starts the next step at 0; enqueued here, it runs while the host waits
        stream.synchronize()
        if int(host[0]) == 0:
            t_applied += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the practical ceiling of the update's read/write mix: the library's probe
    # with the same accesses and no arithmetic, on the same buffers (it leaves
    # the state as it is), timed with HIP events on the same stream
    probe_ms = None
    try:
        hpo.hpo_stream_probe(hset, stream)
    except hpo.HpoError:
        log("stream probe: not applicable to this storage")
    else:
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in pev:
            a.record(stream)
            hpo.hpo_stream_probe(hset, stream)
            b.record(stream)
        torch.cuda.synchronize()
        probe_ms = statistics.median(a.elapsed_time(b) for a, b in pev)
    # the timed steps carry no instrumentation; the kernel times come from a
    # second, shorter run of the same steps with HIP events around the calls
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(min(args.steps, 50))]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    norm_v = float(host[1:2].view(torch.float32)[0])
    gradpass_ms = [e[0].elapsed_time(e[1]) for e in evs]
    update_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    upd = statistics.mean(update_ms)
    gp = statistics.mean(gradpass_ms)
    ub = update_bytes(w)
    upd_gbps = ub * N / (upd * 1e-3) / 1e9
    gp_gbps = gradpass_bytes(w) * N / (gp * 1e-3) / 1e9
    step_gbps = (ub + gradpass_bytes(w)) * N / (ms_step * 1e-3) / 1e9
    traffic = measured_traffic(w.name, N)
    traffic_gb = None if traffic is None else round(traffic / 1e9, 3)
    ceil_gbps = None if probe_ms is None else ub * N / (probe_ms * 1e-3) / 1e9
    clock = measured_clock(w.name, N)
    log(f"norm {norm_v:.6g}, applied steps {t_applied}; step {ms_step:.3f} ms, update {upd:.3f} ms "
        f"({upd_gbps:.0f} GB/s), grad pass {gp:.3f} ms ({gp_gbps:.0f} GB/s)")
    out = {
        "metric": METRIC,
        "value": round(N / (ms_step * 1e-3) / 1e9, 3),
        "unit": "G params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "numel": N, "n_tensors": w.n_tensors, "param_dtype": w.param_dtype,
                   "state": f"{w.master_dtype} master, {w.grad_dtype} main_grad, {w.state_dtype} exp_avg/exp_avg_sq",
                   "max_norm": w.max_norm,
                   "lr": w.lr, "weight_decay": w.weight_decay, "loss_scale": w.loss_scale,
                   "parallelism": "one GPU (one data-parallel rank's shard)"},
        "hbm_full_step": {"GBps": round(step_gbps, 1), "frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
                          "bytes_per_elem": ub + gradpass_bytes(w)},
        "kernels": {"adam_update": {"ms": round(upd, 4), "GBps": round(upd_gbps, 1), "bytes_per_elem": ub,
                                    **spread(update_ms)},
                    "grad_pass+finalize": {"ms": round(gp, 4), "GBps": round(gp_gbps, 1),
                                           "bytes_per_elem": gradpass_bytes(w), **spread(gradpass_ms)}},
        "roofline": {"bound": "hbm", "achieved": round(upd_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(upd_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic_gb,
                     "traffic_unit": "GB per launch of the update kernel (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1, "
                                     "scales from a device copy of known size); algorithmic: "
                                     f"{ub * N / 1e9:.1f} GB",
                     "ceiling": None if ceil_gbps is None else round(ceil_gbps, 1),
                     "frac_of_ceiling": None if ceil_gbps is None else round(upd_gbps / ceil_gbps, 4),
                     "ceiling_unit": "GB/s of the library's stream probe: the update's accesses (same chunks, launch "
                                     "shape, streaming loads/stores) with no arithmetic, same buffers, HIP events, "
                                     "median of 5",
                     "clock_GHz": clock,
                     "clock_unit": "shader clock under each kernel, rocprofv3 GRBM_GUI_ACTIVE per XCD over the "
                                   "dispatch time (committed summary of the same kernels, else null)",
                     "target": {"frac_of_peak_full_step": 0.80,
                                "met": bool(step_gbps / PEAK_HBM_GBPS >= 0.80)}},
        "device": device_info(torch),
    }
    # the same step with the scaler, skip decision and step counter on the
    # device: no host round trip per step (hpo_step_device); constant scale 1
    from mixed_precision_optimizer_amd import DeviceAdamW
    dopt = DeviceAdamW(hset, w.groups(), beta1=w.beta1, beta2=w.beta2, eps=w.eps, mode=w.mode,
                       max_norm=w.max_norm, loss_scale=1.0 if w.loss_scale is None else w.loss_scale,
                       dynamic=False, applied_steps=t_applied, stream=stream)
    for _ in range(args.warmup):
        dopt.step()
    dopt.sync()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dopt.step()
    torch.cuda.synchronize()
    dev_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dst = dopt.sync()
    log(f"device-resident step: {dev_ms:.3f} ms ({dst.applied_steps} applied)")
    out["device_resident_step"] = {"ms_per_step": round(dev_ms, 4), "value": round(N / (dev_ms * 1e-3) / 1e9, 3),
                                   "unit": "G params/s",
                                   "note": "hpo_step_device: no per-step host sync; steps re-read the state every 32"}
    # the same step captured in a HIP graph and replayed (DeviceAdamW.graph): no launch cost per step;
    # the graph covers HPO_MAX_WINDOW values of t, so it is captured again (after a read of the state)
    # every HPO_MAX_WINDOW replays, inside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    done = 0
    while done < args.steps:
        graph = dopt.graph()
        k = min(hpo.HPO_MAX_WINDOW, args.steps - done)
        for _ in range(k):
            graph.replay()
        done += k
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    gst = dopt.sync()
    if gst.error or gst.applied_steps != dst.applied_steps + args.steps:
        raise RuntimeError(f"graph replays: applied {gst.applied_steps - dst.applied_steps} of {args.steps}, "
                           f"error {gst.error}")
    log(f"graph-replayed device step: {graph_ms:.3f} ms")
    out["graph_step"] = {"ms_per_step": round(graph_ms, 4), "value": round(N / (graph_ms * 1e-3) / 1e9, 3),
                         "unit": "G params/s",
                         "note": f"the device-resident step captured once per {hpo.HPO_MAX_WINDOW} steps in a "
                                 "HIP graph (torch.cuda.CUDAGraph) and replayed; captures and state reads timed"}
    hset.close()
    if sample is not None:
        threads = max(1, min(args.cpu_threads, host_cpu().get("cpus_allowed") or 1))
        log(f"cpu baseline on {sample[0].size} elements, {threads} threads")
        out["cpu_baseline"] = cpu_baseline_threads(sample, w, args.cpu_steps, threads)
        one = tuple(a[:max(1, a.size // 8)].copy() for a in sample)
        del sample
        log(f"cpu baseline on {one[0].size} elements, 1 thread")
        out["cpu_baseline_1thread"] = cpu_baseline(one, w, args.cpu_steps)
    print(json.dumps(out), flush=True)


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MUON_METRIC = "G params/s per full chained AdamW + Muon step (bf16 MFMA Newton-Schulz)"


def muon_cpu_baseline(matrices, steps=1):
    """The Muon oracle (numpy, bf16 reading with exact sums; BLAS-threaded)
    on one matrix of the workload: its momentum, NS and update."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import oracle.muon as mu
    from mixed_precision_optimizer_amd import inputs
    oracle.lib()
    name, (r, c), std = next(m for m in matrices if m[0].endswith(".k"))
    W = inputs.seeded_matrix((r, c), 5, 1.0)
    G = inputs.seeded_matrix((r, c), 6, std)
    T = mu.OMatrix.fresh(W)
    times = []
    for k in range(steps + 1):
        t0 = time.perf_counter()
        mu.muon_matrix_step(T, G, mu.MuonCfg(), 1e-3, 0.1, 1.0, False, 1.0, "bf16")
        if k > 0:
            times.append(time.perf_counter() - t0)
    ms = 1e3 * statistics.median(times)
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    return {"value": round(r * c / (ms * 1e-3) / 1e9, 5), "unit": "G params/s", "cores": threads, "kind": "oracle",
            "sample": f"one {r}x{c} Muon matrix ({name}) of the same workload: momentum, 5-step bf16-reading NS "
                      f"(numpy binary64 matmuls over bf16 values, {threads} BLAS threads), decayed scaled update, "
                      f"bf16 write-back; median of {steps} after 1 warm-up", "ms_per_step": round(ms, 2),
            "cpu_model": host_cpu_model()}


def main_muon(args, dev):
    """Llama-8B-shaped chained step: AdamW on the embedding, output head and
    1-D gains (1.05e9 params), Muon on the 224 hidden matrices (6.98e9),
    device-resident (hpo_step_device_chain), constant loss scale 1, clip 1.0."""
    import torch

    from mixed_precision_optimizer_amd import hpo, inputs
    wa, mats = inputs.llama8b_chain()
    n_adam = wa.numel
    n_muon = sum(r * c for _, (r, c), _ in mats)
    N = n_adam + n_muon
    log(f"chain: AdamW {n_adam} params in {wa.n_tensors} tensors, Muon {n_muon} in {len(mats)} matrices; "
        f"allocating {(18 * n_adam + 14 * n_muon) / 1e9:.1f} GB")
    bufs = inputs.allocate(wa, dev)
    inputs.fill_grads_(bufs, 1)
    aset = make_set(bufs)
    mb = inputs.allocate_muon(mats, dev)
    mset = hpo.hpo_muon_set_create(mb.views(mb.param), mb.views(mb.master), mb.views(mb.grad),
                                   mb.views(mb.momentum), workspace_bytes=args.muon_workspace)
    torch.cuda.synchronize()
    log(f"Muon set: {mset.info().device_bytes / 1e9:.2f} GB of tables and NS workspace")
    acfg = hpo.make_cfg(wa.beta1, wa.beta2, wa.eps, wa.mode)
    mcfg = hpo.make_muon_cfg()
    groups = wa.groups()
    mgroups = [(wa.lr, wa.weight_decay)]
    scfg = hpo.make_scaler_cfg(dynamic=False)
    stream = torch.cuda.current_stream()
    d_state = hpo.new_scaler_state(dev)
    hpo.hpo_scaler_state_init(d_state, 1.0, 1, 0, stream)
    st = {"t_first": 1, "window": 0}

    def step():
        if st["window"] == hpo.HPO_MAX_WINDOW:
            s = hpo.read_scaler_state(d_state)
            if s.error:
                raise RuntimeError("device step window overrun")
            st["t_first"], st["window"] = s.applied_steps + 1, 0
        st["window"] += 1
        hpo.hpo_step_device_chain(aset, acfg, groups, mset, mcfg, mgroups, wa.max_norm, scfg, d_state,
                                  st["t_first"], st["window"], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    s = hpo.read_scaler_state(d_state)
    if s.error or s.applied_steps != args.warmup + args.steps:
        raise RuntimeError(f"unexpected device state: applied {s.applied_steps}, error {s.error}")
    log(f"chained step {wall_ms:.2f} ms (events {ev_ms:.2f} ms), norm {s.grad_norm:.5g}, applied {s.applied_steps}")
    # live per-launch timing of the Muon kernels over a few more steps
    hpo.hpo_muon_profile_enable(mset, True)
    n_prof = max(2, min(5, args.steps))
    torch.cuda.synchronize()
    for _ in range(n_prof):
        step()
    prof = hpo.hpo_muon_profile_read(mset)
    hpo.hpo_muon_profile_enable(mset, False)
    kernels = {}
    for k, v in prof.items():
        ms = v["ms"] / n_prof
        ent = {"ms_per_step": round(ms, 4), "launches_per_step": v["launches"] // n_prof}
        if v["flops"]:
            ent["TFLOPs"] = round(v["flops"] / n_prof / (ms * 1e-3) / 1e12, 1)
        if v["bytes"]:
            ent["GBps"] = round(v["bytes"] / n_prof / (ms * 1e-3) / 1e9, 1)
        kernels[k] = ent
    gemm_ms = sum(prof[k]["ms"] for k in ("gram", "poly", "step", "update")) / n_prof
    gemm_fl = sum(prof[k]["flops"] for k in ("gram", "poly", "step", "update")) / n_prof
    dom = max(("gram", "poly", "step", "update"), key=lambda k: prof[k]["ms"])
    dom_ms = prof[dom]["ms"] / max(1, prof[dom]["launches"])
    dom_fl = prof[dom]["flops"] / max(1, prof[dom]["launches"])
    achieved = dom_fl / (dom_ms * 1e-3) / 1e12
    log(f"NS GEMMs {gemm_ms:.2f} ms per step = {gemm_fl / (gemm_ms * 1e-3) / 1e12:.1f} TFLOP/s; "
        f"dominant {dom}: {dom_ms:.3f} ms per launch, {achieved:.1f} TFLOP/s")
    out = {
        "metric": MUON_METRIC,
        "value": round(N / (wall_ms * 1e-3) / 1e9, 3),
        "unit": "G params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (NS matmuls), f32 (momentum, masters, AdamW)",
        "data": "synthetic",
        "config": {"workload": "llama8b_chain_adamw_muon", "params": N, "adamw_params": n_adam,
                   "muon_params": n_muon, "muon_matrices": len(mats), "ns_steps": 5, "max_norm": wa.max_norm,
                   "lr": wa.lr, "weight_decay": wa.weight_decay, "loss_scale": 1.0,
                   "parallelism": "one GPU (whole model, no data-parallel sharding)"},
        "kernels": kernels,
        "ns_gemms": {"ms_per_step": round(gemm_ms, 3), "TFLOPs": round(gemm_fl / (gemm_ms * 1e-3) / 1e12, 1),
                     "flops_per_step": gemm_fl},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": f"k_ns_gemm ({dom}), algorithmic flops per launch {dom_fl:.4g}"},
        "device": device_info(torch),
    }
    tr = measured_muon_traffic() if dom == "step" else None
    if tr is not None:
        out["roofline"]["traffic"] = round(tr[0] / 1e9, 3)
        out["roofline"]["traffic_unit"] = (
            "GB per launch of the step GEMM (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1, scales from a device copy "
            f"of known size); algorithmic {tr[1] / 1e9:.3f} GB: B and X read once, X' and X'^T written")
    aset.close()
    mset.close()
    if args.cpu_sample != 0:
        out["cpu_baseline"] = muon_cpu_baseline(mats, args.cpu_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
