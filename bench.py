#!/usr/bin/env python3
"""Benchmark of the fused partition reduce-scatter + Adam step on one GPU.

Default workload: GPT-2-small parameter list (124,439,808 elements), 8
data-parallel replicas of bf16 gradients resident in HBM, reduce_bucket_size
5e8, fp32 partitions of 1/8.  One step is one rank's whole share of the hot
path: the fused kernel reads the 8 replica windows of partition k, reduces
them (pre-divide by 8, rank order), and applies Adam to partition k's fp32
master / m / v with a bf16 param writeback.  Steps rotate k = 0..7 over eight
independent state sets, so consecutive launches never reuse cached data.

Prints ONE JSON line.  ``value`` is achieved HBM GB/s: algorithmic bytes of a
step (N*s + 26 bytes per partition element) divided by the measured time per
step, inputs already resident in HBM.  ``roofline`` prices the dominant
kernel's average launch duration (HIP events on the launch stream) against
MI355X's 8 TB/s; ``cpu_baseline`` times the CPU oracle on one rank's
partition.  Other workloads (``--workload``) are for characterisation.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for fused partition reduce-scatter+Adam step"
PEAK_GBS = 8000.0
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def traffic_for(kernel_key):
    """HBM bytes per launch measured by rocprofv3 counters for this exact
    kernel source, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    from zero_partition_aware_amd.build import source_hash
    entry = t.get(kernel_key)
    if not entry or entry.get("kernel_src_sha") != source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


class Timer:
    """Counts launches per kernel label; when a step launches more than one
    kind of kernel it also brackets every launch with HIP events (on the
    launch stream, torch's current stream) to split the time per kernel."""

    def __init__(self, torch, per_launch):
        self.torch = torch
        self.per_launch = per_launch
        self.ev = []
        self.count = {}

    def launch(self, fn, label):
        self.count[label] = self.count.get(label, 0) + 1
        if not self.per_launch:
            fn()
            return
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.ev.append((a, b, label))

    def per_label_ms(self):
        out = {}
        for a, b, label in self.ev:
            out.setdefault(label, []).append(a.elapsed_time(b))
        return out


# --------------------------------------------------------------- workloads

def setup_gpt2(torch, zr, workloads):
    name = "gpt2-small"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R = w.groups[0][0]
    reps = [workloads.device_normal(workloads.seed_for(name, r), T, w.grad_sigma, "cuda", "bf16")
            for r in range(R)]
    states = []
    for k in range(R):
        master = workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                         w.master_sigma, "cuda")
        states.append(dict(master=master, m=torch.zeros_like(master),
                           v=torch.zeros_like(master),
                           pbf16=torch.empty(P, dtype=torch.bfloat16, device="cuda")))
    bytes_per_step = (R * 2 + 26) * P

    def step(i, timer):
        k = i % R
        s = states[k]
        timer.launch(lambda: zr.zr_reduce_scatter_adam(
            plan, 0, -1, k, reps, s["master"], s["m"], s["v"], s["pbf16"], None,
            step=i // R + 1, **HP), "fused")

    cfg = {"workload": name, "params": len(w.numels), "total_elems": T,
           "replicas": R, "grad_dtype": "bf16", "reduce_bucket_size": w.reduce_bucket_size,
           "partition_elems": P, "divisor": D, "share": "one rank's partition per step, k = step mod 8",
           "bytes_per_step": bytes_per_step}
    launch_bytes = {"fused": bytes_per_step}

    def cpu_leg():
        return cpu_oracle_fused(torch, workloads, plan, name, w, reps, states[0]["master"], P, R)

    return step, bytes_per_step, P, cfg, launch_bytes, "fused", cpu_leg


def setup_llama(torch, zr, workloads, ipg=False):
    name = "llama3-8b"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R = w.groups[0][0]
    k = 0
    lo = k * P
    mgs = [workloads.device_normal(workloads.seed_for(name, r, 9), P, 2 * w.grad_sigma, "cuda")
           for r in range(R)]
    cfg = {"workload": name + ("-ipg" if ipg else ""), "params": len(w.numels),
           "total_elems": T, "replicas": R, "reduce_bucket_size": w.reduce_bucket_size,
           "partition_elems": P, "divisor": D, "share": "rank 0's partition window"}
    if ipg:
        offs = [zr.zr_plan_param_offset(plan, p) for p in range(len(w.numels))]
        pids = [p for p in range(len(w.numels)) if offs[p] < lo + P and offs[p] + w.numels[p] > lo]
        n = sum(w.numels[p] for p in pids)
        bufs = [workloads.device_normal(workloads.seed_for(name, r, 0), n, w.grad_sigma,
                                        "cuda", "bf16") for r in range(R)]
        views = []
        for b in bufs:
            vs, a = [], 0
            for p in pids:
                vs.append(b[a:a + w.numels[p]])
                a += w.numels[p]
            views.append(vs)
        bytes_per_step = w.micro_batches * R * 10 * P

        def step(i, timer):
            for mu in range(w.micro_batches):
                for r in range(R):
                    timer.launch(lambda: zr.zr_ipg_accumulate(plan, pids, views[r], mgs[r],
                                                              window_base=lo), "ipg")

        cfg.update(micro_batches=w.micro_batches, grad_dtype="bf16 -> fp32 main_grad",
                   bytes_per_step=bytes_per_step)
        return step, bytes_per_step, P * w.micro_batches * R, cfg, \
            {"ipg": 10 * P}, "ipg", None

    master = workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                      w.master_sigma, "cuda")
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    pbf16 = torch.empty(P, dtype=torch.bfloat16, device="cuda")
    reps = [(x, lo) for x in mgs]
    bytes_per_step = (R * 4 + 26) * P

    def step(i, timer):
        timer.launch(lambda: zr.zr_reduce_scatter_adam(
            plan, 0, -1, k, reps, master, m, v, pbf16, None, step=i + 1, **HP), "fused")

    cfg.update(grad_dtype="fp32 main_grad", bytes_per_step=bytes_per_step)
    return step, bytes_per_step, P, cfg, {"fused": bytes_per_step}, "fused", None


def setup_moe(torch, zr, workloads):
    name = "moe-16l"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    groups = []
    total_bytes = 0
    for g, (R, sp) in enumerate(w.groups):
        T, L, P, D = zr.zr_plan_group_info(plan, g)
        reps = [workloads.device_normal(workloads.seed_for(name, r + 100 * g), T, w.grad_sigma,
                                        "cuda") for r in range(R)]
        states = []
        for k in range(R):
            master = workloads.device_normal(workloads.seed_for(name, 10 * g + k, master=True),
                                             P, w.master_sigma, "cuda")
            states.append(dict(master=master, m=torch.zeros_like(master),
                               v=torch.zeros_like(master),
                               pbf16=torch.empty(P, dtype=torch.bfloat16, device="cuda")))
        groups.append(dict(R=R, P=P, D=D, reps=reps, states=states, bytes=(R * 4 + 26) * P))
        total_bytes += (R * 4 + 26) * P

    def step(i, timer):
        for g, gr in enumerate(groups):
            k = i % gr["R"]
            s = gr["states"][k]
            timer.launch(lambda: zr.zr_reduce_scatter_adam(
                plan, g, -1, k, gr["reps"], s["master"], s["m"], s["v"], s["pbf16"], None,
                step=i // gr["R"] + 1, **HP), f"fused_g{g}")

    cfg = {"workload": name, "params": len(w.numels), "groups": w.groups,
           "reduce_bucket_size": w.reduce_bucket_size,
           "partition_elems": [gr["P"] for gr in groups], "divisors": [gr["D"] for gr in groups],
           "grad_dtype": "fp32", "bytes_per_step": total_bytes}
    return step, total_bytes, sum(gr["P"] for gr in groups), cfg, \
        {f"fused_g{g}": gr["bytes"] for g, gr in enumerate(groups)}, "fused_g1", None


def setup_ring(torch, zr, workloads):
    c = workloads.RING_1GIB
    N, M = c["ranks"], c["elems_per_rank"]
    C = M // N
    bufs = [workloads.device_normal(workloads.seed_for("ring-1gib", r), M, c["sigma"], "cuda")
            for r in range(N)]
    bytes_per_step = 12 * C * N

    def step(i, timer):
        timer.launch(lambda: zr.zr_ring_rs_step(bufs, C, i % (N - 1)), "ring")

    cfg = {"workload": "ring-1gib", "ranks": N, "chunk_elems": C, "bytes_per_step": bytes_per_step}
    return step, bytes_per_step, C * N, cfg, {"ring": bytes_per_step}, "ring", None


def setup_copy(torch, zr, workloads):
    n = (4 << 30) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    bytes_per_step = 8 * n

    def step(i, timer):
        timer.launch(lambda: dst.copy_(src), "copy")

    cfg = {"workload": "copy-4gib (torch copy_, practical ceiling)", "bytes_per_step": bytes_per_step}
    return step, bytes_per_step, n, cfg, {"copy": bytes_per_step}, "copy", None


# ------------------------------------------------------------ CPU baseline

def cpu_oracle_fused(torch, workloads, plan, name, w, reps, master_dev, P, R):
    """Time the CPU oracle (reduce-scatter, Adam, bf16 writeback) on rank 0's
    whole partition, single-threaded numpy, inputs already on the host."""
    import numpy as np
    from oracle.adam import adam_oracle
    from oracle.bf16 import bf16_rne_oracle
    from oracle.plan import plan_oracle
    from oracle.reduce import reduce_scatter_oracle

    ref = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    win = [r[:P].cpu().view(torch.int16).numpy().view(np.uint16) for r in reps]
    th = master_dev.cpu().numpy()
    z = np.zeros(P, np.float32)
    t0 = time.perf_counter()
    g = reduce_scatter_oracle(ref, 0, win, True, dst=0)[0]
    th1, m1, v1 = adam_oracle(g, th, z, z, step=1, **HP)
    bf16_rne_oracle(th1)
    dt = time.perf_counter() - t0
    byts = (R * 2 + 26) * P
    return {"value": byts / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "elements_per_s": P / dt, "seconds": dt,
            "sample": f"rank 0's whole partition: {P} elements x {R} bf16 replicas "
                      "(reduce-scatter + Adam + bf16 writeback), numpy single thread",
            "host_cores_available": len(os.sched_getaffinity(0))}


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--workload", default="gpt2-small",
                    choices=["gpt2-small", "llama3-8b", "llama3-8b-ipg", "moe-16l",
                             "ring-1gib", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the data-parallel replicas are resident in one "
              "GPU's HBM and the reduction is a local kernel; runs on more than one GPU "
              "are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from zero_partition_aware_amd import workloads, zr

    torch.cuda.set_device(0)
    setup = {"gpt2-small": setup_gpt2, "llama3-8b": setup_llama,
             "llama3-8b-ipg": lambda *a: setup_llama(*a, ipg=True), "moe-16l": setup_moe,
             "ring-1gib": setup_ring, "copy": setup_copy}[args.workload]
    step, bytes_per_step, elems_per_step, cfg, launch_bytes, dominant, cpu_leg = \
        setup(torch, zr, workloads)
    torch.cuda.synchronize()

    per_launch = len(launch_bytes) > 1
    warm = Timer(torch, per_launch)
    for i in range(args.warmup):
        step(i, warm)
    torch.cuda.synchronize()

    timer = Timer(torch, per_launch)
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region0.record()
    for i in range(args.steps):
        step(args.warmup + i, timer)
    region1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_s = 1e-3 * region0.elapsed_time(region1)

    if per_launch:
        ms = timer.per_label_ms()
        per_label_s = {k: (len(v), 1e-3 * sum(v) / len(v)) for k, v in ms.items()}
    else:
        # One kernel per step: its average launch duration is the event-timed
        # region divided by the launches in it (gaps between launches count).
        (label, n), = timer.count.items()
        per_label_s = {label: (n, region_s / n)}
    launches = {k: {"count": n, "avg_us": 1e6 * t,
                    "achieved_GBps": launch_bytes[k] / t / 1e9}
                for k, (n, t) in per_label_s.items()}
    gpu_step_s = region_s / args.steps
    wall_step_s = elapsed / args.steps
    dom = launches[dominant]
    roof = {"bound": "hbm", "achieved": round(dom["achieved_GBps"], 1), "peak": PEAK_GBS,
            "unit": "GB/s", "frac": round(dom["achieved_GBps"] / PEAK_GBS, 4),
            "traffic": traffic_for(f"{args.workload}:{dominant}"),
            "kernel": dominant, "avg_launch_us": round(dom["avg_us"], 2),
            "algorithmic_bytes_per_launch": launch_bytes[dominant]}

    out = {
        "metric": METRIC,
        "value": round(bytes_per_step / wall_step_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall_step_s, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": cfg,
        "pct_of_peak": round(100 * bytes_per_step / wall_step_s / 1e9 / PEAK_GBS, 2),
        "gpu_region_GBps": round(bytes_per_step / gpu_step_s / 1e9, 1),
        "elements_per_s": round(elems_per_step / wall_step_s),
        "launches": launches,
        "roofline": roof,
        "device": torch.cuda.get_device_name(0),
    }
    if cpu_leg is not None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_leg()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
