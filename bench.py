#!/usr/bin/env python3
"""Benchmark of the fused partition reduce-scatter + Adam step on one GPU.

Default run (``--workload headline``): the Llama-3-8B-shaped parameter list
(291 tensors, 8,030,261,248 elements), 8 data-parallel replicas, rank 0's
share: the fused step reads the 8 fp32 main_grad windows of partition 0
(1,003,782,656 elements), reduces them (pre-divide by 8, rank order) and
applies Adam to the partition's fp32 master / m / v with a bf16 param
writeback -- 58 bytes per partition element, 58.2 GB per step.  The same JSON
line also carries, each with its own roofline, same-run parity and CPU
baseline, the GPT-2-small rank shares (8 bf16 replicas, 42 B per element,
steps rotating over the 8 ranks' state sets) and the MoE step (dense group of
8 replicas with divisor 4, expert group of 2 with divisor 1, fp32), and a
same-run copy ceiling (the library's copy kernel moving a 4 GB bucket).

Prints ONE JSON line.  ``value`` is achieved HBM GB/s of the headline
workload: algorithmic bytes of a step divided by the measured time per step,
inputs already resident in HBM.  ``roofline`` prices the dominant call's
average duration (HIP events on the launch stream) against MI355X's 8 TB/s;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same work;
``parity_ok`` says whether sampled outputs of the timed run (and of one more
call with the reduced gradient written) match the oracle.  Other workloads
(``--workload``) are for characterisation.
"""

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for fused partition reduce-scatter+Adam step"
PEAK_GBS = 8000.0
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# Workloads whose dominant launches are exactly another workload's (same
# kernel, same bytes per launch) share its counter measurement.
TRAFFIC_SAME_AS = {}


def traffic_for(kernel_key):
    """HBM bytes per launch measured by rocprofv3 counters on exactly the
    kernel that runs now (its fingerprint in the built library), or None when
    absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    from zero_partition_aware_amd.build import kernel_hashes
    entry = t.get(kernel_key)
    if not entry or not entry.get("kernel_sha"):
        return None
    now = kernel_hashes()
    if any(now.get(name) != h for name, h in entry["kernel_sha"].items()):
        return None
    return entry.get("hbm_bytes_per_call")


def reduce_dispatches(zr, plan, group, dst, grad_dtype, fused):
    """Kernel launches one reduce call over every bucket makes (the library's
    own launch-shape query), so a call's event-timed average can be set
    beside a profiler's per-dispatch average."""
    nb = zr.zr_plan_num_buckets(plan)
    return zr.zr_plan_reduce_launches(plan, group, 0, nb, dst, grad_dtype, fused)[1]


# Calls actually made per label over the whole run (every timer), reported
# by single-workload runs so counter totals can be divided per call.
CALLS = {}


class Timer:
    """Counts launches per kernel label.  With ``only`` set, launches of other
    labels are skipped, so one kernel of a multi-kernel step can be timed
    back to back on its own."""

    def __init__(self, only=None):
        self.only = only
        self.count = {}

    def launch(self, fn, label):
        if self.only is not None and label != self.only:
            return
        self.count[label] = self.count.get(label, 0) + 1
        CALLS[label] = CALLS.get(label, 0) + 1
        fn()


class EventTimer(Timer):
    """Records a pair of HIP events around every launch of one label (other
    labels are skipped), for per-launch durations."""

    def __init__(self, torch, only, limit):
        super().__init__(only)
        self.torch, self.limit, self.pairs = torch, limit, []

    def launch(self, fn, label):
        if label != self.only or len(self.pairs) >= self.limit:
            return
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        CALLS[label] = CALLS.get(label, 0) + 1
        e0.record()
        fn()
        e1.record()
        self.pairs.append((e0, e1))


def median_launch_us(torch, step, first, label, reps=21):
    """Median duration of ``reps`` launches of one label, each bracketed by
    its own HIP events (three unrecorded warm-up launches first)."""
    for i in range(3):
        step(first + i, Timer(only=label))
    timer = EventTimer(torch, label, reps)
    i = first + 3
    while len(timer.pairs) < reps:
        n = len(timer.pairs)
        step(i, timer)
        i += 1
        if len(timer.pairs) == n:       # the label is not launched by this step
            break
    torch.cuda.synchronize()
    d = sorted(1e3 * a.elapsed_time(b) for a, b in timer.pairs)
    return round(d[len(d) // 2], 2) if d else None


def timed_region(torch, step, first, steps, only=None):
    """Run ``steps`` steps between two HIP events on the launch stream (torch's
    current stream); returns (wall seconds, event seconds, launch counts)."""
    timer = Timer(only)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(first + i, timer)
    ev1.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, 1e-3 * ev0.elapsed_time(ev1), timer.count


# ------------------------------------------------------------ same-run parity

PARITY_SAMPLE = 40000     # random partition elements checked per state set


def sample_indices(P, seed, edges=()):
    """Random partition offsets plus the partition's first and last 2048
    elements and +-8 elements around each given offset (slice edges)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    idx = set(rng.integers(0, P, size=PARITY_SAMPLE).tolist())
    idx.update(range(0, min(P, 2048)))
    idx.update(range(max(0, P - 2048), P))
    for e in edges:
        idx.update(range(max(0, e - 8), min(P, e + 8)))
    return np.array(sorted(idx), dtype=np.int64)


def gather(torch, t, idx):
    """Values of device tensor t at host indices idx as host numpy (fp32, or
    the uint16 patterns of bf16)."""
    import numpy as np
    g = t[torch.from_numpy(idx).to(t.device)]
    if g.dtype == torch.bfloat16:
        return g.cpu().view(torch.int16).numpy().view(np.uint16)
    return g.cpu().numpy()


def track_state(torch, state, idx):
    """Prepares a state set for the same-run check: the sampled offsets, the
    initial master there, and a log of the Adam step numbers applied."""
    state["idx"] = idx
    state["th0"] = gather(torch, state["master"], idx)
    state["steps"] = []


def check_state(torch, state, xs, is_bf16, D, call):
    """Checks one state set after the timed run, on its sampled offsets:
    (1) the oracle replays every logged Adam step from the initial master
    (m = v = 0) with the oracle's reduced gradient of the replica values
    ``xs`` (host arrays at the offsets), and the GPU's master, m, v and bf16
    param must match (Adam within rel 1e-6 / abs 1e-7, v relative only; bf16 =
    round-to-nearest-even of the GPU's master); (2) one more call,
    ``call(grad_out, step)``, with the reduced gradient written: bit-exact
    against the oracle, and its Adam outputs checked the same way."""
    import numpy as np
    from oracle.adam import adam_oracle
    from oracle.bf16 import bf16_rne_oracle
    from oracle.ipg import widen_bf16
    from oracle.reduce import rank_order_mean
    idx = state["idx"]
    g = rank_order_mean([widen_bf16(x) if is_bf16 else x for x in xs], D)
    th = state["th0"].copy()
    m = np.zeros_like(th)
    v = np.zeros_like(th)
    for t in state["steps"]:
        th, m, v = adam_oracle(g, th, m, v, step=t, **HP)
    worst = {"master": 0.0, "m": 0.0, "v": 0.0}

    def compare(want_th, want_m, want_v):
        ok = True
        for name, want, atol in (("master", want_th, 1e-7), ("m", want_m, 1e-7), ("v", want_v, 0.0)):
            got = gather(torch, state[name], idx).astype(np.float64)
            w = want.astype(np.float64)
            err = np.abs(got - w)
            ok &= bool(np.all(err <= atol + 1e-6 * np.abs(w)))
            rel = float(np.max(err / np.maximum(np.abs(w), 1e-30)))
            worst[name] = max(worst[name], rel)
        pb = gather(torch, state["pbf16"], idx)
        ok &= bool(np.array_equal(pb, bf16_rne_oracle(gather(torch, state["master"], idx))))
        return ok

    ok_timed = compare(th, m, v)
    t = (state["steps"][-1] if state["steps"] else 0) + 1
    gout = torch.empty_like(state["master"])
    call(gout, t)
    torch.cuda.synchronize()
    got_g = gather(torch, gout, idx)
    ok_g = bool(np.array_equal(got_g.view(np.uint32), g.view(np.uint32)))
    th, m, v = adam_oracle(g, th, m, v, step=t, **HP)
    ok_next = compare(th, m, v)
    del gout
    return {"ok": ok_timed and ok_g and ok_next, "elements": int(idx.size),
            "adam_steps_replayed": len(state["steps"]),
            "timed_outputs_ok": ok_timed, "reduced_gradient_bit_exact": ok_g,
            "next_step_ok": ok_next,
            "max_rel_err": {k: float(f"{x:.3g}") for k, x in worst.items()}}


def combine_checks(checks):
    return {"ok": all(c["ok"] for c in checks.values()), "state_sets": checks}


# --------------------------------------------------------------- workloads

def setup_gpt2(torch, zr, workloads, all_ranks=False):
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
    checked = (0, R - 1)                 # state sets the same-run check covers
    for k in checked:
        track_state(torch, states[k], sample_indices(P, 100 + k))

    def step(i, timer):
        k = i % R
        s = states[k]
        t = i // R + 1

        def call():
            if "steps" in s:
                s["steps"].append(t)
            zr.zr_reduce_scatter_adam(plan, 0, -1, k, reps, s["master"], s["m"], s["v"],
                                      s["pbf16"], None, step=t, **HP)
        timer.launch(call, "fused")

    def parity():
        out = {}
        for k in checked:
            s = states[k]
            xs = [gather(torch, r_[k * P:(k + 1) * P], s["idx"]) for r_ in reps]
            out[f"rank {k}"] = check_state(
                torch, s, xs, True, D,
                lambda gout, t: zr.zr_reduce_scatter_adam(plan, 0, -1, k, reps, s["master"], s["m"],
                                                          s["v"], s["pbf16"], gout, step=t, **HP))
        return combine_checks(out)

    step.parity = parity
    step.dispatches = {"fused": reduce_dispatches(zr, plan, 0, 0, "bf16", True)}

    cfg = {"workload": name, "params": len(w.numels), "total_elems": T,
           "replicas": R, "grad_dtype": "bf16", "reduce_bucket_size": w.reduce_bucket_size,
           "partition_elems": P, "divisor": D, "share": "one rank's partition per step, k = step mod 8",
           "bytes_per_step": bytes_per_step}
    launch_bytes = {"fused": bytes_per_step}

    def cpu_leg():
        return cpu_oracle_fused(torch, workloads, plan, name, w, reps, states, P, R)

    if all_ranks:
        # Every rank's partition in one fused launch (dst = -1): the Adam
        # state spans the whole padded flat space, partition k from k*P;
        # 5.23 GB per step.
        del states
        L = R * P
        master = torch.empty(L, device="cuda")
        for k in range(R):
            workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                    w.master_sigma, "cuda", out=master[k * P:(k + 1) * P])
        master[T:] = 0.0
        m, v = torch.zeros_like(master), torch.zeros_like(master)
        pbf16 = torch.empty(L, dtype=torch.bfloat16, device="cuda")

        def step_all(i, timer):
            timer.launch(lambda: zr.zr_reduce_scatter_adam(
                plan, 0, -1, -1, reps, master, m, v, pbf16, None, step=i + 1, **HP), "fused")

        step_all.dispatches = {"fused": reduce_dispatches(zr, plan, 0, -1, "bf16", True)}
        cfg.update(workload=name + "-all-ranks", bytes_per_step=R * bytes_per_step,
                   share="all 8 ranks' partitions in one fused call per step")
        return step_all, R * bytes_per_step, R * P, cfg, {"fused": R * bytes_per_step}, \
            "fused", None
    return step, bytes_per_step, P, cfg, launch_bytes, "fused", cpu_leg


def setup_gpt2_unfused(torch, zr, workloads, copy_only=False):
    """The same rank shares as the default, as separate launches: the
    reduce-scatter with its fused store into the partition (a3+a4), then the
    standalone partition Adam (a5); or only the standalone copy of a reduced
    bucket-layout buffer into the partition (a4)."""
    name = "gpt2-small"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R = w.groups[0][0]
    if copy_only:
        src = workloads.device_normal(workloads.seed_for(name, 0, 7), T, w.grad_sigma, "cuda")
        parts = [torch.empty(P, device="cuda") for _ in range(R)]

        def step(i, timer):
            k = i % R
            timer.launch(lambda: zr.zr_copy_grads_in_partition(plan, 0, 0, k, src, parts[k]),
                         "copy")

        cfg = {"workload": name + "-copy-in-partition", "partition_elems": P,
               "bytes_per_step": 8 * P, "share": "one rank's slices of the one bucket"}
        return step, 8 * P, P, cfg, {"copy": 8 * P}, "copy", None
    reps = [workloads.device_normal(workloads.seed_for(name, r), T, w.grad_sigma, "cuda", "bf16")
            for r in range(R)]
    states = []
    for k in range(R):
        master = workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                         w.master_sigma, "cuda")
        states.append(dict(master=master, m=torch.zeros_like(master),
                           v=torch.zeros_like(master), g=torch.empty_like(master),
                           pbf16=torch.empty(P, dtype=torch.bfloat16, device="cuda")))
    rb, ab = (R * 2 + 4) * P, 30 * P

    def step(i, timer):
        k = i % R
        s = states[k]
        timer.launch(lambda: zr.zr_reduce_scatter_local(plan, 0, -1, k, reps, [s["g"]]), "reduce")
        timer.launch(lambda: zr.zr_adam_partition(s["g"], s["master"], s["m"], s["v"], s["pbf16"],
                                                  step=i // R + 1, **HP), "adam")

    cfg = {"workload": name + "-unfused", "replicas": R, "grad_dtype": "bf16",
           "partition_elems": P, "bytes_per_step": rb + ab,
           "share": "one rank's partition per step: reduce-scatter, then Adam"}
    return step, rb + ab, P, cfg, {"reduce": rb, "adam": ab}, "reduce", None


def setup_llama_copy(torch, zr, workloads):
    """The standalone copy into the partition (a4) at a size where a launch's
    ramp does not matter: Llama-3-8B's first bucket (5e8 elements, all of it
    inside rank 0's partition), bucket layout -> partition, 4 GB per launch."""
    name = "llama3-8b"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    n = sum(s[6] for s in zr.zr_plan_slices(plan, 0) if s[2] == 0)
    src = workloads.device_normal(workloads.seed_for(name, 0, 7), w.reduce_bucket_size,
                                  w.grad_sigma, "cuda")
    part = torch.empty(P, device="cuda")

    def step(i, timer):
        timer.launch(lambda: zr.zr_copy_grads_in_partition(plan, 0, 0, 0, src, part), "copy")

    cfg = {"workload": name + "-copy-in-partition", "copied_elems": n,
           "bytes_per_step": 8 * n, "share": "rank 0's slices of the first bucket"}
    return step, 8 * n, n, cfg, {"copy": 8 * n}, "copy", None


def setup_gpt2_allgather(torch, zr, workloads):
    """Parameter all-gather after the update: one rank rebuilds the full bf16
    parameter vector (124,439,808 elements) from the 8 updated partitions."""
    name = "gpt2-small"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R = w.groups[0][0]
    parts = [workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                     w.master_sigma, "cuda", "bf16") for k in range(R)]
    outs = [torch.empty(T, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    b = 4 * T

    def step(i, timer):
        timer.launch(lambda: zr.zr_all_gather_params(plan, 0, parts, outs[i % 2]), "allgather")

    cfg = {"workload": name + "-allgather", "total_elems": T, "replicas": R,
           "bytes_per_step": b, "share": "one rank's full bf16 parameter vector"}
    return step, b, T, cfg, {"allgather": b}, "allgather", None


def setup_gpt2_dp(torch, zr, workloads):
    """Plain data parallelism on one GPU's share, the baseline the method
    replaces: the all-reduce average of the whole flat vector (every
    partition of the reduce-scatter, written contiguously), then Adam over
    every parameter (optimizer state not partitioned)."""
    name = "gpt2-small"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R = w.groups[0][0]
    reps = [workloads.device_normal(workloads.seed_for(name, r), T, w.grad_sigma, "cuda", "bf16")
            for r in range(R)]
    g = torch.empty(L, device="cuda")
    parts = [g[k * P:(k + 1) * P] for k in range(R)]
    master = workloads.device_normal(workloads.seed_for(name, 0, master=True), L, w.master_sigma,
                                     "cuda")
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    pb = torch.empty(L, dtype=torch.bfloat16, device="cuda")
    rb, ab = (R * 2 + 4) * L, 30 * L

    def step(i, timer):
        timer.launch(lambda: zr.zr_reduce_scatter_local(plan, 0, -1, -1, reps, parts), "allreduce")
        timer.launch(lambda: zr.zr_adam_partition(g, master, m, v, pb, step=i + 1, **HP), "adam")

    cfg = {"workload": name + "-dp-baseline", "replicas": R, "total_elems": T,
           "bytes_per_step": rb + ab,
           "share": "plain DP: full averaged gradient and Adam on every parameter"}
    return step, rb + ab, L, cfg, {"allreduce": rb, "adam": ab}, "adam", None


def setup_ring_allreduce(torch, zr, workloads):
    """Ring all-reduce emulation: the 7 reduce-scatter steps then the 7
    all-gather steps, all 8 ranks resident (the all-reduce baseline)."""
    c = workloads.RING_1GIB
    N, M = c["ranks"], c["elems_per_rank"]
    C = M // N
    bufs = [workloads.device_normal(workloads.seed_for("ring-1gib", r), M, c["sigma"], "cuda")
            for r in range(N)]
    rs, ag = 12 * C * N, 8 * C * N

    def step(i, timer):
        for s in range(N - 1):
            timer.launch(lambda: zr.zr_ring_rs_step(bufs, C, s), "ring_rs")
        for s in range(N - 1):
            timer.launch(lambda: zr.zr_ring_ag_step(bufs, C, s), "ring_ag")

    b = (N - 1) * (rs + ag)
    cfg = {"workload": "ring-1gib-allreduce", "ranks": N, "chunk_elems": C,
           "bytes_per_step": b}
    return step, b, M * N, cfg, {"ring_rs": rs, "ring_ag": ag}, "ring_rs", None


def run_placement(torch, zr, workloads, args):
    """The headline call on freshly allocated buffers, ``--sets`` times in
    one process: each set allocates rank 0's 8 fp32 replica windows and its
    state as the headline does, times ``--calls`` calls (each between its own
    pair of events, after two untimed ones), then frees everything and
    returns the memory to the driver before the next set.  The virtual
    addresses usually repeat; the physical pages behind them need not, so the
    spread over the sets is the part of the headline's run-to-run spread that
    follows the allocation."""
    name = "llama3-8b"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R = w.groups[0][0]
    byts = (R * 4 + 26) * P
    sets = []
    for s_ in range(args.sets):
        mgs = [workloads.device_normal(workloads.seed_for(name, r, 9), P, 2 * w.grad_sigma, "cuda")
               for r in range(R)]
        master = workloads.device_normal(workloads.seed_for(name, 0, master=True), P,
                                          w.master_sigma, "cuda")
        m, v = torch.zeros_like(master), torch.zeros_like(master)
        pbf16 = torch.empty(P, dtype=torch.bfloat16, device="cuda")
        reps = [(x, 0) for x in mgs]
        t = 0
        for _ in range(2):
            t += 1
            zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, master, m, v, pbf16, None,
                                      step=t, **HP)
        torch.cuda.synchronize()
        rates = []
        for _ in range(args.calls):
            t += 1
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, master, m, v, pbf16, None,
                                      step=t, **HP)
            b_.record()
            torch.cuda.synchronize()
            rates.append(byts / (a_.elapsed_time(b_) * 1e-3) / 1e9)
        ptrs = [x.data_ptr() for x in mgs] + [master.data_ptr(), m.data_ptr(), v.data_ptr()]
        sets.append({"median_GBps": round(statistics.median(rates), 1),
                     "min_GBps": round(min(rates), 1), "max_GBps": round(max(rates), 1),
                     "lowest_address": hex(min(ptrs))})
        print(f"placement set {s_}: median {sets[-1]['median_GBps']} GB/s "
              f"(min {sets[-1]['min_GBps']}, max {sets[-1]['max_GBps']}), lowest address "
              f"{sets[-1]['lowest_address']}", file=sys.stderr, flush=True)
        del mgs, master, m, v, pbf16, reps
        torch.cuda.empty_cache()
    med = [x["median_GBps"] for x in sets]
    print(json.dumps({"metric": "achieved HBM GB/s of the headline call per fresh allocation",
                      "value": None, "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                      "data": "synthetic",
                      "config": {"workload": "llama3-8b-placement", "partition_elems": P,
                                 "replicas": R, "bytes_per_call": byts, "sets": args.sets,
                                 "calls_per_set": args.calls},
                      "sets": sets, "min_of_medians": min(med), "max_of_medians": max(med),
                      "spread": round(max(med) / min(med) - 1, 4)}), flush=True)


def run_overlap(torch, zr, workloads, args):
    """Overlapped bucketed reduction behind a simulated backward, for one rank.

    The plan is built over the Llama-3-8B list in gradient-ready order (last
    layer first).  Stream A runs the backward stand-in: for every param a
    weight-gradient GEMM (dY^T X over 2048 tokens, bf16, torch matmul) and
    the IPG fill of that gradient into this rank's full fp32 main_grad
    (``--backward ipg``: the IPG fill alone, each gradient a view of one
    pre-drawn bf16 buffer).  As
    soon as a bucket is complete its fused reduce-scatter + Adam for this
    rank's partition is launched on stream B after an event from stream A;
    the other 7 replicas' windows are resident; the per-bucket calls go
    through prepared calls (arguments marshalled once).  Backward-only, reduce-only
    and serial times are taken on one stream; the overlapped run uses two.
    Besides the plain two-stream run, each value of ``--reduce-cus`` splits
    the compute units between the streams (CU-masked streams: the reduction
    on that many, the backward on the rest), and each nonzero value of
    ``--reduce-wgs`` caps the overlapped reductions' launches at that many
    workgroups.  The hidden fraction, (serial - overlapped) / reduce-only, is
    always measured against the unpartitioned, uncapped serial step and may
    be negative.  Checks that every overlapped result equals the serial one
    bit for bit."""
    name = "llama3-8b"
    w = workloads.get(name)
    order = list(range(len(w.numels)))[::-1]
    numels = [w.numels[p] for p in order]
    shapes = [w.shapes[p] for p in order]
    R, k, tok = 8, 0, args.tokens
    ipg_only = args.backward == "ipg"
    dev = "cuda"
    hip = ctypes.CDLL("libamdhip64.so.7")     # the runtime torch already holds
    created = []

    def new_stream(cus=None):
        """A default-priority, non-blocking HIP stream created through the
        runtime torch holds (no torch stream pool), destroyed after each
        configuration.  ``cus``: the compute units (bit indices of the
        runtime's CU mask) the stream's kernels may use; None = all."""
        h = ctypes.c_void_p()
        if cus is None:
            err = hip.hipStreamCreateWithFlags(ctypes.byref(h), ctypes.c_uint(1))
        else:
            words = [0] * ((n_cus + 31) // 32)
            for c in cus:
                words[c // 32] |= 1 << (c % 32)
            mask = (ctypes.c_uint32 * len(words))(*words)
            err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(len(words)),
                                                   mask)
        if err != 0:
            raise RuntimeError(f"stream creation failed with HIP error {err}")
        created.append(h)
        return torch.cuda.ExternalStream(h.value)

    def destroy_stream(ext):
        """Destroys one stream made by new_stream (CU-masked streams each
        hold a hardware queue of their own, so they are not kept around)."""
        torch.cuda.synchronize()
        for i, h in enumerate(created):
            if h.value == ext.cuda_stream:
                hip.hipStreamDestroy(created.pop(i))
                return

    def destroy_streams():
        torch.cuda.synchronize()
        while created:
            hip.hipStreamDestroy(created.pop())

    n_cus = torch.cuda.get_device_properties(0).multi_processor_count

    def reduce_cu_set(n):
        """n compute units for the reduction stream: the lowest n bits of the
        CU mask.  The runtime deals mask bits out to the 8 XCDs in turn, so
        these are n/8 CUs on every XCD (a mask that leaves an XCD without CUs
        cannot be given to a stream: every queue dispatches to every XCD)."""
        if n % 8:
            raise SystemExit("--reduce-cus values must be multiples of 8 (one CU per XCD)")
        return list(range(n))

    o_max = max(s[0] for s in shapes if len(s) == 2)
    # Contiguous operands only (one activation matrix per input width).
    X = {i: (torch.randn(tok, i, device=dev) * 0.1).to(torch.bfloat16)
         for i in sorted({s[-1] for s in shapes})}
    dYt = (torch.randn(o_max, tok, device=dev) * 0.1).to(torch.bfloat16)
    # IPG-only backward: every param's gradient is a view of one bf16 buffer.
    gbuf = (workloads.device_normal(workloads.seed_for(name, 0, 5), max(numels), w.grad_sigma,
                                    dev, "bf16") if ipg_only else None)
    results = {}
    ref_master = None
    s_full = torch.cuda.current_stream()      # serial reference on every CU
    for B in args.buckets:
        plan = zr.zr_plan_buckets(numels, [0] * len(numels), [(R, 1)], B)
        T, L, P, D = zr.zr_plan_group_info(plan, 0)
        nb = zr.zr_plan_num_buckets(plan)
        lo = k * P
        mg = torch.empty(T, device=dev)
        others = [workloads.device_normal(workloads.seed_for(name, r, 7), P, 2 * w.grad_sigma, dev)
                  for r in range(1, R)]
        reps = [(mg, 0)] + [(x, lo) for x in others]
        master0 = workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                          w.master_sigma, dev)
        state = {"master": torch.empty_like(master0), "m": torch.empty_like(master0),
                 "v": torch.empty_like(master0),
                 "pb": torch.empty(P, dtype=torch.bfloat16, device=dev)}
        # One prepared call per workgroup cap: arguments checked and marshalled
        # once, so a per-bucket call costs the C library's validation and
        # launch only.  reset() refills the same state tensors in place.
        prepared = {}

        def prep(cap):
            if cap not in prepared:
                prepared[cap] = zr.prepare_reduce_scatter_adam(
                    plan, 0, k, reps, state["master"], state["m"], state["v"], state["pb"],
                    None, max_workgroups=cap, **HP)
            return prepared[cap]

        pos, ends = 0, []
        for ne in numels:
            pos += ne
            ends.append(pos)

        def reset():
            mg.zero_()
            state["master"].copy_(master0)
            state["m"].zero_()
            state["v"].zero_()
            torch.cuda.synchronize()

        def reduce_bucket(b, cap=0):
            prep(cap)(b, 1)

        def backward(on_bucket):
            done = 0
            for p, (ne, shp) in enumerate(zip(numels, shapes)):
                if ipg_only:
                    g = gbuf[:ne]
                elif len(shp) == 2:
                    g = torch.matmul(dYt[:shp[0]], X[shp[1]]).view(-1)
                else:
                    g = X[shp[0]][0].clone()
                zr.zr_ipg_accumulate(plan, [p], [g], mg, window_base=0)
                while done < nb and ((done + 1) * B <= ends[p] or ends[p] == T):
                    on_bucket(done)
                    done += 1

        def timed(fn):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            return time.perf_counter() - t0

        def run_serial():
            with torch.cuda.stream(s_full):
                backward(lambda b: None)
                for b in range(nb):
                    reduce_bucket(b)

        def run_overlap_once(cap, sa, sb):
            def on_bucket(b):
                ev = torch.cuda.Event()
                ev.record(sa)
                sb.wait_event(ev)
                with torch.cuda.stream(sb):
                    reduce_bucket(b, cap)
            with torch.cuda.stream(sa):
                backward(on_bucket)
            sa.wait_stream(sb)

        def run_backward(stream=s_full):
            with torch.cuda.stream(stream):
                backward(lambda b: None)

        def run_reduce(cap=0, stream=s_full):
            with torch.cuda.stream(stream):
                for b in range(nb):
                    reduce_bucket(b, cap)

        reset(); run_serial(); torch.cuda.synchronize()       # warm-up
        reset(); t_bwd = timed(run_backward)
        t_red = timed(run_reduce)
        reset(); t_ser = timed(run_serial)
        serial_master = state["master"].clone()
        if ref_master is None:
            ref_master = serial_master
        same_across_b = bool(torch.equal(ref_master.view(torch.int32),
                                         serial_master.view(torch.int32)))
        # Configurations: CU-partitioned streams (reduction on ncu compute
        # units, backward on the rest) and grid caps on unpartitioned streams.
        configs = ([(ncu, 0) for ncu in args.reduce_cus] +
                   [(0, cap) for cap in args.reduce_wgs if cap])
        for ncu, cap in configs:
            # One pair of streams per configuration, destroyed after it: a
            # CU-masked stream holds a hardware queue of its own, and a
            # process has few.
            if ncu:
                red_set = reduce_cu_set(ncu)
                rest = sorted(set(range(n_cus)) - set(red_set))
                xa, xb = new_stream(rest), new_stream(red_set)
            else:
                xa, xb = new_stream(), new_stream()
            t_bwd_cfg = t_bwd if ncu == 0 else timed(lambda: run_backward(xa))
            t_red_cfg = (t_red if (ncu, cap) == (0, 0)
                         else timed(lambda: run_reduce(cap, xb)))
            reset(); run_overlap_once(cap, xa, xb); torch.cuda.synchronize()
            reset(); t_ovl = timed(lambda: run_overlap_once(cap, xa, xb))
            same = bool(torch.equal(serial_master.view(torch.int32),
                                    state["master"].view(torch.int32)))
            results[f"B={B},cus={ncu},wgs={cap}"] = {
                "reduce_bucket_size": B, "buckets": nb, "reduce_cus": ncu,
                "reduce_max_workgroups": cap,
                "t_backward_ms": 1e3 * t_bwd, "t_backward_this_config_ms": 1e3 * t_bwd_cfg,
                "t_reduce_ms": 1e3 * t_red, "t_reduce_this_config_ms": 1e3 * t_red_cfg,
                "t_serial_ms": 1e3 * t_ser, "t_overlap_ms": 1e3 * t_ovl,
                "hidden_fraction": (t_ser - t_ovl) / t_red,
                "overlap_bitwise_equal_serial": same,
                "equal_across_bucket_sizes": same_across_b}
            print(f"overlap B={B} cus={ncu} wgs={cap}: {nb} buckets, backward "
                  f"{1e3 * t_bwd:.1f} ms (this config {1e3 * t_bwd_cfg:.1f}), reduce "
                  f"{1e3 * t_red:.1f} ms (this config {1e3 * t_red_cfg:.1f}), serial "
                  f"{1e3 * t_ser:.1f} ms, overlapped {1e3 * t_ovl:.1f} ms, hidden "
                  f"{(t_ser - t_ovl) / t_red:.3f}, equal {same}", file=sys.stderr, flush=True)
            destroy_stream(xa)
            destroy_stream(xb)
        del mg, others, reps, master0, state, prepared
        destroy_streams()
        torch.cuda.empty_cache()
    ok = all(r["overlap_bitwise_equal_serial"] and r["equal_across_bucket_sizes"]
             for r in results.values())
    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
           "higher_is_better": True, "data": "synthetic",
           "config": {"workload": "llama3-8b-overlap", "rank": k, "tokens": tok,
                      "backward": "ipg" if ipg_only else "weight-gradient gemm + ipg",
                      "ready_order": "last layer first"},
           "overlap": results, "parity_ok": ok,
           "device": torch.cuda.get_device_name(0)}
    print(json.dumps(out), flush=True)
    if not ok:
        sys.exit(1)


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
        # The first micro-batch writes the window it would have added into
        # after the step's zeroing (6 B per element: bf16 read, fp32
        # written); the others add into it (10 B: bf16 read, fp32 read and
        # written).
        bytes_per_step = R * P * (6 + 10 * (w.micro_batches - 1))

        def step(i, timer):
            for r in range(R):
                timer.launch(lambda: zr.zr_ipg_accumulate_first(plan, pids, views[r], mgs[r],
                                                                window_base=lo), "ipg_first")
            for mu in range(1, w.micro_batches):
                for r in range(R):
                    timer.launch(lambda: zr.zr_ipg_accumulate(plan, pids, views[r], mgs[r],
                                                              window_base=lo), "ipg")

        cfg.update(micro_batches=w.micro_batches, grad_dtype="bf16 -> fp32 main_grad",
                   first_micro_batch="zr_ipg_accumulate_first (main_grad not read)",
                   bytes_per_step=bytes_per_step)
        return step, bytes_per_step, P * w.micro_batches * R, cfg, \
            {"ipg_first": 6 * P, "ipg": 10 * P}, "ipg", None

    master = workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                      w.master_sigma, "cuda")
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    pbf16 = torch.empty(P, dtype=torch.bfloat16, device="cuda")
    reps = [(x, lo) for x in mgs]
    bytes_per_step = (R * 4 + 26) * P
    state = dict(master=master, m=m, v=v, pbf16=pbf16)
    edges = [s_[5] for s_ in zr.zr_plan_slices(plan) if s_[2] == k]     # slice starts
    track_state(torch, state, sample_indices(P, 200, edges))

    def step(i, timer):
        def call():
            state["steps"].append(i + 1)
            zr.zr_reduce_scatter_adam(plan, 0, -1, k, reps, master, m, v, pbf16, None,
                                      step=i + 1, **HP)
        timer.launch(call, "fused")

    def parity():
        xs = [gather(torch, x, state["idx"]) for x in mgs]
        return combine_checks({f"rank {k}": check_state(
            torch, state, xs, False, D,
            lambda gout, t: zr.zr_reduce_scatter_adam(plan, 0, -1, k, reps, master, m, v, pbf16,
                                                      gout, step=t, **HP))})

    step.parity = parity
    step.dispatches = {"fused": reduce_dispatches(zr, plan, 0, k, "fp32", True)}
    cfg.update(grad_dtype="fp32 main_grad", bytes_per_step=bytes_per_step)
    def cpu_leg():
        return cpu_oracle_chunk(torch, mgs, master, P, R, D, 1 << 26)

    return step, bytes_per_step, P, cfg, {"fused": bytes_per_step}, "fused", cpu_leg


def setup_share(torch, zr, workloads, P):
    """The fused step on one rank's share of P elements with 8 fp32
    replicas (one parameter of 8P elements, one bucket), for how the rate
    depends on the share size: 58 B per partition element."""
    R = 8
    plan = zr.zr_plan_buckets([R * P], [0], [(R, 1)], 1 << 62)
    name = f"share-{P}"
    reps = [(workloads.device_normal(9_100_000 + r, P, 1e-3, "cuda"), 0) for r in range(R)]
    master = workloads.device_normal(9_199_000, P, 0.02, "cuda")
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    pbf16 = torch.empty(P, dtype=torch.bfloat16, device="cuda")
    bytes_per_step = (R * 4 + 26) * P

    def step(i, timer):
        timer.launch(lambda: zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, master, m, v, pbf16,
                                                       None, step=i + 1, **HP), "fused")

    step.dispatches = {"fused": reduce_dispatches(zr, plan, 0, 0, "fp32", True)}
    cfg = {"workload": name, "replicas": R, "partition_elems": P, "grad_dtype": "fp32",
           "bytes_per_step": bytes_per_step}
    return step, bytes_per_step, P, cfg, {"fused": bytes_per_step}, "fused", None


SHARE_SIZES = {"share-15m": 15_554_976, "share-125m": 125_000_000, "share-500m": 500_000_000,
               "share-1b": 1_003_782_656}


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

    slices = zr.zr_plan_slices(plan)
    for g, gr in enumerate(groups):
        for k in (0, gr["R"] - 1):
            edges = [s_[5] for s_ in slices if s_[1] == g and s_[2] == k]
            track_state(torch, gr["states"][k], sample_indices(gr["P"], 300 + 10 * g + k, edges))

    def step(i, timer):
        for g, gr in enumerate(groups):
            k = i % gr["R"]
            s = gr["states"][k]
            t = i // gr["R"] + 1

            def call(g=g, gr=gr, k=k, s=s, t=t):
                if "steps" in s:
                    s["steps"].append(t)
                zr.zr_reduce_scatter_adam(plan, g, -1, k, gr["reps"], s["master"], s["m"],
                                          s["v"], s["pbf16"], None, step=t, **HP)
            timer.launch(call, f"fused_g{g}")

    def parity():
        out = {}
        for g, gr in enumerate(groups):
            P_ = gr["P"]
            for k in (0, gr["R"] - 1):
                s = gr["states"][k]
                xs = [gather(torch, r_[k * P_:(k + 1) * P_], s["idx"]) for r_ in gr["reps"]]
                out[f"group {g} rank {k}"] = check_state(
                    torch, s, xs, False, gr["D"],
                    lambda gout, t, g=g, gr=gr, k=k, s=s: zr.zr_reduce_scatter_adam(
                        plan, g, -1, k, gr["reps"], s["master"], s["m"], s["v"], s["pbf16"],
                        gout, step=t, **HP))
        return combine_checks(out)

    step.parity = parity
    step.dispatches = {f"fused_g{g}": reduce_dispatches(zr, plan, g, 0, "fp32", True)
                       for g in range(len(groups))}

    cfg = {"workload": name, "params": len(w.numels), "groups": w.groups,
           "reduce_bucket_size": w.reduce_bucket_size,
           "partition_elems": [gr["P"] for gr in groups], "divisors": [gr["D"] for gr in groups],
           "grad_dtype": "fp32", "bytes_per_step": total_bytes}

    def cpu_leg():
        # The expert group's rank 0 (the dominant launch): its partition
        # starts at flat offset 0, so the replicas' first elements are its own.
        gr = groups[1]
        return cpu_oracle_chunk(torch, gr["reps"], gr["states"][0]["master"], gr["P"],
                                gr["R"], gr["D"], 1 << 26)

    return step, total_bytes, sum(gr["P"] for gr in groups), cfg, \
        {f"fused_g{g}": gr["bytes"] for g, gr in enumerate(groups)}, "fused_g1", cpu_leg


def setup_moe_bucketed(torch, zr, workloads, graph=False, per_bucket=False, fused=False):
    """The MoE step through the bucketed path of the pages' IPG design, for
    rank 0 of each group: reduce-scatter calls into the rank's fp32 gradient
    partitions (269 buckets of 5e6 elements, both groups interleaved), then
    Adam over each partition.  By default each call takes every bucket
    completed since the previous one (zr_reduce_scatter_local_range), a call
    per group after each layer's 17 parameters, taken in list order as the
    ready order; with ``per_bucket`` one call per (bucket, group) holding
    slices for the rank.  With ``fused`` each range call also applies Adam to
    the partition elements it reduces (zr_reduce_scatter_adam_range): Adam is
    elementwise, so updating an element as soon as its reduced gradient
    exists gives the same numbers as one Adam pass after the last bucket, and
    the reduced gradient never goes through HBM.  With ``graph`` the whole
    step is captured once in a HIP graph (torch.cuda.CUDAGraph) and each step
    is one replay."""
    name = "moe-16l"
    w = workloads.get(name)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    nb = zr.zr_plan_num_buckets(plan)
    k = 0
    groups = []
    total_bytes = 0
    for g, (R, sp) in enumerate(w.groups):
        T, L, P, D = zr.zr_plan_group_info(plan, g)
        reps = [workloads.device_normal(workloads.seed_for(name, r + 100 * g), T, w.grad_sigma,
                                        "cuda") for r in range(R)]
        master = workloads.device_normal(workloads.seed_for(name, 10 * g + k, master=True),
                                         P, w.master_sigma, "cuda")
        groups.append(dict(R=R, P=P, reps=reps, grad=torch.empty(P, device="cuda"),
                           master=master, m=torch.zeros_like(master),
                           v=torch.zeros_like(master),
                           pbf16=torch.empty(P, dtype=torch.bfloat16, device="cuda")))
        total_bytes += (R * 4 + 26 if fused else R * 4 + 4 + 30) * P
    if per_bucket:
        # (bucket, group) selections holding slices for rank k, plus the last
        # bucket of every group (it also writes the group's padding).
        calls = []
        for b in range(nb):
            sl = zr.zr_plan_slices(plan, b)
            for g in range(len(groups)):
                if b == nb - 1 or any(s[1] == g and s[2] == k for s in sl):
                    calls.append((g, b, 1))
    else:
        # Ranges: after each layer, the buckets completed since the last call.
        per_layer = 17
        B = w.reduce_bucket_size
        calls, done, pos = [], 0, 0
        for p, ne in enumerate(w.numels):
            pos += ne
            if (p + 1) % per_layer == 0 or p + 1 == len(w.numels):
                full = nb if p + 1 == len(w.numels) else pos // B
                if full > done:
                    calls += [(g, done, full - done) for g in range(len(groups))]
                    done = full
        assert done == nb

    def eager(t, timer):
        if fused:
            for g, b, n in calls:
                gr = groups[g]
                timer.launch(lambda: zr.zr_reduce_scatter_adam_range(
                    plan, g, b, n, k, gr["reps"], gr["master"], gr["m"], gr["v"], gr["pbf16"],
                    step=t, **HP), "fused")
            return
        for g, b, n in calls:
            gr = groups[g]
            timer.launch(lambda: zr.zr_reduce_scatter_local_range(plan, g, b, n, k, gr["reps"],
                                                                  [gr["grad"]]), "reduce")
        for gr in groups:
            timer.launch(lambda: zr.zr_adam_partition(gr["grad"], gr["master"], gr["m"],
                                                      gr["v"], gr["pbf16"], step=t, **HP),
                         "adam")

    # Per-call bytes of each kind, averaged over the step's calls of it.
    if fused:
        launch_bytes = {"fused": round(total_bytes / len(calls))}
    else:
        launch_bytes = {"reduce": round(sum((gr["R"] * 4 + 4) * gr["P"] for gr in groups) /
                                        len(calls)),
                        "adam": round(sum(30 * gr["P"] for gr in groups) / len(groups))}
    cfg = {"workload": name + ("-per-bucket" if per_bucket else "-bucketed") +
           ("-fused" if fused else "") + ("-graph" if graph else ""),
           "params": len(w.numels), "groups": w.groups, "rank": k,
           "reduce_bucket_size": w.reduce_bucket_size, "buckets": nb,
           "trigger": "one call per (bucket, group) with slices for the rank" if per_bucket
           else "after each layer, one call per group for the buckets completed since the last",
           "reduce_calls_per_step": len(calls), "adam_calls_per_step": 0 if fused else len(groups),
           "partition_elems": [gr["P"] for gr in groups], "grad_dtype": "fp32",
           "bytes_per_step": total_bytes, "launch_sizes": "mixed"}
    if not graph:
        return (lambda i, timer: eager(i + 1, timer)), total_bytes, \
            sum(gr["P"] for gr in groups), cfg, launch_bytes, "fused" if fused else "reduce", None

    # Capture one step (Adam step number fixed at capture) after an eager
    # step has built the plan's launch tables.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        eager(1, Timer())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        eager(1, Timer())
    torch.cuda.synchronize()
    cfg["graph"] = "one captured step per replay (Adam step number fixed at capture)"
    del cfg["launch_sizes"]                   # one replay per step
    return (lambda i, timer: timer.launch(cg.replay, "graph")), total_bytes, \
        sum(gr["P"] for gr in groups), cfg, {"graph": total_bytes}, "graph", None


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

    cfg = {"workload": "copy-4gib (torch copy_, for reference)", "bytes_per_step": bytes_per_step}
    return step, bytes_per_step, n, cfg, {"copy": bytes_per_step}, "copy", None


# ------------------------------------------------------------ CPU baseline

CPU_MIN_SECONDS = 10.0   # single-thread work per CPU baseline (whole passes)
CPU_MAX_PASSES = 8


def _timed_passes(fn):
    """Runs fn() until at least CPU_MIN_SECONDS have been spent (whole
    passes, at most CPU_MAX_PASSES); returns (seconds, passes)."""
    total, passes = 0.0, 0
    while passes < CPU_MAX_PASSES and (passes == 0 or total < CPU_MIN_SECONDS):
        t0 = time.perf_counter()
        fn()
        total += time.perf_counter() - t0
        passes += 1
    return total, passes


def cpu_oracle_fused(torch, workloads, plan, name, w, reps, states, P, R):
    """Time the CPU oracle (plan-driven reduce-scatter, Adam, bf16 writeback)
    on every rank's partition of the step (the whole step of all R ranks),
    inputs already on the host (copies untimed), in whole passes until at
    least CPU_MIN_SECONDS of single-thread work.  Two runs of the same
    oracle code: one thread, ranks one after another; then one thread per
    rank (up to the host cores available), all ranks at once -- numpy's
    elementwise loops release the interpreter lock, so the threads run on
    separate cores."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle.adam import adam_oracle
    from oracle.bf16 import bf16_rne_oracle
    from oracle.ipg import widen_bf16
    from oracle.plan import plan_oracle
    from oracle.reduce import rank_order_mean, reduce_scatter_oracle

    ref = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    D = ref.groups[0].divisor
    assert all(s_.numel == P for s_ in ref.slices)    # one slice per partition
    z = np.zeros(P, np.float32)
    wins = [[r[k * P:(k + 1) * P].cpu().view(torch.int16).numpy().view(np.uint16)
             for r in reps] for k in range(R)]
    masters = [workloads.device_normal(workloads.seed_for(name, k, master=True), P,
                                       w.master_sigma, "cuda").cpu().numpy()
               for k in range(R)]

    def one_rank(k):
        g = reduce_scatter_oracle(ref, 0, wins[k], True, dst=k, flat_bases=[k * P] * R)[k]
        th1, _, _ = adam_oracle(g, masters[k], z, z, step=1, **HP)
        bf16_rne_oracle(th1)

    def whole_step():
        for k in range(R):
            one_rank(k)

    total, passes = _timed_passes(whole_step)
    # Parallel leg: every core of the affinity set, each rank's partition
    # (one slice of the single bucket) cut into pieces, the oracle's per-slice
    # steps on each piece (numpy's elementwise loops release the interpreter
    # lock, so the threads run on separate cores).
    avail = len(os.sched_getaffinity(0))
    threads = max(1, avail)
    cuts = max(1, -(-threads // R))
    jobs = [(k, P * i // cuts, P * (i + 1) // cuts) for k in range(R) for i in range(cuts)]

    def piece(job):
        k, a, b = job
        g = rank_order_mean([widen_bf16(x[a:b]) for x in wins[k]], D)
        th1, _, _ = adam_oracle(g, masters[k][a:b], z[a:b], z[a:b], step=1, **HP)
        bf16_rne_oracle(th1)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda k: None, range(threads)))          # start the threads
        t0 = time.perf_counter()
        for _ in range(passes):
            list(ex.map(piece, jobs))
        par = time.perf_counter() - t0
    byts = (R * 2 + 26) * P * R * passes
    elems = P * R * passes
    return {"value": round(byts / total / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "elements_per_s": round(elems / total), "seconds": round(total, 3),
            "sample": f"{passes} passes over all {R} ranks' partitions of the step: {R} x {P} "
                      f"elements x {R} bf16 replicas (reduce-scatter + Adam + bf16 writeback), "
                      "numpy single thread",
            "parallel": {"value": round(byts / par / 1e9, 3), "unit": "GB/s", "cores": threads,
                         "elements_per_s": round(elems / par), "seconds": round(par, 3),
                         "sample": f"the same {passes} passes, each rank's partition in "
                                   f"{cuts} pieces, {threads} threads"},
            "host_cores_available": avail}


def cpu_oracle_chunk(torch, windows, master, P, R, D, chunk):
    """Time the CPU oracle on a fixed chunk of one rank's share: the first
    ``chunk`` partition elements lie inside one slice, so the oracle's
    per-slice steps apply directly (rank-order pre-divided sum of the R fp32
    replica values, Adam, bf16 writeback); inputs already on the host; whole
    passes until at least CPU_MIN_SECONDS.  One thread, then one thread per
    eighth of the chunk."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle.adam import adam_oracle
    from oracle.bf16 import bf16_rne_oracle
    from oracle.reduce import rank_order_mean

    n = min(chunk, P)
    xs = [w_[:n].cpu().numpy() for w_ in windows]
    th = master[:n].cpu().numpy()
    z = np.zeros(n, np.float32)

    def part(a, b):
        g = rank_order_mean([x[a:b] for x in xs], D)
        th1, _, _ = adam_oracle(g, th[a:b], z[a:b], z[a:b], step=1, **HP)
        bf16_rne_oracle(th1)

    one, passes = _timed_passes(lambda: part(0, n))
    avail = len(os.sched_getaffinity(0))
    threads = max(1, avail)
    cuts = [n * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda i: None, range(threads)))
        t0 = time.perf_counter()
        for _ in range(passes):
            list(ex.map(lambda i: part(cuts[i], cuts[i + 1]), range(threads)))
        par = time.perf_counter() - t0
    byts = (R * 4 + 26) * n * passes
    return {"value": round(byts / one / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "elements_per_s": round(n * passes / one), "seconds": round(one, 3),
            "sample": f"{passes} passes over the first {n} elements of rank 0's partition "
                      f"({R} fp32 replicas, divisor {D:g}; reduce + Adam + bf16 writeback), "
                      "numpy single thread",
            "parallel": {"value": round(byts / par / 1e9, 3), "unit": "GB/s", "cores": threads,
                         "elements_per_s": round(n * passes / par), "seconds": round(par, 3),
                         "sample": f"the same {passes} passes, the chunk in {threads} pieces, "
                                   "one thread each"},
            "host_cores_available": avail}


# --------------------------------------------------------------------- main

def measure(torch, zr, workloads, setup, steps, warmup, workload, cpu=True, check=True):
    """Times one workload: ``warmup`` untimed steps, then exactly ``steps``
    steps between HIP events on the launch stream; returns the result dict
    (value, roofline, launches, same-run parity, CPU baseline)."""
    step, bytes_per_step, elems_per_step, cfg, launch_bytes, dominant, cpu_leg = \
        setup(torch, zr, workloads)
    torch.cuda.synchronize()

    for i in range(warmup):
        step(i, Timer())
    torch.cuda.synchronize()

    # The whole step: value and ms_per_step.
    elapsed, region_s, counts = timed_region(torch, step, warmup, steps)
    # Average duration of each kind of call: the event-timed region divided by
    # its calls.  When a step makes more than one kind of call, each kind is
    # also run back to back on its own (same steps, other calls skipped), so
    # no event ever sits between two different kernels.
    per_label_s = {}
    if len(counts) == 1:
        (label, n), = counts.items()
        per_label_s[label] = (n, region_s / n)
    else:
        for label in counts:
            _, r_s, c = timed_region(torch, step, warmup, steps, only=label)
            per_label_s[label] = (c[label], r_s / c[label])
    launches = {k: {"count": n, "avg_us": 1e6 * t,
                    "achieved_GBps": launch_bytes[k] / t / 1e9}
                for k, (n, t) in per_label_s.items()}
    # Supplementary: the median of 21 calls of each kind, each bracketed by
    # its own events (includes the events' own overhead).  Skipped where one
    # kind of call comes in several sizes (a median of those means nothing).
    for k in launches:
        launches[k]["median_us_event_per_launch"] = None if cfg.get("launch_sizes") == \
            "mixed" else median_launch_us(torch, step, warmup + steps, k)
    gpu_step_s = region_s / steps
    wall_step_s = elapsed / steps
    dom = launches[dominant]
    roof = {"bound": "hbm", "achieved": round(dom["achieved_GBps"], 1), "peak": PEAK_GBS,
            "unit": "GB/s", "frac": round(dom["achieved_GBps"] / PEAK_GBS, 4),
            "traffic": traffic_for(f"{TRAFFIC_SAME_AS.get(workload, workload)}:{dominant}"),
            "kernel": dominant, "avg_launch_us": round(dom["avg_us"], 2),
            "median_launch_us_event_per_launch": dom["median_us_event_per_launch"],
            "algorithmic_bytes_per_launch": launch_bytes[dominant]}
    # A call may be several equal kernel launches (calls over ~2 GiB are cut):
    # the per-dispatch average is what a kernel trace reports.
    dpc = getattr(step, "dispatches", {}).get(dominant)
    if dpc:
        roof["dispatches_per_call"] = dpc
        roof["avg_dispatch_us"] = round(dom["avg_us"] / dpc, 2)
    out = {"value": round(bytes_per_step / wall_step_s / 1e9, 1), "unit": "GB/s",
           "steps": steps, "warmup": warmup, "ms_per_step": round(1e3 * wall_step_s, 4),
           "config": cfg,
           "pct_of_peak": round(100 * bytes_per_step / wall_step_s / 1e9 / PEAK_GBS, 2),
           "gpu_region_GBps": round(bytes_per_step / gpu_step_s / 1e9, 1),
           "elements_per_s": round(elems_per_step / wall_step_s),
           "launches": launches, "roofline": roof}
    parity = getattr(step, "parity", None) if check else None
    if parity is not None:
        out["parity"] = parity()
        out["parity_ok"] = out["parity"]["ok"]
    if cpu_leg is not None and cpu:
        out["cpu_baseline"] = cpu_leg()
    del step, cpu_leg, parity
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


HEADLINE = "llama3-8b"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "gpt2-small", "gpt2-small-unfused", "gpt2-small-copy",
                             "gpt2-small-allgather", "gpt2-small-dp", "ring-1gib-allreduce",
                             "llama3-8b-overlap", "llama3-8b-placement",
                             "llama3-8b", "llama3-8b-ipg", "moe-16l", "moe-16l-bucketed",
                             "moe-16l-bucketed-fused", "moe-16l-per-bucket", "moe-16l-per-bucket-graph",
                             *SHARE_SIZES,
                             "llama3-8b-copy", "gpt2-small-all-ranks",
                             "ring-1gib", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the same-run parity check (counter runs: its extra call "
                         "would be counted with the timed ones)")
    ap.add_argument("--buckets", type=lambda t: [int(float(x)) for x in t.split(",")],
                    default=[int(5e7), int(5e8)],
                    help="reduce_bucket_size values for --workload llama3-8b-overlap")
    ap.add_argument("--backward", choices=["gemm", "ipg"], default="gemm",
                    help="backward stand-in of llama3-8b-overlap: weight-gradient GEMMs "
                         "plus IPG fills, or IPG fills alone")
    ap.add_argument("--tokens", type=int, default=2048,
                    help="tokens of the backward GEMM stand-in (llama3-8b-overlap)")
    ap.add_argument("--reduce-wgs", type=lambda t: [int(x) for x in t.split(",")],
                    default=[0],
                    help="workgroup caps of the overlapped reductions, each run on "
                         "unpartitioned streams (llama3-8b-overlap; 0 = none)")
    ap.add_argument("--reduce-cus", type=lambda t: [int(x) for x in t.split(",")],
                    default=[0],
                    help="compute units given to the reduction stream, the rest to the "
                         "backward stream (llama3-8b-overlap; 0 = no partition)")
    ap.add_argument("--sets", type=int, default=10,
                    help="fresh buffer allocations (llama3-8b-placement)")
    ap.add_argument("--calls", type=int, default=8,
                    help="timed calls per allocation (llama3-8b-placement)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the data-parallel replicas are resident in one "
              "GPU's HBM and the reduction is a local kernel, so there is no multi-GPU "
              "run of this benchmark.", file=sys.stderr)
        sys.exit(2)
    if args.sets < 1 or args.calls < 1:
        ap.error("--sets and --calls must be at least 1")

    import torch
    from zero_partition_aware_amd import workloads, zr

    torch.cuda.set_device(0)
    if args.workload == "llama3-8b-overlap":
        run_overlap(torch, zr, workloads, args)
        return
    if args.workload == "llama3-8b-placement":
        run_placement(torch, zr, workloads, args)
        return
    setups = {"gpt2-small": setup_gpt2, "llama3-8b": setup_llama,
              "gpt2-small-unfused": setup_gpt2_unfused,
              "gpt2-small-allgather": setup_gpt2_allgather,
              "gpt2-small-dp": setup_gpt2_dp,
              "ring-1gib-allreduce": setup_ring_allreduce,
              "gpt2-small-copy": lambda *a: setup_gpt2_unfused(*a, copy_only=True),
              "llama3-8b-ipg": lambda *a: setup_llama(*a, ipg=True), "moe-16l": setup_moe,
              "moe-16l-bucketed": setup_moe_bucketed,
              "moe-16l-bucketed-fused": lambda *a: setup_moe_bucketed(*a, fused=True),
              **{k: (lambda P: lambda *a: setup_share(*a, P))(P) for k, P in SHARE_SIZES.items()},
              "llama3-8b-copy": setup_llama_copy,
              "gpt2-small-all-ranks": lambda *a: setup_gpt2(*a, all_ranks=True),
              "moe-16l-per-bucket": lambda *a: setup_moe_bucketed(*a, per_bucket=True),
              "moe-16l-per-bucket-graph": lambda *a: setup_moe_bucketed(*a, graph=True,
                                                                          per_bucket=True),
              "ring-1gib": setup_ring, "copy": setup_copy}
    cpu = not args.no_cpu_baseline
    head_name = HEADLINE if args.workload == "headline" else args.workload
    check = not args.no_parity
    head = measure(torch, zr, workloads, setups[head_name], args.steps, args.warmup,
                   head_name, cpu, check)
    out = {"metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"),
           "n_gpus": 1, "steps": head.pop("steps"), "warmup": head.pop("warmup"),
           "ms_per_step": head.pop("ms_per_step"), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": head.pop("config")}
    out.update(head)
    if args.workload == "headline":
        # The practical ceiling of a plain stream on this machine, in this run:
        # the library's own copy kernel moving a 2 GB bucket (5e8 fp32
        # elements) into a partition, 4 GB of traffic per call.
        copy = measure(torch, zr, workloads, setup_llama_copy, max(args.steps, 10),
                       args.warmup, "llama3-8b-copy", False)
        out["copy_ceiling"] = {"GBps": copy["roofline"]["achieved"],
                               "frac_of_peak": copy["roofline"]["frac"],
                               "avg_call_us": copy["roofline"]["avg_launch_us"],
                               "bytes_per_call": copy["roofline"]["algorithmic_bytes_per_launch"],
                               "steps": copy["steps"],
                               "what": "zr_copy_grads_in_partition of a 5e8-element fp32 "
                                       "bucket into a partition (2 GB read + 2 GB written)"}
        out["frac_of_copy_ceiling"] = round(out["roofline"]["achieved"] / copy["roofline"]["achieved"], 4)
        # The other bandwidth workloads, each with its own roofline, parity
        # and CPU baseline; steps raised so each timed region spans tens of ms.
        others = {}
        for name, k_min in (("gpt2-small", 400), ("moe-16l", 20)):
            steps = max(args.steps, k_min)
            others[name] = measure(torch, zr, workloads, setups[name], steps,
                                   max(args.warmup, steps // 10), name, cpu, check)
        out["other_configs"] = others
        if check:
            checks = [out.get("parity_ok")] + [o.get("parity_ok") for o in others.values()]
            out["parity_ok"] = all(c is True for c in checks)
    else:
        out["calls_made"] = dict(CALLS)
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out), flush=True)
    if out.get("parity_ok") is False:
        sys.exit(1)


if __name__ == "__main__":
    main()
