"""Stream ordering and host-thread safety of the C ABI.

Every kernel is enqueued on the caller's stream (here a non-default torch
stream); the plan's launch tables are built on first use under a lock, so
several host threads may call into one plan at once."""

import threading

import numpy as np
import pytest

from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, empty_f32, host_f32, to_dev  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _case():
    numels = [5000, 1234, 777, 9000]
    groups = [(4, 1)]
    ref = plan_oracle(numels, [0] * 4, groups, 3000)
    rng = np.random.default_rng(0)
    reps = [(rng.standard_normal(ref.groups[0].total) * 1e-2).astype(np.float32) for _ in range(4)]
    return numels, groups, ref, reps


def test_side_stream_work_is_ordered():
    numels, groups, ref, reps = _case()
    plan = zr.zr_plan_buckets(numels, [0] * 4, groups, 3000)
    want = reduce_scatter_oracle(ref, 0, reps, False)
    P = ref.groups[0].part_numel
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dreps = [to_dev(x) for x in reps]
        outs = [torch.full((P,), float("nan"), device="cuda") for _ in range(4)]
        # a long producer on the same stream, then the reduction, then a consumer
        for k in range(4):
            zr.zr_reduce_scatter_local(plan, 0, -1, k, dreps, [outs[k]])
        copies = [o.clone() for o in outs]
    s.synchronize()
    for k in range(4):
        assert_bits_equal(host_f32(copies[k]), want[k], f"dst {k}")


def test_concurrent_host_threads_share_one_plan():
    numels, groups, ref, reps = _case()
    plan = zr.zr_plan_buckets(numels, [0] * 4, groups, 3000)
    want = reduce_scatter_oracle(ref, 0, reps, False)
    P = ref.groups[0].part_numel
    dreps = [to_dev(x) for x in reps]
    torch.cuda.synchronize()
    n_threads = 8
    results, errors = {}, []
    barrier = threading.Barrier(n_threads)

    def worker(t):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [empty_f32(P) for _ in range(4)]
                barrier.wait()
                for b in [-1] + list(range(zr.zr_plan_num_buckets(plan))):
                    for k in range(4):
                        zr.zr_reduce_scatter_local(plan, 0, b, k, dreps, [outs[k]])
            s.synchronize()
            results[t] = [host_f32(o) for o in outs]
        except Exception as e:  # noqa: BLE001
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    assert len(results) == n_threads
    for t, outs in results.items():
        for k in range(4):
            assert_bits_equal(outs[k], want[k], f"thread {t} dst {k}")
