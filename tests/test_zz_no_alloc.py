"""The no-allocation fused call (zr_reduce_scatter_adam_noalloc) against the
allocating one (zr_reduce_scatter_adam): same selection, same inputs, separate
copies of the state; every output bit for bit, and the reduced gradient
against the oracle.  Two calls in a row, the second with a smaller input, so
the second stages a shorter table over what the first left in the array."""

import numpy as np
import pytest

from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load
from zero_partition_aware_amd import workloads

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, host_f32, to_dev  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _case(numels, R, B, dst, is_bf16, seed, bucket=-1, offset=0):
    """Runs one selection through both entry points; returns the segment count
    the selection stages (merged slices + padding segments)."""
    rng = np.random.default_rng(seed)
    ref = plan_oracle(numels, [0] * len(numels), [(R, 1)], B)
    plan = zr.zr_plan_buckets(numels, [0] * len(numels), [(R, 1)], B)
    info = ref.groups[0]
    T, P, L = info.total, info.part_numel, info.padded
    xs = []
    for _ in range(R):
        x = (rng.standard_normal(T) * 1e-3).astype(np.float32)
        if is_bf16:
            x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        xs.append(x)
    reps = [to_dev(x, offset) for x in xs]
    n = L if dst < 0 else P
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    mm = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    vv = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    outs = {}
    for fn in (zr.zr_reduce_scatter_adam, zr.zr_reduce_scatter_adam_noalloc):
        st = [to_dev(th), to_dev(mm), to_dev(vv)]
        pb = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        go = torch.full((n,), float("nan"), device="cuda")
        fn(plan, 0, bucket, dst, reps, *st, pb, go, step=3, **HP)
        torch.cuda.synchronize()
        outs[fn.__name__] = [host_f32(t) for t in st] + [pb.cpu().view(torch.int16).numpy(),
                                                           host_f32(go)]
    a, b = outs["zr_reduce_scatter_adam"], outs["zr_reduce_scatter_adam_noalloc"]
    for name, x, y in zip(("master", "m", "v"), a[:3], b[:3]):
        assert_bits_equal(y, x, f"{name} (no-allocation call vs allocating call)")
    assert np.array_equal(a[3], b[3]), "bf16 param differs"
    assert_bits_equal(b[4], a[4], "reduced gradient (no-allocation vs allocating)")
    want = reduce_scatter_oracle(ref, 0, xs, is_bf16, bucket=bucket, dst=dst)
    for k, part in want.items():
        got = b[4][k * P:(k + 1) * P] if dst < 0 else b[4]
        sel = ~np.isnan(part)
        assert_bits_equal(got[sel], part[sel], f"reduced partition {k} vs oracle")
    segs = sum(1 for s in ref.slices if (dst < 0 or s.dst == dst)
               and (bucket < 0 or s.bucket == bucket))
    return segs


def test_noalloc_equals_allocating_call_twice_second_smaller():
    # first call: every partition of a many-slice plan (hundreds of segments,
    # several staging launches), bf16 replicas one element off
    n1 = _case([30011, 17, 12345, 7777, 40000, 3, 999], 8, 613, -1, True, 1, offset=1)
    assert n1 > 128
    # second call: a smaller input and a shorter table over the first's
    n2 = _case([1000, 333], 4, 450, 1, False, 2)
    assert 0 < n2 < n1


def test_noalloc_single_bucket_and_large_selection():
    # one bucket of a rank's selection, then a large two-segment selection
    # (the last partition's slice and its padding, 8.4M elements)
    _case([70000, 5000, 33], 4, 20000, 2, False, 3, bucket=1)
    _case([4 * 8400000], 4, 1 << 40, 3, True, 4)
