"""Bucket-range calls (zr_reduce_scatter_local_range, zr_reduce_scatter_adam_range):
random plans cut into random ranges of consecutive buckets must give, bit for
bit, what one call per bucket gives, and the oracle's reduce-scatter; fused and
unfused, every destination, bf16 and fp32, pointers off by an element."""

import random

import numpy as np
import pytest

from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, empty_f32, host_f32, host_u16, to_dev  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _case(seed):
    rng = random.Random(seed)
    groups = [(rng.choice([2, 3, 4, 8]), 1) for _ in range(rng.choice([1, 2]))]
    n = rng.randint(2, 10)
    numels = [rng.choice([17, rng.randint(1, 40000)]) for _ in range(n)]
    pg = [rng.randrange(len(groups)) for _ in range(n)]
    B = rng.choice([777, 5000, 12345])
    return rng, numels, pg, groups, B


def _draw(nprng, n, is_bf16):
    x = (nprng.standard_normal(n) * 1e-2).astype(np.float32)
    if is_bf16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("is_bf16", [False, True])
def test_ranges_equal_per_bucket_calls_and_oracle(seed, is_bf16):
    rng, numels, pg, groups, B = _case(seed)
    ref = plan_oracle(numels, pg, groups, B)
    plan = zr.zr_plan_buckets(numels, pg, groups, B)
    nb = ref.num_buckets
    cuts = sorted(rng.sample(range(1, nb), min(nb - 1, rng.randint(1, 4)))) if nb > 1 else []
    ranges = list(zip([0] + cuts, cuts + [nb]))
    nprng = np.random.default_rng(seed)
    off = seed % 2
    for g, info in enumerate(ref.groups):
        R, P = info.world, info.part_numel
        if info.total == 0:              # a group no param belongs to
            continue
        xs = [_draw(nprng, info.total, is_bf16) for _ in range(R)]
        reps = [to_dev(x, off) for x in xs]
        want = reduce_scatter_oracle(ref, g, xs, is_bf16)
        for dst in sorted({0, R - 1, -1}):
            ks = range(R) if dst < 0 else [dst]
            # unfused: ranges vs one call per bucket vs the oracle
            by_range = [empty_f32(P, off) for _ in ks]
            by_bucket = [empty_f32(P, off) for _ in ks]
            for a, b in ranges:
                zr.zr_reduce_scatter_local_range(plan, g, a, b - a, dst, reps, by_range)
            for bk in range(nb):
                zr.zr_reduce_scatter_local(plan, g, bk, dst, reps, by_bucket)
            for i, k in enumerate(ks):
                got = host_f32(by_range[i])
                assert_bits_equal(got, host_f32(by_bucket[i]), f"group {g} dst {k}: range vs bucket")
                assert_bits_equal(got, want[k], f"group {g} dst {k}: range vs oracle")
            # fused: ranges vs one call per bucket, every output bitwise
            n = P if dst >= 0 else info.padded
            th = (nprng.standard_normal(n) * 0.02).astype(np.float32)
            if dst < 0:
                th[info.total:] = 0.0
            elif (dst + 1) * P > info.total:
                th[max(0, info.total - dst * P):] = 0.0
            outs = []
            for mode in ("range", "bucket"):
                st = [to_dev(th, off), to_dev(np.zeros(n, np.float32), off),
                      to_dev(np.zeros(n, np.float32), off)]
                pb = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
                go = empty_f32(n, off)
                if mode == "range":
                    for a, b in ranges:
                        zr.zr_reduce_scatter_adam_range(plan, g, a, b - a, dst, reps, *st, pb, go,
                                                        step=2, **HP)
                else:
                    for bk in range(nb):
                        zr.zr_reduce_scatter_adam(plan, g, bk, dst, reps, *st, pb, go, step=2, **HP)
                outs.append([host_f32(t) for t in st] + [host_u16(pb), host_f32(go)])
            for name, x, y in zip(("master", "m", "v"), outs[0][:3], outs[1][:3]):
                assert_bits_equal(x, y, f"group {g} dst {dst}: fused range vs bucket, {name}")
            assert np.array_equal(outs[0][3], outs[1][3])
            assert_bits_equal(outs[0][4], outs[1][4], f"group {g} dst {dst}: reduced gradient")
            for i, k in enumerate(ks):
                seg = outs[0][4][i * P:(i + 1) * P] if dst < 0 else outs[0][4]
                assert_bits_equal(seg, want[k], f"group {g} dst {k}: fused range vs oracle")
