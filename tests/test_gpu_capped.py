"""The grid-capped fused call (zr_reduce_scatter_adam_capped) against the
oracle and, bit for bit, against the uncapped call: random small plans with
caps from one workgroup to more than the tiles, the every-partition form per
bucket, and a GPT-2-small rank share at full size."""

import random

import numpy as np
import pytest

from oracle.adam import adam_oracle
from oracle.bf16 import bf16_rne_oracle
from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load
from zero_partition_aware_amd import workloads

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import (assert_bits_equal, assert_within, empty_f32,  # noqa: E402
                        host_f32, host_u16, to_dev)

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _draw(rng, n, is_bf16, sigma):
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    if is_bf16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x


def _case(seed):
    rng = random.Random(seed)
    R = rng.choice([2, 3, 4, 8, 12])
    sp = rng.choice([d for d in (1, 2, 4) if R % d == 0])
    n = rng.randint(1, 10)
    numels = [rng.choice([1, 17, rng.randint(1, 40000)]) for _ in range(n)]
    B = rng.choice([1000, 7777, 1 << 30])
    return numels, [0] * n, [(R, sp)], B


def _state(rng, n, total_real):
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    th[total_real:] = m[total_real:] = v[total_real:] = 0.0
    return th, m, v


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("is_bf16", [False, True])
@pytest.mark.parametrize("cap", [1, 3, 64, 1 << 30])
def test_capped_equals_uncapped_and_oracle(seed, is_bf16, cap):
    numels, pg, groups, B = _case(300 + seed)
    ref = plan_oracle(numels, pg, groups, B)
    plan = zr.zr_plan_buckets(numels, pg, groups, B)
    info = ref.groups[0]
    P, R, T = info.part_numel, info.world, info.total
    rng = np.random.default_rng(seed)
    reps = [_draw(rng, T, is_bf16, 1e-3) for _ in range(R)]
    dreps = [to_dev(x, seed % 3) for x in reps]
    want_g = reduce_scatter_oracle(ref, 0, reps, is_bf16)
    for k in sorted({0, R // 2, R - 1}):
        th, m, v = _state(rng, P, max(0, min(P, T - k * P)))
        outs = {}
        for name in ("capped", "uncapped"):
            dth, dm, dv = to_dev(th), to_dev(m), to_dev(v)
            pb = torch.zeros(P, dtype=torch.bfloat16, device="cuda")
            go = empty_f32(P)
            if name == "capped":
                zr.zr_reduce_scatter_adam_capped(plan, 0, -1, k, dreps, dth, dm, dv, pb, go,
                                                 max_workgroups=cap, step=2, **HP)
            else:
                zr.zr_reduce_scatter_adam(plan, 0, -1, k, dreps, dth, dm, dv, pb, go,
                                          step=2, **HP)
            outs[name] = [host_f32(t) for t in (go, dth, dm, dv)] + [host_u16(pb)]
        for a, b, nm in zip(outs["capped"], outs["uncapped"], ("grad", "master", "m", "v", "bf16")):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
                f"{nm} of partition {k}: capped ({cap}) vs uncapped"
        got = outs["capped"]
        assert_bits_equal(got[0], want_g[k], f"grad of partition {k} vs oracle")
        w_th, w_m, w_v = adam_oracle(want_g[k], th, m, v, step=2, **HP)
        assert_within(got[1], w_th, what="master vs oracle")
        assert_within(got[2], w_m, what="m vs oracle")
        assert_within(got[3], w_v, atol=0.0, what="v vs oracle")
        assert np.array_equal(got[4], bf16_rne_oracle(got[1]))


@pytest.mark.parametrize("cap", [2, 256])
def test_capped_every_partition_per_bucket(cap):
    """dst = -1, one capped call per bucket, equals the oracle on every
    partition."""
    numels = [37, 64 * 33, 129, 5000, 3]
    ref = plan_oracle(numels, [0] * 5, [(4, 1)], 1000)
    plan = zr.zr_plan_buckets(numels, [0] * 5, [(4, 1)], 1000)
    info = ref.groups[0]
    P, R, L, T = info.part_numel, info.world, info.padded, info.total
    rng = np.random.default_rng(7)
    reps = [_draw(rng, T, False, 1.0) for _ in range(R)]
    dreps = [to_dev(x) for x in reps]
    want_g = reduce_scatter_oracle(ref, 0, reps, False)
    th, m, v = _state(rng, L, T)
    ath, am, av, ago = to_dev(th), to_dev(m), to_dev(v), empty_f32(L)
    apb = torch.zeros(L, dtype=torch.bfloat16, device="cuda")
    for b in range(ref.num_buckets):
        zr.zr_reduce_scatter_adam_capped(plan, 0, b, -1, dreps, ath, am, av, apb, ago,
                                         max_workgroups=cap, step=2, **HP)
    got = [host_f32(t) for t in (ago, ath, am, av)] + [host_u16(apb)]
    for k in range(R):
        sl = slice(k * P, (k + 1) * P)
        assert_bits_equal(got[0][sl], want_g[k], f"grad of partition {k}")
        w_th, w_m, w_v = adam_oracle(want_g[k], th[sl], m[sl], v[sl], step=2, **HP)
        assert_within(got[1][sl], w_th, what=f"master of partition {k}")
        assert_within(got[2][sl], w_m, what=f"m of partition {k}")
        assert_within(got[3][sl], w_v, atol=0.0, what=f"v of partition {k}")
        assert np.array_equal(got[4][sl], bf16_rne_oracle(got[1][sl]))


def test_capped_gpt2_small_rank_share_equals_uncapped():
    """Full GPT-2-small share of the last rank (8 bf16 replicas, 15.55M
    elements): a 256-workgroup launch gives the uncapped launch's results
    bit for bit."""
    w = workloads.get("gpt2-small")
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    T, L, P, D = zr.zr_plan_group_info(plan, 0)
    R, k = 8, 7
    reps = [workloads.device_normal(workloads.seed_for("gpt2-small", r), T, w.grad_sigma,
                                    "cuda", "bf16") for r in range(R)]
    master0 = workloads.device_normal(workloads.seed_for("gpt2-small", k, master=True), P,
                                      w.master_sigma, "cuda")
    res = []
    for cap in (None, 256):
        th, m, v = master0.clone(), torch.zeros(P, device="cuda"), torch.zeros(P, device="cuda")
        pb = torch.empty(P, dtype=torch.bfloat16, device="cuda")
        go = torch.empty(P, device="cuda")
        if cap is None:
            zr.zr_reduce_scatter_adam(plan, 0, -1, k, reps, th, m, v, pb, go, **HP)
        else:
            zr.zr_reduce_scatter_adam_capped(plan, 0, -1, k, reps, th, m, v, pb, go,
                                             max_workgroups=cap, **HP)
        res.append((go, th, m, v, pb))
    torch.cuda.synchronize()
    for a, b, nm in zip(res[0], res[1], ("grad", "master", "m", "v", "bf16")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
