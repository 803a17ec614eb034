"""Prepared fused calls (arguments marshalled once, bucket and step per call)
give the direct calls' results bit for bit, uncapped and grid-capped, over
every bucket and two Adam steps; and the direct results equal the oracle."""

import numpy as np
import pytest

from oracle.adam import adam_oracle
from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, assert_within, empty_f32, host_f32, to_dev  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


@pytest.mark.parametrize("cap", [0, 3])
@pytest.mark.parametrize("dst", [1, -1])
def test_prepared_equals_direct(cap, dst):
    numels = [37, 64 * 33, 129, 9000, 5]
    groups = [(4, 1)]
    ref = plan_oracle(numels, [0] * 5, groups, 1000)
    plan = zr.zr_plan_buckets(numels, [0] * 5, groups, 1000)
    info = ref.groups[0]
    P, R, L, T = info.part_numel, info.world, info.padded, info.total
    n = P if dst >= 0 else L
    rng = np.random.default_rng(11)
    reps = [(rng.standard_normal(T) * 1e-3).astype(np.float32) for _ in range(R)]
    dreps = [to_dev(x, 1) for x in reps]
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    real = T - dst * P if dst >= 0 else T
    th[max(0, min(n, real)):] = 0.0
    outs = {}
    for how in ("prepared", "direct"):
        dth, dm, dv = to_dev(th), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
        pb = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        go = empty_f32(n)
        call = zr.prepare_reduce_scatter_adam(plan, 0, dst, dreps, dth, dm, dv, pb, go,
                                              max_workgroups=cap, **HP)
        for step in (1, 2):
            for b in range(ref.num_buckets):
                if how == "prepared":
                    call(b, step)
                elif cap:
                    zr.zr_reduce_scatter_adam_capped(plan, 0, b, dst, dreps, dth, dm, dv, pb, go,
                                                     max_workgroups=cap, step=step, **HP)
                else:
                    zr.zr_reduce_scatter_adam(plan, 0, b, dst, dreps, dth, dm, dv, pb, go,
                                              step=step, **HP)
        outs[how] = [host_f32(t) for t in (go, dth, dm, dv)] + [
            pb.cpu().view(torch.int16).numpy()]
    for a, b_, nm in zip(outs["prepared"], outs["direct"], ("grad", "master", "m", "v", "bf16")):
        assert np.array_equal(a.view(np.uint8), b_.view(np.uint8)), f"{nm}: prepared vs direct"
    # two steps of the same gradient against the oracle
    want = reduce_scatter_oracle(ref, 0, reps, False)
    g = want[dst] if dst >= 0 else np.concatenate([want[d] for d in range(R)])
    w_th, w_m, w_v = adam_oracle(g, th, np.zeros(n, np.float32), np.zeros(n, np.float32),
                                 step=1, **HP)
    w_th, w_m, w_v = adam_oracle(g, w_th, w_m, w_v, step=2, **HP)
    got = outs["direct"]
    assert_bits_equal(got[0], g, "grad vs oracle")
    assert_within(got[1], w_th, what="master vs oracle")
    assert_within(got[2], w_m, what="m vs oracle")
    assert_within(got[3], w_v, atol=0.0, what="v vs oracle")
