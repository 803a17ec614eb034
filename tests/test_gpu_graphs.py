"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) replay to the
same bits as the same calls made eagerly: the bucketed step (one
reduce-scatter per bucket and group into a rank's gradient partition, then
Adam on each partition) is captured once and replayed several times, with
eager library work between the replays, each replay starting from the same
state as the eager reference."""

import numpy as np
import pytest

from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, host_f32, host_u16, to_dev  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def test_bucketed_step_graph_replays_equal_eager():
    rng = np.random.default_rng(3)
    numels = [int(x) for x in rng.integers(1, 9000, size=40)]
    pg = [int(x) for x in rng.integers(0, 2, size=40)]
    groups = [(4, 2), (2, 1)]
    plan = zr.zr_plan_buckets(numels, pg, groups, 3000)
    nb = zr.zr_plan_num_buckets(plan)
    k = 1
    state = []
    for g, (R, _) in enumerate(groups):
        T, _, P, _ = zr.zr_plan_group_info(plan, g)
        reps = [to_dev((rng.standard_normal(T) * 1e-3).astype(np.float32)) for _ in range(R)]
        state.append(dict(reps=reps, P=P,
                          master=to_dev((rng.standard_normal(P) * 0.02).astype(np.float32)),
                          m=to_dev((rng.standard_normal(P) * 1e-4).astype(np.float32)),
                          v=to_dev(np.abs(rng.standard_normal(P) * 1e-8).astype(np.float32)),
                          grad=torch.empty(P, device="cuda"),
                          pbf16=torch.empty(P, dtype=torch.bfloat16, device="cuda")))
    pairs = []
    for b in range(nb):
        sl = zr.zr_plan_slices(plan, b)
        for g in range(len(groups)):
            if b == nb - 1 or any(s[1] == g and s[2] == k for s in sl):
                pairs.append((b, g))
    assert len(pairs) > 20

    def step():
        for b, g in pairs:
            st = state[g]
            zr.zr_reduce_scatter_local(plan, g, b, k, st["reps"], [st["grad"]])
        for st in state:
            zr.zr_adam_partition(st["grad"], st["master"], st["m"], st["v"], st["pbf16"],
                                 step=2, **HP)

    keys = ("master", "m", "v", "grad", "pbf16")
    start = [{key: st[key].clone() for key in keys} for st in state]

    def restore():
        for st, s0 in zip(state, start):
            for key in keys:
                st[key].copy_(s0[key])

    def snapshot():
        torch.cuda.synchronize()
        return [{key: (host_u16(st[key]) if key == "pbf16" else host_f32(st[key]).copy())
                 for key in keys} for st in state]

    step()
    want = snapshot()

    restore()
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        step()
    torch.cuda.synchronize()

    other = torch.empty(state[0]["P"], device="cuda")
    for replay in range(3):
        restore()
        # Eager library work between replays (not part of the graph).
        zr.zr_reduce_scatter_local(plan, 0, -1, 0, state[0]["reps"], [other])
        cg.replay()
        got = snapshot()
        for g, (gw, gg) in enumerate(zip(want, got)):
            for key in keys:
                what = f"replay {replay}, group {g}, {key}"
                if key == "pbf16":
                    assert np.array_equal(gg[key], gw[key]), what
                else:
                    assert_bits_equal(gg[key], gw[key], what)
