"""The XCD-weighted tile order of the reduce kernels.  Selections of 2 or more
replicas hand their tiles out in cycles of 256 workgroups of which the 4
odd-slot ones of the last 8 take no tile; a launch ends after the workgroup
that holds its last tile.  Launches whose tile counts end at every kind of
place in a cycle (first workgroup, mid-cycle, the last 8 with and without
their idle slots) must give, element by element, what the grid-capped call
(equal shares, a grid-stride walk) gives and the oracle: reduced gradient
bit-exact, Adam within rel 1e-6 / abs 1e-7 (v relative only), bf16 param =
RNE of the kernel's own master.  Fused bf16 and fp32 and the bf16
reduce-scatter at 8 replicas; fused fp32 and the fp32 reduce-scatter at 2."""

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
from tests._gpu import assert_bits_equal, assert_within, host_f32, host_u16  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
DEV = "cuda"
CYCLE = 252            # tiles per cycle of 256 workgroups


def _partition_for_tiles(tiles, tile):
    # a one-segment selection of n elements spans (n + 63 + tile - 1) // tile
    # tiles; the largest such n for the given count
    return tiles * tile - 63


@pytest.mark.parametrize("R,is_bf16,fused", [(8, False, True), (8, True, True), (8, True, False),
                                            (2, False, True), (2, False, False)])
@pytest.mark.parametrize("rem", [1, 100, 247, 248, 249, 251, 252])
def test_every_cycle_tail_matches_equal_shares_and_oracle(R, is_bf16, fused, rem):
    tile = 512 if is_bf16 and fused else 256
    tiles = 2 * CYCLE + rem
    P = _partition_for_tiles(tiles, tile)
    assert (P + 63 + tile - 1) // tile == tiles
    numels = [R * P]
    ref = plan_oracle(numels, [0], [(R, 1)], 1 << 40)
    plan = zr.zr_plan_buckets(numels, [0], [(R, 1)], 1 << 40)
    assert ref.groups[0].part_numel == P
    dst = min(3, R - 1)
    lo = dst * P
    dt = "bf16" if is_bf16 else "fp32"
    seed = 700 + rem + (10 if is_bf16 else 0) + (20 if fused else 0) + (1000 if R == 2 else 0)
    wins = [workloads.device_normal(seed * 100 + r, P, 1e-3, DEV, dt) for r in range(R)]
    reps = [(w, lo) for w in wins]
    xs = [host_u16(w) if is_bf16 else host_f32(w) for w in wins]
    want = reduce_scatter_oracle(ref, 0, xs, is_bf16, dst=dst, flat_bases=[lo] * R)[dst]
    if not fused:
        out = torch.full((P,), float("nan"), device=DEV)
        zr.zr_reduce_scatter_local(plan, 0, -1, dst, reps, [out])
        assert_bits_equal(host_f32(out), want, "reduced partition")
        return
    master0 = workloads.device_normal(seed * 100 + 99, P, 0.02, DEV)
    th0 = host_f32(master0)
    outs = {}
    for name, cap in (("weighted", None), ("equal", 1 << 20)):
        master = master0.clone()
        m, v = torch.zeros(P, device=DEV), torch.zeros(P, device=DEV)
        pb = torch.empty(P, dtype=torch.bfloat16, device=DEV)
        go = torch.full((P,), float("nan"), device=DEV)
        if cap is None:
            zr.zr_reduce_scatter_adam(plan, 0, -1, dst, reps, master, m, v, pb, go, **HP)
        else:
            zr.zr_reduce_scatter_adam_capped(plan, 0, -1, dst, reps, master, m, v, pb, go,
                                             max_workgroups=cap, **HP)
        outs[name] = [host_f32(go), host_f32(master), host_f32(m), host_f32(v), host_u16(pb)]
    for a, b, what in zip(outs["weighted"], outs["equal"], ["grad", "master", "m", "v", "bf16"]):
        if what == "bf16":
            assert np.array_equal(a, b), what
        else:
            assert_bits_equal(a, b, what + " (weighted vs equal shares)")
    g, th, mm, vv, pbh = outs["weighted"]
    assert_bits_equal(g, want, "reduced gradient")
    z = np.zeros(P, np.float32)
    w_th, w_m, w_v = adam_oracle(want, th0, z, z, step=1, **HP)
    assert_within(th, w_th, what="master")
    assert_within(mm, w_m, what="m")
    assert_within(vv, w_v, atol=0.0, what="v")
    assert np.array_equal(pbh, bf16_rne_oracle(th)), "bf16 param"
