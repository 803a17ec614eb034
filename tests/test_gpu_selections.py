"""Large rank selections of one to three segments -- one slice, a slice plus
the last partition's padding, a share cut by a bucket border -- checked on
every element against the oracle, fused and unfused, bf16 and fp32, with 4,
8 and 16 replicas (all in the XCD-weighted order), including
selections cut into several launches (a launch carries at most ~2 GiB of
traffic).  Reduced gradients bit-exact; Adam within rel 1e-6 / abs 1e-7 (v
relative only); bf16 param = RNE of the kernel's own master.

The launch shape follows from the library's rules, stated here so the cases
can be checked by hand: a tile is 512 elements for the bf16 fused step and
256 otherwise, a segment of n elements spans (n + 63 + tile - 1) // tile
tiles, and a selection of T tiles moving b bytes per tile is cut into
ceil(T / floor(2^31 / b)) equal launches."""

import gc

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


def _tiles(n, tile):
    return (n + 63 + tile - 1) // tile


def _launch_split(total_tiles, tile_bytes):
    per = (2 ** 31) // tile_bytes
    nl = -(-total_tiles // per)
    return nl, -(-total_tiles // nl)


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(numels, R, B, dst, is_bf16, fused, seed, expect_segs, expect_launches):
    ref = plan_oracle(numels, [0] * len(numels), [(R, 1)], B)
    plan = zr.zr_plan_buckets(numels, [0] * len(numels), [(R, 1)], B)
    info = ref.groups[0]
    T, P = info.total, info.part_numel
    # the case is what it claims to be (derived from the oracle plan)
    segs = [s for s in ref.slices if s.dst == dst]
    pad = max(0, min(P, (dst + 1) * P - T))
    nseg = len(segs) + (1 if pad else 0)
    assert nseg == expect_segs
    s_in = 2 if is_bf16 else 4
    tile = 512 if is_bf16 and fused else 256
    tiles = sum(_tiles(s.numel, tile) for s in segs) + (_tiles(pad, tile) if pad else 0)
    tile_bytes = tile * (R * s_in + (30 if fused else 4))
    nl, _ = _launch_split(tiles, tile_bytes)
    assert nl == expect_launches
    # the library's own launch-shape query agrees (fused calls here write grad_out)
    nb = zr.zr_plan_num_buckets(plan)
    assert zr.zr_plan_reduce_launches(plan, 0, 0, nb, dst, "bf16" if is_bf16 else "fp32",
                                      fused, fused) == (tiles, nl)
    # replica windows of partition dst, drawn on the device from seeds
    lo, n_real = dst * P, min(P, max(0, T - dst * P))
    dt = "bf16" if is_bf16 else "fp32"
    wins = [workloads.device_normal(seed * 100 + r, n_real, 1e-3, DEV, dt) for r in range(R)]
    reps = [(w, lo) for w in wins]
    xs = [host_u16(w) if is_bf16 else host_f32(w) for w in wins]
    want = reduce_scatter_oracle(ref, 0, xs, is_bf16, dst=dst, flat_bases=[lo] * R)[dst]
    assert not np.isnan(want).any()
    if not fused:
        out = torch.full((P,), float("nan"), device=DEV)
        zr.zr_reduce_scatter_local(plan, 0, -1, dst, reps, [out])
        assert_bits_equal(host_f32(out), want, "reduced partition")
        return
    master = workloads.device_normal(seed * 100 + 99, P, 0.02, DEV)
    th = host_f32(master)
    th[n_real:] = 0.0
    master[n_real:] = 0.0
    m, v = torch.zeros(P, device=DEV), torch.zeros(P, device=DEV)
    pbf16 = torch.empty(P, dtype=torch.bfloat16, device=DEV)
    gout = torch.empty(P, device=DEV)
    zr.zr_reduce_scatter_adam(plan, 0, -1, dst, reps, master, m, v, pbf16, gout, **HP)
    assert_bits_equal(host_f32(gout), want, "reduced gradient")
    z = np.zeros(P, np.float32)
    w_th, w_m, w_v = adam_oracle(want, th, z, z, step=1, **HP)
    g_th = host_f32(master)
    assert_within(g_th, w_th, what="master")
    assert_within(host_f32(m), w_m, what="m")
    assert_within(host_f32(v), w_v, atol=0.0, what="v")
    assert np.array_equal(host_u16(pbf16), bf16_rne_oracle(g_th)), "bf16 param"


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("is_bf16", [False, True])
def test_one_segment(fused, is_bf16):
    # one param of 4 x 9,000,000: partition 1 is one slice (35,157 tiles of
    # 256 elements, 17,579 of 512 for the bf16 fused step)
    _run([36_000_000], 4, 1 << 40, 1, is_bf16, fused, 1, 1, 1)
    _free()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("is_bf16", [False, True])
def test_two_segments_slice_and_padding(fused, is_bf16):
    # the last partition: a slice of 8,999,994 elements and 6 of padding
    _run([36_000_000 - 6], 4, 1 << 40, 3, is_bf16, fused, 2, 2, 1)
    _free()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("is_bf16", [False, True])
def test_two_segments_cut_by_a_bucket_border(fused, is_bf16):
    # partition 1 = [9M, 18M) is cut by the bucket border at 13.5M
    _run([36_000_000], 4, 13_500_000, 1, is_bf16, fused, 3, 2, 1)
    _free()


@pytest.mark.parametrize("is_bf16", [False, True])
def test_eight_replicas_weighted_order(is_bf16):
    # 8 replicas of 8,389,000 elements, fused and not
    _run([8 * 8_389_000], 8, 1 << 40, 5, is_bf16, True, 4, 1, 1)
    _run([8 * 8_389_000], 8, 1 << 40, 6, is_bf16, False, 5, 1, 1)
    _free()


@pytest.mark.parametrize("is_bf16", [False, True])
def test_sixteen_replicas(is_bf16):
    # 16 replicas of 4,000,000 elements (15,626 tiles of 256, 7,813 of 512),
    # fused and not, in the 16-replica kernels
    _run([16 * 4_000_000], 16, 1 << 40, 9, is_bf16, True, 8, 1, 1)
    _run([16 * 4_000_000], 16, 1 << 40, 14, is_bf16, False, 9, 1, 1)
    _free()


def test_two_launches_one_segment():
    # fp32, 8 replicas, 40M-element partition: 156,251 tiles of 15,872 bytes
    # (fused, reduced gradient written) -> two launches of 78,126 tiles
    _run([8 * 40_000_000], 8, 1 << 40, 2, False, True, 6, 1, 2)
    _free()


def test_two_launches_three_segments():
    # the last partition cut by a bucket border, plus 10 elements of padding
    _run([8 * 40_000_000 - 10], 8, 290_000_000, 7, False, True, 7, 3, 2)
    _free()
