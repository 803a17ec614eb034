"""Parameter all-gather and the ring all-gather step against the oracle
(bit-exact: pure data movement)."""

import random

import numpy as np
import pytest

from oracle.allgather import all_gather_window_oracle
from oracle.plan import plan_oracle
from oracle.ring import ring_all_gather_oracle, ring_reduce_scatter_oracle
from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, host_f32, host_u16, to_dev  # noqa: E402


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("bf16", [False, True])
def test_all_gather_params_windows(seed, bf16):
    rng = random.Random(seed)
    R = rng.choice([1, 2, 3, 4, 8, 16])
    numels = [rng.randint(1, 9000) for _ in range(rng.randint(1, 6))]
    align = rng.choice([1, 4])
    ref = plan_oracle(numels, [0] * len(numels), [(R, 1)], 1 << 30, align)
    plan = zr.zr_plan_buckets(numels, [0] * len(numels), [(R, 1)], 1 << 30, 0, align)
    info = ref.groups[0]
    T, P = info.total, info.part_numel
    nrng = np.random.default_rng(seed)
    if bf16:
        parts = [nrng.integers(0, 1 << 16, size=P).astype(np.uint16) for _ in range(R)]
    else:
        parts = [nrng.standard_normal(P).astype(np.float32) for _ in range(R)]
    dparts = [to_dev(x, (k + seed) % 3) for k, x in enumerate(parts)]
    for base, length in [(0, T), (min(T - 1, 5), max(1, T // 3)), (T // 2, T - T // 2), (T - 1, 1)]:
        length = min(length, T - base)
        want = all_gather_window_oracle(parts, T, base, length)
        dt = torch.bfloat16 if bf16 else torch.float32
        out = torch.zeros(length + 8, dtype=dt, device="cuda")[seed % 2: seed % 2 + length]
        zr.zr_all_gather_params(plan, 0, dparts, out, out_base=base)
        got = host_u16(out) if bf16 else host_f32(out)
        if bf16:
            assert np.array_equal(got, want), (base, length)
        else:
            assert_bits_equal(got, want, f"window {base}+{length}")


def test_all_gather_rejects_window_past_real_elements():
    plan = zr.zr_plan_buckets([10], [0], [(4, 1)], 100)      # T = 10, L = 12
    parts = [to_dev(np.zeros(3, np.float32)) for _ in range(4)]
    out = torch.zeros(12, device="cuda")
    with pytest.raises(zr.ZrError, match="real elements"):
        zr.zr_all_gather_params(plan, 0, parts, out, out_base=0, out_len=12)


@pytest.mark.parametrize("n,chunk", [(8, 4096 * 3 + 5), (3, 1000), (2, 7)])
def test_ring_all_reduce_steps(n, chunk):
    rng = np.random.default_rng(n)
    bufs = [rng.standard_normal(n * chunk).astype(np.float32) for _ in range(n)]
    dev = [to_dev(b) for b in bufs]
    for s in range(n - 1):
        zr.zr_ring_rs_step(dev, chunk, s)
    for s in range(n - 1):
        zr.zr_ring_ag_step(dev, chunk, s)
    rs, _ = ring_reduce_scatter_oracle(bufs)
    want, _ = ring_all_gather_oracle(rs)
    for k in range(n):
        assert_bits_equal(host_f32(dev[k]), want[k], f"rank {k}")


def test_ring_all_reduce_integer_equals_sum_everywhere():
    n, chunk = 8, 3000
    rng = np.random.default_rng(1)
    bufs = [rng.integers(-999, 999, size=n * chunk).astype(np.float32) for _ in range(n)]
    dev = [to_dev(b) for b in bufs]
    for s in range(n - 1):
        zr.zr_ring_rs_step(dev, chunk, s)
    for s in range(n - 1):
        zr.zr_ring_ag_step(dev, chunk, s)
    total = sum(b.astype(np.int64) for b in bufs).astype(np.float32)
    for k in range(n):
        assert np.array_equal(host_f32(dev[k]), total)


# Rank buffers starting at different offsets within a 16-byte line: no phase
# aligns a chunk of one rank with the same chunk of the previous one, so the
# steps take their dword-aligned variants.  RS then AG against the oracle.
@pytest.mark.parametrize("n,chunk", [(8, 4096 * 2 + 3), (3, 999)])
def test_ring_steps_with_misaligned_rank_buffers(n, chunk):
    rng = np.random.default_rng(100 + n)
    bufs = [rng.standard_normal(n * chunk).astype(np.float32) for _ in range(n)]
    dev = [to_dev(b, k % 4) for k, b in enumerate(bufs)]
    for s in range(n - 1):
        zr.zr_ring_rs_step(dev, chunk, s)
    rs, _ = ring_reduce_scatter_oracle(bufs)
    for k in range(n):
        assert_bits_equal(host_f32(dev[k]), rs[k], f"rank {k} after reduce-scatter")
    for s in range(n - 1):
        zr.zr_ring_ag_step(dev, chunk, s)
    want, _ = ring_all_gather_oracle(rs)
    for k in range(n):
        assert_bits_equal(host_f32(dev[k]), want[k], f"rank {k} after all-gather")
