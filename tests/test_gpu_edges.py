"""GPU edge cases: the kernel's bf16 rounding on a stratified sample of all
2^32 fp32 patterns, checkpoint/resume, empty selections, bucket-size
invariance of the reduced partitions."""

import numpy as np
import pytest

from oracle.bf16 import bf16_rne_oracle
from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, empty_f32, host_f32, host_u16, to_dev  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def test_bf16_writeback_on_stratified_bit_patterns():
    # With g = m = v = 0 Adam leaves theta unchanged (upd = lr*0/eps = 0), so
    # the bf16 output is the kernel's rounding of arbitrary fp32 patterns.
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000,
                     0x1234, 0xFEDC], dtype=np.uint32)
    rng = np.random.default_rng(0)
    bits = np.concatenate([(hi[:, None] | lows[None, :]).ravel(),
                           rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)])
    n = bits.size
    th = bits.view(np.float32)
    z = np.zeros(n, np.float32)
    dth, dg, dm, dv = to_dev(th), to_dev(z), to_dev(z), to_dev(z)
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    zr.zr_adam_partition(dg, dth, dm, dv, pb, **HP)
    got_th = host_f32(dth)
    # theta unchanged (NaNs stay NaN)
    nan = np.isnan(th)
    assert np.array_equal(got_th.view(np.uint32)[~nan], bits[~nan])
    assert np.isnan(got_th[nan]).all()
    assert np.array_equal(host_u16(pb), bf16_rne_oracle(got_th))


def test_bf16_writeback_on_every_fp32_pattern():
    """The same identity over all 2^32 fp32 bit patterns, drawn on the device
    in chunks: theta comes back unchanged bit for bit (NaNs stay NaN) and the
    bf16 output equals the oracle's rounding of the kernel's own theta."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 28
    z = torch.zeros(chunk, device="cuda")
    pb = torch.empty(chunk, dtype=torch.bfloat16, device="cuda")
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    piece = chunk // threads
    for c in range((1 << 32) // chunk):
        x = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda")
        x = torch.where(x >= (1 << 31), x - (1 << 32), x).to(torch.int32)
        th = x.view(torch.float32)
        del x
        zr.zr_adam_partition(z, th, z.clone(), z.clone(), pb, **HP)
        got_th = host_f32(th)
        got_pb = host_u16(pb)
        bits = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32)

        def check(i):
            a, b = i * piece, (i + 1) * piece
            gt = got_th[a:b]
            nan = np.isnan(gt)
            assert np.array_equal(np.isnan(bits[a:b].view(np.float32)), nan)
            assert np.array_equal(gt.view(np.uint32)[~nan], bits[a:b][~nan])
            assert np.array_equal(got_pb[a:b], bf16_rne_oracle(gt))

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(check, range(threads)))
        del th


def test_checkpoint_resume_is_bitwise():
    numels = [5000, 333, 12000]
    plan = zr.zr_plan_buckets(numels, [0] * 3, [(4, 1)], 7000)
    ref = plan_oracle(numels, [0] * 3, [(4, 1)], 7000)
    P = ref.groups[0].part_numel
    rng = np.random.default_rng(1)
    steps = [[to_dev((rng.standard_normal(ref.groups[0].total) * 1e-3).astype(np.float32))
              for _ in range(4)] for _ in range(2)]
    th0 = (rng.standard_normal(P) * 0.02).astype(np.float32)
    # two straight steps
    a = [to_dev(th0), torch.zeros(P, device="cuda"), torch.zeros(P, device="cuda")]
    for t, reps in enumerate(steps, 1):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 2, reps, *a, step=t, **HP)
    # step, save to host, reload into fresh buffers, step
    b = [to_dev(th0), torch.zeros(P, device="cuda"), torch.zeros(P, device="cuda")]
    zr.zr_reduce_scatter_adam(plan, 0, -1, 2, steps[0], *b, step=1, **HP)
    saved = [host_f32(x).copy() for x in b]
    del b
    c = [to_dev(x) for x in saved]
    zr.zr_reduce_scatter_adam(plan, 0, -1, 2, steps[1], *c, step=2, **HP)
    for x, y in zip(a, c):
        assert_bits_equal(host_f32(x), host_f32(y))


def test_empty_selections_are_noops():
    # group 1 has no slice in bucket 0 (the first param, all of bucket 0, is
    # in group 0); an IPG window that misses every param writes nothing.
    numels, pg = [100, 50], [0, 1]
    plan = zr.zr_plan_buckets(numels, pg, [(2, 1), (2, 1)], 100)
    reps = [to_dev(np.ones(50, np.float32)) for _ in range(2)]
    out = empty_f32(25, fill=7.0)
    zr.zr_reduce_scatter_local(plan, 1, 0, 0, reps, [out])
    m = empty_f32(25, fill=7.0)
    zr.zr_reduce_scatter_adam(plan, 1, 0, 0, reps, m, m, m)
    mg = empty_f32(10, fill=3.0)
    zr.zr_ipg_accumulate(plan, [0], [to_dev(np.ones(100, np.float32))], mg,
                         window_base=0, window_len=0)
    zr.zr_adam_partition(out, out, out, out, n=0)
    assert (host_f32(out) == 7.0).all() and (host_f32(m) == 7.0).all()
    assert (host_f32(mg) == 3.0).all()


@pytest.mark.parametrize("is_bf16", [False, True])
def test_bucket_size_invariance_on_gpu(is_bf16):
    numels = [1000, 1, 4099, 77, 2048]
    rng = np.random.default_rng(2)
    T = sum(numels)
    reps = [(rng.standard_normal(T) * 1e-2).astype(np.float32) for _ in range(4)]
    if is_bf16:
        reps = [torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                for x in reps]
    dreps = [to_dev(x) for x in reps]
    ref = plan_oracle(numels, [0] * 5, [(4, 2)], 1 << 40)
    want = reduce_scatter_oracle(ref, 0, reps, is_bf16)
    for B in (1, 7, 1000, 1 << 40):
        plan = zr.zr_plan_buckets(numels, [0] * 5, [(4, 2)], B)
        outs = [empty_f32(ref.groups[0].part_numel) for _ in range(4)]
        zr.zr_reduce_scatter_local(plan, 0, -1, -1, dreps, outs)
        for k in range(4):
            assert_bits_equal(host_f32(outs[k]), want[k], f"B={B} dst {k}")


def test_binding_rejects_strided_and_host_tensors():
    """A strided view or a host tensor never reaches the C call (the kernels
    would read it as dense device memory); outputs stay untouched."""
    plan = zr.zr_plan_buckets([1000], [0], [(2, 1)], 1 << 20)
    P = zr.zr_plan_group_info(plan, 0)[2]
    reps = [to_dev(np.ones(1000, np.float32)) for _ in range(2)]
    master = torch.zeros(P, device="cuda")
    m, v = torch.zeros(P, device="cuda"), torch.zeros(P, device="cuda")
    strided = torch.zeros(2 * P, device="cuda")[::2]
    with pytest.raises(zr.ZrError, match="contiguous"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, strided, m, v)
    with pytest.raises(zr.ZrError, match="device tensor"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, torch.zeros(P), m, v)
    with pytest.raises(zr.ZrError, match="replica 0 must be contiguous"):
        zr.zr_reduce_scatter_local(plan, 0, -1, 0,
                                   [torch.ones(2000, device="cuda")[::2], reps[1]], [master])
    torch.cuda.synchronize()
    assert not master.any() and not m.any() and not v.any()
