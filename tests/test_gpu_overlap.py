"""The overlapped bucketed schedule ([ZeRO-RS blog] §四: each IPG bucket is
reduced as soon as it is full while the backward continues; [Megatron DP]
"梯度缓冲区+分桶+overlap"): stream A runs the IPG fills of every replica in
ready order; as soon as every param feeding a bucket has been accumulated
(zr_plan_param_buckets says which buckets a param feeds), an event recorded
on A orders stream B's fused reduce-scatter + Adam of the buckets completed
since the last trigger (one range call).  The result must equal, bit for
bit, the same calls made in the same order on one stream, and the oracle
chain (IPG fills, partition reduce-scatter, Adam) element by element."""

import numpy as np
import pytest

from oracle.adam import adam_oracle
from oracle.bf16 import bf16_rne_oracle
from oracle.ipg import ipg_accumulate_oracle
from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests._lib import load

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import assert_bits_equal, assert_within, host_f32, host_u16  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
DEV = "cuda"


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _schedule(plan, numels, R, k, grads, mgs, state, mb, stream_a, stream_b):
    """IPG fills on stream_a, triggered range calls on stream_b (streams may
    be the same).  grads[mu][r][p]: device bf16 gradient of param p."""
    nb = zr.zr_plan_num_buckets(plan)
    feeds = [zr.zr_plan_param_buckets(plan, p) for p in range(len(numels))]
    remaining = [0] * nb
    for a, b in feeds:
        for bk in range(a, b + 1):
            remaining[bk] += 1
    done = 0
    for mu in range(mb):
        for p in range(len(numels)):
            for r in range(R):
                zr.zr_ipg_accumulate(plan, [p], [grads[mu][r][p]], mgs[r], stream=stream_a)
            if mu < mb - 1:
                continue
            a, b = feeds[p]
            for bk in range(a, b + 1):
                remaining[bk] -= 1
            full = done
            while full < nb and remaining[full] == 0:
                full += 1
            if full > done:
                if stream_b is not stream_a:
                    ev = torch.cuda.Event()
                    ev.record(stream_a)
                    stream_b.wait_event(ev)
                zr.zr_reduce_scatter_adam_range(plan, 0, done, full - done, k, mgs, *state,
                                                step=1, stream=stream_b, **HP)
                done = full
    assert done == nb
    if stream_b is not stream_a:
        stream_a.wait_stream(stream_b)


@pytest.mark.parametrize("k", [0, 3])
def test_overlapped_schedule_matches_serial_and_oracle(k):
    rng = np.random.default_rng(10 + k)
    numels = [31, 70000, 5, 12345, 40000, 1, 25000, 64, 33333, 7, 60001, 999]
    R, B, mb = 4, 20000, 2
    ref = plan_oracle(numels, [0] * len(numels), [(R, 1)], B)
    plan = zr.zr_plan_buckets(numels, [0] * len(numels), [(R, 1)], B)
    info = ref.groups[0]
    T, P = info.total, info.part_numel
    assert ref.num_buckets >= 8
    host_g = [[[_bf16((rng.standard_normal(n) * 1e-2).astype(np.float32)) for n in numels]
               for _ in range(R)] for _ in range(mb)]
    dev_g = [[[torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV) for x in per_r]
              for per_r in per_mu] for per_mu in host_g]
    th0 = (rng.standard_normal(P) * 0.02).astype(np.float32)
    th0[max(0, T - k * P):] = 0.0                    # padding of the last partition
    results = []
    for overlapped in (True, False):
        mgs = [torch.zeros(T, device=DEV) for _ in range(R)]
        state = [torch.from_numpy(th0.copy()).to(DEV), torch.zeros(P, device=DEV),
                 torch.zeros(P, device=DEV), torch.zeros(P, dtype=torch.bfloat16, device=DEV),
                 torch.full((P,), float("nan"), device=DEV)]
        torch.cuda.synchronize()
        sa = torch.cuda.Stream()
        sb = torch.cuda.Stream() if overlapped else sa
        _schedule(plan, numels, R, k, dev_g, mgs, state, mb, sa, sb)
        torch.cuda.synchronize()
        results.append([host_f32(t) for t in (state[0], state[1], state[2], state[4])] +
                       [host_u16(state[3])])
        del mgs, state
    ovl, ser = results
    for name, x, y in zip(("master", "m", "v", "reduced gradient"), ovl[:4], ser[:4]):
        assert_bits_equal(x, y, f"overlapped vs serial: {name}")
    assert np.array_equal(ovl[4], ser[4]), "overlapped vs serial: bf16 param"
    # the oracle chain
    offs = [ref.param_offset[p] for p in range(len(numels))]
    mg = []
    for r in range(R):
        acc = np.zeros(T, np.float32)
        for mu in range(mb):
            ipg_accumulate_oracle(acc, 0, offs, list(range(len(numels))), host_g[mu][r], True)
        mg.append(acc)
    g = reduce_scatter_oracle(ref, 0, mg, False, dst=k)[k]
    assert_bits_equal(ovl[3], g, "reduced gradient vs oracle")
    z = np.zeros(P, np.float32)
    w_th, w_m, w_v = adam_oracle(g, th0, z, z, step=1, **HP)
    assert_within(ovl[0], w_th, what="master vs oracle")
    assert_within(ovl[1], w_m, what="m vs oracle")
    assert_within(ovl[2], w_v, atol=0.0, what="v vs oracle")
    assert np.array_equal(ovl[4], bf16_rne_oracle(ovl[0])), "bf16 param vs RNE of master"
