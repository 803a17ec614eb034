"""Planted mistakes in the oracle must be caught by its pins.

Each test builds a deliberately wrong variant of one oracle function (on the
CPU, never touching the HIP path) and checks that the same checks that pin
the real oracle reject it.  This is what gives the pins their value: a
plausible mistake anywhere (a dropped term, a wrong sign or index, a swapped
operand, a different summation order) fails at least one of them.
"""

import numpy as np
import pytest
import torch

from oracle import adam as adam_mod
from oracle import bf16 as bf16_mod
from oracle import plan as plan_mod
from oracle import reduce as reduce_mod
from oracle.ipg import widen_bf16
from zero_partition_aware_amd import workloads

F = np.float32


# ---------------------------------------------------------------- reduce

def _pins_for_mean(fn):
    """The reduce pins of tests/test_oracle_reduce.py, as a predicate."""
    vals = [np.array([v], F) for v in (2.0 ** 24, 1.0, 1.0, -(2.0 ** 24))]
    if fn(vals, 1)[0] != 0.0:
        return False
    rng = np.random.default_rng(5)
    for R, D in [(4, 4), (6, 6), (3, 1)]:
        xs = [rng.integers(-1000, 1000, size=64) * D for _ in range(R)]
        want = [float(sum(int(x[i]) // D for x in xs)) for i in range(64)]
        if fn([x.astype(F) for x in xs], D).tolist() != want:
            return False
    big = fn([np.array([3e38], F)] * 4, 4)
    if not (np.isfinite(big[0]) and big[0] == F(3e38)):
        return False
    z = fn([np.array([-0.0], F)] * 2, 2)
    return bool(np.signbit(z[0]))


def test_real_rank_order_mean_passes():
    assert _pins_for_mean(reduce_mod.rank_order_mean)


@pytest.mark.parametrize("mutant", ["reverse_order", "pairwise", "drop_last", "sum_first",
                                    "start_from_zero", "no_divide", "negate_one"])
def test_reduce_mutants_are_caught(mutant):
    def fn(values, divisor):
        d = F(divisor)
        vs = list(values)
        if mutant == "reverse_order":
            vs = vs[::-1]
        if mutant == "drop_last":
            vs = vs[:-1]
        if mutant == "pairwise":
            qs = [np.divide(x, d, dtype=F) for x in vs]
            while len(qs) > 1:
                qs = [np.add(qs[i], qs[i + 1], dtype=F) if i + 1 < len(qs) else qs[i]
                      for i in range(0, len(qs), 2)]
            return qs[0]
        if mutant == "sum_first":
            acc = vs[0].copy()
            with np.errstate(over="ignore"):
                for x in vs[1:]:
                    acc = np.add(acc, x, dtype=F)
            return np.divide(acc, d, dtype=F)
        acc = np.zeros_like(vs[0]) if mutant == "start_from_zero" else None
        for i, x in enumerate(vs):
            q = x if mutant == "no_divide" else np.divide(x, d, dtype=F)
            if mutant == "negate_one" and i == 1:
                q = -q
            acc = q if acc is None else np.add(acc, q, dtype=F)
        return acc
    assert not _pins_for_mean(fn)


# ------------------------------------------------------------------ plan

def _tiny_plan_pin(build):
    w = workloads.get("tiny")
    plan = build(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    got = [(s.bucket, s.dst, s.bucket_offset, s.flat_offset, s.part_offset, s.numel)
           for s in plan.slices]
    want = [(0, 0, 0, 0, 0, 570), (0, 1, 570, 570, 0, 430), (1, 1, 0, 1000, 430, 140),
            (1, 2, 140, 1140, 0, 570), (1, 3, 710, 1710, 0, 290), (2, 3, 0, 2000, 290, 278)]
    gso = [plan.grad_start_offset[1][k] for k in plan.param_to_partition_ids[1]]
    return got == want and gso == [0, 533, 1103, 1673]


def _mutated_plan(kind):
    def build(numels, param_groups, groups, B, align=1):
        plan = plan_mod.plan_oracle(numels, param_groups, groups, B, align)
        S = plan_mod.Slice
        if kind == "swap_offsets":
            plan.slices = [S(s.bucket, s.group, s.dst, s.flat_offset, s.bucket_offset,
                             s.part_offset, s.numel) for s in plan.slices]
        elif kind == "no_merge":
            # cut every slice at param borders (what skipping the merge gives)
            out = []
            starts = set(plan.param_offset)
            for s in plan.slices:
                cut = [f for f in sorted(starts) if s.flat_offset < f < s.flat_offset + s.numel]
                edges = [s.flat_offset] + cut + [s.flat_offset + s.numel]
                for a, b in zip(edges, edges[1:]):
                    out.append(S(s.bucket, s.group, s.dst, s.bucket_offset + a - s.flat_offset,
                                 a, s.part_offset + a - s.flat_offset, b - a))
            plan.slices = out
        elif kind == "gso_off_by_one":
            plan.grad_start_offset = [{k: v + (1 if v else 0) for k, v in d.items()}
                                      for d in plan.grad_start_offset]
        elif kind == "part_offset_from_bucket":
            plan.slices = [S(s.bucket, s.group, s.dst, s.bucket_offset, s.flat_offset,
                             s.bucket_offset, s.numel) for s in plan.slices]
        return plan
    return build


def test_real_plan_passes():
    assert _tiny_plan_pin(plan_mod.plan_oracle)


@pytest.mark.parametrize("kind", ["swap_offsets", "no_merge", "gso_off_by_one",
                                  "part_offset_from_bucket"])
def test_plan_mutants_are_caught(kind):
    assert not _tiny_plan_pin(_mutated_plan(kind))


# ------------------------------------------------------------------ adam

def _adam_pin(fn):
    """Two steps against torch.optim.Adam on the CPU (the library routine)."""
    n = 20000
    g1 = workloads.host_normal(1, n, 1e-3)
    g2 = workloads.host_normal(2, n, 1e-3)
    th0 = workloads.host_normal(3, n, 0.02)
    z = np.zeros(n, F)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    th1, m1, v1 = fn(g1, th0, z, z, step=1, **hp)
    th2, m2, v2 = fn(g2, th1, m1, v1, step=2, **hp)
    p = torch.nn.Parameter(torch.from_numpy(th0.copy()))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, foreach=False)
    for g in (g1, g2):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    ok = lambda a, b, atol: np.all(np.abs(np.float64(a) - np.float64(b)) <= atol + 1e-6 * np.abs(np.float64(b)))
    return (ok(th2, p.detach().numpy(), 1e-7) and ok(m2, st["exp_avg"].numpy(), 1e-7)
            and ok(v2, st["exp_avg_sq"].numpy(), 0.0))


def test_real_adam_passes():
    assert _adam_pin(adam_mod.adam_oracle)


@pytest.mark.parametrize("kind", ["eps_inside_sqrt", "no_bias_correction", "betas_swapped",
                                  "v_uses_g_not_g2", "sign_flip", "t_from_zero"])
def test_adam_mutants_are_caught(kind):
    def fn(grad, master, m, v, lr, beta1, beta2, eps, step):
        g = np.asarray(grad, np.float64)
        th = np.asarray(master, np.float64)
        b1, b2 = (beta2, beta1) if kind == "betas_swapped" else (beta1, beta2)
        t = step - 1 if kind == "t_from_zero" else step
        m1 = b1 * m + (1 - b1) * g
        v1 = b2 * v + (1 - b2) * (np.abs(g) if kind == "v_uses_g_not_g2" else g * g)
        if kind == "no_bias_correction":
            mh, vh = m1, v1
        else:
            mh = m1 / (1 - b1 ** t) if t > 0 else m1
            vh = v1 / (1 - b2 ** t) if t > 0 else v1
        den = np.sqrt(vh + eps) if kind == "eps_inside_sqrt" else np.sqrt(vh) + eps
        upd = lr * mh / den
        th1 = th + upd if kind == "sign_flip" else th - upd
        return th1.astype(F), m1.astype(F), v1.astype(F)
    assert not _adam_pin(fn)


# ------------------------------------------------------------------ bf16

def _bf16_pin(fn):
    cases = {1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82, 3.4028235e38: 0x7F80,
             -0.0: 0x8000}
    for v, want in cases.items():
        if fn(np.array([v], F))[0] != want:
            return False
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(F)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    return bool(np.array_equal(fn(x)[~nan], ref[~nan]))


def test_real_bf16_passes():
    assert _bf16_pin(bf16_mod.bf16_rne_oracle)


@pytest.mark.parametrize("kind", ["truncate", "ties_away", "ties_down"])
def test_bf16_mutants_are_caught(kind):
    def fn(x):
        b = np.ascontiguousarray(x, F).view(np.uint32).astype(np.uint64)
        if kind == "truncate":
            return (b >> 16).astype(np.uint16)
        if kind == "ties_away":
            return ((b + 0x8000) >> 16).astype(np.uint16)
        return ((b + 0x7FFF) >> 16).astype(np.uint16)
    assert not _bf16_pin(fn)


def test_widen_mutant_is_caught():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    wrong = (bits.astype(np.uint32) << 15).view(F)        # shifted one bit short
    assert not np.array_equal(np.nan_to_num(wrong), np.nan_to_num(ref))
    assert np.array_equal(np.nan_to_num(widen_bf16(bits)), np.nan_to_num(ref))
