"""Pins for oracle O5 (Adam on the fp32 partition)."""

import numpy as np
import pytest
import torch

from oracle.adam import adam_oracle, adam_oracle_f64, bias_corrections
from zero_partition_aware_amd import workloads

F = np.float32
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def within(got, want, rtol=1e-6, atol=1e-7):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return np.all(np.abs(got - want) <= atol + rtol * np.abs(want))


def _torch_adam(grads, master, lr, beta1, beta2, eps):
    p = torch.nn.Parameter(torch.from_numpy(master.copy()))
    opt = torch.optim.Adam([p], lr=lr, betas=(beta1, beta2), eps=eps,
                           foreach=False, fused=False)
    for g in grads:
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("sigma", [1.0, 1e-3, 1e-4])
def test_two_steps_match_torch_adam(sigma):
    n = 50_000
    g1 = workloads.host_normal(1, n, sigma)
    g2 = workloads.host_normal(2, n, sigma)
    th0 = workloads.host_normal(3, n, 0.02)
    z = np.zeros(n, F)
    th1, m1, v1 = adam_oracle(g1, th0, z, z, step=1, **HP)
    th2, m2, v2 = adam_oracle(g2, th1, m1, v1, step=2, **HP)
    tth, tm, tv = _torch_adam([g1, g2], th0, **HP)
    assert within(th2, tth)
    assert within(m2, tm)
    # v ~ sigma^2 can be far below the absolute term; compare relatively.
    assert within(v2, tv, atol=0.0, rtol=1e-6)


def test_step1_closed_form():
    # From m = v = 0: mh = g, vh = g^2, so theta' = theta - lr*g/(|g| + eps).
    n = 10_000
    g = workloads.host_normal(4, n, 1.0)
    th = workloads.host_normal(5, n, 0.02)
    z = np.zeros(n, F)
    th1, m1, v1 = adam_oracle(g, th, z, z, step=1, **HP)
    g64 = g.astype(np.float64)
    want = th.astype(np.float64) - 1e-3 * g64 / (np.abs(g64) + 1e-8)
    assert within(th1, want)
    assert within(m1, 0.1 * g64, rtol=1e-6, atol=0)


def test_zero_gradient_leaves_everything_unchanged():
    th = workloads.host_normal(6, 100, 0.02)
    z = np.zeros(100, F)
    for step in (1, 2, 50):
        th1, m1, v1 = adam_oracle(z, th, z, z, step=step, **HP)
        assert np.array_equal(th1, th) and not m1.any() and not v1.any()
    # padding: theta = m = v = g = 0 stays 0
    th1, m1, v1 = adam_oracle(z, z, z, z, step=3, **HP)
    assert not th1.any()


def test_fp64_twin_within_tolerance():
    n = 20_000
    rng = np.random.default_rng(9)
    g = workloads.host_normal(7, n, 1e-3)
    th = workloads.host_normal(8, n, 0.02)
    m = (rng.standard_normal(n) * 1e-4).astype(F)
    v = (np.abs(rng.standard_normal(n)) * 1e-7).astype(F)
    a = adam_oracle(g, th, m, v, step=7, **HP)
    b = adam_oracle_f64(g, th, m, v, step=7, **HP)
    assert within(a[0], b[0])
    # m' = b1*m + (1-b1)*g may cancel: bound the error by the terms' size
    # (a few fp32 roundings of each term, 4u with u = 2^-24).
    terms = 0.9 * np.abs(m.astype(np.float64)) + 0.1 * np.abs(g.astype(np.float64))
    assert np.all(np.abs(a[1] - b[1]) <= 4 * 2.0 ** -24 * terms)
    # v' is a sum of non-negative terms: plain relative error.
    assert within(a[2], b[2], atol=0)


def test_constants_rounded_once_from_float64():
    bc1, bc2 = bias_corrections(0.9, 0.999, 1)
    assert bc1 == F(0.1) and bc2 == F(0.001)
    bc1, _ = bias_corrections(0.9, 0.999, 3)
    assert bc1 == F(1.0 - 0.9 ** 3) == F(0.271)
