"""The bench's same-run parity check, driven on the CPU with a stand-in for
the device call (the oracle writing the state), must pass on correct state
and fail on each planted mistake: a wrong master, m or v value at a sampled
offset, a wrong bf16 param, a wrong reduced gradient in the extra call, or a
logged Adam step that was not applied."""

import importlib.util
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.adam import adam_oracle  # noqa: E402
from oracle.bf16 import bf16_rne_oracle  # noqa: E402
from oracle.reduce import rank_order_mean  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

P, R, D = 6000, 4, 4.0


def _setup(monkeypatch, seed):
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    rng = np.random.default_rng(seed)
    xs_full = [(rng.standard_normal(P) * 1e-3).astype(np.float32) for _ in range(R)]
    g_full = rank_order_mean(xs_full, D)
    th = (rng.standard_normal(P) * 0.02).astype(np.float32)
    state = {"master": torch.from_numpy(th.copy()), "m": torch.zeros(P), "v": torch.zeros(P),
             "pbf16": torch.zeros(P, dtype=torch.bfloat16)}
    bench.track_state(torch, state, bench.sample_indices(P, seed, edges=[1000, 4000]))

    def apply(t, gout=None, bad_g=False):
        th_, m_, v_ = adam_oracle(g_full, state["master"].numpy(), state["m"].numpy(),
                                  state["v"].numpy(), step=t, **bench.HP)
        state["master"].copy_(torch.from_numpy(th_))
        state["m"].copy_(torch.from_numpy(m_))
        state["v"].copy_(torch.from_numpy(v_))
        pb = bf16_rne_oracle(th_).view(np.int16)
        state["pbf16"].copy_(torch.from_numpy(pb.copy()).view(torch.bfloat16))
        if gout is not None:
            g = g_full.copy()
            if bad_g:
                g[state["idx"][3]] = np.nextafter(g[state["idx"][3]], np.float32(1))
            gout.copy_(torch.from_numpy(g))

    for t in (1, 2):                      # the "timed" steps
        state["steps"].append(t)
        apply(t)
    xs = [x[state["idx"]] for x in xs_full]
    return state, xs, apply


def _check(state, xs, apply, bad_g=False):
    return bench.check_state(torch, state, xs, False, D,
                             lambda gout, t: apply(t, gout, bad_g))


def test_correct_state_passes(monkeypatch):
    state, xs, apply = _setup(monkeypatch, 1)
    res = _check(state, xs, apply)
    assert res["ok"] and res["reduced_gradient_bit_exact"], res


@pytest.mark.parametrize("what", ["master", "m", "v", "pbf16", "grad", "step"])
def test_planted_mistakes_fail(monkeypatch, what):
    state, xs, apply = _setup(monkeypatch, 2)
    j = int(state["idx"][len(state["idx"]) // 2])
    if what in ("master", "m", "v"):
        state[what][j] = state[what][j] * 1.001 + 1e-6
    elif what == "pbf16":
        pb = state["pbf16"].view(torch.int16)
        pb[j] = pb[j] + 1
    elif what == "step":
        state["steps"].append(3)          # logged but never applied
    res = _check(state, xs, apply, bad_g=(what == "grad"))
    assert not res["ok"], (what, res)
