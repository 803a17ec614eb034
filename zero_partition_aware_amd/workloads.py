"""Seeded synthetic workloads: parameter lists and random inputs.

This module is shared by the HIP path's tests/bench and by the oracle's
tests.  It holds only shapes, seeds and random-number draws, none of the
method's arithmetic (no plan, no reduction, no optimizer step).

Parameter lists use public architecture hyper-parameters only (no weights are
loaded; gradients are random stand-ins for backward gradients):

* ``tiny``      -- N=4, params [37], [64,33], [129]; fp32 grads; bucket 1000.
* ``gpt2-small``-- 12 layers, d=768, vocab 50257, 1024 positions, tied head;
  8 bf16 replicas; bucket 5e8.
* ``ring-1gib`` -- 8 ranks x 1 GiB fp32 (no parameter list).
* ``llama3-8b`` -- 32 layers, d=4096, ffn 14336, GQA with 8 KV heads of 128,
  vocab 128256, untied head; 8 replicas x 4 bf16 micro-batches; bucket 5e8.
* ``moe-16l``   -- 16 layers, d=2048: dense attention block reduced over 8
  replicas with sequence-parallel 2, and this rank's 2 of 8 experts
  (ffn 8192) reduced over an expert-data-parallel group of 2 with
  sequence-parallel 2; fp32 grads; bucket 5e6.

Seed scheme: replica r, micro-batch mu of workload c gets
``c*100000 + mu*1000 + r``; rank k's master weights get
``c*100000 + 99000 + k``.
"""

from dataclasses import dataclass

import numpy as np

WORKLOAD_IDS = {"tiny": 1, "gpt2-small": 2, "ring-1gib": 3, "llama3-8b": 4,
                "moe-16l": 5}


@dataclass
class Workload:
    name: str
    numels: list          # per param, list (ready) order
    shapes: list          # per param
    param_groups: list    # per param: group index
    groups: list          # (world, sp) per group
    reduce_bucket_size: int
    grad_dtype: str       # "fp32" or "bf16"
    grad_sigma: float
    master_sigma: float
    micro_batches: int    # 0: replicas hold reduced-ready grads directly


def _numel(shape):
    n = 1
    for d in shape:
        n *= d
    return n


def _tiny():
    shapes = [(37,), (64, 33), (129,)]
    return Workload("tiny", [_numel(s) for s in shapes], shapes, [0, 0, 0],
                    [(4, 1)], 1000, "fp32", 1.0, 0.02, 0)


def _gpt2_small():
    d, vocab, pos, layers = 768, 50257, 1024, 12
    shapes = [(vocab, d), (pos, d)]
    for _ in range(layers):
        shapes += [(d,), (d,), (d, 3 * d), (3 * d,), (d, d), (d,),
                   (d,), (d,), (d, 4 * d), (4 * d,), (4 * d, d), (d,)]
    shapes += [(d,), (d,)]
    return Workload("gpt2-small", [_numel(s) for s in shapes], shapes,
                    [0] * len(shapes), [(8, 1)], 500_000_000, "bf16", 1e-3,
                    0.02, 0)


def _llama3_8b():
    d, ffn, vocab, layers, kv = 4096, 14336, 128256, 32, 8 * 128
    shapes = [(vocab, d)]
    for _ in range(layers):
        shapes += [(d,), (d, d), (kv, d), (kv, d), (d, d), (d,),
                   (ffn, d), (ffn, d), (d, ffn)]
    shapes += [(d,), (vocab, d)]
    return Workload("llama3-8b", [_numel(s) for s in shapes], shapes,
                    [0] * len(shapes), [(8, 1)], 500_000_000, "bf16", 1e-4,
                    0.02, 4)


def _moe_16l():
    d, ffn, layers, experts_here = 2048, 8192, 16, 2
    shapes, groups_of = [], []
    for _ in range(layers):
        dense = [(d,), (d,), (3 * d, d), (3 * d,), (d, d), (d,), (d,), (d,),
                 (8, d)]
        shapes += dense
        groups_of += [0] * len(dense)
        for _e in range(experts_here):
            exp = [(ffn, d), (ffn,), (d, ffn), (d,)]
            shapes += exp
            groups_of += [1] * len(exp)
    return Workload("moe-16l", [_numel(s) for s in shapes], shapes, groups_of,
                    [(8, 2), (2, 2)], 5_000_000, "fp32", 1e-3, 0.02, 0)


def get(name):
    return {"tiny": _tiny, "gpt2-small": _gpt2_small,
            "llama3-8b": _llama3_8b, "moe-16l": _moe_16l}[name]()


RING_1GIB = {"ranks": 8, "elems_per_rank": (1 << 30) // 4, "sigma": 1.0}


def seed_for(name, replica=0, micro_batch=0, master=False):
    """Seed of replica ``replica``'s micro-batch ``micro_batch`` gradients, or
    (``master=True``) of rank ``replica``'s master weights."""
    c = WORKLOAD_IDS[name]
    if master:
        return c * 100000 + 99000 + replica
    return c * 100000 + micro_batch * 1000 + replica


# ---------------------------------------------------------------- host draws

def host_normal(seed, n, sigma):
    """float32 N(0, sigma) (sigma is the standard deviation)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n, dtype=np.float32) * np.float32(sigma))


def host_bf16_normal(seed, n, sigma):
    """bf16 N(0, sigma) as uint16 bit patterns (drawn in fp32, converted by
    torch's CPU conversion)."""
    import torch
    x = torch.from_numpy(host_normal(seed, n, sigma))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def host_int_valued(seed, n, lo, hi, multiple=1):
    """float32 integers uniformly in [lo, hi], multiples of ``multiple``."""
    rng = np.random.default_rng(seed)
    v = rng.integers(lo // multiple, hi // multiple + 1, size=n)
    return (v * multiple).astype(np.float32)


def host_special_values(seed, n):
    """A mix of +-0, subnormals, tiny normals, near-overflow values, +-inf,
    NaN and ordinary values, as float32."""
    rng = np.random.default_rng(seed)
    pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39, 1.2e-38,
                     -1.1754944e-38, 3e38, -3e38, 3.4028235e38, np.inf,
                     -np.inf, np.nan, 1.0, -2.5, 1e-3, 7e-8],
                    dtype=np.float32)
    pick = rng.integers(0, pool.shape[0], size=n)
    out = pool[pick].copy()
    normal = rng.random(n) < 0.3
    out[normal] = rng.standard_normal(int(normal.sum()), dtype=np.float32)
    return out


# -------------------------------------------------------------- device draws

def device_normal(seed, n, sigma, device, dtype="fp32", out=None):
    """N(0, sigma) drawn on the device with torch's generator; returns a
    torch tensor of float32 or bfloat16 (``dtype`` "fp32"/"bf16").  Large
    draws are made in chunks so that no fp32 temporary above 1 GiB exists."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty(n, dtype=tdt, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    chunk = 1 << 28
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        t = torch.randn(hi - lo, generator=gen, device=device,
                        dtype=torch.float32)
        t.mul_(sigma)
        out[lo:hi].copy_(t)
    return out
