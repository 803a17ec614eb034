"""Pins for oracle O6 (fp32 -> bf16 round to nearest even) against torch's
CPU conversion, a library routine: on a stratified sample of bit patterns and
on all 2^32 of them."""

import numpy as np
import torch

from oracle.bf16 import bf16_rne_oracle


def _torch_bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _compare(bits):
    x = bits.view(np.float32)
    mine = bf16_rne_oracle(x)
    ref = _torch_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(mine[~nan], ref[~nan])
    # NaN stays NaN, quiet, with sign and top payload kept.
    m = mine[nan].astype(np.uint32)
    assert ((m & 0x7F80) == 0x7F80).all() and ((m & 0x7F) != 0).all()
    assert ((m & 0x40) != 0).all()
    assert np.array_equal(m >> 15, (bits[nan] >> 31).astype(np.uint32))


def test_every_high_half_with_boundary_low_halves():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000,
                     0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    _compare(bits)


def test_random_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    _compare(bits)


def test_hand_cases():
    cases = {
        1.0: 0x3F80,
        # 1 + 2^-8 is exactly half way between 1 and 1 + 2^-7: tie to even (1).
        1.0 + 2.0 ** -8: 0x3F80,
        # 1 + 3*2^-8 is half way between 1+2^-7 (odd) and 1+2^-6: goes up.
        1.0 + 3 * 2.0 ** -8: 0x3F82,
        -0.0: 0x8000,
        3.4028235e38: 0x7F80,      # rounds past the largest bf16 -> inf
    }
    for v, want in cases.items():
        got = bf16_rne_oracle(np.array([v], np.float32))[0]
        assert got == want, (v, hex(got), hex(want))


def test_every_fp32_pattern():
    """All 2^32 fp32 bit patterns, in chunks on the host's cores (numpy and
    torch release the interpreter lock inside their loops): the oracle equals
    torch's conversion on every non-NaN value, and every NaN stays NaN with
    its sign and top payload bits."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 22

    def run(i):
        _compare(np.arange(i * chunk, (i + 1) * chunk, dtype=np.uint64).astype(np.uint32))

    threads = max(1, min(8, len(os.sched_getaffinity(0))))
    prev = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, range((1 << 32) // chunk)))
    finally:
        torch.set_num_threads(prev)
