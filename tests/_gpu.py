"""Helpers shared by the GPU parity tests (device placement and comparison).
No method arithmetic lives here."""

import numpy as np
import torch

DEV = "cuda"


def to_dev(arr, offset_elems=0):
    """numpy float32 or uint16 (bf16 patterns) -> device tensor, placed
    ``offset_elems`` elements into a larger allocation (to exercise
    misaligned pointers)."""
    if arr.dtype == np.uint16:
        host = torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)
    else:
        host = torch.from_numpy(np.ascontiguousarray(arr, np.float32))
    buf = torch.empty(host.numel() + offset_elems + 8, dtype=host.dtype, device=DEV)
    view = buf[offset_elems: offset_elems + host.numel()]
    view.copy_(host)
    return view


def empty_f32(n, offset_elems=0, fill=float("nan")):
    buf = torch.full((n + offset_elems + 8,), fill, dtype=torch.float32, device=DEV)
    return buf[offset_elems: offset_elems + n]


def host_f32(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()


def host_u16(t):
    torch.cuda.synchronize()
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def assert_bits_equal(got, want, what=""):
    """Bit-exact fp32 comparison; NaNs must sit at the same places."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    diff = (got.view(np.uint32) != want.view(np.uint32)) & ~gn
    if diff.any():
        i = int(np.flatnonzero(diff)[0])
        raise AssertionError(f"{what}: {int(diff.sum())} of {got.size} elements differ; "
                             f"first at {i}: got {got[i]!r} want {want[i]!r}")


def assert_within(got, want, rtol=1e-6, atol=1e-7, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    ok = np.abs(got - want) <= atol + rtol * np.abs(want)
    ok |= gn | (np.isinf(got) & (got == want))
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {got.size} out of tolerance; "
                             f"first at {i}: got {got[i]!r} want {want[i]!r}")


def max_ulp(got, want):
    g = np.asarray(got, np.float32).view(np.int32).astype(np.int64)
    w = np.asarray(want, np.float32).view(np.int32).astype(np.int64)
    fin = np.isfinite(np.asarray(want, np.float32))
    return int(np.abs(g - w)[fin].max()) if fin.any() else 0
