"""Oracle O2: IPG / contiguous fp32 gradient-buffer accumulation.
TEST INFRASTRUCTURE ONLY.

[Megatron DP] "深入：朴素 DP 的 all-reduce" section, step 2: a backward hook adds
each param's grad into its view ``param.main_grad`` of one preallocated
contiguous fp32 buffer with ``add_`` (fp32 because repeated bf16 accumulation
loses precision); [ZeRO-RS blog §四]: each grad is copied into the contiguous
reduce bucket as soon as it is produced.

Per element: main_grad[f] = fl(main_grad[f] + widen(grad[f - o_p])), one fp32
add per micro-batch, in the order the calls are made.  ``widen`` turns a bf16
bit pattern into the fp32 number it denotes (exact: bf16 is the top half of
an fp32).  The caller zeroes main_grad at the start of a step.
"""

import numpy as np


def widen_bf16(bits_u16):
    """bf16 bit patterns (uint16) -> the float32 values they denote.

    A bf16 number is an fp32 number whose low 16 mantissa bits are zero, so
    its fp32 encoding is the bf16 pattern followed by 16 zero bits."""
    b = np.asarray(bits_u16, dtype=np.uint16).astype(np.uint32)
    return (b * np.uint32(65536)).view(np.float32)


def ipg_accumulate_oracle(main_grad, window_base, param_offsets, param_ids,
                          grads, grad_is_bf16):
    """Add each listed param's grad into the fp32 window ``main_grad`` that
    covers flat elements [window_base, window_base + len(main_grad)) of one
    group, clipping each param to the window.  Works in place; returns it.

    ``param_offsets[p]`` is o_p; ``grads[i]`` is param ``param_ids[i]``'s
    gradient (uint16 bf16 patterns if ``grad_is_bf16`` else float32)."""
    assert main_grad.dtype == np.float32
    wlen = main_grad.shape[0]
    for pid, g in zip(param_ids, grads):
        o = param_offsets[pid]
        vals = widen_bf16(g) if grad_is_bf16 else np.asarray(g, np.float32)
        n = vals.shape[0]
        lo = max(o, window_base)
        hi = min(o + n, window_base + wlen)
        if lo >= hi:
            continue
        dst = main_grad[lo - window_base: hi - window_base]
        src = vals[lo - o: hi - o]
        # one fp32 add per element, written back in place
        np.add(dst, src, out=dst, dtype=np.float32)
    return main_grad
