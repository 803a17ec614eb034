"""Oracle for the parameter all-gather after the partition update.
TEST INFRASTRUCTURE ONLY.

[Megatron DP] "通信模式" section: after each card has updated its own 1/DP
slice with its fp32 master, an all-gather stitches the updated parameters
back into complete weights for the next forward.  [Collectives Q&A]
"三种集合通信原语", AllGather: each GPU holds one segment; afterwards every GPU
holds the whole data.

Definition used: the full flat vector of a group is the concatenation of its
R_g partitions in rank order, truncated to the T_g real elements (the padding
at the end of the last partition is not a parameter).
"""

import numpy as np


def all_gather_oracle(parts, total):
    """parts: list of R equal-length arrays (partition k at index k);
    returns the first ``total`` elements of their concatenation."""
    full = np.concatenate([np.asarray(p) for p in parts])
    assert total <= full.shape[0]
    return full[:total].copy()


def all_gather_window_oracle(parts, total, base, length):
    """Elements [base, base + length) of the gathered vector, clipped to the
    real elements (a shorter result when the window runs into padding)."""
    full = all_gather_oracle(parts, total)
    return full[base:min(base + length, total)].copy()
