"""Oracle O7: literal ring reduce-scatter (and all-gather) message passing.
TEST INFRASTRUCTURE ONLY.

[Megatron DP] "深入：all-reduce 底层算法（NCCL）" section, Ring All-Reduce: N
cards form a ring, the vector is cut into N chunks; in the reduce-scatter
phase every step passes one partial chunk to the next card, which adds its
own copy; after N-1 steps card k holds the complete sum of chunk k.  The
all-gather phase passes completed chunks around once more.  Per-card traffic
is 2(N-1)/N of the vector for the whole all-reduce ([Megatron DP], same
section; [Collectives Q&A] "三种集合通信原语").

Schedule used (the reading that makes card k own chunk k): in step s
(0 <= s <= N-2) card k sends its partial chunk (k - s - 1) mod N to card
k + 1, which sets chunk[c] = fl(chunk[c] + received).  So chunk k is summed in
ring order k+1, k+2, ..., k (mod N).  Messages are copies taken before the
receiver adds, exactly as if they crossed a wire.
"""

import numpy as np


def ring_reduce_scatter_oracle(bufs, steps=None):
    """``bufs``: list of N float32 arrays (one per card), each of N equal
    chunks.  Returns (new buffers, elements sent per card).  ``steps`` limits
    the number of steps run (default N-1, the whole reduce-scatter)."""
    N = len(bufs)
    M = bufs[0].shape[0]
    assert M % N == 0
    C = M // N
    cur = [np.array(b, dtype=np.float32, copy=True) for b in bufs]
    sent = [0] * N
    nsteps = N - 1 if steps is None else steps
    for s in range(nsteps):
        messages = []
        for k in range(N):
            c = (k - s - 1) % N
            messages.append((k, (k + 1) % N, c,
                             cur[k][c * C:(c + 1) * C].copy()))
            sent[k] += C
        for _, dst, c, payload in messages:
            seg = cur[dst][c * C:(c + 1) * C]
            np.add(seg, payload, out=seg, dtype=np.float32)
    return cur, sent


def ring_all_gather_oracle(bufs):
    """Second ring phase: card k starts owning chunk k; after N-1 steps every
    card holds every chunk.  Returns (new buffers, elements sent per card)."""
    N = len(bufs)
    C = bufs[0].shape[0] // N
    cur = [np.array(b, dtype=np.float32, copy=True) for b in bufs]
    sent = [0] * N
    for s in range(N - 1):
        messages = []
        for k in range(N):
            c = (k - s) % N
            messages.append(((k + 1) % N, c, cur[k][c * C:(c + 1) * C].copy()))
            sent[k] += C
        for dst, c, payload in messages:
            cur[dst][c * C:(c + 1) * C] = payload
    return cur, sent


def ring_order_sum(bufs, k):
    """Chunk k summed in the ring's own order k+1, ..., k (mod N), one fp32
    add at a time: what card k must hold after the reduce-scatter."""
    N = len(bufs)
    C = bufs[0].shape[0] // N
    chunk = lambda r: np.asarray(bufs[r][k * C:(k + 1) * C], np.float32)
    acc = chunk((k + 1) % N).copy()
    for i in range(2, N + 1):
        acc = np.add(acc, chunk((k + i) % N), dtype=np.float32)
    return acc
